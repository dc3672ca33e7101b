"""mk_prefill_batched_noalloc (the batched prefill in the library's fixed per-device
scratch array) against mk_prefill_batched (scratch the handle allocates), through the
C ABI: two handles built from the same weights take the same calls, and every result
must agree bit for bit, since both run the same kernels on the same inputs:

* a first call of 70 positions (chunks of 64 and a ragged 6), then a second, smaller
  call of 23 positions that continues behind it, so the second call finds the first
  one's words in the array;
* the first ids, the hidden states of every prompt position after every layer, the
  positions, and four greedy decode steps after the two calls (which read every cache
  entry the calls wrote);
* a call on a new handle after the others are destroyed (the array outlives them).

Every shape with a built kernel body fits the array (the hidden-2048 body needs about
41 MiB of its 48), so MK_ERR_SCRATCH, the refusal of a larger shape, has no case here.
"""
import numpy as np
import pytest

from persistent_megakernel_loop_amd import workload as wl
from tests.parity import make_inputs

pytestmark = pytest.mark.gpu


def _calls(dec, shape, inp, noalloc):
    import torch

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    L, H = shape.n_layers, shape.hidden
    firsts, hidden = [], []
    for a, b in ((0, 70), (70, 93)):
        ids, rows, pos3 = t(inp.prompt_ids[a:b]), t(inp.prompt_rows[a:b]), t(inp.prompt_pos3[a:b])
        hid = torch.zeros((b - a, L + 1, H), dtype=torch.float32, device="cuda")
        out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        dec.set_debug(hid, None)
        if noalloc:
            dec.prefill_batched_noalloc(ids, out, rows, pos3)
        else:
            dec.prefill(ids, rows, pos3, out=out, batched=True)
        torch.cuda.synchronize()
        dec.set_debug(None, None)
        dec.check()
        firsts.append(int(out.cpu()[0]))
        hidden.append(hid.cpu().numpy())
    pos = dec.position
    steps = dec.decode(4)
    torch.cuda.synchronize()
    dec.check()
    return firsts, hidden, pos, steps.cpu().numpy()


def test_noalloc_matches_allocating_prefill():
    from persistent_megakernel_loop_amd.binding import Decoder, weights_to_device

    shape = wl.TALKER_0P6B.replace(name="talker-2l-noalloc", n_layers=2, prompt_len=93, steps=4)
    print(f"[case] {shape.name}: mk_prefill_batched_noalloc vs mk_prefill_batched, calls of 70 then 23",
          flush=True)
    inp = make_inputs(shape)
    dw = weights_to_device(wl.make_weights(shape))
    ref_dec, dec = Decoder(shape, dw), Decoder(shape, dw)
    ref = _calls(ref_dec, shape, inp, noalloc=False)
    got = _calls(dec, shape, inp, noalloc=True)
    ref_dec.close()
    dec.close()
    assert got[0] == ref[0]
    for g, r in zip(got[1], ref[1]):
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32))
    assert got[2] == ref[2] == 93
    assert np.array_equal(got[3], ref[3])
    # the array outlives the handles: a new handle's call still matches
    print(f"[case] {shape.name}: new handle after destroy", flush=True)
    again = Decoder(shape, dw)
    got2 = _calls(again, shape, inp, noalloc=True)
    again.close()
    assert got2[0] == ref[0] and np.array_equal(got2[3], ref[3])
    for g, r in zip(got2[1], ref[1]):
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32))

