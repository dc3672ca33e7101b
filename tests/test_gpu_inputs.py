"""GPU tests of the input side and the host-visible state of the C ABI.

* mk_embed_sum (the 17-row talker input sum on the device) is bit-exact against
  the oracle's float32 sum, at the talker's real table sizes and on a ragged f32
  case with ids outside their tables;
* progress, position and status after prefill/decode calls.
"""
import numpy as np
import pytest

from oracle import embed_sum17
from persistent_megakernel_loop_amd import workload as wl

pytestmark = pytest.mark.gpu


def test_embed_sum_talker_tables_bit_exact():
    import torch
    from persistent_megakernel_loop_amd.binding import embed_sum, to_device

    print("[case] embed_sum talker tables hidden 1024, 96 positions", flush=True)
    tables = wl.make_talker_tables(1024)
    ids = wl.make_talker_ids(96)
    rows = embed_sum(to_device(tables["codebooks"]), to_device(tables["text"]), torch.from_numpy(ids).cuda())
    got = rows.cpu().numpy()
    want = np.stack([embed_sum17(tables["codebooks"], tables["text"], t) for t in ids])
    assert got.dtype == np.float32 and got.shape == want.shape
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_embed_sum_f32_ragged_with_bad_ids():
    import torch
    from persistent_megakernel_loop_amd.binding import embed_sum

    print("[case] embed_sum f32 n_cb=3 hidden 320 with bad ids", flush=True)
    rng = np.random.default_rng(7)
    n_cb, cb_size, text_vocab, hidden, n = 3, 50, 70, 320, 9
    cb = rng.standard_normal((n_cb, cb_size, hidden)).astype(np.float32)
    tx = rng.standard_normal((text_vocab, hidden)).astype(np.float32)
    ids = np.concatenate([rng.integers(0, cb_size, (n, n_cb)), rng.integers(0, text_vocab, (n, 1))], 1).astype(np.int32)
    ids[2, 1] = cb_size       # past its codebook
    ids[5, 0] = -3            # negative
    ids[7, n_cb] = text_vocab  # past the text table
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows = embed_sum(torch.from_numpy(cb).cuda(), torch.from_numpy(tx).cuda(), torch.from_numpy(ids).cuda(), bad=bad)
    # documented rule: an id outside its table reads row 0 of that table and is counted
    fixed = ids.copy()
    fixed[2, 1] = fixed[5, 0] = fixed[7, n_cb] = 0
    want = np.stack([embed_sum17(cb, tx, t) for t in fixed])
    assert np.array_equal(rows.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert int(bad.cpu()[0]) == 3


def test_embed_sum_empty_is_a_no_op():
    import torch
    from persistent_megakernel_loop_amd.binding import embed_sum

    cb = torch.zeros((2, 4, 64), dtype=torch.float32, device="cuda")
    tx = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    ids = torch.zeros((0, 3), dtype=torch.int32, device="cuda")
    rows = torch.full((1, 64), 5.0, device="cuda")
    embed_sum(cb, tx, ids, rows=rows)
    torch.cuda.synchronize()
    assert float(rows[0, 0].cpu()) == 5.0


def test_progress_position_status():
    import torch
    from persistent_megakernel_loop_amd.binding import Decoder, MkError, weights_to_device

    print("[case] progress/position/status on tiny-f32", flush=True)
    shape = wl.TINY
    dec = Decoder(shape, weights_to_device(wl.make_weights(shape)))
    ids = torch.from_numpy(wl.make_prompt_ids(shape)).cuda()
    assert dec.position == 0
    with pytest.raises(MkError):  # feedback decode with no previous id
        dec.decode(4)
    first = dec.prefill(ids)
    torch.cuda.synchronize()
    assert dec.progress() == 1 and dec.position == len(ids)
    out = dec.decode(7)
    torch.cuda.synchronize()
    assert dec.progress() == 7 and dec.position == len(ids) + 7
    dec.check()
    # feedback continues across calls: one launch of 7+5 equals 7 then 5
    more = dec.decode(5)
    torch.cuda.synchronize()
    dec.reset()
    dec.prefill(ids)
    both = dec.decode(12)
    torch.cuda.synchronize()
    dec.check()
    assert np.array_equal(np.concatenate([out.cpu().numpy(), more.cpu().numpy()]), both.cpu().numpy())
    assert int(first.cpu()[0]) >= 0
    # capacity: position + n beyond max_seq is refused on the host
    with pytest.raises(MkError):
        dec.decode(shape.capacity)
    dec.close()
