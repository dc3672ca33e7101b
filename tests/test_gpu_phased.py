"""The launch-per-phase decode (mk_decode_phased): the persistent kernel's phase bodies,
one kernel launch per phase, must give the persistent kernel's results bit for bit (ids,
every layer's hidden state, and the cache entries, which the decode steps after it read),
and through it the oracle's.  Cases: the talker (rows, three rotary streams) and the
text model (greedy feedback), two layers and all 28, and a body with no phased form
refused."""
import numpy as np
import pytest

from persistent_megakernel_loop_amd import workload as wl
from tests.parity import compare, make_inputs, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

MK_ERR_UNSUPPORTED = -2


def _case(shape, oracle=False):
    import torch
    from persistent_megakernel_loop_amd.binding import Decoder, weights_to_device

    print(f"[case] {shape.name}: phased decode of {shape.steps} steps against the persistent kernel", flush=True)
    weights = wl.make_weights(shape)
    dw = weights_to_device(weights)
    inp = make_inputs(shape)
    a, b = Decoder(shape.replace(max_seq=shape.capacity + 4), dw), Decoder(shape.replace(max_seq=shape.capacity + 4), dw)
    ref = run_gpu(shape, dw, inp, dec=a)
    got = run_gpu(shape, dw, inp, dec=b, phased=True)
    assert got.first_id == ref.first_id
    assert np.array_equal(got.ids, ref.ids)
    assert np.array_equal(got.hidden.view(np.uint32), ref.hidden.view(np.uint32))
    # four more persistent steps on each handle read every cache entry the two wrote
    nxt = []
    for d in (a, b):
        o = d.decode(4)
        torch.cuda.synchronize()
        d.check()
        nxt.append(o.cpu().numpy())
        d.close()
    assert np.array_equal(nxt[0], nxt[1])
    if oracle:
        summary = compare(got, run_oracle(shape, weights, inp, got))
        print(f"[case] {shape.name}: phased against the oracle {summary}", flush=True)


def test_talker_two_layers():
    _case(wl.TALKER_0P6B.replace(name="talker-2l-phased", n_layers=2, steps=12))


def test_text_two_layers_feedback():
    _case(wl.TEXT_0P6B.replace(name="q06-2l-v1000-phased", n_layers=2, vocab=1000, steps=12))


def test_full_talker_0p6b():
    _case(wl.TALKER_0P6B.replace(name="talker-0.6b-phased", steps=8), oracle=True)


def test_other_bodies_refused():
    import torch
    from persistent_megakernel_loop_amd.binding import Decoder, MkError, weights_to_device

    print("[case] tiny-f32: phased decode refused", flush=True)
    shape = wl.TINY
    dec = Decoder(shape, weights_to_device(wl.make_weights(shape)))
    dec.prefill(torch.from_numpy(wl.make_prompt_ids(shape)).cuda())
    with pytest.raises(MkError) as e:
        dec.decode_phased(4)
    assert e.value.code == MK_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    dec.close()
