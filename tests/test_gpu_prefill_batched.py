"""GPU parity of the batched prompt prefill (mk_prefill_batched) through the C ABI.

* the matrix-core product it is built on, against a float64 product on the CPU, over
  shapes that span one and several K runs, 1..64 positions and ragged position tiles;
* whole prompts against the oracle: the talker (row inputs, multi-section rotary
  streams) and the text model (id inputs) on the hidden-1024 body, the hidden-2048
  body, prompts over one and several 64-position chunks, behind a pre-filled cache;
* against the position-by-position prefill on the same handle: same first id (unless
  the oracle's top two logits are within rounding of each other), hidden states and
  the following decode steps within the parity tolerance;
* the smallest prompt (one position), the full text vocabulary in the first id's LM
  head, the progress word and greedy feedback after the call, and a float32-weight
  handle refused with MK_ERR_UNSUPPORTED.
"""
import numpy as np
import pytest

from persistent_megakernel_loop_amd import workload as wl
from tests.parity import HIDDEN_RTOL, compare, make_inputs, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

MK_ERR_UNSUPPORTED = -2


@pytest.mark.parametrize("rows,k,n", [(32, 64, 1), (64, 256, 16), (96, 512, 17), (4096, 1024, 31),
                                      (1024, 3072, 64), (2048, 6144, 33)])
def test_product_against_float64(rows, k, n):
    import torch
    from persistent_megakernel_loop_amd.binding import selftest_gemm

    print(f"[case] product rows={rows} k={k} n={n}", flush=True)
    g = torch.Generator().manual_seed(rows * 7 + k + n)
    w = (torch.randn(rows, k, generator=g) * 0.05).to(torch.bfloat16)
    x = torch.randn(n, k, generator=g) * 3.0
    y = selftest_gemm(w.cuda(), x.cuda()).cpu().double()
    ref = x.double() @ w.double().T
    # each activation keeps ~17 significant bits after the hi/lo split; the sums run in
    # float32 over k terms
    scale = x.double().abs() @ w.double().abs().T
    err = (y - ref).abs() / scale.clamp_min(1e-30)
    assert float(err.max()) < 2e-5, f"max error {float(err.max()):.3e} (in units of sum |x||w|)"


def _case(shape, prompt_len=None, kv_prefill=None, n_steps=None):
    from persistent_megakernel_loop_amd.binding import weights_to_device

    print(f"[case] {shape.name} batched prefill: prompt={prompt_len or shape.prompt_len} "
          f"kv={kv_prefill if kv_prefill is not None else shape.kv_prefill}", flush=True)
    weights = wl.make_weights(shape)
    inp = make_inputs(shape, n_steps=n_steps, prompt_len=prompt_len, kv_prefill=kv_prefill)
    dw = weights_to_device(weights)
    gpu = run_gpu(shape, dw, inp, batched=True)
    ref = run_gpu(shape, dw, inp, batched=False)
    del dw
    orc = run_oracle(shape, weights, inp, gpu)
    summary = compare(gpu, orc)
    P = len(inp.prompt_ids)
    g, r = gpu.hidden[:P].astype(np.float64), ref.hidden[:P].astype(np.float64)
    rel = np.linalg.norm(g - r, axis=-1) / np.maximum(np.linalg.norm(r, axis=-1), 1e-30)
    summary["max_rel_l2_vs_per_position"] = float(rel.max())
    print(f"[case] {shape.name}: {summary}", flush=True)
    assert rel.max() <= HIDDEN_RTOL
    return gpu, ref, orc


def test_talker_two_layers_prompt32():
    shape = wl.TALKER_0P6B.replace(name="talker-2l-pb", n_layers=2, prompt_len=32, steps=8)
    _case(shape)


def test_text_two_layers_ids_ragged_vocab():
    shape = wl.TEXT_0P6B.replace(name="q06-2l-v1000-pb", n_layers=2, vocab=1000, prompt_len=20, steps=8)
    _case(shape)


def test_talker_two_layers_several_chunks_behind_cache():
    """150 prompt positions behind 70 cached ones: chunks of 64, 64 and 22 (ragged last
    tile), then the first id's LM head over the last position."""
    shape = wl.TALKER_0P6B.replace(name="talker-2l-pb150", n_layers=2, kv_prefill=70, prompt_len=150, steps=6)
    _case(shape)


def test_talker_two_layers_behind_long_cache():
    """A prompt behind 2100 cached positions: the attention takes the key-range path
    (MFMA tiles per range of keys, then the ranges' merge), chunks of 64 and 1."""
    shape = wl.TALKER_0P6B.replace(name="talker-2l-pb-kv2100", n_layers=2, kv_prefill=2100, prompt_len=65, steps=3)
    _case(shape)


def test_q17_talker_two_layers():
    shape = wl.TALKER_1P7B.replace(name="talker-1.7b-2l-pb", n_layers=2, kv_prefill=40, prompt_len=24, steps=6)
    _case(shape)


def test_full_talker_0p6b_prompt():
    """All 28 layers at the benchmark's prompt: every prompt position against the oracle."""
    shape = wl.TALKER_0P6B.replace(name="talker-0.6b-pb", steps=4)
    _case(shape)


def test_one_position_prompt():
    """The smallest prompt: one position, a single 16-column tile with one live column."""
    shape = wl.TALKER_0P6B.replace(name="talker-2l-pb1", n_layers=2, prompt_len=1, steps=4)
    _case(shape)


def test_text_vocab_lm_head_two_layers():
    """The full 151936-row text vocabulary in the first id's LM head."""
    shape = wl.TEXT_0P6B.replace(name="q06-2l-pbV", n_layers=2, prompt_len=12, steps=2)
    _case(shape)


def test_progress_and_feedback_after_batched_prefill():
    """The first id is published like a decode step's: the progress word reads 1 and a
    feedback decode continues from it exactly as after mk_prefill with the same id."""
    import torch
    from persistent_megakernel_loop_amd.binding import Decoder, weights_to_device

    shape = wl.TEXT_0P6B.replace(name="q06-2l-v1000-fb", n_layers=2, vocab=1000, prompt_len=10, steps=6)
    print(f"[case] {shape.name}: progress word and greedy feedback after the batched prefill", flush=True)
    dec = Decoder(shape, weights_to_device(wl.make_weights(shape)))
    ids = torch.from_numpy(wl.make_prompt_ids(shape)).cuda()
    first = dec.prefill(ids, batched=True)
    torch.cuda.synchronize()
    assert dec.progress() == 1
    out = dec.decode(shape.steps)
    torch.cuda.synchronize()
    dec.check()
    # the same prompt position by position, decoded teacher-forced from the batched first id
    dec.reset()
    dec.prefill(ids)
    steps = torch.cat([first, out[:-1]]).to(torch.int32)
    ref = dec.decode(shape.steps, steps)
    torch.cuda.synchronize()
    dec.check()
    dec.close()
    # the cache entries differ by rounding order only: the greedy ids agree on this case
    assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy())


def test_float32_weights_refused():
    import torch
    from persistent_megakernel_loop_amd.binding import Decoder, MkError, weights_to_device

    print("[case] tiny-f32: batched prefill refused", flush=True)
    shape = wl.TINY
    dec = Decoder(shape, weights_to_device(wl.make_weights(shape)))
    ids = torch.from_numpy(wl.make_prompt_ids(shape)).cuda()
    with pytest.raises(MkError) as e:
        dec.prefill(ids, batched=True)
    assert e.value.code == MK_ERR_UNSUPPORTED
    assert dec.position == 0
    dec.close()


def _batched_prefill_hidden(dec, shape, ids, rows=None, pos3=None):
    import torch

    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    L, H = shape.n_layers, shape.hidden
    dec.reset()
    hid = torch.zeros((len(ids), L + 1, H), dtype=torch.float32, device="cuda")
    dec.set_debug(hid, None)
    first = dec.prefill(t(ids), t(rows), t(pos3), batched=True)
    torch.cuda.synchronize()
    code = dec.status()
    dec.set_debug(None, None)
    return code, int(first.cpu()[0]), hid.cpu().numpy()


def test_bad_id_and_position_flagged_and_read_as_zero():
    """As on the persistent path: an id past the vocabulary and a rotary stream past the
    table are flagged in the device error word (MK_ERR_DEVICE) and read as 0; the prompt
    then equals, bit for bit, the prompt with 0 in their place."""
    from persistent_megakernel_loop_amd.binding import Decoder, weights_to_device

    MK_ERR_DEVICE = -7
    shape = wl.TALKER_0P6B.replace(name="talker-2l-pbbad", n_layers=2, prompt_len=20, steps=1)
    print(f"[case] {shape.name}: batched prompt with a bad id, then a bad position stream", flush=True)
    inp = make_inputs(shape)
    dec = Decoder(shape, weights_to_device(wl.make_weights(shape)))
    ids, fixed = inp.prompt_ids.copy(), inp.prompt_ids.copy()
    ids[5], fixed[5] = shape.vocab + 7, 0
    a = _batched_prefill_hidden(dec, shape, ids, inp.prompt_rows, inp.prompt_pos3)
    b = _batched_prefill_hidden(dec, shape, fixed, inp.prompt_rows, inp.prompt_pos3)
    assert a[0] == MK_ERR_DEVICE and b[0] == 0
    assert a[1] == b[1] and np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))
    pos, pfixed = inp.prompt_pos3.copy(), inp.prompt_pos3.copy()
    pos[7, 1], pfixed[7, 1] = 1 << 24, 0
    c = _batched_prefill_hidden(dec, shape, inp.prompt_ids, inp.prompt_rows, pos)
    d = _batched_prefill_hidden(dec, shape, inp.prompt_ids, inp.prompt_rows, pfixed)
    dec.close()
    assert c[0] == MK_ERR_DEVICE and d[0] == 0
    assert c[1] == d[1] and np.array_equal(c[2].view(np.uint32), d[2].view(np.uint32))
