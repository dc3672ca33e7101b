"""GPU parity: the HIP decode path (through the C ABI) against the oracle.

Small cases span several tiles and a ragged vocabulary tail and run the oracle
over every position; full-size cases run the launch configuration the
benchmark times (one workgroup per CU, the whole prompt and a block of decode
steps in single launches) and compare every position the oracle replays.
"""
import numpy as np
import pytest

from persistent_megakernel_loop_amd import workload as wl
from tests.parity import check_free_run, compare, make_inputs, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _case(shape, n_steps=None, prompt_len=None, kv_prefill=None, steps_checked=None, random_gains=False,
          logits_every=1, free_run=False):
    from persistent_megakernel_loop_amd.binding import weights_to_device

    print(f"[case] {shape.name} L={shape.n_layers} V={shape.vocab} steps={n_steps} prompt={prompt_len} "
          f"kv={kv_prefill}", flush=True)
    weights = wl.make_weights(shape, random_gains=random_gains)
    inp = make_inputs(shape, n_steps=n_steps, prompt_len=prompt_len, kv_prefill=kv_prefill)
    dw = weights_to_device(weights)
    gpu = run_gpu(shape, dw, inp)
    del dw
    orc = run_oracle(shape, weights, inp, gpu, steps=steps_checked, logits_every=logits_every)
    summary = compare(gpu, orc)
    if free_run:
        summary["free_run_ids_equal"] = check_free_run(shape, weights, inp, gpu, orc)
    print(f"[case] {shape.name}: {summary}", flush=True)
    return gpu, summary


def test_tiny_fp32_full_run():
    """The tiny fp32 decoder: 8 prompt ids, 32 greedy steps; the oracle's own free run
    gives the GPU's ids up to its first low-margin step."""
    _case(wl.TINY, free_run=True)


def test_tiny_random_gains_ragged_vocab():
    shape = wl.TINY.replace(name="tiny-97", vocab=97)
    _case(shape, n_steps=12, random_gains=True)


def test_q06_text_two_layers_ragged_vocab():
    shape = wl.TEXT_0P6B.replace(name="q06-2l-v1000", n_layers=2, vocab=1000, prompt_len=16, steps=24)
    _case(shape)


def test_q06_talker_two_layers():
    shape = wl.TALKER_0P6B.replace(name="talker-2l", n_layers=2, prompt_len=32, steps=16)
    _case(shape)


def test_q06_talker_long_chunks_two_layers():
    """Positions past 32 x 56 use all 32 attention chunks of an XCD (the last one ragged)."""
    shape = wl.TALKER_0P6B.replace(name="talker-2l-kv1800", n_layers=2, kv_prefill=1800, prompt_len=0, steps=8)
    _case(shape)


def test_q17_talker_two_layers():
    """The hidden-2048 body (register-resident tiles) on two layers with a short pre-filled cache."""
    shape = wl.TALKER_1P7B.replace(name="talker-1.7b-2l", n_layers=2, kv_prefill=40, prompt_len=8, steps=8)
    _case(shape)


@pytest.mark.parametrize("shape", [
    wl.TALKER_0P6B.replace(name="talker-2l-fbrows", n_layers=2, prompt_len=8, steps=24),
    wl.TALKER_1P7B.replace(name="talker-1.7b-2l-fbrows", n_layers=2, kv_prefill=0, prompt_len=8, steps=12),
], ids=lambda s: s.name)
def test_greedy_feedback_plus_frame_rows(shape):
    """Greedy feedback with rows: each step's input is the fed-back id's embedding plus
    the step's row (the frame's other embeddings); the oracle replays the GPU's ids."""
    import dataclasses

    from persistent_megakernel_loop_amd.binding import weights_to_device

    print(f"[case] {shape.name}: greedy feedback + rows, {shape.steps} steps", flush=True)
    weights = wl.make_weights(shape)
    inp = dataclasses.replace(make_inputs(shape), step_ids=None)
    gpu = run_gpu(shape, weights_to_device(weights), inp)
    print(f"[case] {shape.name}: {compare(gpu, run_oracle(shape, weights, inp, gpu))}", flush=True)


def test_determinism_bitwise():
    from persistent_megakernel_loop_amd.binding import weights_to_device

    shape = wl.TEXT_0P6B.replace(name="q06-2l-det", n_layers=2, vocab=1000, prompt_len=16, steps=16)
    weights = wl.make_weights(shape)
    inp = make_inputs(shape)
    dw = weights_to_device(weights)
    a = run_gpu(shape, dw, inp)
    b = run_gpu(shape, dw, inp)
    assert a.first_id == b.first_id
    assert np.array_equal(a.ids, b.ids)
    assert np.array_equal(a.hidden.view(np.uint32), b.hidden.view(np.uint32))


def test_full_talker_0p6b():
    """The 0.6B talker exactly as the benchmark launches it: 32-row prompt, then ONE
    launch of 256 decode steps; every step's id and every layer at every position compared."""
    _case(wl.TALKER_0P6B, n_steps=256)


def test_full_text_0p6b():
    """The Qwen3-0.6B-shaped text decoder (151936-row tied head) exactly as the benchmark
    launches it: 16 prompt ids, one launch of 256 greedy steps; every layer at every position
    and every id (the full head each step), and the oracle's own free run against the GPU's
    ids up to the first low-margin step."""
    _, summary = _case(wl.TEXT_0P6B, n_steps=256, free_run=True)
    assert summary["ids_checked"] == 256


def test_full_talker_long_context():
    """The talker with 4096 pre-filled positions exactly as the benchmark launches it: one
    launch of 512 decode steps (positions 4096..4607, all 28 attention chunks), every step's
    id and every layer's hidden state against the oracle."""
    _, summary = _case(wl.TALKER_0P6B_LONG, n_steps=512)
    assert summary["ids_checked"] == 512


def test_full_talker_1p7b():
    """The 1.7B-scale talker (hidden 2048) with 2048 pre-filled positions exactly as the
    benchmark launches it: one launch of 512 steps, every step's id and every layer's hidden
    state against the oracle."""
    _, summary = _case(wl.TALKER_1P7B, n_steps=512)
    assert summary["ids_checked"] == 512


def _sweep_cases():
    rng = np.random.default_rng(20261202)
    cases = []
    for i in range(6):
        p = int(rng.integers(1, 101))
        kv = int(rng.choice([0, int(rng.integers(1, 401))]))
        n = int(rng.integers(1, 17))
        cases.append((f"sweep{i}-p{p}-kv{kv}-n{n}", p, kv, n, bool(i % 2)))
    return cases


@pytest.mark.parametrize("name,prompt_len,kv_prefill,n_steps,batched", _sweep_cases(), ids=lambda c: str(c))
def test_seeded_shape_sweep(name, prompt_len, kv_prefill, n_steps, batched):
    """Seeded prompt lengths (ragged position tiles, several prefill chunks), pre-filled
    caches and step counts on the 2-layer talker, both prefill paths, against the oracle."""
    from persistent_megakernel_loop_amd.binding import weights_to_device

    shape = wl.TALKER_0P6B.replace(name=name, n_layers=2, prompt_len=prompt_len, kv_prefill=kv_prefill,
                                   steps=n_steps)
    print(f"[case] {name} ({'batched' if batched else 'per-position'} prefill)", flush=True)
    weights = wl.make_weights(shape)
    inp = make_inputs(shape)
    gpu = run_gpu(shape, weights_to_device(weights), inp, batched=batched)
    print(f"[case] {name}: {compare(gpu, run_oracle(shape, weights, inp, gpu))}", flush=True)


def test_whole_attention_form_equals_chunked_below_56():
    """A decode launch whose positions all lie below 56 runs the whole-attention form of
    the hidden-1024 body (every workgroup of an XCD computes the group's attention; no
    chunk exchange).  Below 56 positions the chunked form has exactly one chunk, so both
    forms compute the same sums in the same order: the first 20 steps of a 30-step launch
    (which crosses 56 and runs the chunked form) must equal a 20-step launch (the whole
    form) bit for bit, ids and every layer's hidden state; both follow the oracle."""
    from persistent_megakernel_loop_amd.binding import weights_to_device

    shape = wl.TALKER_0P6B.replace(name="talker-2l-whole", n_layers=2, prompt_len=32, steps=30)
    print(f"[case] {shape.name}: 20 steps (whole-attention form) against the first 20 of 30 (chunked)", flush=True)
    weights = wl.make_weights(shape)
    dw = weights_to_device(weights)
    inp = make_inputs(shape)
    chunked = run_gpu(shape, dw, inp)
    short = inp.__class__(**{**inp.__dict__, "step_ids": inp.step_ids[:20], "step_rows": inp.step_rows[:20],
                             "step_pos3": inp.step_pos3[:20], "n_steps": 20})
    whole = run_gpu(shape, dw, short)
    del dw
    assert np.array_equal(whole.ids, chunked.ids[:20])
    assert np.array_equal(whole.hidden.view(np.uint32), chunked.hidden[:32 + 20].view(np.uint32))
    summary = compare(chunked, run_oracle(shape, weights, inp, chunked))
    print(f"[case] {shape.name}: {summary}", flush=True)
