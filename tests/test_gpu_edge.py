"""GPU edge cases of the decode path, through the C ABI.

* a decode call of zero steps is refused on the host and changes nothing;
* a one-position prompt (the smallest prefill) against the oracle, on the fp32 body
  and on the bf16 talker body;
* an id outside the vocabulary in a teacher-forced step is flagged in the device error
  word (mk_status returns MK_ERR_DEVICE) and read as id 0: the run equals, bit for bit,
  the run with 0 in its place;
* a position stream outside the rotary table is flagged the same way and read as
  position 0;
* a wait that gives up (a spin limit of one poll round, set from the host) ends the
  launch cleanly, is reported as MK_ERR_TIMEOUT, and the handle recovers after mk_reset.
"""
import ctypes

import numpy as np
import pytest

from persistent_megakernel_loop_amd import workload as wl
from tests.parity import compare, make_inputs, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

MK_ERR_DEVICE = -7
MK_ERR_TIMEOUT = -8


def _decoder(shape):
    from persistent_megakernel_loop_amd.binding import Decoder, weights_to_device
    return Decoder(shape, weights_to_device(wl.make_weights(shape)))


def test_decode_zero_steps_refused():
    import torch
    from persistent_megakernel_loop_amd.binding import MkError

    print("[case] decode(0) on tiny-f32", flush=True)
    shape = wl.TINY
    dec = _decoder(shape)
    dec.prefill(torch.from_numpy(wl.make_prompt_ids(shape)).cuda())
    torch.cuda.synchronize()
    pos = dec.position
    with pytest.raises(MkError):
        dec.decode(0)
    assert dec.position == pos
    dec.check()
    dec.close()


@pytest.mark.parametrize("shape", [
    wl.TINY.replace(name="tiny-p1", prompt_len=1, steps=12),
    wl.TALKER_0P6B.replace(name="talker-2l-p1", n_layers=2, prompt_len=1, steps=8),
], ids=lambda s: s.name)
def test_one_position_prompt(shape):
    from persistent_megakernel_loop_amd.binding import weights_to_device

    print(f"[case] {shape.name}: one prompt position, {shape.steps} steps", flush=True)
    weights = wl.make_weights(shape)
    inp = make_inputs(shape)
    gpu = run_gpu(shape, weights_to_device(weights), inp)
    print(f"[case] {shape.name}: {compare(gpu, run_oracle(shape, weights, inp, gpu))}", flush=True)


def _teacher_forced(dec, shape, prompt, steps, rows=None, pos3=None, prompt_rows=None, prompt_pos3=None):
    """Prefill then a teacher-forced decode; returns (status, ids, hidden) without raising."""
    import torch

    L, H = shape.n_layers, shape.hidden
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    dec.reset()
    dec.prefill(t(prompt), t(prompt_rows), t(prompt_pos3))
    dec.check()
    hid = torch.zeros((len(steps), L + 1, H), dtype=torch.float32, device="cuda")
    dec.set_debug(hid, None)
    out = dec.decode(len(steps), t(steps), t(rows), t(pos3))
    torch.cuda.synchronize()
    code = dec.status()
    dec.set_debug(None, None)
    return code, out.cpu().numpy(), hid.cpu().numpy()


def test_id_outside_vocab_flagged_and_read_as_zero():
    print("[case] tiny-f32: teacher-forced id past the vocabulary", flush=True)
    shape = wl.TINY
    dec = _decoder(shape)
    prompt = wl.make_prompt_ids(shape)
    steps = wl.make_prompt_ids(shape, 6, seed=11)
    bad, fixed = steps.copy(), steps.copy()
    bad[2], fixed[2] = shape.vocab + 3, 0
    code_b, ids_b, hid_b = _teacher_forced(dec, shape, prompt, bad)
    code_f, ids_f, hid_f = _teacher_forced(dec, shape, prompt, fixed)
    dec.close()
    assert code_b == MK_ERR_DEVICE and code_f == 0
    assert np.array_equal(ids_b, ids_f)
    assert np.array_equal(hid_b.view(np.uint32), hid_f.view(np.uint32))


def test_position_outside_rotary_table_flagged_and_read_as_zero():
    shape = wl.TALKER_0P6B.replace(name="talker-2l-pos", n_layers=2, prompt_len=4, steps=4)
    print(f"[case] {shape.name}: a position stream past the rotary table", flush=True)
    inp = make_inputs(shape)
    dec = _decoder(shape)
    bad, fixed = inp.step_pos3.copy(), inp.step_pos3.copy()
    bad[1, 2], fixed[1, 2] = 1 << 24, 0
    args = dict(prompt_rows=inp.prompt_rows, prompt_pos3=inp.prompt_pos3, rows=inp.step_rows)
    code_b, ids_b, hid_b = _teacher_forced(dec, shape, inp.prompt_ids, inp.step_ids, pos3=bad, **args)
    code_f, ids_f, hid_f = _teacher_forced(dec, shape, inp.prompt_ids, inp.step_ids, pos3=fixed, **args)
    dec.close()
    assert code_b == MK_ERR_DEVICE and code_f == 0
    assert np.array_equal(ids_b, ids_f)
    assert np.array_equal(hid_b.view(np.uint32), hid_f.view(np.uint32))


@pytest.mark.parametrize("shape", [
    wl.TINY,
    wl.TALKER_0P6B.replace(name="talker-2l-timeout", n_layers=2, prompt_len=4, steps=8),
    wl.TALKER_1P7B.replace(name="talker-1.7b-2l-timeout", n_layers=2, kv_prefill=0, prompt_len=4, steps=8),
], ids=lambda s: s.name)
def test_forced_timeout_reported_and_recovered(shape):
    """A spin limit of one poll round makes the first wait for another workgroup give up:
    the launch still completes (every wave leaves at the same barrier), mk_status reports
    MK_ERR_TIMEOUT with the place recorded, and after mk_reset with the default limit the
    handle decodes exactly as before, also when mk_reset is called without reading the
    status first (each body: fp32 LDS tiles, bf16 LDS tiles, register
    rings)."""
    import torch
    from persistent_megakernel_loop_amd.binding import lib

    print(f"[case] {shape.name}: spin limit 1 (forced timeout), then recovery", flush=True)
    dec = _decoder(shape)
    inp = make_inputs(shape)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    prompt = (t(inp.prompt_ids), t(inp.prompt_rows), t(inp.prompt_pos3))
    steps = (t(inp.step_ids), t(inp.step_rows), t(inp.step_pos3))
    dec.prefill(*prompt)
    ref = dec.decode(inp.n_steps, *steps)
    torch.cuda.synchronize()
    dec.check()
    ref = ref.cpu().numpy()

    dec.reset()
    dec.set_spin_limit(1)
    dec.prefill(*prompt)
    dec.decode(inp.n_steps, *steps)
    torch.cuda.synchronize()
    assert dec.status() == MK_ERR_TIMEOUT
    info = (ctypes.c_int32 * 5)()
    assert lib().mk_error_info(dec.handle, info) == 0
    assert info[0] == 1 and 0 <= info[1] < 256  # recorded, by a workgroup of the grid

    dec.set_spin_limit(0)
    dec.reset()
    dec.prefill(*prompt)
    again = dec.decode(inp.n_steps, *steps)
    torch.cuda.synchronize()
    dec.check()
    assert np.array_equal(again.cpu().numpy(), ref)

    # mk_reset alone re-arms the handle: a timed-out launch, no mk_status, then reset
    dec.reset()
    dec.set_spin_limit(1)
    dec.prefill(*prompt)
    dec.decode(inp.n_steps, *steps)
    dec.set_spin_limit(0)
    dec.reset()
    dec.prefill(*prompt)
    third = dec.decode(inp.n_steps, *steps)
    torch.cuda.synchronize()
    assert dec.status() == 0
    dec.close()
    assert np.array_equal(third.cpu().numpy(), ref)


@pytest.mark.parametrize("batched", [False, True], ids=["per-position", "batched"])
def test_fill_to_capacity_then_refuse(batched):
    """The cache filled to its last slot (capacity = prompt + steps exactly), against the
    oracle up to that slot; one more step is refused on the host (MK_ERR_CAPACITY) and
    the position stays at the capacity."""
    from persistent_megakernel_loop_amd.binding import Decoder, MkError, weights_to_device

    MK_ERR_CAPACITY = -4
    shape = wl.TALKER_0P6B.replace(name="talker-2l-full", n_layers=2, prompt_len=20, steps=12)
    assert shape.capacity == 32
    print(f"[case] {shape.name}: cache filled to capacity {shape.capacity} ({'batched' if batched else 'per-position'} "
          "prefill), then one step more", flush=True)
    weights = wl.make_weights(shape)
    inp = make_inputs(shape)
    dec = Decoder(shape, weights_to_device(weights))
    gpu = run_gpu(shape, None, inp, dec=dec, batched=batched)
    print(f"[case] {shape.name}: {compare(gpu, run_oracle(shape, weights, inp, gpu))}", flush=True)
    assert dec.position == shape.capacity
    with pytest.raises(MkError) as e:
        dec.decode(1)
    assert e.value.code == MK_ERR_CAPACITY and dec.position == shape.capacity
    dec.close()
