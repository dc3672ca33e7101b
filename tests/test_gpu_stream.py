"""Host-side streaming of the decode ids (mk_progress / mk_read_ids / mk_query) on the
full 28-layer talker: the chunks arrive while the launch is still running, together
they are exactly the launch's device output, and every streamed id passes the parity
rule against the oracle run on the same inputs."""
import time

import numpy as np
import pytest

from persistent_megakernel_loop_amd import workload as wl
from oracle import Decoder as OracleDecoder
from tests.parity import check_id, make_inputs

pytestmark = pytest.mark.gpu


def test_stream_chunks_arrive_while_running():
    import torch
    from persistent_megakernel_loop_amd.binding import Decoder, weights_to_device

    shape = wl.TALKER_0P6B.replace(name="talker-0.6b-stream", steps=64)
    print(f"[case] {shape.name}: 64 steps streamed in chunks of 8", flush=True)
    inp = make_inputs(shape)
    weights = wl.make_weights(shape)
    dec = Decoder(shape, weights_to_device(weights))
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    prompt = (t(inp.prompt_ids), t(inp.prompt_rows), t(inp.prompt_pos3))
    steps = (t(inp.step_ids), t(inp.step_rows), t(inp.step_pos3))
    dec.prefill(*prompt, batched=True)
    out = torch.empty(inp.n_steps, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    chunks, arrive = [], []
    for c in dec.stream(inp.n_steps, *steps, chunk=8, out=out):
        chunks.append(c)
        arrive.append(time.perf_counter() - t0)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    got = np.concatenate(chunks)
    print(f"[case] {len(chunks)} chunks, first after {arrive[0] * 1e3:.2f} ms, last after {arrive[-1] * 1e3:.2f} ms, "
          f"launch {total * 1e3:.2f} ms", flush=True)
    assert np.array_equal(got, out.cpu().numpy())
    assert all(len(c) >= 8 for c in chunks[:-1])
    # 64 steps take about 29 ms; the first 8 ids are out after about an eighth of that
    assert arrive[0] < 0.5 * arrive[-1]
    # the pinned mirror holds exactly the published ids: the whole launch reads back,
    # one more is refused
    from persistent_megakernel_loop_amd.binding import MkError
    assert np.array_equal(dec.read_ids(0, inp.n_steps), got)
    with pytest.raises(MkError):
        dec.read_ids(0, inp.n_steps + 1)
    # the same inputs again through a plain decode give the same ids
    dec.reset()
    dec.prefill(*prompt, batched=True)
    again = dec.decode(inp.n_steps, *steps)
    torch.cuda.synchronize()
    dec.check()
    dec.close()
    assert np.array_equal(again.cpu().numpy(), got)
    # the streamed ids against the oracle: the talker's inputs are sentinel rows, so the
    # oracle runs the same positions on its own (no feedback to replay)
    orc = OracleDecoder.from_shape(shape, weights)
    orc.prefill(inp.prompt_ids, inp.prompt_rows, inp.prompt_pos3)
    strict = 0
    for s in range(inp.n_steps):
        logits, _ = orc.step(orc.input_row(int(inp.step_ids[s]), inp.step_rows[s]), inp.step_pos3[s])
        strict += check_id(int(got[s]), logits, f"streamed step {s}")
    print(f"[case] streamed ids against the oracle: {inp.n_steps} checked, {strict} strict", flush=True)
