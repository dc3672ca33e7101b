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


def test_speak_through_the_stub_codec():
    """The streaming loop: prompt, one decode launch, every chunk of ids into the stub
    codec as it is published; the codec gets every frame in order (the launch's output),
    80 ms of audio each, and the talker runs faster than real time."""
    import torch
    from persistent_megakernel_loop_amd.binding import Decoder, weights_to_device
    from persistent_megakernel_loop_amd.codec import StubCodec, speak

    shape = wl.TALKER_0P6B.replace(name="talker-0.6b-speak", steps=96)
    print(f"[case] {shape.name}: prompt + 96 frames through the stub codec in chunks of 4", flush=True)
    inp = make_inputs(shape)
    dec = Decoder(shape, weights_to_device(wl.make_weights(shape)))
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    prompt = (t(inp.prompt_ids), t(inp.prompt_rows), t(inp.prompt_pos3))
    steps = (t(inp.step_ids), t(inp.step_rows), t(inp.step_pos3))
    torch.cuda.synchronize()
    codec, pcm = StubCodec(codebook_size=shape.vocab), []
    st = speak(dec, inp.n_steps, *steps, prompt=prompt, chunk=4, codec=codec, on_audio=pcm.append)
    torch.cuda.synchronize()
    print(f"[case] ttfc {st.ttfc_ms:.2f} ms, total {st.total_ms:.2f} ms for {st.audio_s:.2f} s of audio: "
          f"rtf {st.rtf:.4f}, {st.chunks} chunks", flush=True)
    ids = dec.read_ids(0, inp.n_steps)
    dec.close()
    assert st.frames == inp.n_steps and codec.frames == [int(v) for v in ids]
    assert sum(len(a) for a in pcm) == inp.n_steps * codec.samples_per_frame
    assert st.chunks >= inp.n_steps // 4 and st.ttfc_ms < st.total_ms
    assert st.rtf < 0.3  # the theaicatchup article's real-time target


def test_ring_wraps_on_a_long_call():
    """5000 ids through the 4096-entry ring in one launch, no synchronization: a reader
    that keeps up streams all of them; one that lags more than the ring falls back to
    the device output; the entry of id 0 is overwritten by id 4096 (MK_ERR_OVERRUN)."""
    import torch
    from persistent_megakernel_loop_amd.binding import MK_ERR_OVERRUN, Decoder, MkError, weights_to_device

    shape = wl.TINY.replace(name="tiny-ring", steps=5000)
    print(f"[case] {shape.name}: 5000 greedy steps streamed through the id ring", flush=True)
    dec = Decoder(shape, weights_to_device(wl.make_weights(shape)))
    ids = torch.from_numpy(wl.make_prompt_ids(shape)).cuda()

    def run(lag_s):
        dec.reset()
        dec.prefill(ids)
        out = torch.empty(5000, dtype=torch.int32, device="cuda")
        chunks = []
        for c in dec.stream(5000, chunk=64, out=out):
            chunks.append(c)
            if lag_s and len(chunks) == 1:
                time.sleep(lag_s)
        torch.cuda.synchronize()
        return np.concatenate(chunks), out.cpu().numpy()

    got, out = run(0.0)
    assert np.array_equal(got, out)
    assert np.array_equal(dec.read_ids(4096, 904), out[4096:])
    with pytest.raises(MkError) as e:
        dec.read_ids(0, 1)
    assert e.value.code == MK_ERR_OVERRUN
    lagged, out2 = run(1.0)  # the launch ends while the reader sleeps
    dec.close()
    assert np.array_equal(lagged, out2) and np.array_equal(out2, out)
