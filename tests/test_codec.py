"""The stub codec (host only): 80 ms of audio per code at 12.5 frames per second, the
pitch each code sets, phase carried across chunks, codes outside the codebook refused."""
import numpy as np
import pytest

from persistent_megakernel_loop_amd.codec import FRAME_MS, SAMPLE_RATE, SpeechStats, StubCodec


def test_frame_length_and_rate():
    c = StubCodec(codebook_size=3072)
    assert c.samples_per_frame == 1920 and FRAME_MS == 80.0 and SAMPLE_RATE == 24000
    pcm = c.decode([0, 5, 3071])
    assert pcm.dtype == np.float32 and pcm.shape == (3 * 1920,)
    assert c.frames == [0, 5, 3071] and c.seconds == pytest.approx(0.24)


def test_pitch_follows_the_code():
    # one second of a code: its spectrum peaks at base * 2^(code / codebook_size) (1 Hz bins)
    for code in (0, 1024, 2047, 3071):
        c = StubCodec(codebook_size=3072)
        pcm = c.decode([code] * 13)[:SAMPLE_RATE].astype(np.float64)
        peak = int(np.argmax(np.abs(np.fft.rfft(pcm))))
        assert abs(peak - 110.0 * 2.0 ** (code / 3072)) <= 1.0


def test_chunks_join_like_one_call():
    codes = np.random.default_rng(7).integers(0, 3072, size=40)
    whole = StubCodec().decode(codes)
    c = StubCodec()
    parts = np.concatenate([c.decode(codes[a:a + 7]) for a in range(0, 40, 7)])
    assert np.allclose(parts, whole, atol=1e-5)
    # no jump at a frame boundary larger than one sample's step at the highest pitch
    step = 2 * np.pi * 220.0 / SAMPLE_RATE * 0.2
    assert np.abs(np.diff(parts.astype(np.float64))).max() <= step * 1.01


def test_codes_outside_the_codebook_refused():
    with pytest.raises(ValueError):
        StubCodec(codebook_size=16).decode([16])
    with pytest.raises(ValueError):
        StubCodec(codebook_size=16).decode([-1])


def test_rtf_is_compute_over_audio():
    s = SpeechStats(frames=25, chunks=5, ttfc_ms=3.0, total_ms=500.0, audio_s=2.0)
    assert s.rtf == pytest.approx(0.25)
