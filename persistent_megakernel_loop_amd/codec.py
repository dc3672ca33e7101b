"""Stub audio codec and the streaming speech loop around the decode kernel.

The talker emits one codebook-0 code per decode step, and a step is one codec frame:
audio codes come at 12.5 frames per second (the theaicatchup article, "Why Does a
Single Kernel Even Matter for TTS?"), so a frame is 80 ms of audio.  The stage that
turns frames into sound is stubbed here, as it was in the dev.to article's build (its
opening scope note): ``StubCodec`` maps each code to 80 ms of a tone whose pitch is
set by the code, so its output has the length and timing real audio would have and a
test can check that every frame reached it, in order.

``speak`` is the streaming loop of the dev.to article's "Making it talk end-to-end":
the prompt, then one decode launch whose ids leave in chunks while the kernel runs
(``Decoder.stream``), each chunk handed to the codec as soon as it is published.  It
measures the two figures the theaicatchup article's FAQ defines: time to the first
audio chunk (TTFC) and the real-time factor, compute time over audio duration (RTF).
The codec is a stand-in costing microseconds, so the RTF measured here is the
talker's own.
"""
from __future__ import annotations

import time
from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np

FRAME_RATE_HZ = 12.5
FRAME_MS = 1000.0 / FRAME_RATE_HZ
# The pages give no sample rate; 24 kHz is taken as the codec's output rate.
SAMPLE_RATE = 24000


class StubCodec:
    """Codes -> float32 PCM, ``samples_per_frame`` samples per code: a sine at
    ``base_hz * 2**(code / codebook_size)`` with its phase carried across frames (so
    consecutive chunks join without a click).  ``frames`` records every code received,
    in order."""

    def __init__(self, codebook_size: int = 3072, sample_rate: int = SAMPLE_RATE,
                 frame_rate_hz: float = FRAME_RATE_HZ, base_hz: float = 110.0, amplitude: float = 0.2):
        spf = sample_rate / frame_rate_hz
        if spf != int(spf):
            raise ValueError("sample_rate must be a whole multiple of the frame rate")
        self.codebook_size = int(codebook_size)
        self.sample_rate = int(sample_rate)
        self.samples_per_frame = int(spf)
        self.base_hz = float(base_hz)
        self.amplitude = float(amplitude)
        self.frames: List[int] = []
        self._phase = 0.0

    def decode(self, codes) -> np.ndarray:
        codes = np.asarray(codes, dtype=np.int64).reshape(-1)
        if codes.size and (codes.min() < 0 or codes.max() >= self.codebook_size):
            raise ValueError("code outside the codebook")
        n = self.samples_per_frame
        out = np.empty(codes.size * n, dtype=np.float32)
        k = np.arange(n, dtype=np.float64)
        for j, c in enumerate(codes):
            step = 2.0 * np.pi * self.base_hz * 2.0 ** (float(c) / self.codebook_size) / self.sample_rate
            out[j * n:(j + 1) * n] = self.amplitude * np.sin(self._phase + step * k)
            self._phase = float(np.fmod(self._phase + step * n, 2.0 * np.pi))
        self.frames.extend(int(c) for c in codes)
        return out

    @property
    def seconds(self) -> float:
        return len(self.frames) / (self.sample_rate / self.samples_per_frame)


@dataclass
class SpeechStats:
    frames: int
    chunks: int
    ttfc_ms: float            # prompt enqueue -> first audio chunk out of the codec
    total_ms: float           # prompt enqueue -> last audio chunk out of the codec
    audio_s: float
    chunk_ms: List[float] = field(default_factory=list)  # when each audio chunk came out

    @property
    def rtf(self) -> float:
        """Compute time over audio duration (below 1: faster than real time)."""
        return (self.total_ms / 1e3) / self.audio_s if self.audio_s else float("inf")


def speak(dec, n_frames: int, ids=None, rows=None, pos3=None, prompt=None, chunk: int = 4,
          codec: Optional[StubCodec] = None, on_audio: Optional[Callable[[np.ndarray], None]] = None,
          batched_prefill: bool = True) -> SpeechStats:
    """One utterance: the prompt (``prompt`` = (ids, rows, pos3) device tensors, or None
    to continue from the handle's state), then ``n_frames`` decode steps in one launch,
    streamed in chunks of ``chunk`` ids through ``codec`` (a new StubCodec by default);
    every PCM chunk goes to ``on_audio``.  The clock starts when the prompt is enqueued."""
    codec = codec if codec is not None else StubCodec(codebook_size=dec.shape.vocab)
    t0 = time.perf_counter()
    if prompt is not None:
        dec.prefill(*prompt, batched=batched_prefill)
    marks: List[float] = []
    frames = 0
    for codes in dec.stream(n_frames, ids, rows, pos3, chunk=chunk):
        pcm = codec.decode(codes)
        marks.append((time.perf_counter() - t0) * 1e3)
        frames += len(codes)
        if on_audio is not None:
            on_audio(pcm)
    return SpeechStats(frames=frames, chunks=len(marks), ttfc_ms=marks[0] if marks else float("nan"),
                       total_ms=marks[-1] if marks else float("nan"), audio_s=frames * FRAME_MS / 1e3,
                       chunk_ms=marks)
