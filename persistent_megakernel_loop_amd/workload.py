"""Seeded synthetic workloads for the batch-1 talker decode path.

This module only draws random numbers and lays them out.  It holds none of the
decoder's arithmetic: no norm, no rotation, no attention, no sum of embedding
rows.  Both the GPU path and the CPU oracle read what it returns.

Shapes follow the decoders the pages describe:
  * the Qwen3 text decoder whose body the TTS talker copies (same hidden size,
    layers and heads; "Why Does a Single Kernel Even Matter for TTS?" on the
    theaicatchup article),
  * the talker itself: vocab of 3072 audio codes, an untied LM head
    ("Porting it to Qwen3-TTS-1.7B", dev.to article), multi-section rotary
    position streams, and inputs that are sums of 17 embedding rows
    (16 codebooks + text, theaicatchup article, same section).

Recipe (every draw is a numpy PCG64 stream with its own sub-seed, so the order
in which tensors are drawn never changes their values):
  * weights: N(0, 0.02^2) float32, rounded to bf16 (round-to-nearest-even, done
    by torch's dtype cast) for bf16 bodies; RMSNorm gains are exactly 1.0
    unless ``random_gains`` asks for N(1, 0.1^2);
  * prompt ids: uniform over the vocab (seed 1);
  * talker input ids: 16 codebook ids uniform in [0, 2048) and one text id
    uniform in [0, 151936) per position (seed 2); the tables are drawn like
    weights;
  * pre-filled KV cache: bf16(N(0, 1)) (seed 3);
  * rotary position streams for position p: (p, p // 2, p // 3).
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, List, Optional

import numpy as np

WEIGHT_SEED = 0
PROMPT_SEED = 1
TALKER_ID_SEED = 2
KV_SEED = 3

N_CODEBOOKS = 16
CODEBOOK_SIZE = 2048
TEXT_VOCAB = 151936


@dataclasses.dataclass(frozen=True)
class DecoderShape:
    """Static description of one decoder and of the workload run on it."""

    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    tied: bool
    weight_dtype: str          # "f32" | "bf16"
    kv_dtype: str              # "f32" | "bf16"
    rms_eps: float
    rope_theta: float
    sections: tuple            # rotary pairs per position stream; sum == head_dim // 2
    # workload
    prompt_len: int            # prompt positions run by prefill
    steps: int                 # decode steps after prefill
    inputs: str                # "ids" (prompt ids, then greedy feedback) | "talker" (summed rows)
    kv_prefill: int = 0        # positions pre-filled in the KV cache before the prompt
    max_seq: int = 0           # KV capacity; 0 -> kv_prefill + prompt_len + steps

    @property
    def capacity(self) -> int:
        return self.max_seq or (self.kv_prefill + self.prompt_len + self.steps)

    def replace(self, **kw) -> "DecoderShape":
        return dataclasses.replace(self, **kw)


# The five workloads.  Index 0 is the tiny fp32 decoder, 1 the Qwen3-0.6B-shaped
# text decoder, 2 the 0.6B-shaped talker, 3 the same talker at long context,
# 4 the 1.7B-scale talker.
TINY = DecoderShape("tiny-f32", 2, 256, 4, 2, 64, 768, 512, True, "f32", "f32",
                    1e-6, 1e4, (32,), 8, 32, "ids")
TEXT_0P6B = DecoderShape("qwen3-0.6b-text", 28, 1024, 16, 8, 128, 3072, 151936, True,
                         "bf16", "bf16", 1e-6, 1e6, (64,), 16, 256, "ids")
TALKER_0P6B = DecoderShape("talker-0.6b", 28, 1024, 16, 8, 128, 3072, 3072, False,
                           "bf16", "bf16", 1e-6, 1e6, (24, 20, 20), 32, 256, "talker")
TALKER_0P6B_LONG = TALKER_0P6B.replace(name="talker-0.6b-kv4096", kv_prefill=4096,
                                       prompt_len=0, steps=512)
TALKER_1P7B = DecoderShape("talker-1.7b", 28, 2048, 16, 8, 128, 6144, 3072, False,
                           "bf16", "bf16", 1e-6, 1e6, (24, 20, 20), 0, 512, "talker",
                           kv_prefill=2048)

WORKLOADS: List[DecoderShape] = [TINY, TEXT_0P6B, TALKER_0P6B, TALKER_0P6B_LONG, TALKER_1P7B]
BY_NAME: Dict[str, DecoderShape] = {w.name: w for w in WORKLOADS}


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([seed, zlib.crc32(name.encode())])


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even, via torch's cast) and return the raw uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _normal(seed: int, name: str, shape, std: float, dtype: str, mean: float = 0.0) -> np.ndarray:
    a = _rng(seed, name).standard_normal(int(np.prod(shape)), dtype=np.float32)
    a *= np.float32(std)
    if mean:
        a += np.float32(mean)
    a = a.reshape(shape)
    return _to_bf16_bits(a) if dtype == "bf16" else a


def _gain(seed: int, name: str, n: int, dtype: str, random_gains: bool) -> np.ndarray:
    if random_gains:
        return _normal(seed, name, (n,), 0.1, dtype, mean=1.0)
    ones = np.ones(n, dtype=np.float32)
    return _to_bf16_bits(ones) if dtype == "bf16" else ones


def make_weights(shape: DecoderShape, seed: int = WEIGHT_SEED,
                 random_gains: bool = False) -> Dict[str, object]:
    """Weights in HF layout: every matrix row-major [out][in].

    Returns a dict with ``embed`` [V][H], ``lm_head`` [V][H] (absent when tied),
    ``final_norm`` [H] and ``layers``: a list of dicts with ``in_norm`` [H],
    ``wq`` [n_q*d][H], ``wk`` [n_kv*d][H], ``wv`` [n_kv*d][H], ``q_norm`` [d],
    ``k_norm`` [d], ``wo`` [H][n_q*d], ``post_norm`` [H], ``w_gate`` [I][H],
    ``w_up`` [I][H], ``w_down`` [H][I].  Arrays are float32 for an f32 body and
    uint16 bf16 bit patterns for a bf16 body.
    """
    H, d, I, V = shape.hidden, shape.head_dim, shape.intermediate, shape.vocab
    dt = shape.weight_dtype
    w: Dict[str, object] = {
        "embed": _normal(seed, "embed", (V, H), 0.02, dt),
        "final_norm": _gain(seed, "final_norm", H, dt, random_gains),
    }
    if not shape.tied:
        w["lm_head"] = _normal(seed, "lm_head", (V, H), 0.02, dt)
    layers = []
    for l in range(shape.n_layers):
        p = f"layers.{l}."
        layers.append({
            "in_norm": _gain(seed, p + "in_norm", H, dt, random_gains),
            "wq": _normal(seed, p + "wq", (shape.n_q_heads * d, H), 0.02, dt),
            "wk": _normal(seed, p + "wk", (shape.n_kv_heads * d, H), 0.02, dt),
            "wv": _normal(seed, p + "wv", (shape.n_kv_heads * d, H), 0.02, dt),
            "q_norm": _gain(seed, p + "q_norm", d, dt, random_gains),
            "k_norm": _gain(seed, p + "k_norm", d, dt, random_gains),
            "wo": _normal(seed, p + "wo", (H, shape.n_q_heads * d), 0.02, dt),
            "post_norm": _gain(seed, p + "post_norm", H, dt, random_gains),
            "w_gate": _normal(seed, p + "w_gate", (I, H), 0.02, dt),
            "w_up": _normal(seed, p + "w_up", (I, H), 0.02, dt),
            "w_down": _normal(seed, p + "w_down", (H, I), 0.02, dt),
        })
    w["layers"] = layers
    return w


def make_prompt_ids(shape: DecoderShape, n: Optional[int] = None, seed: int = PROMPT_SEED) -> np.ndarray:
    n = shape.prompt_len if n is None else n
    return _rng(seed, "prompt").integers(0, shape.vocab, size=n, dtype=np.int64).astype(np.int32)


def make_talker_tables(hidden: int, dtype: str = "bf16", seed: int = WEIGHT_SEED,
                       text_vocab: int = TEXT_VOCAB, codebook_size: int = CODEBOOK_SIZE,
                       n_codebooks: int = N_CODEBOOKS) -> Dict[str, np.ndarray]:
    """The 16 codebook tables [n_codebooks][codebook_size][H] and the text table [text_vocab][H]."""
    cb = np.stack([_normal(seed, f"codebook.{c}", (codebook_size, hidden), 0.02, dtype)
                   for c in range(n_codebooks)])
    text = _normal(seed, "text_embed", (text_vocab, hidden), 0.02, dtype)
    return {"codebooks": cb, "text": text}


def make_talker_ids(n_positions: int, seed: int = TALKER_ID_SEED, text_vocab: int = TEXT_VOCAB,
                    codebook_size: int = CODEBOOK_SIZE, n_codebooks: int = N_CODEBOOKS) -> np.ndarray:
    """[n_positions][17] int32: 16 codebook ids then one text id per position."""
    r = _rng(seed, "talker_ids")
    cb = r.integers(0, codebook_size, size=(n_positions, n_codebooks), dtype=np.int64)
    tx = r.integers(0, text_vocab, size=(n_positions, 1), dtype=np.int64)
    return np.concatenate([cb, tx], axis=1).astype(np.int32)


def make_kv_prefill(shape: DecoderShape, n_pos: Optional[int] = None, seed: int = KV_SEED) -> np.ndarray:
    """[L][2][n_kv][n_pos][d] cache contents (K then V), already rotated; bf16 bits or float32."""
    n_pos = shape.kv_prefill if n_pos is None else n_pos
    shp = (shape.n_layers, 2, shape.n_kv_heads, n_pos, shape.head_dim)
    return _normal(seed, "kv_prefill", shp, 1.0, shape.kv_dtype)


def position_streams(start: int, n: int, n_streams: int = 3) -> np.ndarray:
    """[n][3] int32 rotary position streams (p, p//2, p//3) for p = start..start+n-1.

    With a single rotary section only stream 0 is read.  Distinct streams make a
    mix-up between sections visible; equal offsets would cancel in q.k.
    """
    p = np.arange(start, start + n, dtype=np.int64)
    cols = [p, p // 2, p // 3][:n_streams]
    return np.stack(cols, axis=1).astype(np.int32)


def sentinel_ids(n: int) -> np.ndarray:
    """Per-step ids that all say "read the precomputed row" (any negative value)."""
    return np.full(n, -1, dtype=np.int32)
