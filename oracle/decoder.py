"""Plain CPU forward pass of the Qwen3-style talker decoder, one position at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Sources, as pages of the
subject and the section each function follows:

* [P1] dev.to, "Porting a 1,200-line persistent CUDA megakernel to Qwen3-TTS":
  - "The idea: one kernel that never exits": the ops of one decode step
    (embedding lookup, attention, MLP, norms, sampling).
  - "Porting it to Qwen3-TTS-1.7B": untied embeddings (the final projection
    reads its own matrix) and multi-section rotary embeddings (the rotary
    pairs of a head are split into sections, each driven by its own position).
* [P3] theaicatchup, "I made a single CUDA kernel speak":
  - "Why Does a Single Kernel Even Matter for TTS?": the talker copies the
    Qwen3-0.6B body (so the Qwen3 layer: RMSNorm, per-head q/k RMSNorm, GQA,
    SwiGLU MLP, 28 layers); inputs are sums of 17 embeddings (16 codebooks +
    text); a non-negative id is a table lookup, a negative id means "take the
    precomputed row".
  - "So, What's the Catch with These Megakernels?": rotary frequencies come
    from host-side tables.

Readings where the pages are silent (each is listed with its basis in the
design notes): q/k norm over head_dim before the rotation; rotate-half pairing
(i, i + d/2); sections are contiguous runs of pairs with the global frequency
index; attention is causal over positions 0..p inclusive with scale 1/sqrt(d);
the KV cache stores bf16 (round-to-nearest-even) for bf16 bodies and attention
reads the rounded values back, including position p; ties in argmax go to the
lowest index; the 17 rows are summed in float32 in the order codebook 0..15,
then text.

Precision: float64 for all arithmetic by default.  Two quantities decide a
discrete result and are taken in the kernel's precision (float32) on both
sides: the bf16 rounding of K/V entries (value rounded to float32 first), and
the argmax over logits (logits rounded to float32 first).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np


# ---------------------------------------------------------------- bf16 helpers
def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bit patterns (uint16) to float32 exactly: bf16 is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value, ties to even, returned as float32.

    The value is first rounded to float32 (the kernel's precision for this
    decision), then the low 16 bits of its encoding are rounded away.  NaN stays
    NaN; overflow rounds to infinity as IEEE rounding does.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out.reshape(f.shape)


# ------------------------------------------------------------- the operations
def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """y = g * x / sqrt(mean(x^2) + eps) over the last axis (Qwen3 RMSNorm, [P3] body)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return g * (x / np.sqrt(ms + eps))


def rope_angles(positions: Sequence[int], sections: Sequence[int], head_dim: int,
                theta: float, dtype=np.float64):
    """cos and sin of the rotation angle of every rotary pair i < head_dim/2.

    Pair i turns at frequency theta^(-2i/d) (the global index i, not restarted
    per section) and is driven by the position of the section it falls in:
    sections are contiguous runs of pairs, run k reads positions[k] ([P1]
    "Porting it to Qwen3-TTS-1.7B": one band split into sections).  A single
    section covering all pairs is ordinary RoPE.
    """
    half = head_dim // 2
    if sum(sections) != half:
        raise ValueError(f"sections {tuple(sections)} must sum to head_dim/2 = {half}")
    pos_of_pair = np.empty(half, dtype=np.float64)
    start = 0
    for k, n in enumerate(sections):
        pos_of_pair[start:start + n] = float(positions[k])
        start += n
    i = np.arange(half, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / head_dim)
    ang = pos_of_pair * inv_freq
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rotate_half_apply(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pair (v_i, v_{i+d/2}) by the angle of pair i, over the last axis."""
    half = v.shape[-1] // 2
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def gqa_decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Softmax attention of one query position over cached positions.

    q: [n_q][d]; K, V: [n_kv][n_pos][d] (positions 0..p, the current one
    included).  Query head h reads KV head h // (n_q / n_kv).  Scores are
    q.K_j / sqrt(d); the softmax subtracts its maximum.
    """
    n_q, d = q.shape
    n_kv = K.shape[0]
    group = n_q // n_kv
    out = np.empty_like(q)
    for h in range(n_q):
        g = h // group
        s = (K[g] @ q[h]) / np.sqrt(d)
        w = np.exp(s - s.max())
        w /= w.sum()
        out[h] = w @ V[g]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def embed_sum17(codebooks: np.ndarray, text: np.ndarray, ids: Sequence[int]) -> np.ndarray:
    """One talker input row: sum of 16 codebook rows and one text row, in float32.

    codebooks: [16][C][H] (bf16 bits or float32); text: [T][H]; ids: 16 codebook
    ids then the text id.  The rows are widened to float32 and added one at a
    time, codebook 0 first and the text row last ([P3], sum of 17 embeddings).
    """
    def row(tbl, i):
        r = tbl[i]
        return bf16_bits_to_float(r) if r.dtype == np.uint16 else np.asarray(r, np.float32)

    n_cb = codebooks.shape[0]
    acc = row(codebooks[0], int(ids[0])).copy()
    for c in range(1, n_cb):
        acc = (acc + row(codebooks[c], int(ids[c]))).astype(np.float32)
    acc = (acc + row(text, int(ids[n_cb]))).astype(np.float32)
    return acc


def argmax_lowest(logits: np.ndarray) -> int:
    """Greedy pick on float32 logits; among equal maxima the lowest index wins."""
    l32 = np.asarray(logits, dtype=np.float32)
    return int(np.argmax(l32))   # numpy returns the first maximum


def top2_margin(logits: np.ndarray) -> float:
    """top1 - top2 of the float32 logits (0 when the maximum is repeated)."""
    l32 = np.asarray(logits, dtype=np.float32)
    top = np.partition(l32, -2)[-2:]
    return float(top[1] - top[0])


# ------------------------------------------------------------------ the model
def _widen(a, dtype):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = bf16_bits_to_float(a)
    return np.ascontiguousarray(a, dtype=dtype)


class Decoder:
    """The decoder with its KV cache; ``step`` runs one position.

    ``weights`` is the dict of ``persistent_megakernel_loop_amd.workload
    .make_weights`` (HF layout, [out][in]); bf16 arrays arrive as uint16 bit
    patterns and are widened exactly.  ``kv_dtype`` "bf16" rounds each cache
    entry to bf16 when it is written.
    """

    def __init__(self, n_layers: int, hidden: int, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, intermediate: int, vocab: int, tied: bool,
                 kv_dtype: str, rms_eps: float, rope_theta: float,
                 sections: Sequence[int], capacity: int,
                 weights: Dict[str, object], dtype=np.float64):
        if n_q_heads % n_kv_heads:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        if sum(sections) != head_dim // 2:
            raise ValueError("sections must cover head_dim/2 rotary pairs")
        self.L, self.H, self.nq, self.nkv, self.d = n_layers, hidden, n_q_heads, n_kv_heads, head_dim
        self.I, self.V, self.tied = intermediate, vocab, tied
        self.kv_bf16 = kv_dtype == "bf16"
        self.eps, self.theta, self.sections = float(rms_eps), float(rope_theta), tuple(sections)
        self.capacity, self.dtype = int(capacity), dtype
        W = lambda a: _widen(a, dtype)  # noqa: E731
        self.embed = W(weights["embed"])
        self.lm_head = self.embed if tied else W(weights["lm_head"])
        self.final_norm = W(weights["final_norm"])
        self.layers: List[Dict[str, np.ndarray]] = [
            {k: W(v) for k, v in lw.items()} for lw in weights["layers"]]
        self.K = np.zeros((n_layers, n_kv_heads, self.capacity, head_dim), dtype)
        self.V_ = np.zeros_like(self.K)
        self.pos = 0

    @classmethod
    def from_shape(cls, shape, weights, dtype=np.float64, capacity: Optional[int] = None,
                   kv_dtype: Optional[str] = None):
        return cls(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                   shape.intermediate, shape.vocab, shape.tied, kv_dtype or shape.kv_dtype,
                   shape.rms_eps, shape.rope_theta, shape.sections,
                   capacity if capacity is not None else shape.capacity, weights, dtype)

    # -- state
    def reset(self):
        self.K[:] = 0
        self.V_[:] = 0
        self.pos = 0

    def load_kv(self, kv: np.ndarray):
        """Install n pre-computed (already rotated) positions: kv is [L][2][n_kv][n][d]."""
        n = kv.shape[3]
        if n > self.capacity:
            raise ValueError("pre-fill exceeds the cache capacity")
        vals = _widen(kv, np.float32)
        self.K[:, :, :n] = vals[:, 0]
        self.V_[:, :, :n] = vals[:, 1]
        self.pos = n

    def _kvround(self, x):
        return bf16_round(x).astype(self.dtype) if self.kv_bf16 else x

    # -- one position
    def input_row(self, token_id: int, row: Optional[np.ndarray] = None) -> np.ndarray:
        """Sentinel rule: id >= 0 reads the embedding table, id < 0 the precomputed row."""
        if token_id >= 0:
            return self.embed[token_id].copy()
        if row is None:
            raise ValueError("a negative id needs a precomputed row")
        return np.asarray(row, dtype=np.float32).astype(self.dtype)

    def feedback_row(self, token_id: int, rest: np.ndarray) -> np.ndarray:
        """Greedy feedback with a precomputed row: the fed-back id's embedding plus the
        rest of the frame's embeddings ([P3] "Why Does a Single Kernel Even Matter for
        TTS?": the input is the sum of 16 codebook rows and a text row; the talker's own
        table gives the fed-back codebook-0 row, the caller sums the other 16)."""
        return self.embed[token_id] + np.asarray(rest, dtype=np.float32).astype(self.dtype)

    def step(self, x0: np.ndarray, pos3: Optional[Sequence[int]] = None,
             want_logits: bool = True):
        """Run position ``self.pos`` on input row x0.

        Returns (logits or None, hidden [L+1][H]) where hidden[0] is the input
        and hidden[l+1] the residual stream after layer l.
        """
        p = self.pos
        if p >= self.capacity:
            raise ValueError("KV cache full")
        streams = [p] * len(self.sections) if pos3 is None else [int(v) for v in pos3[:len(self.sections)]]
        cos, sin = rope_angles(streams, self.sections, self.d, self.theta, self.dtype)
        x = np.asarray(x0, dtype=self.dtype).copy()
        hidden = np.empty((self.L + 1, self.H), dtype=self.dtype)
        hidden[0] = x
        for l, w in enumerate(self.layers):
            a = rms_norm(x, w["in_norm"], self.eps)
            q = (w["wq"] @ a).reshape(self.nq, self.d)
            k = (w["wk"] @ a).reshape(self.nkv, self.d)
            v = (w["wv"] @ a).reshape(self.nkv, self.d)
            q = rotate_half_apply(rms_norm(q, w["q_norm"], self.eps), cos, sin)
            k = rotate_half_apply(rms_norm(k, w["k_norm"], self.eps), cos, sin)
            self.K[l, :, p] = self._kvround(k)
            self.V_[l, :, p] = self._kvround(v)
            o = gqa_decode_attention(q, self.K[l, :, :p + 1], self.V_[l, :, :p + 1])
            x = x + w["wo"] @ o.reshape(-1)
            b = rms_norm(x, w["post_norm"], self.eps)
            x = x + w["w_down"] @ (silu(w["w_gate"] @ b) * (w["w_up"] @ b))
            hidden[l + 1] = x
        self.pos = p + 1
        logits = None
        if want_logits:
            logits = self.lm_head @ rms_norm(x, self.final_norm, self.eps)
        return logits, hidden

    # -- runs
    def prefill(self, ids: Sequence[int], rows: Optional[np.ndarray] = None,
                pos3: Optional[np.ndarray] = None):
        """Run the prompt position by position; logits only at the last one.

        Returns (first_id, logits_last, hiddens [n][L+1][H]).
        """
        n = len(ids)
        hiddens = []
        logits = None
        for t in range(n):
            x0 = self.input_row(int(ids[t]), None if rows is None else rows[t])
            logits, h = self.step(x0, None if pos3 is None else pos3[t], want_logits=(t == n - 1))
            hiddens.append(h)
        first = argmax_lowest(logits) if logits is not None else None
        return first, logits, np.stack(hiddens) if hiddens else None

    def decode(self, ids: Sequence[int], rows: Optional[np.ndarray] = None,
               pos3: Optional[np.ndarray] = None):
        """Teacher-forced decode: step s reads ids[s] (or rows[s] when ids[s] < 0).

        Returns (ids_out [n], logits [n][V], hiddens [n][L+1][H]).
        """
        out, lg, hs = [], [], []
        for s in range(len(ids)):
            x0 = self.input_row(int(ids[s]), None if rows is None else rows[s])
            logits, h = self.step(x0, None if pos3 is None else pos3[s])
            out.append(argmax_lowest(logits))
            lg.append(logits)
            hs.append(h)
        return np.array(out, np.int32), np.stack(lg), np.stack(hs)

    def generate(self, first_id: int, n: int, pos3: Optional[np.ndarray] = None):
        """Free-running greedy decode: step s reads the id picked at step s-1."""
        cur, out = int(first_id), []
        for s in range(n):
            logits, _ = self.step(self.input_row(cur), None if pos3 is None else pos3[s])
            cur = argmax_lowest(logits)
            out.append(cur)
        return np.array(out, np.int32)
