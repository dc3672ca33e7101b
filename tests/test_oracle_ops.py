"""Pins for the oracle's single operations, against closed forms, invariants and library routines.

Each test would fail on a plausible slip in the oracle: a dropped epsilon or
gain, a wrong rotation sign or pairing, a section mapped to the wrong stream, a
wrong GQA head map, a missing softmax max-shift, a rounding mode other than
nearest-even.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (argmax_lowest, bf16_bits_to_float, bf16_round, embed_sum17,
                    gqa_decode_attention, rms_norm, rope_angles, rotate_half_apply, silu,
                    top2_margin)


# ------------------------------------------------------------------ bf16
def test_bf16_widen_matches_torch():
    bits = np.random.default_rng(0).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    bits[:4] = [0x0000, 0x8000, 0x7F80, 0xFF80]          # +-0, +-inf
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = bf16_bits_to_float(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_bf16_round_nearest_even_matches_torch():
    r = np.random.default_rng(1)
    x = np.concatenate([
        r.standard_normal(100000).astype(np.float32),
        (r.standard_normal(1000) * 1e30).astype(np.float32),
        (r.standard_normal(1000) * 1e-30).astype(np.float32),
        # exact ties: low 16 bits == 0x8000, with both parities of the kept lsb
        (np.arange(2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([3.0e38, -3.0e38, 0.0, -0.0], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_round_ties_go_to_even():
    # 1 + 2^-8 lies half way between bf16 1.0 and 1 + 2^-7: even mantissa (1.0) wins.
    assert bf16_round(np.float32(1 + 2 ** -8)) == np.float32(1.0)
    # 1 + 3*2^-8 lies half way between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert bf16_round(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)


# ------------------------------------------------------------------ RMSNorm
def test_rms_norm_closed_form_constant_vector():
    for c in (0.5, -3.0, 1e-4):
        x = np.full(64, c)
        y = rms_norm(x, np.ones(64), 1e-6)
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-14)


def test_rms_norm_gain_and_eps_against_torch():
    r = np.random.default_rng(2)
    x, g = r.standard_normal((5, 96)), r.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-15)
    # epsilon matters for small vectors
    small = x * 1e-4
    ref2 = torch.nn.functional.rms_norm(torch.from_numpy(small), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(rms_norm(small, g, 1e-6), ref2, rtol=1e-13, atol=1e-15)


def test_rms_norm_scale_invariant_without_eps():
    x = np.random.default_rng(3).standard_normal(128)
    assert np.allclose(rms_norm(7.5 * x, np.ones(128), 0.0), rms_norm(x, np.ones(128), 0.0), rtol=1e-14)
    assert np.isclose(np.sqrt(np.mean(rms_norm(x, np.ones(128), 0.0) ** 2)), 1.0)


# ------------------------------------------------------------------ RoPE / MRoPE
def test_rope_preserves_norm_and_is_identity_at_zero():
    r = np.random.default_rng(4)
    v = r.standard_normal((3, 128))
    for pos in (0, 1, 17, 4095):
        c, s = rope_angles([pos], [64], 128, 1e6)
        y = rotate_half_apply(v, c, s)
        assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-13)
        if pos == 0:
            assert np.array_equal(y, v)


def test_rope_relative_position_invariance():
    r = np.random.default_rng(5)
    q, k = r.standard_normal(64), r.standard_normal(64)

    def dot(m, n):
        cm, sm = rope_angles([m], [32], 64, 1e4)
        cn, sn = rope_angles([n], [32], 64, 1e4)
        return rotate_half_apply(q, cm, sm) @ rotate_half_apply(k, cn, sn)

    assert np.isclose(dot(10, 3), dot(107, 100), rtol=1e-10)
    assert np.isclose(dot(3, 10), dot(0, 7), rtol=1e-10)
    assert not np.isclose(dot(10, 3), dot(10, 4), rtol=1e-3)


def test_rope_one_hot_pair_turns_by_its_own_angle():
    d, theta, pos = 64, 1e4, 9
    c, s = rope_angles([pos], [32], d, theta)
    for i in (0, 1, 15, 31):
        e = np.zeros(d)
        e[i] = 1.0
        y = rotate_half_apply(e, c, s)
        ang = pos * theta ** (-2.0 * i / d)
        want = np.zeros(d)
        want[i], want[i + d // 2] = math.cos(ang), math.sin(ang)
        assert np.allclose(y, want, atol=1e-14)


def test_rope_matches_transformers_qwen3():
    from transformers.models.qwen3.modeling_qwen3 import apply_rotary_pos_emb, Qwen3RotaryEmbedding
    from transformers import Qwen3Config

    cfg = Qwen3Config(hidden_size=256, num_attention_heads=2, head_dim=128,
                      rope_parameters={"rope_type": "default", "rope_theta": 1e6})
    rot = Qwen3RotaryEmbedding(cfg)
    r = np.random.default_rng(6)
    q = r.standard_normal((1, 2, 5, 128))
    k = r.standard_normal((1, 2, 5, 128))
    pos = torch.tensor([[0, 1, 2, 100, 301]])
    cos, sin = rot(torch.zeros(1, dtype=torch.float64), pos)
    hq, hk = apply_rotary_pos_emb(torch.from_numpy(q), torch.from_numpy(k), cos.double(), sin.double())
    for t, p in enumerate(pos[0].tolist()):
        c, s = rope_angles([p], [64], 128, 1e6)
        # transformers builds its angles in float32: allow that rounding
        assert np.allclose(rotate_half_apply(q[0, :, t], c, s), hq[0, :, t].numpy(), atol=5e-5)
        assert np.allclose(rotate_half_apply(k[0, :, t], c, s), hk[0, :, t].numpy(), atol=5e-5)


def test_mrope_one_section_and_equal_streams_reduce_to_rope():
    c1, s1 = rope_angles([37], [64], 128, 1e6)
    c3, s3 = rope_angles([37, 37, 37], [24, 20, 20], 128, 1e6)
    assert np.array_equal(c1, c3) and np.array_equal(s1, s3)


def test_mrope_sections_read_their_own_stream():
    d, theta, pos3, secs = 128, 1e6, (40, 20, 13), (24, 20, 20)
    c, s = rope_angles(pos3, secs, d, theta)
    bounds = np.cumsum((0,) + secs)
    for k in range(3):
        for i in (bounds[k], bounds[k + 1] - 1):
            ang = pos3[k] * theta ** (-2.0 * i / d)
            assert math.isclose(c[i], math.cos(ang), abs_tol=1e-14)
            assert math.isclose(s[i], math.sin(ang), abs_tol=1e-14)


def test_mrope_layout_matches_transformers_qwen2_vl():
    """Qwen2-VL's multimodal rotation (used as a black box) has the same section layout."""
    from transformers import Qwen2VLTextConfig
    from transformers.models.qwen2_vl import modeling_qwen2_vl as q2

    secs = [24, 20, 20]
    cfg = Qwen2VLTextConfig(hidden_size=2048, num_attention_heads=16, num_key_value_heads=8,
                            rope_parameters={"rope_type": "default", "rope_theta": 1e6,
                                             "mrope_section": secs})
    cfg.head_dim = 128
    rot = q2.Qwen2VLRotaryEmbedding(cfg)
    pos3 = np.array([[300, 150, 100], [7, 3, 2], [0, 5, 9]])
    pid = torch.from_numpy(pos3.T.copy())[:, None, :]               # (3 streams, batch 1, seq)
    cos, sin = rot(torch.zeros(1, dtype=torch.float64), pid)
    r = np.random.default_rng(7)
    q = r.standard_normal((1, 2, 3, 128))
    k = r.standard_normal((1, 2, 3, 128))
    hq, hk = q2.apply_multimodal_rotary_pos_emb(torch.from_numpy(q), torch.from_numpy(k),
                                                cos.double(), sin.double(), secs)
    for t in range(3):
        c, s = rope_angles(pos3[t], secs, 128, 1e6)
        assert np.allclose(rotate_half_apply(q[0, :, t], c, s), hq[0, :, t].numpy(), atol=5e-5)
        assert np.allclose(rotate_half_apply(k[0, :, t], c, s), hk[0, :, t].numpy(), atol=5e-5)


def test_rope_rejects_bad_sections():
    with pytest.raises(ValueError):
        rope_angles([0, 0, 0], [24, 20, 19], 128, 1e6)


# ------------------------------------------------------------------ attention
def _sdpa_ref(q, K, V):
    n_q, n_kv = q.shape[0], K.shape[0]
    Kr = np.repeat(K, n_q // n_kv, axis=0)
    Vr = np.repeat(V, n_q // n_kv, axis=0)
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], torch.from_numpy(Kr), torch.from_numpy(Vr))
    return out[:, 0, :].numpy()


@pytest.mark.parametrize("n_q,n_kv,n_pos", [(4, 2, 9), (16, 8, 300), (4, 4, 5), (8, 1, 33)])
def test_attention_matches_torch_sdpa(n_q, n_kv, n_pos):
    r = np.random.default_rng(8)
    q = r.standard_normal((n_q, 64)) * 3
    K, V = r.standard_normal((n_kv, n_pos, 64)), r.standard_normal((n_kv, n_pos, 64))
    assert np.allclose(gqa_decode_attention(q, K, V), _sdpa_ref(q, K, V), rtol=1e-12, atol=1e-13)


def test_attention_invariants():
    r = np.random.default_rng(9)
    q = r.standard_normal((4, 64))
    K, V = r.standard_normal((2, 7, 64)), r.standard_normal((2, 7, 64))
    # weights sum to one: all-ones values give all-ones output
    assert np.allclose(gqa_decode_attention(q, K, np.ones_like(V)), 1.0, rtol=1e-14)
    # one position: the output is that position's value row, per group
    o1 = gqa_decode_attention(q, K[:, :1], V[:, :1])
    assert np.allclose(o1, np.repeat(V[:, 0], 2, axis=0), rtol=1e-14)
    # equal scores: the output is the mean value row
    o0 = gqa_decode_attention(np.zeros_like(q), K, V)
    assert np.allclose(o0, np.repeat(V.mean(axis=1), 2, axis=0), rtol=1e-13)
    # huge scores do not overflow (max-shift)
    big = gqa_decode_attention(q * 1e4, K, V)
    assert np.all(np.isfinite(big))


def test_attention_gqa_head_map():
    """Query head h reads KV head h // (n_q / n_kv): heads 0,1 -> kv 0; heads 2,3 -> kv 1."""
    r = np.random.default_rng(10)
    q = r.standard_normal((4, 8))
    K = r.standard_normal((2, 3, 8))
    V = np.stack([np.zeros((3, 8)), np.ones((3, 8))])
    o = gqa_decode_attention(q, K, V)
    assert np.allclose(o[:2], 0.0) and np.allclose(o[2:], 1.0)


# ------------------------------------------------------------------ misc ops
def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_embed_sum17_exact_on_integer_grid():
    """On values of a coarse binary grid every float32 partial sum is exact: the sum equals the fp64 sum."""
    r = np.random.default_rng(11)
    cb = (r.integers(-64, 64, size=(16, 10, 32)) / 256.0).astype(np.float32)
    tx = (r.integers(-64, 64, size=(20, 32)) / 256.0).astype(np.float32)
    ids = list(r.integers(0, 10, size=16)) + [int(r.integers(0, 20))]
    want = sum(cb[c, ids[c]].astype(np.float64) for c in range(16)) + tx[ids[16]]
    assert np.array_equal(embed_sum17(cb, tx, ids), want.astype(np.float32))


def test_embed_sum17_reads_bf16_and_orders_adds():
    r = np.random.default_rng(12)
    cb32 = r.standard_normal((16, 8, 64)).astype(np.float32)
    cbb = torch.from_numpy(cb32).to(torch.bfloat16)
    tx = torch.from_numpy(r.standard_normal((9, 64)).astype(np.float32)).to(torch.bfloat16)
    ids = [int(v) for v in r.integers(0, 8, size=16)] + [4]
    got = embed_sum17(cbb.view(torch.int16).numpy().view(np.uint16),
                      tx.view(torch.int16).numpy().view(np.uint16), ids)
    # codebook 0 first, one float32 add at a time, the text row last
    acc = torch.zeros(64, dtype=torch.float32) + cbb[0, ids[0]].float()
    for c in range(1, 16):
        acc = acc + cbb[c, ids[c]].float()
    acc = acc + tx[4].float()
    assert np.array_equal(got, acc.numpy())
    # a single codebook rearranged changes the rounding, so order is pinned by the exact compare above
    assert got.dtype == np.float32


def test_argmax_ties_lowest_and_margin():
    l = np.array([0.1, 3.0, -1.0, 3.0, 2.5], np.float32)
    assert argmax_lowest(l) == 1
    assert top2_margin(l) == 0.0
    l2 = np.array([0.1, 3.0, -1.0, 2.0], np.float32)
    assert argmax_lowest(l2) == 1 and math.isclose(top2_margin(l2), 1.0)
    # float64 logits that differ only below float32 resolution tie in float32
    l3 = np.array([1.0, 1.0 + 1e-12], np.float64)
    assert argmax_lowest(l3) == 0
