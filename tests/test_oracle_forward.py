"""Pins for the oracle's whole decode step.

* transformers' Qwen3 decoder (float64, eager attention, our weights) run over
  the full sequence with no cache must give the oracle's per-position logits
  and per-layer residual stream: pins q/k norm, rotate-half RoPE, the GQA map,
  SwiGLU, the residual wiring, the tied head and the KV-cache bookkeeping.
* the same model with Qwen2-VL's multi-section rotation, an untied head and
  summed-row inputs pins the talker's differences.
* a brute-force recompute of a 1-layer toy (no cache, every position redone)
  pins the cache with bf16 rounding.
* the sentinel, tied/untied and "one section is RoPE" equivalences the pages
  state hold bit-exactly.
"""
import numpy as np
import pytest
import torch

from oracle import Decoder, argmax_lowest, bf16_round, embed_sum17, rms_norm, silu
from persistent_megakernel_loop_amd import workload as wl
from tests.hf_pins import layer_outputs, multimodal_rotary, qwen3_from_weights

SMALL_TEXT = wl.TINY
WIDE_TEXT = wl.TEXT_0P6B.replace(name="wide-2l", n_layers=2, vocab=1000, prompt_len=6, steps=6)


def _run_oracle(shape, weights, ids_prompt, n_steps, kv_dtype="f32"):
    dec = Decoder.from_shape(shape, weights, kv_dtype=kv_dtype)
    first, _, hp = dec.prefill(ids_prompt)
    seq = [first]
    logits_all, hid_all = [], [hp[-1]]
    for s in range(n_steps):
        lg, h = dec.step(dec.input_row(seq[-1]))
        logits_all.append(lg)
        hid_all.append(h)
        seq.append(argmax_lowest(lg))
    return seq, np.stack(logits_all), np.stack(hid_all)


@pytest.mark.parametrize("shape", [SMALL_TEXT, WIDE_TEXT, SMALL_TEXT.replace(name="gains")],
                         ids=["tiny", "wide", "tiny-gains"])
def test_text_forward_matches_transformers_qwen3(shape):
    weights = wl.make_weights(shape, random_gains=(shape.name == "gains"))
    prompt = wl.make_prompt_ids(shape)
    n = min(shape.steps, 8)
    seq, logits, hid = _run_oracle(shape, weights, prompt, n)
    full = np.concatenate([prompt, np.array(seq[:-1], np.int32)])   # every input position
    m = qwen3_from_weights(shape, weights)
    outs, rm = layer_outputs(m)
    with torch.no_grad():
        ref = m(input_ids=torch.from_numpy(full.astype(np.int64))[None]).logits[0].numpy()
    rm()
    P = len(prompt)
    # logits at the last prompt position and at every decode position
    ref_dec = ref[P:]
    assert ref_dec.shape == logits.shape
    scale = np.abs(ref_dec).max()
    assert np.max(np.abs(logits - ref_dec)) <= 1e-5 * scale
    assert argmax_lowest(ref[P - 1]) == seq[0]
    # residual stream after every layer, at the decode positions
    for l in range(shape.n_layers):
        r_l = outs[l][0, P - 1:].numpy()
        o_l = hid[:, l + 1]
        assert np.max(np.abs(o_l - r_l)) <= 1e-5 * np.abs(r_l).max()


def _talker_small():
    return wl.TALKER_0P6B.replace(name="talker-2l", n_layers=2, hidden=256, n_q_heads=4,
                                  n_kv_heads=2, head_dim=64, intermediate=768, vocab=300,
                                  sections=(12, 10, 10), prompt_len=5, steps=7)


def test_talker_forward_matches_transformers_with_multimodal_rotary():
    shape = _talker_small()
    weights = wl.make_weights(shape)
    n = shape.prompt_len + shape.steps
    tables = wl.make_talker_tables(shape.hidden, text_vocab=500, codebook_size=64)
    tids = wl.make_talker_ids(n, text_vocab=500, codebook_size=64)
    rows = np.stack([embed_sum17(tables["codebooks"], tables["text"], tids[t]) for t in range(n)])
    pos3 = wl.position_streams(0, n)
    dec = Decoder.from_shape(shape, weights, kv_dtype="f32")
    ids = wl.sentinel_ids(n)
    logits, hid = [], []
    for t in range(n):
        lg, h = dec.step(dec.input_row(int(ids[t]), rows[t]), pos3[t])
        logits.append(lg)
        hid.append(h)
    logits, hid = np.stack(logits), np.stack(hid)

    m = qwen3_from_weights(shape, weights)
    assert m.lm_head.weight.data_ptr() != m.model.embed_tokens.weight.data_ptr()
    outs, rm = layer_outputs(m)
    with torch.no_grad(), multimodal_rotary(m, shape.sections):
        pid = torch.from_numpy(pos3.T.astype(np.int64).copy())[:, None, :]
        ref = m(inputs_embeds=torch.from_numpy(rows.astype(np.float64))[None], position_ids=pid).logits[0].numpy()
    rm()
    assert np.max(np.abs(logits - ref)) <= 1e-5 * np.abs(ref).max()
    for l in range(shape.n_layers):
        r_l = outs[l][0].numpy()
        assert np.max(np.abs(hid[:, l + 1] - r_l)) <= 1e-5 * np.abs(r_l).max()
    # a section mix-up fails the tolerance above: swapping two streams moves the logits well past it
    dec2 = Decoder.from_shape(shape, weights, kv_dtype="f32")
    lg2 = [dec2.step(dec2.input_row(-1, rows[t]), pos3[t][[0, 2, 1]])[0] for t in range(n)]
    assert np.max(np.abs(np.stack(lg2) - ref)) > 10 * 1e-5 * np.abs(ref).max()


def _brute_force_1layer(w, x_rows, n_q, n_kv, d, eps, theta, kv_bf16):
    """Full causal recompute at every step, with plain loops and no cache object.

    K/V of every earlier position are rebuilt from scratch each time.
    """
    T = len(x_rows)
    outs = []
    for t in range(T):
        Ks, Vs = [], []
        for j in range(t + 1):
            a = rms_norm(x_rows[j], w["in_norm"], eps)
            k = (w["wk"] @ a).reshape(n_kv, d)
            v = (w["wv"] @ a).reshape(n_kv, d)
            k = rms_norm(k, w["k_norm"], eps)
            kr = np.empty_like(k)
            for g in range(n_kv):
                for i in range(d // 2):
                    ang = j * theta ** (-2.0 * i / d)
                    c, s = np.cos(ang), np.sin(ang)
                    kr[g, i] = k[g, i] * c - k[g, i + d // 2] * s
                    kr[g, i + d // 2] = k[g, i + d // 2] * c + k[g, i] * s
            if kv_bf16:
                kr, v = bf16_round(kr).astype(np.float64), bf16_round(v).astype(np.float64)
            Ks.append(kr)
            Vs.append(v)
        a = rms_norm(x_rows[t], w["in_norm"], eps)
        q = rms_norm((w["wq"] @ a).reshape(n_q, d), w["q_norm"], eps)
        o = np.zeros((n_q, d))
        for h in range(n_q):
            g = h // (n_q // n_kv)
            qr = np.empty(d)
            for i in range(d // 2):
                ang = t * theta ** (-2.0 * i / d)
                c, s = np.cos(ang), np.sin(ang)
                qr[i] = q[h, i] * c - q[h, i + d // 2] * s
                qr[i + d // 2] = q[h, i + d // 2] * c + q[h, i] * s
            sc = np.array([qr @ Ks[j][g] for j in range(t + 1)]) / np.sqrt(d)
            e = np.exp(sc - sc.max())
            p = e / e.sum()
            o[h] = sum(p[j] * Vs[j][g] for j in range(t + 1))
        x = x_rows[t] + w["wo"] @ o.reshape(-1)
        b = rms_norm(x, w["post_norm"], eps)
        x = x + w["w_down"] @ (silu(w["w_gate"] @ b) * (w["w_up"] @ b))
        outs.append(x)
    return np.stack(outs)


@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_one_layer_toy_against_brute_force(kv):
    shape = wl.DecoderShape("toy", 1, 64, 4, 2, 16, 96, 50, True, "f32", kv, 1e-6, 1e4, (8,), 0, 0, "ids",
                            max_seq=12)
    weights = wl.make_weights(shape, random_gains=True)
    wd = {k: np.asarray(v, np.float64) for k, v in weights["layers"][0].items()}
    rows = np.random.default_rng(13).standard_normal((12, 64)).astype(np.float32) * 3
    dec = Decoder.from_shape(shape, weights)
    got = np.stack([dec.step(dec.input_row(-1, rows[t]), want_logits=False)[1][1] for t in range(12)])
    ref = _brute_force_1layer(wd, rows.astype(np.float64), 4, 2, 16, 1e-6, 1e4, kv == "bf16")
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.abs(ref).max()


def test_sentinel_row_equals_table_lookup_bit_exact():
    """Backward compatible: a row equal to the embedding row gives the token path's result exactly."""
    shape = WIDE_TEXT
    weights = wl.make_weights(shape)
    ids = wl.make_prompt_ids(shape)
    a = Decoder.from_shape(shape, weights)
    b = Decoder.from_shape(shape, weights)
    fa, la, ha = a.prefill(ids)
    rows = np.stack([a.embed[i].astype(np.float32) for i in ids])
    fb, lb, hb = b.prefill(wl.sentinel_ids(len(ids)), rows)
    assert fa == fb and np.array_equal(la, lb) and np.array_equal(ha, hb)


def test_sentinel_path_equals_explicit_17_table_sum():
    shape = _talker_small()
    weights = wl.make_weights(shape)
    tables = wl.make_talker_tables(shape.hidden, text_vocab=500, codebook_size=64)
    tids = wl.make_talker_ids(4, text_vocab=500, codebook_size=64)
    rows = np.stack([embed_sum17(tables["codebooks"], tables["text"], t) for t in tids])
    # the explicit sum, widened to float64 from the float32 definition and fed as a sentinel row
    explicit = []
    for t in tids:
        acc = np.zeros(shape.hidden, np.float32)
        for c in range(16):
            acc = acc + wl_bf16(tables["codebooks"][c, t[c]])
        acc = acc + wl_bf16(tables["text"][t[16]])
        explicit.append(acc)
    assert np.array_equal(rows, np.stack(explicit))
    d1 = Decoder.from_shape(shape, weights)
    d2 = Decoder.from_shape(shape, weights)
    pos3 = wl.position_streams(0, 4)
    for t in range(4):
        l1, h1 = d1.step(d1.input_row(-1, rows[t]), pos3[t])
        l2, h2 = d2.step(np.asarray(explicit[t], np.float64), pos3[t])
        assert np.array_equal(l1, l2) and np.array_equal(h1, h2)


def wl_bf16(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()


def test_untied_head_equal_to_embedding_reproduces_tied():
    shape = WIDE_TEXT
    weights = wl.make_weights(shape)
    untied = dict(weights, lm_head=weights["embed"].copy())
    a = Decoder.from_shape(shape, weights)
    b = Decoder.from_shape(shape.replace(tied=False), untied)
    ids = wl.make_prompt_ids(shape)
    fa, la, _ = a.prefill(ids)
    fb, lb, _ = b.prefill(ids)
    assert fa == fb and np.array_equal(la, lb)


def test_prefilled_cache_is_read_as_is():
    """Positions installed by load_kv are attended to exactly as given (already rotated)."""
    shape = wl.DecoderShape("toy", 1, 64, 4, 2, 16, 96, 50, False, "f32", "bf16", 1e-6, 1e6, (4, 2, 2),
                            0, 3, "talker", kv_prefill=5)
    weights = wl.make_weights(shape)
    kv = wl.make_kv_prefill(shape)
    dec = Decoder.from_shape(shape, weights)
    dec.load_kv(kv)
    assert dec.pos == 5
    Kf = wl_bf16(kv[0, 0])
    assert np.array_equal(dec.K[0, :, :5], Kf)
    row = np.random.default_rng(14).standard_normal(64).astype(np.float32)
    _, h = dec.step(dec.input_row(-1, row), (5, 2, 1), want_logits=False)
    assert np.all(np.isfinite(h)) and dec.pos == 6


def test_feedback_row_is_the_17_row_sum_with_the_fed_back_codebook0_row():
    """Greedy feedback with rows: when the talker's embedding table holds codebook 0,
    feedback_row(id, rest) is the 17-row input sum with codebook 0 at the fed-back id,
    rest being the other 16 rows (codebooks 1..15 and text), up to the order of the
    float32 additions."""
    shape = _talker_small()
    weights = wl.make_weights(shape)
    tables = wl.make_talker_tables(shape.hidden, text_vocab=500, codebook_size=64)
    cb0 = tables["codebooks"][0]
    dec = Decoder.from_shape(shape, weights)
    dec.embed = np.stack([wl_bf16(cb0[i]) for i in range(cb0.shape[0])]).astype(np.float64)
    zero0 = tables["codebooks"].copy()
    zero0[0] = 0  # bf16 bits of +0.0: the sum without codebook 0
    for t in wl.make_talker_ids(6, text_vocab=500, codebook_size=64):
        full = embed_sum17(tables["codebooks"], tables["text"], t)
        rest = embed_sum17(zero0, tables["text"], t)
        got = dec.feedback_row(int(t[0]), rest)
        np.testing.assert_allclose(got, full, rtol=1e-6, atol=1e-7)
        # a plausible slip (the row of another id, or no row at all) is caught
        assert not np.allclose(dec.feedback_row(int(t[0]) ^ 1, rest), full, rtol=1e-6, atol=1e-7)
        assert not np.allclose(rest, full, rtol=1e-6, atol=1e-7)


def test_generate_matches_transformers_greedy_generate():
    """Decoder.generate (the free-running greedy loop) against transformers' own greedy
    generate on the same weights: an untied tiny decoder whose head is scaled so every
    step's top-1/top-2 margin is decisive, and whose ids vary (a loop that fed back the
    wrong id, or the same id, would diverge)."""
    shape = wl.TINY.replace(name="tiny-untied-gen", tied=False, vocab=300)
    weights = wl.make_weights(shape)
    weights["lm_head"] = (np.asarray(weights["lm_head"], np.float32) * 40.0).astype(np.float32)
    prompt = wl.make_prompt_ids(shape)
    n = 24
    dec = Decoder.from_shape(shape, weights)
    first, logits, _ = dec.prefill(prompt)
    ours = [first] + list(dec.generate(first, n - 1))
    m = qwen3_from_weights(shape, weights)
    with torch.no_grad():
        g = m.generate(torch.from_numpy(prompt.astype(np.int64))[None], max_new_tokens=n, do_sample=False,
                       output_scores=True, return_dict_in_generate=True, pad_token_id=0)
    ref = g.sequences[0, len(prompt):].tolist()
    margins = [float(np.diff(np.sort(s[0].numpy())[-2:])[0]) for s in g.scores]
    assert min(margins) > 1e-3, margins
    assert len(set(ref)) >= 6 and sum(a != b for a, b in zip(ref, ref[1:])) >= n // 2, ref
    assert ours == ref
