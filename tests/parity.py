"""Run the HIP path and the oracle on the same seeded inputs and compare them.

Parity rule (per position): where the oracle's float32 top-1/top-2 logit margin
exceeds 0.05 the GPU id must equal the oracle's; otherwise the GPU id must
have an oracle logit within 0.05 of the top.  Every layer's residual stream,
at every position, must match to a relative L2 error of at most 1e-2.  The
oracle is replayed on the inputs the GPU actually consumed (teacher forcing),
so a near-tie resolved differently cannot derail the rest of the comparison.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from oracle import Decoder as OracleDecoder
from oracle import argmax_lowest, embed_sum17, top2_margin
from persistent_megakernel_loop_amd import workload as wl

MARGIN = 0.05
HIDDEN_RTOL = 1e-2


@dataclasses.dataclass
class Inputs:
    prompt_ids: Optional[np.ndarray]     # [P] ids (>=0 or sentinel)
    prompt_rows: Optional[np.ndarray]    # [P][H] float32
    prompt_pos3: Optional[np.ndarray]
    step_ids: Optional[np.ndarray]       # [n] or None for feedback
    step_rows: Optional[np.ndarray]
    step_pos3: Optional[np.ndarray]
    kv: Optional[np.ndarray]             # pre-filled cache
    n_steps: int


def make_inputs(shape, n_steps: Optional[int] = None, prompt_len: Optional[int] = None,
                kv_prefill: Optional[int] = None, talker_tables=None) -> Inputs:
    n = shape.steps if n_steps is None else n_steps
    P = shape.prompt_len if prompt_len is None else prompt_len
    K = shape.kv_prefill if kv_prefill is None else kv_prefill
    kv = wl.make_kv_prefill(shape, K) if K else None
    if shape.inputs == "ids":
        return Inputs(wl.make_prompt_ids(shape, P), None, None, None, None, None, kv, n)
    # talker: every position reads a summed 17-embedding row
    tables = talker_tables if talker_tables is not None else wl.make_talker_tables(shape.hidden)
    tids = wl.make_talker_ids(P + n)
    rows = np.stack([embed_sum17(tables["codebooks"], tables["text"], tids[t]) for t in range(P + n)])
    pos3 = wl.position_streams(K, P + n)
    return Inputs(wl.sentinel_ids(P) if P else None, rows[:P] if P else None, pos3[:P] if P else None,
                  wl.sentinel_ids(n), rows[P:], pos3[P:], kv, n)


@dataclasses.dataclass
class GpuRun:
    first_id: Optional[int]
    ids: np.ndarray          # [n] decode ids
    hidden: np.ndarray       # [P + n][L+1][H]
    trace: Optional[np.ndarray] = None


def run_gpu(shape, dev_weights, inp: Inputs, trace: bool = False, dec=None, batched: bool = False,
            phased: bool = False, prefill_path: Optional[int] = None) -> GpuRun:
    import torch
    from persistent_megakernel_loop_amd.binding import Decoder, to_device

    dev = "cuda"
    own = dec is None
    if own:
        dec = Decoder(shape, dev_weights)
    if prefill_path is not None:
        dec.set_prefill_path(prefill_path)
    L, H = shape.n_layers, shape.hidden
    P = 0 if inp.prompt_ids is None else len(inp.prompt_ids)
    n = inp.n_steps
    hid = torch.zeros(((P + n), L + 1, H), dtype=torch.float32, device=dev)
    tr = torch.zeros((max(P, n), 256, 2), dtype=torch.int64, device=dev) if trace else None
    if inp.kv is not None:
        dec.load_kv(to_device(inp.kv), inp.kv.shape[3])
    first = None
    t = lambda a, dt=None: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    if P:
        dec.set_debug(hid[:P], None)
        out = dec.prefill(t(inp.prompt_ids), t(inp.prompt_rows), t(inp.prompt_pos3), batched=batched)
        dec.check()
        first = int(out.cpu()[0])
    dec.set_debug(hid[P:], tr)
    ids = (dec.decode_phased if phased else dec.decode)(n, t(inp.step_ids), t(inp.step_rows), t(inp.step_pos3))
    dec.check()
    torch.cuda.synchronize()
    res = GpuRun(first, ids.cpu().numpy().astype(np.int32), hid.cpu().numpy(),
                 tr.cpu().numpy() if trace else None)
    dec.set_debug(None, None)
    if own:
        dec.close()
    return res


@dataclasses.dataclass
class OracleRun:
    first_id: Optional[int]
    first_logits: Optional[np.ndarray]
    logits: np.ndarray       # [n][V]
    hidden: np.ndarray       # [P + n][L+1][H]


def run_oracle(shape, weights, inp: Inputs, gpu: GpuRun, dtype=np.float64, steps: Optional[int] = None,
               logits_every: int = 1) -> OracleRun:
    """Teacher-forced replay of the GPU's realised inputs (feedback ids come from the GPU).

    Every position's hidden states are computed; logits only at decode steps s with
    s % logits_every == 0 and at the last step (rows of NaN elsewhere), since a large
    LM head dominates the oracle's time."""
    dec = OracleDecoder.from_shape(shape, weights, dtype=dtype)
    if inp.kv is not None:
        dec.load_kv(inp.kv)
    hid = []
    first = first_logits = None
    P = 0 if inp.prompt_ids is None else len(inp.prompt_ids)
    if P:
        first, first_logits, hp = dec.prefill(inp.prompt_ids, inp.prompt_rows, inp.prompt_pos3)
        hid.extend(hp)
    n = inp.n_steps if steps is None else steps
    if inp.step_ids is None:  # greedy feedback: step s reads the GPU's id of step s-1
        prev = [gpu.first_id] + list(gpu.ids[:-1])
        ids = np.array(prev[:n], np.int32)
    else:
        ids = inp.step_ids[:n]
    logits = np.full((n, shape.vocab), np.nan)
    for s in range(n):
        if inp.step_ids is None and inp.step_rows is not None:  # feedback id + the frame's other rows
            x0 = dec.feedback_row(int(ids[s]), inp.step_rows[s])
        else:
            x0 = dec.input_row(int(ids[s]), None if inp.step_rows is None else inp.step_rows[s])
        want = s % logits_every == 0 or s == n - 1
        lg, h = dec.step(x0, None if inp.step_pos3 is None else inp.step_pos3[s], want_logits=want)
        if want:
            logits[s] = lg
        hid.append(h)
    return OracleRun(first, first_logits, logits, np.stack(hid))


def check_id(gpu_id: int, logits: np.ndarray, where: str):
    l32 = np.asarray(logits, np.float32)
    top = argmax_lowest(l32)
    m = top2_margin(l32)
    if m > MARGIN:
        assert gpu_id == top, f"{where}: id {gpu_id} != oracle {top} (margin {m:.4f})"
    else:
        assert 0 <= gpu_id < len(l32) and l32[gpu_id] >= l32[top] - MARGIN, \
            f"{where}: id {gpu_id} logit {l32[gpu_id]:.5f} below oracle top {l32[top]:.5f} - {MARGIN}"
    return m > MARGIN


def compare(gpu: GpuRun, orc: OracleRun, n_steps: Optional[int] = None):
    """Assert the parity rule; returns a summary dict."""
    n = orc.logits.shape[0] if n_steps is None else n_steps
    strict = 0
    if orc.first_logits is not None:
        strict += check_id(gpu.first_id, orc.first_logits, "prefill")
    checked = 0
    for s in range(n):
        if np.isnan(orc.logits[s, 0]):
            continue
        strict += check_id(int(gpu.ids[s]), orc.logits[s], f"step {s}")
        checked += 1
    npos = orc.hidden.shape[0]
    g, o = gpu.hidden[:npos].astype(np.float64), orc.hidden
    err = np.linalg.norm(g - o, axis=-1) / np.maximum(np.linalg.norm(o, axis=-1), 1e-30)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= HIDDEN_RTOL, f"hidden rel-L2 {err.max():.3e} at position {worst[0]} layer {worst[1]}"
    return {"ids_checked": checked, "strict_ids": strict, "max_hidden_rel_l2": float(err.max()), "median_hidden_rel_l2": float(np.median(err))}


def check_free_run(shape, weights, inp: Inputs, gpu: GpuRun, orc: OracleRun, dtype=np.float64):
    """The oracle's own free-running greedy decode (``Decoder.generate``) from its own
    prefill gives the GPU's ids up to the first position whose oracle top-1/top-2 margin
    is at most MARGIN (there the two may legitimately part).  Greedy-feedback workloads
    (ids inputs) only.  Returns the number of ids compared."""
    assert inp.step_ids is None and inp.step_rows is None and inp.prompt_ids is not None
    dec = OracleDecoder.from_shape(shape, weights, dtype=dtype)
    if inp.kv is not None:
        dec.load_kv(inp.kv)
    first, first_logits, _ = dec.prefill(inp.prompt_ids)
    if top2_margin(first_logits) <= MARGIN:
        return 0
    assert first == gpu.first_id, f"prefill: oracle {first} != gpu {gpu.first_id}"
    # the teacher-forced replay read the GPU's ids, so its margins are the free run's up to
    # the first difference: ids before the first low-margin step are strict
    n = orc.logits.shape[0]
    m = n
    for s in range(n):
        if np.isnan(orc.logits[s, 0]) or top2_margin(orc.logits[s]) <= MARGIN:
            m = s
            break
    free = dec.generate(first, m)
    assert np.array_equal(free, gpu.ids[:m]), f"the oracle's free run parts from the GPU's ids before step {m}"
    return m
