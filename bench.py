"""Benchmark: batch-1 persistent-kernel decode of the 0.6B-shaped TTS talker on one MI355X.

    python bench.py [--gpus 1] [--steps 256] [--warmup 2] [--workload talker-0.6b]

One "step" is one decode step (one position through all layers, the LM head and
the argmax).  The timed region is ONE mk_decode launch of --steps steps whose
inputs (summed 17-embedding rows, rotary position streams) already sit in HBM;
the 32-row prompt is prefilled, untimed, before it.  Prints one JSON line.

Roofline: the decode kernel is bound by HBM.  Its algorithmic bytes per step are
every weight byte it reads (all layers, norms, LM head) plus the KV cache bytes
of positions 0..p; achieved GB/s = those bytes over the launch, divided by the
launch time measured with HIP events on the launch stream.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from persistent_megakernel_loop_amd import workload as wl  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "batch-1 decode ms/step + achieved HBM GB/s (% of peak); TTFC for first chunk"
FRAME_MS = 80.0  # one talker step = one 12.5 Hz codec frame


def weight_bytes_per_step(s: wl.DecoderShape) -> int:
    """Bytes of weights one decode step reads (the input row excluded)."""
    wb = 2 if s.weight_dtype == "bf16" else 4
    H, D, I, V = s.hidden, s.head_dim, s.intermediate, s.vocab
    layer = (s.n_q_heads * D * H + 2 * s.n_kv_heads * D * H + H * s.n_q_heads * D + 3 * I * H)
    norms = 2 * H + 2 * D
    return (s.n_layers * (layer + norms) + V * H + H) * wb


def kv_bytes_per_position(s: wl.DecoderShape) -> int:
    return 2 * s.n_layers * s.n_kv_heads * s.head_dim * (2 if s.kv_dtype == "bf16" else 4)


def step_bytes(s: wl.DecoderShape, first_pos: int, n: int) -> int:
    """Algorithmic bytes of n decode steps at positions first_pos .. first_pos+n-1."""
    kv = kv_bytes_per_position(s) * sum(p + 1 for p in range(first_pos, first_pos + n))
    return weight_bytes_per_step(s) * n + kv


def gpu_inputs(shape, n_prompt, n_steps, torch):
    """Talker rows built on the GPU by mk_embed_sum from seeded tables and ids; ids-mode prompt otherwise."""
    from persistent_megakernel_loop_amd.binding import embed_sum, to_device

    dev = "cuda"
    kv0 = shape.kv_prefill
    if shape.inputs == "ids":
        return dict(prompt_ids=torch.from_numpy(wl.make_prompt_ids(shape, n_prompt)).to(dev), prompt_rows=None,
                    prompt_pos3=None, step_ids=None, step_rows=None, step_pos3=None)
    tables = wl.make_talker_tables(shape.hidden)
    cb, tx = to_device(tables["codebooks"]), to_device(tables["text"])
    tids = torch.from_numpy(wl.make_talker_ids(n_prompt + n_steps)).to(dev)
    rows = embed_sum(cb, tx, tids)
    pos3 = torch.from_numpy(wl.position_streams(kv0, n_prompt + n_steps)).to(dev)
    sent = torch.full((n_prompt + n_steps,), -1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    del cb, tx
    return dict(prompt_ids=sent[:n_prompt] if n_prompt else None, prompt_rows=rows[:n_prompt] if n_prompt else None,
                prompt_pos3=pos3[:n_prompt] if n_prompt else None, step_ids=sent[n_prompt:],
                step_rows=rows[n_prompt:].contiguous(), step_pos3=pos3[n_prompt:].contiguous())


def stream_ceiling(torch, gib: int = 2, runs: int = 5) -> dict:
    """GB/s of the library's streaming-read kernel over a gib-GiB buffer (best of runs,
    HIP events on the launch stream), with plain and with non-temporal loads."""
    from persistent_megakernel_loop_amd.binding import bench_stream_read

    buf = torch.ones(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(2048, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    out = {}
    for nt in (False, True):
        best = float("inf")
        for _ in range(runs + 1):  # the first run warms up
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            bench_stream_read(buf, nontemporal=nt, sink=sink, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        out["nontemporal_gbps" if nt else "plain_gbps"] = round(buf.numel() / (best * 1e-3) / 1e9, 1)
    del buf, sink
    torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def blas_info():
    """(library, threads) of the BLAS numpy calls, from threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if pools:
            return pools[0].get("internal_api", "blas"), max(int(i.get("num_threads", 1)) for i in pools)
    except Exception:  # pragma: no cover
        pass
    return "unknown", os.cpu_count() or 1


def oracle_steps_per_s(shape, n_prompt, n_steps, dtype, budget_s):
    """The oracle timed on this host on a bounded sample of the workload: the timed
    workload (prefill untimed, then n_steps decode steps) is replayed until about
    budget_s seconds of decode steps have run.  (steps/s, steps, passes, seconds)."""
    from oracle import Decoder as OracleDecoder
    from oracle import embed_sum17

    weights = wl.make_weights(shape)
    dec = OracleDecoder.from_shape(shape, weights, dtype=dtype)
    kv0 = shape.kv_prefill
    kv = wl.make_kv_prefill(shape) if kv0 else None
    if shape.inputs == "talker":
        tables = wl.make_talker_tables(shape.hidden)
        tids = wl.make_talker_ids(n_prompt + n_steps)
        rows = np.stack([embed_sum17(tables["codebooks"], tables["text"], t) for t in tids])
        pos3 = wl.position_streams(kv0, n_prompt + n_steps)

    def start():  # untimed: back to the state the timed launch starts from
        dec.reset()
        if kv is not None:
            dec.load_kv(kv)
        if shape.inputs == "talker":
            if n_prompt:
                dec.prefill(wl.sentinel_ids(n_prompt), rows[:n_prompt], pos3[:n_prompt])
            return None
        first, _, _ = dec.prefill(wl.make_prompt_ids(shape, n_prompt))
        return [first]

    el, done, passes = 0.0, 0, 0
    while el < budget_s:
        cur = start()
        passes += 1
        t0 = time.perf_counter()
        for s in range(n_steps):
            if shape.inputs == "talker":
                logits, _ = dec.step(dec.input_row(-1, rows[n_prompt + s]), pos3[n_prompt + s])
            else:
                logits, _ = dec.step(dec.input_row(cur[-1]), None)
                cur.append(int(np.argmax(logits.astype(np.float32))))
            done += 1
            if time.perf_counter() - t0 + el >= budget_s:
                break
        el += time.perf_counter() - t0
    return done / el, done, passes, el


def cpu_baseline(shape, n_prompt, n_steps, budget_s=10.0):
    """The oracle as it stands, timed on this host's cores: the float64 leg (the oracle
    the parity tests use) is `value`; the same code with float32 arrays is the `fp32`
    leg, the rate a plain single-precision CPU implementation of the step reaches."""
    blas, threads = blas_info()
    v64, n64, p64, t64 = oracle_steps_per_s(shape, n_prompt, n_steps, np.float64, budget_s)
    v32, n32, p32, t32 = oracle_steps_per_s(shape, n_prompt, n_steps, np.float32, budget_s)
    what = f"decode steps of {shape.name} over the {n_steps}-step workload after an untimed {n_prompt}-position prefill"
    return {"value": v64, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n64} {what} ({p64} pass(es); float64 numpy oracle), {t64:.1f} s",
            "cpu_model": cpu_model(), "blas": blas, "blas_threads": int(threads),
            "fp32": {"value": v32, "unit": "steps/s",
                     "sample": f"{n32} {what} ({p32} pass(es); the oracle with float32 arrays), {t32:.1f} s"}}


CSRC = os.path.join(ROOT, "persistent_megakernel_loop_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# The decode kernel's sources: its code and the parameter block the host fills in.
DECODE_SOURCES = ("mk_internal.h", "mk_device.h", "mk_body.h", "mk_kernel.hip")
# The batched prefill's kernels (both forms).
PREFILL_SOURCES = ("mk_internal.h", "mk_device.h", "mk_prefill.h", "mk_prefill.hip", "mk_pprefill.hip")


def csrc_digest(sources=DECODE_SOURCES) -> str:
    """sha256 over the code of the given kernel sources (line comments and blank lines
    dropped): names the kernel build HBM counters were taken on."""
    import hashlib
    import re
    h = hashlib.sha256()
    for n in sources:
        with open(os.path.join(CSRC, n)) as f:
            code = [re.sub(r"//.*", "", ln).rstrip() for ln in f]
        h.update(n.encode() + b"\0" + "\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()


def counters_path(workload: str, steps: int = 256) -> str:
    """The counter summary of one launch of `steps` steps (256: the default run)."""
    tail = "" if steps == 256 else f"_{steps}steps"
    return os.path.join(PROFILES, f"decode_kernel_{workload}{tail}_hbm_counters.txt")


def _read_counters(path: str) -> dict:
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.split()[0] if v.split() else ""
    return kv


def load_traffic(workload: str, steps: int, algo: int):
    """HBM bytes per decode launch from the committed counter summaries, with where they
    come from: the measured bytes when counters were taken at this step count, else the
    measured ratio of HBM bytes to algorithmic bytes of the default (256-step) run times
    this launch's algorithmic bytes.  (None, reason) when no summary applies or the kernel
    sources changed since."""
    exact = counters_path(workload, steps)
    path = exact if os.path.exists(exact) else counters_path(workload)
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = _read_counters(path)
    if kv.get("csrc_sha256") != csrc_digest():
        return None, "kernel sources changed since the counters were taken"
    if kv.get("steps") == str(steps):
        return int(kv["traffic_bytes_per_launch"]), f"FETCH_SIZE + WRITE_SIZE at {steps} steps"
    ratio = float(kv["traffic_over_algorithmic"])
    return int(round(ratio * algo)), (f"ratio {ratio:.4f} of HBM to algorithmic bytes measured at {kv.get('steps')} "
                                      f"steps, times this launch's algorithmic bytes")


def _pmc_mean(csv_path: str, prefix: str):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path)) if r["Kernel_Name"].startswith(prefix)]
    return (sum(vals) / len(vals), vals) if vals else (None, vals)


def hbm_summary(outdir: str, workload: str, steps: int, copy_mib: int, copy_dir: str = "", warmup: int = 2) -> str:
    """Summary text of the four counter passes (decode launches under outdir, a plain copy
    under copy_dir or outdir; FETCH_SIZE and WRITE_SIZE in KiB per dispatch): each decode
    figure is scaled by known/measured of the copy."""
    copy_dir = copy_dir or outdir
    copy_kib = copy_mib * 1024
    f_dec, f_all = _pmc_mean(os.path.join(outdir, "pmc_FETCH_SIZE", "p_counter_collection.csv"), "void mk::decode_kernel")
    w_dec, w_all = _pmc_mean(os.path.join(outdir, "pmc_WRITE_SIZE", "p_counter_collection.csv"), "void mk::decode_kernel")
    f_cp, _ = _pmc_mean(os.path.join(copy_dir, "pmccopy_FETCH_SIZE", "p_counter_collection.csv"), "__amd_rocclr_copyBuffer")
    w_cp, _ = _pmc_mean(os.path.join(copy_dir, "pmccopy_WRITE_SIZE", "p_counter_collection.csv"), "__amd_rocclr_copyBuffer")
    fs, ws = copy_kib / f_cp, copy_kib / w_cp
    fetch_b, write_b = f_dec * fs * 1024, w_dec * ws * 1024
    shape = wl.BY_NAME[workload]
    algo = step_bytes(shape, shape.kv_prefill + shape.prompt_len, steps)
    base = "--ttfc-trials 0 --ablation-steps 0 --no-ceiling --no-cpu-baseline" + (
        "" if workload == "talker-0.6b" else f" --workload {workload}")
    if steps != 256 or warmup != 2:
        base = f"--steps {steps} --warmup {warmup} " + base
    lines = [
        f"# HBM counters of decode_kernel on {workload}: one launch of {steps} decode steps after the prompt",
        "# commands (repository root, TMPDIR=/tmp), one counter per pass:",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {outdir}/pmc_FETCH_SIZE -o p --output-format csv -- python3 bench.py {base}",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {outdir}/pmc_WRITE_SIZE -o p --output-format csv -- python3 bench.py {base}",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {copy_dir}/pmccopy_FETCH_SIZE -o p --output-format csv -- python3 bench.py --copy-calibration {copy_mib}",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {copy_dir}/pmccopy_WRITE_SIZE -o p --output-format csv -- python3 bench.py --copy-calibration {copy_mib}",
        f"# summarised by: python3 bench.py --hbm-summary {outdir}" + ("" if workload == "talker-0.6b" else f" --workload {workload}")
        + ("" if copy_dir == outdir else f" --copy-dir {copy_dir}") + ("" if steps == 256 else f" --steps {steps}")
        + ("" if warmup == 2 else f" --warmup {warmup}"),
        f"workload: {workload}",
        f"steps: {steps}",
        f"csrc_sha256: {csrc_digest()}",
        f"decode_fetch_kib_per_dispatch: {f_dec:.0f} (dispatches: {', '.join(f'{v:.0f}' for v in f_all)})",
        f"decode_write_kib_per_dispatch: {w_dec:.0f} (dispatches: {', '.join(f'{v:.0f}' for v in w_all)})",
        f"copy_fetch_kib: {f_cp:.0f} for {copy_kib} KiB copied, scale {fs:.4f}",
        f"copy_write_kib: {w_cp:.0f} for {copy_kib} KiB copied, scale {ws:.4f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"algorithmic_bytes_per_launch: {algo}",
        f"traffic_over_algorithmic: {(fetch_b + write_b) / algo:.4f}",
    ]
    return "\n".join(lines) + "\n"


PREFILL_PATHS = {"auto": 0, "chain": 1, "persistent": 2}


def prefill_summary(outdir: str, workload: str, calls: int, path: str, copy_mib: int, copy_dir: str = "") -> str:
    """Summary text of the counter passes of `calls` batched prompt calls (--prefill-only)
    under outdir: FETCH_SIZE and WRITE_SIZE per kernel, summed over the calls' dispatches
    and divided by the call count, each scaled by known/measured of the plain copy."""
    import csv
    copy_dir = copy_dir or outdir
    copy_kib = copy_mib * 1024
    f_cp, _ = _pmc_mean(os.path.join(copy_dir, "pmccopy_FETCH_SIZE", "p_counter_collection.csv"), "__amd_rocclr_copyBuffer")
    w_cp, _ = _pmc_mean(os.path.join(copy_dir, "pmccopy_WRITE_SIZE", "p_counter_collection.csv"), "__amd_rocclr_copyBuffer")
    fs, ws = copy_kib / f_cp, copy_kib / w_cp
    per = {}
    order = []
    for counter, scale, col in (("FETCH_SIZE", fs, 0), ("WRITE_SIZE", ws, 1)):
        for r in csv.DictReader(open(os.path.join(outdir, f"pfpmc_{counter}", "p_counter_collection.csv"))):
            name = r["Kernel_Name"]
            if not (name.startswith("mk::") or name.startswith("void mk::")) or "widen_kernel" in name \
                    or "embed_sum" in name or "pp_clear" in name:
                continue
            short = re.sub(r"^void ", "", name)
            short = re.sub(r"mk::\(anonymous namespace\)::|mk::", "", short)
            short = re.sub(r"\(.*$", "", short)
            if short not in per:
                per[short] = [0.0, 0.0]
                order.append(short)
            per[short][col] += float(r["Counter_Value"]) * scale * 1024 / calls
    shape = wl.BY_NAME[workload]
    algo = weight_bytes_per_step(shape)
    base = f"--prefill-only {calls}" + ("" if path == "auto" else f" --prefill-path {path}") + (
        "" if workload == "talker-0.6b" else f" --workload {workload}")
    lines = [
        f"# HBM counters of the batched prompt prefill on {workload}: one {shape.prompt_len}-position prompt call ({path} form)",
        "# commands (repository root, TMPDIR=/tmp), one counter per pass:",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {outdir}/pfpmc_FETCH_SIZE -o p --output-format csv -- python3 bench.py {base}",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {outdir}/pfpmc_WRITE_SIZE -o p --output-format csv -- python3 bench.py {base}",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {copy_dir}/pmccopy_FETCH_SIZE -o p --output-format csv -- python3 bench.py --copy-calibration {copy_mib}",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {copy_dir}/pmccopy_WRITE_SIZE -o p --output-format csv -- python3 bench.py --copy-calibration {copy_mib}",
        f"# summarised by: python3 bench.py --prefill-summary {outdir} --prefill-only {calls}"
        + ("" if path == "auto" else f" --prefill-path {path}") + ("" if workload == "talker-0.6b" else f" --workload {workload}")
        + ("" if copy_dir == outdir else f" --copy-dir {copy_dir}"),
        f"fetch_scale: {fs:.4f}",
        f"write_scale: {ws:.4f}",
        f"csrc_sha256: {csrc_digest(PREFILL_SOURCES)} (the prefill kernels' sources)",
        "kernel | fetch MB per call | write MB per call",
    ]
    tf = tw = 0.0
    for k in order:
        f, w = per[k]
        tf += f
        tw += w
        lines.append(f"{k} | {f / 1e6:.1f} | {w / 1e6:.1f}")
    lines += [f"total | {tf / 1e6:.1f} | {tw / 1e6:.1f}",
              f"algorithmic_bytes_per_call: {algo} (one pass over the layer weights and the LM head; the cache rows are under 1 MB)",
              f"traffic_over_algorithmic: {(tf + tw) / algo:.2f}"]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--repeats", type=int, default=5, help="timed launches of --steps steps; the median is reported")
    ap.add_argument("--workload", default="talker-0.6b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="leave out the read-stream ceiling measurement")
    ap.add_argument("--ttfc-trials", type=int, default=20)
    ap.add_argument("--ablation-steps", type=int, default=32,
                    help="decode steps of the launch-per-phase ablation (0 turns it off)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 3 times (known bytes for scaling HBM counters) and exit")
    ap.add_argument("--hbm-summary", metavar="DIR", help="only print the HBM counter summary of the passes under DIR")
    ap.add_argument("--copy-dir", default="", metavar="DIR",
                    help="with --hbm-summary: where the copy-calibration passes are (default: DIR)")
    ap.add_argument("--prefill-only", type=int, default=0, metavar="N",
                    help="only run the workload's prompt N times through the batched prefill (for profiling) and exit")
    ap.add_argument("--prefill-path", choices=sorted(PREFILL_PATHS), default="auto",
                    help="form of the batched prefill (mk_set_prefill_path) in every run of it")
    ap.add_argument("--prefill-summary", metavar="DIR",
                    help="only print the HBM counter summary of the --prefill-only passes under DIR")
    args = ap.parse_args()
    if args.prefill_summary:
        sys.stdout.write(prefill_summary(args.prefill_summary, args.workload, args.prefill_only or 5, args.prefill_path,
                                         1024, args.copy_dir))
        return
    if args.hbm_summary:
        sys.stdout.write(hbm_summary(args.hbm_summary, args.workload, args.steps, 1024, args.copy_dir, args.warmup))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the decode path runs on a single MI355X; "
                                   "run with --gpus 1"}))
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n, "copies": 3}), flush=True)
        return
    from persistent_megakernel_loop_amd.binding import Decoder, to_device, weights_to_device

    shape = wl.BY_NAME[args.workload]
    K = args.steps
    P = shape.prompt_len
    shape = shape.replace(max_seq=shape.kv_prefill + P + K)
    weights = wl.make_weights(shape)
    dw = weights_to_device(weights)
    dec = Decoder(shape, dw)
    dec.set_prefill_path(PREFILL_PATHS[args.prefill_path])
    del dw
    torch.cuda.empty_cache()
    inp = gpu_inputs(shape, P, K, torch)
    kv = to_device(wl.make_kv_prefill(shape)) if shape.kv_prefill else None
    out = torch.empty(K, dtype=torch.int32, device="cuda")
    first = torch.empty(1, dtype=torch.int32, device="cuda")
    if args.prefill_only:
        times = []
        for _ in range(args.prefill_only):
            dec.reset()
            if kv is not None:
                dec.load_kv(kv, shape.kv_prefill)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            dec.prefill(inp["prompt_ids"], inp["prompt_rows"], inp["prompt_pos3"], out=first, batched=True)
            torch.cuda.synchronize()
            times.append((time.perf_counter() - t0) * 1e3)
        dec.check()
        print(json.dumps({"workload": shape.name, "prompt_positions": P, "batched_prefill_ms": times}), flush=True)
        dec.close()
        return

    def prepare():
        dec.reset()
        if kv is not None:
            dec.load_kv(kv, shape.kv_prefill)
        if P:
            dec.prefill(inp["prompt_ids"], inp["prompt_rows"], inp["prompt_pos3"], out=first)

    def decode():
        dec.decode(K, inp["step_ids"], inp["step_rows"], inp["step_pos3"], out=out)

    for _ in range(args.warmup):
        prepare()
        decode()
    torch.cuda.synchronize()
    dec.check()
    # timed: --repeats decode launches of K steps each, every one after the same untimed
    # prompt, events on the launch stream; the median launch is the measurement
    stream = torch.cuda.current_stream()
    launches, walls = [], []
    for _ in range(args.repeats):
        prepare()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(stream)
        decode()
        e1.record(stream)
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - w0) * 1e3)
        dec.check()
        launches.append(e0.elapsed_time(e1))
    ref_ids = out.clone()  # the persistent kernel's ids of the timed workload
    launch_ms = float(np.median(launches))
    wall_ms = float(np.median(walls))
    ms_step = launch_ms / K
    first_pos = shape.kv_prefill + P
    algo = step_bytes(shape, first_pos, K)
    gbps = algo / (launch_ms * 1e-3) / 1e9

    # time to first chunk: host clock from the prefill enqueue until the host sees k ids;
    # the prompt through the batched prefill (the default) and position by position
    def ttfc_run(batched):
        res = {}
        for kf in (1, 2, 4, 8):
            trials = []
            for _ in range(args.ttfc_trials):
                dec.reset()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                dec.prefill(inp["prompt_ids"], inp["prompt_rows"], inp["prompt_pos3"], out=first, batched=batched)
                if kf == 1:
                    while dec.progress() < 1:
                        pass
                else:
                    dec.decode(kf - 1, inp["step_ids"], inp["step_rows"], inp["step_pos3"], out=out)
                    while dec.progress() < kf - 1:
                        pass
                trials.append((time.perf_counter() - t0) * 1e3)
                torch.cuda.synchronize()
            res[str(kf)] = round(float(np.median(trials)), 3)
        dec.check()
        return res

    def prefill_ms(batched):
        """Median device time of the prompt call alone (events on the launch stream)."""
        trials = []
        for _ in range(args.ttfc_trials):
            dec.reset()
            if kv is not None:
                dec.load_kv(kv, shape.kv_prefill)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dec.prefill(inp["prompt_ids"], inp["prompt_rows"], inp["prompt_pos3"], out=first, batched=batched)
            b.record(stream)
            torch.cuda.synchronize()
            trials.append(a.elapsed_time(b))
        dec.check()
        return round(float(np.median(trials)), 3)

    # the batched prefill serves the bf16 bodies; a float32 body's prompt runs position by position
    batched_ok = shape.weight_dtype == "bf16"
    ttfc, ttfc_pp, pf_ms = {}, {}, {}
    if P and args.ttfc_trials > 0:
        ttfc = ttfc_run(batched_ok)
        ttfc_pp = ttfc_run(False)
        pf_ms = {"batched": prefill_ms(True) if batched_ok else None, "per_position": prefill_ms(False)}

    # launch-per-phase ablation: the same decode steps with the persistent kernel's own phase
    # bodies, one kernel launch per phase (7 per layer and the LM head; mk_decode_phased),
    # after the same prompt and on the same inputs; its ids must equal the persistent ones
    ablation = {}
    n_abl = min(args.ablation_steps, K)
    if P and n_abl > 0 and shape.hidden <= 1024 and batched_ok:
        prepare()
        torch.cuda.synchronize()
        ids_ab = inp["step_ids"][:n_abl] if inp["step_ids"] is not None else None
        rows_ab = inp["step_rows"][:n_abl] if inp["step_rows"] is not None else None
        pos_ab = inp["step_pos3"][:n_abl] if inp["step_pos3"] is not None else None
        out_ab = torch.empty(n_abl, dtype=torch.int32, device="cuda")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(stream)
        dec.decode_phased(n_abl, ids_ab, rows_ab, pos_ab, out=out_ab)
        b.record(stream)
        torch.cuda.synchronize()
        host = (time.perf_counter() - t0) * 1e3 / n_abl
        dec.check()
        per = a.elapsed_time(b) / n_abl
        same = bool(torch.equal(out_ab, ref_ids[:n_abl]))
        ablation = {"ms_per_step": round(per, 4), "host_ms_per_step": round(host, 4),
                    "over_persistent": round(per / ms_step, 2), "steps": n_abl,
                    "launches_per_step": 7 * shape.n_layers + 1, "ids_equal_persistent": same,
                    "kernels": "the persistent kernel's phase bodies (mk_decode_phased)"}

    # the streaming loop: prompt, then the K frames of one launch handed to the stub codec in
    # chunks of 4 as they are published; talker-only RTF from its clock
    speech = {}
    if args.ttfc_trials > 0:
        from persistent_megakernel_loop_amd.codec import StubCodec, speak
        dec.reset()
        if kv is not None:
            dec.load_kv(kv, shape.kv_prefill)
        torch.cuda.synchronize()
        st = speak(dec, K, inp["step_ids"], inp["step_rows"], inp["step_pos3"],
                   prompt=(inp["prompt_ids"], inp["prompt_rows"], inp["prompt_pos3"]) if P else None, chunk=4,
                   codec=StubCodec(codebook_size=shape.vocab), batched_prefill=batched_ok)
        torch.cuda.synchronize()
        dec.check()
        speech = {"rtf": round(st.rtf, 5), "ttfc_ms": round(st.ttfc_ms, 3), "total_ms": round(st.total_ms, 3),
                  "frames": st.frames, "audio_s": round(st.audio_s, 3), "chunk": 4, "codec": "stub (tone per code)"}

    # barrier share: in-kernel wait ticks over position ticks, one separate traced run
    prepare()
    trace = torch.zeros((K, dec.grid_size(), 2), dtype=torch.int64, device="cuda")
    dec.set_debug(None, trace)
    decode()
    torch.cuda.synchronize()
    dec.set_debug(None, None)
    tr = trace.cpu().numpy().astype(np.float64)
    share = float(tr[:, :, 0].sum() / max(tr[:, :, 1].sum(), 1.0))
    per_step = tr[:, :, 0].sum(axis=1) / np.maximum(tr[:, :, 1].sum(axis=1), 1.0)
    share_p99 = float(np.percentile(per_step, 99))
    dec.check()

    # read-stream ceiling: the bandwidth a plain streaming read reaches on this device
    ceiling = {} if args.no_ceiling else stream_ceiling(torch)

    traffic, traffic_src = load_traffic(shape.name, K, algo)
    res = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 2),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.weight_dtype,
        "data": "synthetic",
        "config": {"workload": shape.name, "layers": shape.n_layers, "hidden": shape.hidden, "vocab": shape.vocab,
                   "prompt_positions": P, "kv_prefill": shape.kv_prefill, "decode_steps": K, "batch": 1,
                   "weights": f"{shape.weight_dtype} N(0,0.02) random", "kv_cache": shape.kv_dtype,
                   "launches_timed": args.repeats, "reported": "median launch"},
        "hbm_gbps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "ttfc_ms": ttfc,
        "ttfc_ms_per_position_prefill": ttfc_pp,
        "prefill_ms": pf_ms,
        "launch_per_phase": ablation,
        "rtf_talker_only": speech.get("rtf"),
        "rtf_kernel_only": round(ms_step / FRAME_MS, 5),
        "speech": speech,
        "barrier_share": round(share, 4),
        "barrier_share_p99": round(share_p99, 4),
        "stream_ceiling": dict(ceiling, decode_frac_of_ceiling=round(gbps / max(ceiling.values()), 4)) if ceiling else {},
        "wall_ms_timed_launch": round(wall_ms, 3),
        "launch_ms_all": [round(v, 4) for v in launches],
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "traffic_source": traffic_src,
                     "algorithmic_bytes_per_launch": int(algo), "launch_ms": round(launch_ms, 4)},
    }
    # release every device resource before the interpreter exits: the handle (arena, cache,
    # exchange buffers, pinned progress word and id mirror) and every tensor
    dec.close()
    del dec, inp, kv, out, first, trace, ref_ids
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(shape, P, K)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
