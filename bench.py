#!/usr/bin/env python3
"""Benchmark of one permuted block-sparse attention prefill step on one MI355X.

A step is the whole hot path on one layer's synthetic Q/K/V already resident in HBM:
segment permutation (importance + sort), block mask (pooling + selection) and block-sparse
attention.  Prints ONE JSON line on stdout (progress goes to stderr):

  value         dense-equivalent TFLOP/s of the whole step, 2 N^2 d Hq / t_step
  ms_per_step   mean step time over --steps timed steps
  roofline      the attention kernel against the bf16 MFMA peak: MFMA FLOP executed on computed
                tiles (4 B^2 d per tile) / mean kernel duration (HIP events on its stream)
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample, extrapolated per stage

  subrecords    the 128K layer (tau 0.9 and tau bisected to ~10% density), the 64K early-stop
                layer and the 1K single-head case, each against the library's dense kernel

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b_32k] [--no-subrecords]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
COPY_CALIB_BYTES = 1 << 30  # plain device copy of known size used to scale the byte counters
KERNEL_SOURCES = ("block_sparse_attention_blocks_amd/csrc/attention.hip", "block_sparse_attention_blocks_amd/csrc/attn_device.h",
                  "block_sparse_attention_blocks_amd/csrc/common.h")
TRAFFIC_SUMMARY = "profiles/attn_pipe_kernel_llama8b_32k_traffic.txt"
ATTN_KERNEL = "attn_pipe_kernel<128, 128, false, 2, false>"


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter summary, or None
    when there is none or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            kk, vv = line.split("=", 1)
            vals[kk.strip()] = vv.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return float(vals["traffic_bytes_per_launch"])


def summarize_pmc(fetch_csv: str, write_csv: str, out: str, command: str, kernel: str = ATTN_KERNEL,
                  workload: str = "llama8b_32k") -> int:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of one kernel, scaled by what the same counters
    read for the plain copy of COPY_CALIB_BYTES in the same run."""
    import csv
    import statistics

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        attn = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"].replace("pbsa::", "")]
        copy = [float(r["Counter_Value"]) for r in rows
                if "copy" in r["Kernel_Name"].lower() and float(r["Counter_Value"]) > COPY_CALIB_BYTES / 1024 / 4]
        return statistics.median(attn), statistics.median(copy), len(attn)

    fa, fc, n_f = per_kernel(fetch_csv, "FETCH_SIZE")
    wa, wc, n_w = per_kernel(write_csv, "WRITE_SIZE")
    sf = (COPY_CALIB_BYTES / 1024) / fc   # true KiB per counted KiB, reads
    sw = (COPY_CALIB_BYTES / 1024) / wc   # same for writes
    traffic = (fa * sf + wa * sw) * 1024
    with open(out, "w") as f:
        f.write(f"# {kernel}, {workload} workload: HBM traffic per launch from rocprofv3 byte counters\n")
        f.write(f"# command: {command}\n")
        f.write(f"# FETCH_SIZE / WRITE_SIZE are KiB per dispatch (median of {n_f} / {n_w} dispatches); each is scaled\n")
        f.write(f"# by the ratio true/counted bytes of a plain {COPY_CALIB_BYTES} B device copy in the same run.\n")
        f.write(f"attn_fetch_kib = {fa:.1f}\nattn_write_kib = {wa:.1f}\n")
        f.write(f"copy_fetch_kib = {fc:.1f}\ncopy_write_kib = {wc:.1f}\n")
        f.write(f"fetch_scale = {sf:.4f}\nwrite_scale = {sw:.4f}\n")
        f.write(f"traffic_bytes_per_launch = {traffic:.6g}\n")
        f.write(f"kernel_source_sha256_16 = {kernel_source_hash()}\n")
    print(open(out).read())
    return 0


SQ_COUNTERS = ("SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
               "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAVE_CYCLES")


def summarize_sq(sections, out: str, commands) -> int:
    """Per-kernel SQ counter table from rocprofv3 --pmc counter_collection.csv files: counters summed
    over every dispatch of a kernel; sections = [(title, csv path)].  SQ_INSTS_VALU counts the MFMA
    instructions too, so VALU/MFMA is that count over SQ_INSTS_MFMA."""
    import csv

    def short(name):
        name = name.replace("pbsa::", "").replace("(anonymous namespace)::", "")
        if name.startswith("void "):
            name = name[5:]
        cut = name.find("(")
        return name[:cut] if cut > 0 else name

    with open(out, "w") as f:
        f.write("# rocprofv3 SQ counters per kernel (summed over every dispatch of the kernel in the run)\n")
        f.write("# commands (from the repository root, TMPDIR=/tmp; one --pmc pass each):\n")
        for c in commands:
            f.write(f"#   {c}\n")
        f.write("# ratios: VALU/MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA, LDS/MFMA = SQ_INSTS_LDS / SQ_INSTS_MFMA,\n")
        f.write("# waiting = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of wave cycles spent waiting on s_waitcnt or "
                "a barrier)\n")
        for title, path in sections:
            tot, disp = {}, {}
            for r in csv.DictReader(open(path)):
                k = short(r["Kernel_Name"])
                d = tot.setdefault(k, {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                disp.setdefault(k, set()).add(r.get("Dispatch_Id", r.get("Correlation_Id", len(disp.get(k, ())))))
            f.write(f"\n## {title}\n")
            f.write(f"{'kernel':60s} {'dispatches':>11s} {'SQ_INSTS_MFMA':>14s} {'SQ_INSTS_VALU':>14s} "
                    f"{'SQ_INSTS_LDS':>13s} VALU/MFMA LDS/MFMA waiting\n")
            rows = [(k, d) for k, d in tot.items() if d.get("SQ_INSTS_MFMA", 0.0) > 0]
            for k, d in sorted(rows, key=lambda kd: -kd[1]["SQ_INSTS_MFMA"]):
                mf, va, ld = d["SQ_INSTS_MFMA"], d.get("SQ_INSTS_VALU", 0.0), d.get("SQ_INSTS_LDS", 0.0)
                wt = d.get("SQ_WAIT_INST_ANY", 0.0) / max(d.get("SQ_WAVE_CYCLES", 0.0), 1.0)
                f.write(f"{k[:60]:60s} {len(disp[k]):11d} {mf:14.4g} {va:14.4g} {ld:13.4g} {va / mf:9.2f} "
                        f"{ld / mf:8.2f} {100 * wt:6.1f}%\n")
    print(open(out).read())
    return 0


def summarize_stats(stats_csv: str, bench_out: str, out: str, command: str, workload: str) -> int:
    """Per-kernel table from a rocprofv3 --kernel-trace --stats kernel_stats.csv, with the HIP-event
    kernel time that the bench line of the same run reported beside it."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    kernel_ms = None
    if bench_out and os.path.exists(bench_out):
        for line in open(bench_out):
            line = line.strip()
            if line.startswith("{") and '"roofline"' in line:
                kernel_ms = json.loads(line)["roofline"]["kernel_ms"]

    def short(name):
        own = "pbsa::" in name
        name = name.replace("pbsa::", "").replace("(anonymous namespace)::", "")
        if name.startswith("void "):
            name = name[5:]
        cut = name.find("(")
        if own:
            name = name[:cut] if cut > 0 else name
            for kw, v in (("ImpArgs", ""), ("SelArgs", ""), ("ZArgs", "")):
                name = name.replace(kw, v)
            return name
        return name[:40] + " (torch)"

    total = sum(float(r["TotalDurationNs"]) for r in rows)
    with open(out, "w") as f:
        f.write(f"# rocprofv3 kernel-trace statistics, {workload}\n")
        f.write(f"# command (from the repository root, TMPDIR=/tmp):\n#   {command}\n")
        f.write("# calls include warm-up, timed steps and bench.py's own dense-kernel timing; times in microseconds.\n")
        if kernel_ms is not None:
            f.write(f"# bench.py's HIP-event figure for the block-sparse attention kernel in the same run: "
                    f"kernel_ms = {kernel_ms:.3f}\n")
        f.write(f"{'kernel':62s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}\n")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            f.write(f"{short(r['Name'])[:62]:62s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.1f} "
                    f"{float(r['MinNs']) / 1e3:9.1f} {float(r['MaxNs']) / 1e3:9.1f} "
                    f"{100.0 * float(r['TotalDurationNs']) / total:6.2f}\n")
    print(open(out).read())
    return 0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def make_inputs(w, torch, np):
    from workloads import generate_for
    x = generate_for(w)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    return x, dev


def cpu_baseline(w, x, count, budget_s, np):
    """Time the fp64 oracle on this host: stages 1-2 in full, attention on a seeded sample of
    (head, query block) rows extrapolated by computed-tile count."""
    import oracle
    from workloads import bf16_bits_to_f32
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=cores, user_api="blas")
    except ImportError:  # pragma: no cover
        limit = None
    try:
        return _cpu_baseline(w, x, count, budget_s, np, oracle, bf16_bits_to_f32, cores)
    finally:
        if limit is not None:
            limit.restore_original_limits()


def _cpu_baseline(w, x, count, budget_s, np, oracle, bf16_bits_to_f32, cores):
    q = bf16_bits_to_f32(x["q"]).astype(np.float64)
    k = bf16_bits_to_f32(x["k"]).astype(np.float64)
    v = bf16_bits_to_f32(x["v"]).astype(np.float64)
    B, S = w.block_size, w.segment_size
    t0 = time.perf_counter()
    imp = oracle.key_importance(q, k, B)
    perm = oracle.segment_permutation(imp, S)
    t1 = time.perf_counter()
    cnt_o, idx_o, _ = oracle.block_mask(q, k, perm, B, S, w.mass_tau, w.force_diag, w.force_first)
    t2 = time.perf_counter()
    rng = np.random.default_rng(12345)
    Hq, NB = cnt_o.shape
    rows, tiles, t_att = [], 0, 0.0
    order = rng.permutation(Hq * NB)
    for r in order:
        h, I = divmod(int(r), NB)
        s0 = time.perf_counter()
        oracle.block_sparse_attention(q, k, v, perm, cnt_o, idx_o, B, S, rows=[(h, I)])
        t_att += time.perf_counter() - s0
        tiles += int(cnt_o[h, I])
        rows.append((h, I))
        if t_att > budget_s or len(rows) >= 256:
            break
    total_tiles = int(cnt_o.sum())
    t_att_full = t_att * total_tiles / max(tiles, 1)
    t_step = (t1 - t0) + (t2 - t1) + t_att_full
    return {
        "value": w.dense_causal_flop / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"{cores} cores (the process's affinity mask), BLAS threads set to {cores}; "
                   f"permutation and mask stages in full ({t1 - t0:.2f} s, {t2 - t1:.2f} s); attention on "
                   f"{len(rows)} seeded (head, query-block) rows = {tiles} of {total_tiles} computed tiles "
                   f"({t_att:.2f} s), extrapolated by tile count to {t_att_full:.1f} s; step {t_step:.1f} s"),
        "step_s": t_step,
    }


def _events(torch, stream, fn, reps):
    """Median and minimum of reps timed calls of fn on the stream, after one untimed warm-up call (a
    first call on freshly written inputs runs cold and is never part of a figure)."""
    fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    xs = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median_ms": xs[len(xs) // 2], "min_ms": xs[0]}


def torch_sdpa_ms(torch, q, k, v, stream, reps):
    """Dense causal attention through torch's fused SDPA kernels on the same tensors, as context:
    (median ms, backend) or (None, reason).  Only the flash and memory-efficient backends are
    allowed (the unfused path is never used); K and V are expanded to the query heads."""
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
    except ImportError as e:
        return None, f"unavailable: {e}"
    G = q.shape[0] // k.shape[0]
    qq = q.unsqueeze(0)
    kk = k.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
    vv = v.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
    reason = "no fused kernel"
    try:
        for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
            try:
                with sdpa_kernel([be]):
                    f = lambda: torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True)
                    f()
                    torch.cuda.synchronize()
                    return _events(torch, stream, f, reps)["median_ms"], be.name
            except RuntimeError as e:
                reason = f"{be.name}: {str(e)[:120]}"
        return None, reason
    finally:
        del qq, kk, vv
        torch.cuda.empty_cache()


def suite(args) -> int:
    """Secondary measurements, one JSON object per line into --suite-out:
    128K (as configured and at a bisected ~10% block density), the 64K density sweep with the
    permutation on and off, and the 64K tile-max early-stop workload with calibrated thresholds."""
    import numpy as np
    import torch

    import block_sparse_attention_blocks_amd as pbsa
    from workloads import WORKLOADS, generate_for

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    out_f = open(args.suite_out, "w")

    def emit(rec):
        out_f.write(json.dumps(rec) + "\n")
        out_f.flush()
        log("[suite] " + json.dumps(rec))

    def load(w, seed=None):
        x = generate_for(w, seed=seed)
        return {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}

    class _WithWorkspace:  # every attention call of the suite reuses one preallocated workspace
        def __init__(self, mod, ws):
            self._mod, self._ws = mod, ws

        def __getattr__(self, name):
            return getattr(self._mod, name)

        def block_sparse_attn_prefill(self, *a, **kw):
            kw.setdefault("workspace", self._ws)
            return self._mod.block_sparse_attn_prefill(*a, **kw)

        def s2o_attn_prefill(self, *a, **kw):
            kw.setdefault("workspace", self._ws)
            return self._mod.s2o_attn_prefill(*a, **kw)

        def s2o_prefix_attn_prefill(self, *a, **kw):
            kw.setdefault("workspace", self._ws)
            return self._mod.s2o_prefix_attn_prefill(*a, **kw)

    pbsa = _WithWorkspace(pbsa, torch.empty(4096, dtype=torch.uint8, device="cuda"))
    reps = args.suite_reps
    parts = set(args.suite_parts.split(","))
    if "128k" in parts:
        suite_128k(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps)
    if "sweep" in parts:
        suite_sweep(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps)
    if "earlystop" in parts:
        suite_earlystop(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps)
    if "s2o" in parts:
        suite_s2o(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps)
    if "twopass" in parts:
        suite_s2o(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps, two_pass=True)
    if "qperm" in parts:
        suite_s2o(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps, two_pass=True, qperm=True)
    if "sample" in parts:
        suite_sample(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps)
    out_f.close()
    if args.copy_calib:
        copy_calibration(torch)
    return 0


def copy_calibration(torch):
    """A plain device copy of COPY_CALIB_BYTES, whose byte counters scale the kernels' counters."""
    src = torch.empty(COPY_CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def suite_128k(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps):
    for rec in measure_128k(torch, np, pbsa, WORKLOADS, load, stream, reps):
        emit(rec)


def measure_128k(torch, np, pbsa, WORKLOADS, load, stream, reps, sdpa=True):
    """The 128K layer as configured (tau 0.9) and at tau bisected to ~10% block density: stage times,
    the library's dense causal kernel and the speedups, MFMA fraction on computed tiles."""
    w = WORKLOADS["llama8b_128k"]
    t0 = time.perf_counter()
    d = load(w)
    log(f"[bench] {w.name} inputs in {time.perf_counter() - t0:.1f} s")
    q, k, v = d["q"], d["k"], d["v"]
    B, S, NB, Hq = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads
    causal_tiles = Hq * NB * (NB + 1) // 2
    shape = pbsa.make_shape(q, k, B, S)
    ws_p = torch.empty(pbsa.workspace_size(shape, pbsa.PBSA_OP_PERMUTATION) + 256, dtype=torch.uint8, device="cuda")
    ws_m = torch.empty(pbsa.workspace_size(shape, pbsa.PBSA_OP_MASK) + 256, dtype=torch.uint8, device="cuda")
    perm = torch.empty((w.num_kv_heads, w.seq_len), dtype=torch.int32, device="cuda")
    count = torch.empty((Hq, NB), dtype=torch.int32, device="cuda")
    idx = torch.empty((Hq, NB * (NB + 1) // 2), dtype=torch.int32, device="cuda")
    out = torch.empty((Hq, w.seq_len, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((Hq, w.seq_len), dtype=torch.float32, device="cuda")
    fp = lambda: pbsa.build_segment_permutation(q, k, B, S, perm=perm, workspace=ws_p)
    fp()

    def at_tau(tau, use_perm=True):
        pbsa.estimate_block_mask(q, k, perm if use_perm else None, B, S, tau, out=(count, idx), workspace=ws_m)
        torch.cuda.synchronize()
        return int(count.sum().item()) / causal_tiles

    dense = lambda: pbsa.block_sparse_attn_prefill(q, k, v, None, None, None, B, S, out=out, lse=lse)
    t_dense = _events(torch, stream, dense, max(3, reps))
    sdpa_ms, sdpa_backend = torch_sdpa_ms(torch, q, k, v, stream, 2) if sdpa else (None, "not run")
    t_perm = _events(torch, stream, fp, reps)
    recs = []
    for label, tau in (("as_configured", w.mass_tau), ("density_10pct", None)):
        if tau is None:  # bisect the mass target to a ~10% computed-block fraction
            lo, hi = 0.0, 1.0
            for _ in range(18):
                mid = 0.5 * (lo + hi)
                if at_tau(mid) < 0.10:
                    lo = mid
                else:
                    hi = mid
            tau = hi
        dens = at_tau(tau)
        fm = lambda: pbsa.estimate_block_mask(q, k, perm, B, S, tau, out=(count, idx), workspace=ws_m)
        fa = lambda: pbsa.block_sparse_attn_prefill(q, k, v, perm, count, idx, B, S, out=out, lse=lse)
        t_mask = _events(torch, stream, fm, reps)
        fm()
        t_attn = _events(torch, stream, fa, reps)
        tiles = int(count.sum().item())
        ta = t_attn["median_ms"]
        step = t_perm["median_ms"] + t_mask["median_ms"] + ta
        recs.append({"workload": w.name, "point": label, "mass_tau": tau, "block_density": dens,
              "permutation_ms": t_perm["median_ms"], "mask_ms": t_mask["median_ms"], "attention_ms": ta,
              "step_ms": step, "dense_kernel_ms": t_dense["median_ms"],
              "torch_sdpa_dense_ms": sdpa_ms, "torch_sdpa_backend": sdpa_backend,
              "attention_speedup_vs_dense": t_dense["median_ms"] / ta,
              "step_speedup_vs_dense": t_dense["median_ms"] / step,
              "attention_mfma_tflops": tiles * 4.0 * B * B * w.head_dim / (ta * 1e-3) / 1e12,
              "attention_mfma_frac": tiles * 4.0 * B * B * w.head_dim / (ta * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
              "dense_equiv_tflops_step": w.dense_causal_flop / (step * 1e-3) / 1e12})
    del d, q, k, v, out, lse, ws_p, ws_m, perm, count, idx
    torch.cuda.empty_cache()
    return recs


def suite_sweep(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps):
    w = WORKLOADS["llama8b_64k_sweep"]
    d = load(w)
    q, k, v = d["q"], d["k"], d["v"]
    B, S, NB, Hq = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads
    causal_tiles = Hq * NB * (NB + 1) // 2
    perm = pbsa.build_segment_permutation(q, k, B, S)
    out = torch.empty((Hq, w.seq_len, w.head_dim), dtype=torch.float32, device="cuda")
    dense = lambda: pbsa.block_sparse_attn_prefill(q, k, v, None, None, None, B, S, out=out, return_lse=False)
    t_dense = _events(torch, stream, dense, max(3, reps))["median_ms"]
    for tau in w.taus:
        for use_perm in (True, False):
            pp = perm if use_perm else None
            count, idx = pbsa.estimate_block_mask(q, k, pp, B, S, tau)
            fa = lambda: pbsa.block_sparse_attn_prefill(q, k, v, pp, count, idx, B, S, out=out, return_lse=False)
            ta = _events(torch, stream, fa, reps)["median_ms"]
            tiles = int(count.sum().item())
            emit({"workload": w.name, "mass_tau": tau, "permutation": use_perm, "block_density": tiles / causal_tiles,
                  "attention_ms": ta, "dense_kernel_ms": t_dense, "attention_speedup_vs_dense": t_dense / ta,
                  "attention_mfma_frac": tiles * 4.0 * B * B * w.head_dim / (ta * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
    del d, q, k, v, out, perm
    torch.cuda.empty_cache()


def suite_earlystop(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps):
    emit(measure_earlystop(torch, np, pbsa, WORKLOADS, load, stream, reps))


def measure_earlystop(torch, np, pbsa, WORKLOADS, load, stream, reps):
    """64K tile-max early stop with thresholds calibrated on a second draw (top 64 tiles per query
    block): kept-tile and V-gather fractions, time against the library's dense causal kernel."""
    w = WORKLOADS["llama8b_64k_earlystop"]
    d = load(w)
    cal = load(w, seed=w.calib_seed)
    B, NB, Hq = w.block_size, w.num_blocks, w.num_q_heads
    # offline calibration on the second draw: tile maxima, then the keep-th largest per query block
    tmax = pbsa.tile_max(cal["q"], cal["k"], B)
    theta_t = pbsa.calibrate_thresholds(tmax, cal["q"], cal["k"], B, w.calib_keep)
    del cal, tmax
    q, k, v = d["q"], d["k"], d["v"]
    out = torch.empty((Hq, w.seq_len, w.head_dim), dtype=torch.float32, device="cuda")
    dense = lambda: pbsa.block_sparse_attn_prefill(q, k, v, None, None, None, B, 0, out=out, return_lse=False)
    gated = lambda: pbsa.block_sparse_attn_prefill(q, k, v, None, None, None, B, 0, early_stop_theta=theta_t,
                                                   out=out, return_lse=False)
    t_dense = _events(torch, stream, dense, max(3, reps))["median_ms"]
    t_gate = _events(torch, stream, gated, reps)["median_ms"]
    _, kept = pbsa.block_sparse_attn_prefill(q, k, v, None, None, None, B, 0, early_stop_theta=theta_t,
                                             return_lse=False, return_kept=True)
    bits = np.unpackbits(kept.cpu().numpy().view(np.uint8), bitorder="little").reshape(Hq, -1)
    kept_tiles = int(bits.sum())
    causal_tiles = Hq * NB * (NB + 1) // 2
    # the head-pair kernel gathers a V tile when either head of the pair keeps it
    pairs = bits[0::2] | bits[1::2] if Hq % 2 == 0 and (Hq // w.num_kv_heads) % 2 == 0 else bits
    v_gather = int(pairs.sum()) * (2 if pairs is not bits else 1)
    flop = causal_tiles * 2.0 * B * B * w.head_dim + kept_tiles * 2.0 * B * B * w.head_dim
    rec = {"workload": w.name, "calibration": f"seed {w.calib_seed}, keep top {w.calib_keep} tiles per query block",
           "kept_tile_fraction": kept_tiles / causal_tiles, "v_gather_fraction": v_gather / causal_tiles,
           "attention_ms": t_gate, "dense_kernel_ms": t_dense, "attention_speedup_vs_dense": t_dense / t_gate,
           "mfma_frac": flop / (t_gate * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del d, q, k, v, out
    torch.cuda.empty_cache()
    return rec


def measure_1k(torch, np, pbsa, WORKLOADS, load, stream, reps):
    """The single-head 1K case: the three stages and the library's dense causal kernel."""
    w = WORKLOADS["single_head_1k"]
    d = load(w)
    q, k, v = d["q"], d["k"], d["v"]
    B, S, NB, Hq = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads
    perm = pbsa.build_segment_permutation(q, k, B, S)
    count, idx = pbsa.estimate_block_mask(q, k, perm, B, S, w.mass_tau, w.force_diag, w.force_first)
    out = torch.empty((Hq, w.seq_len, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((Hq, w.seq_len), dtype=torch.float32, device="cuda")
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    fp = lambda: pbsa.build_segment_permutation(q, k, B, S, perm=perm)
    fm = lambda: pbsa.estimate_block_mask(q, k, perm, B, S, w.mass_tau, w.force_diag, w.force_first,
                                          out=(count, idx))
    fa = lambda: pbsa.block_sparse_attn_prefill(q, k, v, perm, count, idx, B, S, out=out, lse=lse, workspace=ws)
    fd = lambda: pbsa.block_sparse_attn_prefill(q, k, v, None, None, None, B, S, out=out, lse=lse, workspace=ws)
    t = {n: _events(torch, stream, f, reps)["median_ms"] for n, f in
         (("permutation", fp), ("mask", fm), ("attention", fa), ("dense", fd))}
    tiles = int(count.sum().item())
    step = t["permutation"] + t["mask"] + t["attention"]
    return {"workload": w.name, "block_density": tiles / (Hq * NB * (NB + 1) // 2), "mass_tau": w.mass_tau,
            "stages_ms": {k_: t[k_] for k_ in ("permutation", "mask", "attention")}, "step_ms": step,
            "dense_kernel_ms": t["dense"], "attention_speedup_vs_dense": t["dense"] / t["attention"],
            "step_speedup_vs_dense": t["dense"] / step}


def suite_s2o(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps, two_pass=False, qperm=False):
    """Marginal-gain early stop at 32K and 128K, and at 32K on inputs drawn without stripe keys
    (there the stop falls in the middle of most lists): over the pooled-logit ranked list (PBS
    permutation + PBSA_MASK_RANKED), or with two_pass over S2O's historical ranking (qperm: with
    the query permutation too, whose build time is added to ranking_ms)."""
    from workloads import generate
    cases = [("llama8b_32k", None), ("llama8b_32k", "no_stripes"), ("llama8b_128k", None)]
    for name, variant in cases:
        w = WORKLOADS[name]
        if variant == "no_stripes":
            x = generate(w.seq_len, w.num_q_heads, w.num_kv_heads, w.head_dim, 0, w.band_width, w.seed + 500)
            d = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
            del x
        else:
            d = load(w)
        q, k, v = d["q"], d["k"], d["v"]
        B, S, NB, Hq = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads
        causal_tiles = Hq * NB * (NB + 1) // 2
        out = torch.empty((Hq, w.seq_len, w.head_dim), dtype=torch.float32, device="cuda")
        lse = torch.empty((Hq, w.seq_len), dtype=torch.float32, device="cuda")
        if two_pass:
            shape = pbsa.make_shape(q, k, B, S)
            ws_r = torch.empty(pbsa.workspace_size(shape, pbsa.PBSA_OP_PREFIX_RANK) + 256, dtype=torch.uint8,
                               device="cuda")
            rank = pbsa.build_prefix_kv_ranking(q, k, B, S, workspace=ws_r)
            qp = pbsa.build_query_permutation(q, k, B, S) if qperm else None

            def fr():
                pbsa.build_prefix_kv_ranking(q, k, B, S, out=rank, workspace=ws_r)
                if qperm:
                    pbsa.build_query_permutation(q, k, B, S, out=qp)
            perm = count = idx = None
        else:
            perm = pbsa.build_segment_permutation(q, k, B, S)
            count, idx = pbsa.estimate_block_mask(q, k, perm, B, S, 1.0, ranked=True)
            fr = lambda: pbsa.estimate_block_mask(q, k, perm, B, S, 1.0, ranked=True, out=(count, idx))
        t_rank = _events(torch, stream, fr, reps)["median_ms"]
        dense = lambda: pbsa.block_sparse_attn_prefill(q, k, v, None, None, None, B, S, out=out, lse=lse)
        t_dense = _events(torch, stream, dense, max(3, reps))["median_ms"]
        for gain_tau in (0.001, 0.01, 0.05):
            if two_pass:
                fa = lambda: pbsa.s2o_prefix_attn_prefill(q, k, v, rank, B, S, gain_tau, out=out, lse=lse, qperm=qp)
                _, _, kept = pbsa.s2o_prefix_attn_prefill(q, k, v, rank, B, S, gain_tau, return_kept=True, qperm=qp)
            else:
                fa = lambda: pbsa.s2o_attn_prefill(q, k, v, perm, count, idx, B, S, gain_tau, out=out, lse=lse)
                _, _, kept = pbsa.s2o_attn_prefill(q, k, v, perm, count, idx, B, S, gain_tau, return_kept=True)
            ta = _events(torch, stream, fa, reps)["median_ms"]
            tiles = int(np.unpackbits(kept.cpu().numpy().view(np.uint8)).sum())
            emit({"workload": w.name + ("" if variant is None else "_" + variant), "gain_tau": gain_tau,
                  "lists": ("two-pass historical ranking" + (", query permutation" if qperm else "")) if two_pass
                  else "pooled-logit ranked",
                  "processed_fraction": tiles / causal_tiles, "ranking_ms": t_rank, "attention_ms": ta,
                  "dense_kernel_ms": t_dense, "attention_speedup_vs_dense": t_dense / ta,
                  "attention_mfma_frac": tiles * 4.0 * B * B * w.head_dim / (ta * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
        del d, q, k, v, out, lse, perm, count, idx
        if two_pass:
            del rank, ws_r, qp
        torch.cuda.empty_cache()


def suite_sample(args, torch, np, pbsa, WORKLOADS, load, emit, stream, reps):
    """SampleAttention's mask (8 trunks of 16 sampled rows per query head) at 32K and 128K for a few
    CIA targets: estimator time, mask density and attention time on the mask against dense."""
    nt, rpt = 8, 16
    for name in ("llama8b_32k", "llama8b_128k"):
        w = WORKLOADS[name]
        d = load(w)
        q, k, v = d["q"], d["k"], d["v"]
        B, NB, Hq = w.block_size, w.num_blocks, w.num_q_heads
        causal_tiles = Hq * NB * (NB + 1) // 2
        ws = torch.empty(pbsa.sample_mask_workspace_size(q, k, B, nt, rpt) + 256, dtype=torch.uint8, device="cuda")
        count = torch.empty((Hq, NB), dtype=torch.int32, device="cuda")
        idx = torch.empty((Hq, NB * (NB + 1) // 2), dtype=torch.int32, device="cuda")
        out = torch.empty((Hq, w.seq_len, w.head_dim), dtype=torch.float32, device="cuda")
        lse = torch.empty((Hq, w.seq_len), dtype=torch.float32, device="cuda")
        dense = lambda: pbsa.block_sparse_attn_prefill(q, k, v, None, None, None, B, 0, out=out, lse=lse)
        t_dense = _events(torch, stream, dense, max(3, reps))["median_ms"]
        for tau in (0.5, 0.8, 0.95):
            fm = lambda: pbsa.sample_attention_mask(q, k, B, tau, nt, rpt, out=(count, idx), workspace=ws)
            t_mask = _events(torch, stream, fm, reps)["median_ms"]
            fm()
            fa = lambda: pbsa.block_sparse_attn_prefill(q, k, v, None, count, idx, B, 0, out=out, lse=lse)
            ta = _events(torch, stream, fa, reps)["median_ms"]
            tiles = int(count.sum().item())
            emit({"workload": w.name, "estimator": f"SampleAttention, {nt} trunks x {rpt} rows", "cia_tau": tau,
                  "block_density": tiles / causal_tiles, "mask_ms": t_mask, "attention_ms": ta,
                  "dense_kernel_ms": t_dense, "attention_speedup_vs_dense": t_dense / ta,
                  "step_speedup_vs_dense": t_dense / (t_mask + ta),
                  "attention_mfma_frac": tiles * 4.0 * B * B * w.head_dim / (ta * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
        del d, q, k, v, out, lse, ws, count, idx
        torch.cuda.empty_cache()


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--mass-tau", type=float, default=None, help="override the workload's mass target")
    ap.add_argument("--no-subrecords", action="store_true",
                    help="time only the main workload (no 128K, 64K early-stop and 1K sub-records)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle attention sampling")
    ap.add_argument("--copy-calib", action="store_true",
                    help="after timing, copy %d bytes on the device (byte-counter calibration)" % COPY_CALIB_BYTES)
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 --pmc counter_collection.csv files")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "BENCH_OUT"),
                    help="write a kernel table from a rocprofv3 kernel_stats.csv and the bench line of that run")
    ap.add_argument("--summarize-sq", nargs="+", metavar="TITLE=CSV",
                    help="write the SQ counter table from rocprofv3 --pmc counter_collection.csv files")
    ap.add_argument("--summary-out", default=TRAFFIC_SUMMARY)
    ap.add_argument("--summary-command", default="")
    ap.add_argument("--summary-kernel", default=ATTN_KERNEL, help="kernel whose counters --summarize-pmc reads")
    ap.add_argument("--summary-label", default="", help="workload description in a --summarize-stats header")
    ap.add_argument("--suite", action="store_true", help="run the secondary measurements instead")
    ap.add_argument("--suite-out", default="bench_suite.jsonl")
    ap.add_argument("--suite-reps", type=int, default=5)
    ap.add_argument("--suite-parts", default="128k,sweep,earlystop,s2o,twopass,qperm,sample",
                    help="comma-separated subset of 128k, sweep, earlystop, s2o, twopass, qperm, sample")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (got --gpus {args.gpus}); "
              "query heads split across GPUs with no exchange between them, each GPU running this same step "
              "on its heads",
              file=sys.stderr)
        return 2

    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.summary_out, args.summary_command,
                             args.summary_kernel, args.workload)
    if args.summarize_sq:
        secs = [tuple(x.split("=", 1)) for x in args.summarize_sq]
        return summarize_sq(secs, args.summary_out, [c for c in args.summary_command.split(" ;; ") if c])
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats[0], args.summarize_stats[1], args.summary_out,
                               args.summary_command, args.summary_label or f"{args.workload} workload")
    if args.suite:
        os.makedirs(os.path.dirname(os.path.abspath(args.suite_out)), exist_ok=True)
        return suite(args)

    import numpy as np
    import torch

    import block_sparse_attention_blocks_amd as pbsa
    from workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.mass_tau is not None:
        import dataclasses
        w = dataclasses.replace(w, mass_tau=args.mass_tau)
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    torch.cuda.set_device(0)
    log(f"[bench] workload {w.name}: N={w.seq_len} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"B={w.block_size} S={w.segment_size} tau={w.mass_tau}")
    t = time.perf_counter()
    x, dev = make_inputs(w, torch, np)
    log(f"[bench] inputs ready in {time.perf_counter() - t:.1f} s")
    q, k, v = dev["q"], dev["k"], dev["v"]
    B, S = w.block_size, w.segment_size
    Hq, Hkv, N, d = w.num_q_heads, w.num_kv_heads, w.seq_len, w.head_dim
    NB = w.num_blocks
    dv = q.device

    # preallocated outputs and workspaces: the timed step allocates nothing
    shape = pbsa.make_shape(q, k, B, S)
    ws_p = torch.empty(pbsa.workspace_size(shape, pbsa.PBSA_OP_PERMUTATION) + 256, dtype=torch.uint8, device=dv)
    ws_m = torch.empty(pbsa.workspace_size(shape, pbsa.PBSA_OP_MASK) + 256, dtype=torch.uint8, device=dv)
    ws_a = torch.empty(pbsa.workspace_size(shape, pbsa.PBSA_OP_ATTENTION) + 256, dtype=torch.uint8, device=dv)
    perm = torch.empty((Hkv, N), dtype=torch.int32, device=dv)
    count = torch.empty((Hq, NB), dtype=torch.int32, device=dv)
    idx = torch.empty((Hq, NB * (NB + 1) // 2), dtype=torch.int32, device=dv)
    out = torch.empty((Hq, N, d), dtype=torch.float32, device=dv)
    lse = torch.empty((Hq, N), dtype=torch.float32, device=dv)

    def stage_perm():
        pbsa.build_segment_permutation(q, k, B, S, perm=perm, workspace=ws_p)

    def stage_mask():
        pbsa.estimate_block_mask(q, k, perm, B, S, w.mass_tau, w.force_diag, w.force_first, out=(count, idx),
                                 workspace=ws_m)

    def stage_attn():
        pbsa.block_sparse_attn_prefill(q, k, v, perm, count, idx, B, S, out=out, lse=lse, workspace=ws_a)

    def step():
        stage_perm()
        stage_mask()
        stage_attn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    log(f"[bench] step {t_step * 1e3:.3f} ms")

    # per-stage times with HIP events on the stream the kernels are launched on
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    reps = max(args.steps, 5)
    ms_perm = timed(stage_perm, reps)
    ms_mask = timed(stage_mask, reps)
    ms_attn = timed(stage_attn, reps)

    def dense():
        pbsa.block_sparse_attn_prefill(q, k, v, None, None, None, B, S, out=out, lse=lse, workspace=ws_a)

    dense()
    ms_dense = timed(dense, max(3, reps // 2))
    stage_attn()  # leave the sparse result in `out`
    torch.cuda.synchronize()
    sdpa_ms, sdpa_backend = torch_sdpa_ms(torch, q, k, v, stream, 3)

    tiles = int(count.sum().item())
    causal_tiles = Hq * NB * (NB + 1) // 2
    flop_tile = 4.0 * B * B * d
    t_attn = sum(ms_attn) / len(ms_attn) * 1e-3
    achieved = tiles * flop_tile / t_attn / 1e12
    med = lambda xs: sorted(xs)[len(xs) // 2]

    res = {
        "metric": "attention prefill ms + dense-equivalent TFLOP/s at 32K/128K; % bf16 MFMA peak",
        "value": w.dense_causal_flop / t_step / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V with planted stripe keys and a local band)",
        "config": {"workload": w.name, "seq_len": N, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d,
                   "block_size": B, "segment_size": S, "mass_tau": w.mass_tau, "batch": 1,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": ATTN_KERNEL, "kernel_ms": t_attn * 1e3,
                     "flop_per_launch": tiles * flop_tile},
        "stages_ms": {"permutation": med(ms_perm), "mask": med(ms_mask), "attention": med(ms_attn)},
        "attention_ms": t_attn * 1e3,
        "attention_dense_equiv_tflops": w.dense_causal_flop / t_attn / 1e12,
        "block_density": tiles / causal_tiles,
        "dense_kernel_ms": med(ms_dense),
        "speedup_vs_dense_kernel": med(ms_dense) / (t_attn * 1e3),
        "dense_kernel_tflops": w.dense_causal_flop / (med(ms_dense) * 1e-3) / 1e12,
        "torch_sdpa_dense": {"ms": sdpa_ms, "backend": sdpa_backend,
                             "step_speedup": None if sdpa_ms is None else sdpa_ms / (t_step * 1e3)},
    }
    if args.copy_calib:
        copy_calibration(torch)
    res["roofline"]["traffic"] = read_traffic() if w.name == "llama8b_32k" and args.mass_tau is None else None
    if not args.no_subrecords:
        # the other workloads, timed after the main one (their inputs are generated here)
        del dev, q, k, v, out, lse, ws_p, ws_m, ws_a, perm, idx
        torch.cuda.empty_cache()
        from workloads import generate_for

        def load(wl, seed=None):
            xx = generate_for(wl, seed=seed)
            return {n: torch.from_numpy(xx[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}

        sub = {}
        t_sub = time.perf_counter()
        recs = measure_128k(torch, np, pbsa, WORKLOADS, load, stream, 5, sdpa=False)
        sub["llama8b_128k"] = {r["point"]: {kk: vv for kk, vv in r.items() if kk not in ("workload", "point")}
                               for r in recs}
        log(f"[bench] llama8b_128k: {json.dumps(sub['llama8b_128k'])}")
        sub["llama8b_64k_earlystop"] = measure_earlystop(torch, np, pbsa, WORKLOADS, load, stream, 5)
        log(f"[bench] llama8b_64k_earlystop: {json.dumps(sub['llama8b_64k_earlystop'])}")
        sub["single_head_1k"] = measure_1k(torch, np, pbsa, WORKLOADS, load, stream, 20)
        log(f"[bench] single_head_1k: {json.dumps(sub['single_head_1k'])}")
        log(f"[bench] sub-records in {time.perf_counter() - t_sub:.1f} s")
        res["subrecords"] = sub
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (bounded sample)")
        cb = cpu_baseline(w, x, count.cpu().numpy(), args.cpu_budget, np)
        res["cpu_baseline"] = {kk: cb[kk] for kk in ("value", "unit", "cores", "kind", "sample")}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
