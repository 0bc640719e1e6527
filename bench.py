"""Benchmark of the SageSLA hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
sage_quant_qk -> sla_block_mask -> sage_sla_attn_fwd (linear states, complement
GEMM and the sparse attention kernel). Inputs are resident in HBM before the
timed region. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0   # MI355X dense INT8 MFMA, published
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
HEAD_DIM = 128


def effective_ops(kidx, N, nqb, nkb, dense, BH=1):
    """4*D*sum over computed (query block, key block) pairs of valid-token
    products: QK^T and PV multiply-adds over the blocks actually computed, over
    all B*H heads (kidx [B][H][nqb][keep] covers them; a dense run has BH heads
    of every pair)."""
    nq = np.minimum(128, N - 128 * np.arange(nqb)).astype(np.float64)
    nk = np.minimum(64, N - 64 * np.arange(nkb)).astype(np.float64)
    if dense:
        per_head = nq.sum() * nk.sum()
        return 4.0 * HEAD_DIM * per_head * BH, None
    kid = kidx.reshape(-1, nqb, kidx.shape[-1])
    tot = (nk[kid].sum(axis=2) * nq[None, :]).sum()
    return 4.0 * HEAD_DIM * tot, None


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(q, k, v, w, keep, kidx_np):
    """The oracle timed on the host's cores over heads 0 and H-1 of the
    workload (quantization, block mask, linear states, sparse + linear
    attention rows of every query block), extrapolated over the heads (all
    heads do the same work up to the mask's tail-block choices)."""
    import oracle
    from bit_sparse_attention_amd.workloads import bf16_bits

    nthreads = oracle.threads()
    N, H, B = w.N, w.H, w.B
    nqb, nkb = (N + 127) // 128, (N + 63) // 64
    heads = sorted({0, B * H - 1})
    t_heads = 0.0
    for bh in heads:
        b, h = divmod(bh, H)
        qb = bf16_bits(q[b, h:h + 1]).reshape(1, N, 128)
        kb = bf16_bits(k[b, h:h + 1]).reshape(1, N, 128)
        vb = bf16_bits(v[b, h:h + 1]).reshape(1, N, 128)
        t0 = time.perf_counter()
        quant = oracle.quant_qk(qb, kb, nthreads)
        kh = None
        if not w.dense:
            kh, _ = oracle.block_mask_head(qb, kb, 0, keep, np.arange(nqb))
        hs = zs = None
        if not w.dense:
            hs, zs = oracle.linear_states(kb, vb, 0, nthreads)
        toks = np.arange(N)
        oracle.sparse_rows(*quant[:4], vb, 0, toks, kh, want=("decl",), nthreads=nthreads)
        if not w.dense:
            oracle.linear_rows(qb, hs, zs, 0, toks, kh, nthreads)
        t_heads += time.perf_counter() - t0
    t_full = t_heads / len(heads) * B * H
    ops_full, _ = effective_ops(kidx_np, N, nqb, nkb, w.dense, B * H)
    return {
        "value": ops_full / t_full / 1e12,
        "unit": "TOPS",
        "cores": nthreads,
        "kind": "oracle",
        "sample": (f"heads {heads} of {B * H} in full (quantization, block mask, linear states, "
                   f"sparse and linear attention rows of all {nqb} query blocks): {t_heads:.1f} s "
                   f"on {nthreads} threads (the job's CPU share) of {_cpu_model()}, extrapolated "
                   f"x{B * H / len(heads):g} over heads to {t_full:.0f} s for the workload"),
    }


# The dominant kernel of each benchmark and the sources that define it; an
# HBM-traffic record taken with rocprofv3 counters is valid only while these
# are unchanged.
ATTN_KERNEL = "sagesla_attn_kernel"
W8_KERNEL = "w8a8_gemm_kernel"
KERNEL_SOURCES = {
    ATTN_KERNEL: ("bit_sparse_attention_amd/csrc/attn.hip", "bit_sparse_attention_amd/csrc/common.hpp"),
    W8_KERNEL: ("bit_sparse_attention_amd/csrc/w8a8.hip", "bit_sparse_attention_amd/csrc/common.hpp"),
}
RECORD_PREFIX = {ATTN_KERNEL: "attn_kernel", W8_KERNEL: "w8a8_gemm"}
COPY_KERNEL = "copyBuffer"
TRAFFIC_UNIT = ("bytes past L2 per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled): "
                "HBM and Infinity Cache (MALL) together")
XCDS = 8


def _md_value(path, pattern):
    if not os.path.exists(path):
        return None
    m = re.search(pattern, open(path).read())
    return float(m.group(1)) if m else None


def mfma_bound(workload, ops, kern_ms):
    """The attention kernel's matrix-core bound at the sustained clock.

    The clock is GRBM_GUI_ACTIVE per XCD over the kernel's mean duration, both
    from the committed records of the same workload (a counter run and a
    kernel trace). The bound is the time the MFMAs alone take at that clock:
    half the effective ops are INT8 (QK^T) at the INT8 rate, half bf16 (PV) at
    half that rate."""
    cpath = os.path.join(ROOT, "profiles", f"attn_kernel_counters_{workload}.md")
    tpath = os.path.join(ROOT, "profiles", f"kernel_time_{workload}.md")
    grbm = _md_value(cpath, r"sagesla_attn_kernel[^|]*\| GRBM_GUI_ACTIVE \| \d+ \| ([0-9.e+]+)")
    t_us = _md_value(tpath, r"sagesla_attn_kernel[^|]*` \| \d+ \| ([0-9.]+)")
    if grbm is None or t_us is None:
        return None
    ghz = grbm / XCDS / (t_us * 1e3)
    scale = ghz / 2.4
    ms = ((ops / 2) / (INT8_PEAK_TOPS * 1e12 * scale) + (ops / 2) / (INT8_PEAK_TOPS / 2 * 1e12 * scale)) * 1e3
    return {"clock_ghz": round(ghz, 4), "ms": ms, "frac": ms / kern_ms if kern_ms else None,
            "frac_of_int8_peak": ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS,
            "source": f"profiles/attn_kernel_counters_{workload}.md (GRBM_GUI_ACTIVE per XCD) over "
                      f"profiles/kernel_time_{workload}.md (mean kernel time)"}


def sources_sha256(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_record_path(workload, kernel=ATTN_KERNEL):
    return os.path.join(ROOT, "profiles", f"{RECORD_PREFIX[kernel]}_hbm_traffic_{workload}.md")


def traffic_from_record(workload, kernel=ATTN_KERNEL):
    """HBM bytes per launch of the kernel from the committed counter record,
    or None when there is none or the kernel's sources changed since."""
    path = traffic_record_path(workload, kernel)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel") != kernel or rec.get("sources_sha256") != sources_sha256(kernel):
        return None
    k = rec["kernels"].get(kernel)
    return None if k is None else k["fetch_bytes"] + k["write_bytes"]


def _pmc_per_kernel(path, counter):
    """Per-dispatch values of a counter for each kernel in a rocprofv3
    counter_collection.csv (each value summed over the counter's instances)."""
    per_dispatch = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per_dispatch.items():
        out.setdefault(name, []).append(v)
    return out


def pmc_summary(fetch_csv, write_csv, copy_mib, workload, command, kernel=ATTN_KERNEL):
    """Markdown record of HBM traffic per launch from a FETCH_SIZE run and a
    WRITE_SIZE run, each scaled by what the same counter reads for a plain
    device copy of copy_mib MiB (which moves exactly that much each way)."""
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    # the calibration copies are the largest copy dispatches of the run
    cf = [max(v) for n, v in fetch.items() if COPY_KERNEL in n]
    cw = [max(v) for n, v in write.items() if COPY_KERNEL in n]
    if not cf or not cw:
        raise SystemExit("no copy-kernel dispatch in the counter files")
    sf, sw = copy_kib / max(cf), copy_kib / max(cw)
    fetch = {n: (len(v), sum(v) / len(v)) for n, v in fetch.items() if COPY_KERNEL not in n}
    write = {n: (len(v), sum(v) / len(v)) for n, v in write.items() if COPY_KERNEL not in n}
    lines = [f"# HBM traffic per launch, {workload}", "",
             "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over instances), "
             "each from its own rocprofv3 --pmc run, scaled by the factor that makes the same "
             f"counter read exactly {copy_mib} MiB for a device-to-device copy of {copy_mib} MiB "
             "in the same run.", "",
             f"Scale: FETCH x{sf:.4f}, WRITE x{sw:.4f} (the largest copy dispatch read "
             f"{max(cf):.0f} KiB and wrote {max(cw):.0f} KiB for {copy_kib:.0f} KiB moved).", "",
             "Commands:", ""]
    lines += [f"    {c}" for c in command]
    lines += ["", "| kernel | dispatches | FETCH KiB | WRITE KiB | scaled read MB | scaled write MB |",
              "|---|---|---|---|---|---|"]
    rec = {"workload": workload, "copy_mib": copy_mib, "fetch_scale": sf, "write_scale": sw,
           "kernel": kernel, "sources_sha256": sources_sha256(kernel), "kernels": {}}
    for name in sorted(fetch, key=lambda n: -fetch[n][1]):
        n, f = fetch[name]
        w = write.get(name, (0, float("nan")))[1]
        short = re.sub(r"\(.*", "", name)
        lines.append(f"| `{short}` | {n} | {f:.0f} | {w:.0f} | {f * sf * 1024 / 1e6:.1f} | "
                     f"{w * sw * 1024 / 1e6:.1f} |")
        if kernel in name:
            rec["kernels"][kernel] = {"fetch_bytes": f * sf * 1024, "write_bytes": w * sw * 1024}
    lines += ["", "```json", json.dumps(rec), "```", ""]
    return "\n".join(lines)


def trace_summary(stats_csv, workload, command):
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel_stats.csv."""
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# Kernel time per launch, {workload}", "", "Command:", ""]
    lines += [f"    {c}" for c in command]
    lines += ["", "| kernel | calls | avg us | min us | max us | % of GPU time |",
              "|---|---|---|---|---|---|"]
    for r in rows:
        short = re.sub(r"\(.*", "", r["Name"])
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    return "\n".join(lines) + "\n"


def pmc_table(csvs, workload, command, kernel_filter):
    """Markdown table: mean value per dispatch of every counter in the given
    rocprofv3 counter_collection.csv files, for kernels matching the filter."""
    vals = {}
    for path in csvs:
        per = {}
        for r in csv.DictReader(open(path)):
            if kernel_filter not in r["Kernel_Name"]:
                continue
            key = (re.sub(r"\(.*", "", r["Kernel_Name"]), r["Counter_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (kern, ctr, _), v in per.items():
            vals.setdefault((kern, ctr), []).append(v)
    lines = [f"# Counters per dispatch, {workload}", "", "Commands:", ""]
    lines += [f"    {c}" for c in command]
    lines += ["", "| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
    for (kern, ctr), v in sorted(vals.items()):
        lines.append(f"| `{kern}` | {ctr} | {len(v)} | {sum(v) / len(v):.6g} |")
    return "\n".join(lines) + "\n"


def copy_calibration(mib):
    """A plain device-to-device copy of `mib` MiB, three times, for scaling
    HBM byte counters."""
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"# copy calibration: 3 x {mib} MiB device copies", file=sys.stderr, flush=True)


def bench_w8a8(args):
    """The W8A8 linear layer (page 5, Pillar Three) on the 14B / 720p linear
    shape: per step, the block quantization of the activations and the
    block-dequantized INT8 product with weights quantized once beforehand."""
    import torch

    import bit_sparse_attention_amd as ssa
    from bit_sparse_attention_amd.workloads import (LINEAR_BENCH_WORKLOAD, LINEAR_WORKLOADS,
                                                    make_linear_workload)

    wl = LINEAR_WORKLOADS[args.workload or LINEAR_BENCH_WORKLOAD]
    dev = torch.device("cuda:0")
    print(f"# generating {wl.name}", file=sys.stderr, flush=True)
    x, wt = make_linear_workload(wl)
    xd, wd = x.to(dev), wt.to(dev)
    wq, sw = ssa.w8a8_quant(wd)
    xq, sx = ssa.w8a8_quant(xd)
    for _ in range(args.warmup):
        xq, sx = ssa.w8a8_quant(xd)
        y = ssa.w8a8_gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record()
        xq, sx = ssa.w8a8_quant(xd)
        e1.record()
        y = ssa.w8a8_gemm(xq, sx, wq, sw)
        e2.record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    q_ms = [a.elapsed_time(b) for a, b, _ in ev]
    g_ms = [b.elapsed_time(c) for _, b, c in ev]
    ops = 2.0 * wl.M * wl.N * wl.K
    g_mean = float(np.mean(g_ms))
    g_tops = ops / (g_mean * 1e-3) / 1e12
    line = {
        "metric": "W8A8 linear (block-128x128 INT8) ms/call + TOPS (% INT8 MFMA peak), 14B-720p linear shape, 1 GPU",
        "value": ops / (ms_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x int8 -> int32 per 128-block, fp32 dequantized accumulation",
        "data": "synthetic (seeded; x ~ N(0,1) with 1% of channels x20, w ~ N(0,1)/sqrt(K))",
        "config": {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K, "block": 128},
        "quant_ms": float(np.mean(q_ms)),
        "gemm_ms": g_mean,
        "gemm_ms_pct": {f"p{p}": float(np.percentile(g_ms, p)) for p in (10, 50, 90)},
        "roofline": {"bound": "mfma", "achieved": g_tops, "peak": INT8_PEAK_TOPS,
                     "unit": "TOP/s", "frac": g_tops / INT8_PEAK_TOPS,
                     "traffic": traffic_from_record(wl.name, W8_KERNEL),
                     "traffic_unit": TRAFFIC_UNIT},
    }
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    if not args.no_cpu_baseline:
        import oracle
        from bit_sparse_attention_amd.workloads import bf16_bits

        nthreads = oracle.threads()
        xb = bf16_bits(x).reshape(wl.M, wl.K)
        wb = bf16_bits(wt).reshape(wl.N, wl.K)
        t0 = time.perf_counter()
        oxq, osx = oracle.w8a8_quant(xb, nthreads)
        owq, osw = oracle.w8a8_quant(wb, nthreads)
        tq = time.perf_counter() - t0
        rows = np.arange(0, wl.M, max(1, wl.M // 512))
        t0 = time.perf_counter()
        oracle.w8a8_gemm(oxq, osx, owq, osw, rows=rows, nthreads=nthreads)
        tg = time.perf_counter() - t0
        t_full = tq + tg * wl.M / len(rows)
        line["cpu_baseline"] = {
            "value": ops / t_full / 1e12, "unit": "TOPS", "cores": nthreads, "kind": "oracle",
            "sample": (f"quantization of x and w in full ({tq:.1f} s) and the product for "
                       f"{len(rows)} of {wl.M} rows ({tg:.1f} s) on {nthreads} threads (the job's "
                       f"CPU share) of "
                       f"{_cpu_model()}, extrapolated over the rows to {t_full:.0f} s"),
        }
    print(json.dumps(line), flush=True)


BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def bench_bwd(args):
    """The SageSLA backward (sage_sla_attn_bwd) on the benchmarked workload:
    per step, the gradients of Q, K, V for a seeded dL/dO, from the forward's
    quantized tensors, selection, fp32 output and row statistics (the forward
    runs once before timing, as in training, where it precedes the backward).
    Useful work = the four gradient products per computed block pair,
    8*D*n_q*n_k (dP, dV, dQ, dK; the recomputed scores not counted)."""
    import ctypes as C

    import torch

    import bit_sparse_attention_amd as ssa
    from bit_sparse_attention_amd.workloads import BENCH_WORKLOAD, WORKLOADS, make_workload

    w = WORKLOADS[args.workload or BENCH_WORKLOAD]
    dev = torch.device("cuda:0")
    print(f"# generating {w.name}", file=sys.stderr, flush=True)
    q, k, v = make_workload(w)
    # the forward keeps its fp32 output and row statistics for the backward
    plan = ssa.SageSLAPlan(w.B, w.H, w.N, w.topk, linear=True, device=dev, want_f32=True,
                           want_lse=True)
    plan.bind(q.to(dev), k.to(dev), v.to(dev))
    plan.run()
    g = torch.Generator().manual_seed(1)
    dout = torch.randn(w.B, w.H, w.N, HEAD_DIM, generator=g).to(torch.bfloat16).to(dev)
    grads = [torch.empty((w.B, w.H, w.N, HEAD_DIM), dtype=torch.float32, device=dev)
             for _ in range(3)]
    L = ssa._load()
    ws_n = ssa.workspace_bytes(ssa.OP_BWD, plan.shape, plan.keep, plan.branches)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    p = lambda t: None if t is None else C.c_void_p(t.data_ptr())  # noqa: E731

    def step():
        st = L.sage_sla_attn_bwd(p(plan.q), p(plan.k), p(plan.v), plan.shape, p(plan.q_i8),
                                 p(plan.q_scale), p(plan.k_i8), p(plan.k_scale), p(plan.kidx),
                                 plan.keep, plan.branches, plan.sm_scale, p(dout),
                                 p(plan.out32), p(plan.lse), *map(p, grads), p(ws), ws_n,
                                 C.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(L.ssa_last_error().decode())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    ev_ms = e0.elapsed_time(e1) / K
    kidx_np = None if plan.dense else plan.kidx.cpu().numpy()
    fwd_ops, _ = effective_ops(kidx_np, w.N, plan.nqb, plan.nkb, plan.dense, w.B * w.H)
    ops = 2.0 * fwd_ops  # 8*D*n_q*n_k against the forward's 4*D*n_q*n_k
    tflops = ops / (ms_step * 1e-3) / 1e12
    line = {
        "metric": "SageSLA backward ms/call + effective TFLOP/s (% bf16 MFMA peak), 14B-720p shape, 1 GPU",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "event_ms_per_step": ev_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 score recompute; bf16 x bf16 -> fp32 gradient products; fp32 linear branch",
        "data": "synthetic (seeded; the forward's inputs, dL/dO ~ N(0,1))",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": HEAD_DIM,
                   "topk": w.topk, "keep": plan.keep, "branches": "sparse+linear"
                   if plan.branches == 3 else "sparse", "call": "sage_sla_attn_bwd"},
        "effective_ops": ops,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS, "traffic": None,
                     "note": "whole backward call (statistics pass, prep, dq, dk/dv and linear "
                             "kernels) against the bf16 peak; per-kernel times in profiles/"},
    }
    if not args.no_cpu_baseline:
        import oracle
        from bit_sparse_attention_amd.workloads import bf16_bits, make_qkv

        # one head, the first 100 query blocks (12800 tokens) at the same keep fraction
        Ns = 12800
        qs, ks_, vs = make_qkv(1, 1, Ns, HEAD_DIM, seed=0)
        gs = torch.randn(1, 1, Ns, HEAD_DIM, generator=g).to(torch.bfloat16)
        qb, kb, vb, gb = (bf16_bits(t).reshape(1, Ns, HEAD_DIM) for t in (qs, ks_, vs, gs))
        nthreads = oracle.threads()
        t0 = time.perf_counter()
        quant = oracle.quant_qk(qb, kb, nthreads)[:4]
        keep_s = oracle.keep_blocks(Ns, w.topk)
        kh, _ = oracle.block_mask_head(qb, kb, 0, keep_s)
        oracle.sagesla_bwd(qb, kb, vb, quant, 0, gb, kh, plan.branches, nthreads=nthreads)
        ts = time.perf_counter() - t0
        sops, _ = effective_ops(kh[None], Ns, (Ns + 127) // 128, (Ns + 63) // 64, False, 1)
        t_full = ts * ops / (2.0 * sops)
        line["cpu_baseline"] = {
            "value": ops / t_full / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": (f"one head of {Ns} tokens at keep {keep_s} (quantization, mask and the "
                       f"fp64 backward): {ts:.1f} s on {nthreads} threads (the job's CPU share) "
                       f"of {_cpu_model()}, extrapolated by the computed-pair work to "
                       f"{t_full:.0f} s for the workload"),
        }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stages", action="store_true",
                    help="also time each staged ABI call on its own, and the staged step")
    ap.add_argument("--staged", action="store_true",
                    help="time the three staged calls instead of the one-call step")
    ap.add_argument("--flush", type=int, default=0, metavar="MIB",
                    help="after the timed steps, time K more, each after overwriting a MIB-MiB "
                         "buffer (evicts L2 and the Infinity Cache); reported as 'flushed'")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run a plain MIB-MiB device copy (for counter scaling)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic record from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_STATS_CSV",
                    help="print a kernel-time table from a rocprofv3 --stats run and exit")
    ap.add_argument("--pmc-table", nargs="+", metavar="COUNTER_CSV",
                    help="print a per-dispatch counter table for the attention kernel and exit")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="command line recorded in the summary outputs")
    ap.add_argument("--w8a8", action="store_true",
                    help="benchmark the W8A8 linear layer instead (its own JSON line)")
    ap.add_argument("--bwd", action="store_true",
                    help="benchmark the SageSLA backward instead (its own JSON line)")
    args = ap.parse_args()
    if args.pmc_summary or args.trace_summary or args.pmc_table:
        from bit_sparse_attention_amd.workloads import BENCH_WORKLOAD, LINEAR_BENCH_WORKLOAD
        # --bwd: every kernel the counter files hold (the runs select them)
        kernel = W8_KERNEL if args.w8a8 else ("" if args.bwd else ATTN_KERNEL)
        wl = args.workload or (LINEAR_BENCH_WORKLOAD if args.w8a8 else BENCH_WORKLOAD)
        if args.pmc_summary:
            print(pmc_summary(*args.pmc_summary, args.copy_calibration or 1024, wl,
                              args.pmc_command, kernel))
        elif args.trace_summary:
            print(trace_summary(args.trace_summary, wl, args.pmc_command))
        else:
            print(pmc_table(args.pmc_table, wl, args.pmc_command, kernel))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the SageSLA path is "
              "per-head independent and this build measures one GPU's share; no multi-GPU "
              "figure is produced.", file=sys.stderr)
        sys.exit(2)

    if args.w8a8:
        bench_w8a8(args)
        return
    if args.bwd:
        bench_bwd(args)
        return

    import torch

    import bit_sparse_attention_amd as ssa
    from bit_sparse_attention_amd.workloads import BENCH_WORKLOAD, WORKLOADS, make_workload

    w = WORKLOADS[args.workload or BENCH_WORKLOAD]
    dev = torch.device("cuda:0")
    print(f"# generating {w.name}", file=sys.stderr, flush=True)
    q, k, v = make_workload(w)
    plan = ssa.SageSLAPlan(w.B, w.H, w.N, w.topk, linear=True, device=dev, fused=not args.staged)
    plan.bind(q.to(dev), k.to(dev), v.to(dev))
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    K = args.steps
    with ssa.KernelTimer(K) as timer:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            plan.run()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kern_ms = timer.read()
    ms_step = (t1 - t0) * 1e3 / K
    print(f"# timed {K} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    flushed = None
    if args.flush:
        junk = torch.empty(args.flush << 20, dtype=torch.uint8, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        with ssa.KernelTimer(K) as ftimer:
            for e0, e1 in ev:
                junk.fill_(1)
                e0.record()
                plan.run()
                e1.record()
            torch.cuda.synchronize()
            fk = ftimer.read()
        fs = [a.elapsed_time(b) for a, b in ev]
        flushed = {"flush_mib": args.flush, "ms_per_step": float(np.mean(fs)),
                   "attn_kernel_ms": float(np.mean(fk)) if fk else None}
        del junk

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    stages = None
    if args.stages:
        stages = {}
        for name, fn in (("sage_quant_qk", plan.quant), ("sla_block_mask", plan.mask),
                         ("sage_sla_attn_fwd", plan.attn), ("staged_step", plan.run_staged),
                         ("sage_sla_fwd", plan.step)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(K):
                fn()
            e1.record()
            torch.cuda.synchronize()
            stages[name] = round(e0.elapsed_time(e1) / K, 4)

    kidx_np = None if plan.dense else plan.kidx.cpu().numpy()
    ops, _ = effective_ops(kidx_np, w.N, plan.nqb, plan.nkb, plan.dense, w.B * w.H)
    k_ms = float(np.mean(kern_ms)) if kern_ms else float("nan")
    k_pct = ({f"p{p}": float(np.percentile(kern_ms, p)) for p in (10, 50, 90)}
             if kern_ms else None)
    k_tops = ops / (k_ms * 1e-3) / 1e12
    line = {
        "metric": "SageSLA attn ms/call + effective INT8 TOPS (% MFMA peak), 14B-720p shape, 1 GPU",
        "value": ops / (ms_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 QK^T + bf16 PV (fp32 softmax/accumulate)",
        "data": "synthetic (seeded; Q,V ~ N(0,1), K ~ N(0,1) + per-channel N(0,3) offset)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": HEAD_DIM,
                   "topk": w.topk, "keep": plan.keep, "branches": "sparse+linear"
                   if plan.branches == 3 else "sparse", "spikes": w.spikes,
                   "call": "sage_sla_fwd" if plan.fused else "staged"},
        "attn_kernel_ms": k_ms,
        "attn_kernel_ms_pct": k_pct,
        "attn_kernel_tops": k_tops,
        "effective_ops": ops,
        "roofline": {"bound": "mfma", "achieved": k_tops, "peak": INT8_PEAK_TOPS,
                     "unit": "TOP/s", "frac": k_tops / INT8_PEAK_TOPS, "traffic": traffic_from_record(w.name),
                     "traffic_unit": TRAFFIC_UNIT},
    }
    bound = mfma_bound(w.name, ops, k_ms)
    if bound is not None:
        line["mfma_bound"] = bound
    if stages is not None:
        line["stages_ms"] = stages
    if flushed is not None:
        line["flushed"] = flushed
    if not args.no_cpu_baseline:
        print("# timing the oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(q, k, v, w, plan.keep, kidx_np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
