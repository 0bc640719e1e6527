"""Benchmark of the SageSLA hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
sage_quant_qk -> sla_block_mask -> sage_sla_attn_fwd (linear states, complement
GEMM and the sparse attention kernel). Inputs are resident in HBM before the
timed region. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0   # MI355X dense INT8 MFMA, published
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
HEAD_DIM = 128


def effective_ops(kidx, N, nqb, nkb, dense):
    """4*D*sum over computed (query block, key block) pairs of valid-token
    products: QK^T and PV multiply-adds over the blocks actually computed."""
    nq = np.minimum(128, N - 128 * np.arange(nqb)).astype(np.float64)
    nk = np.minimum(64, N - 64 * np.arange(nkb)).astype(np.float64)
    if dense:
        per_head = nq.sum() * nk.sum()
        return 4.0 * HEAD_DIM * per_head, None
    kid = kidx.reshape(-1, nqb, kidx.shape[-1])
    tot = (nk[kid].sum(axis=2) * nq[None, :]).sum()
    return 4.0 * HEAD_DIM * tot, None


def cpu_baseline(q, k, v, w, keep, kidx_np, budget_blocks=128):
    """Oracle timed on the host: head 0, full quantization / linear states of
    that head and `budget_blocks` query blocks of mask + attention rows,
    extrapolated to the whole workload."""
    import oracle
    from bit_sparse_attention_amd.workloads import bf16_bits

    nthreads = min(16, os.cpu_count() or 1)
    N, H, B = w.N, w.H, w.B
    nqb, nkb = (N + 127) // 128, (N + 63) // 64
    qb = bf16_bits(q[0, :1]).reshape(1, N, 128)
    kb = bf16_bits(k[0, :1]).reshape(1, N, 128)
    vb = bf16_bits(v[0, :1]).reshape(1, N, 128)
    t0 = time.perf_counter()
    quant = oracle.quant_qk(qb, kb, nthreads)
    t_quant = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    blocks = np.sort(rng.choice(nqb, size=min(budget_blocks, nqb), replace=False))
    t0 = time.perf_counter()
    if w.dense:
        kh = None
    else:
        kh_rows, _ = oracle.block_mask_head(qb, kb, 0, keep, blocks)
        kh = np.zeros((nqb, keep), np.int32)
        kh[blocks] = kh_rows
    t_mask = time.perf_counter() - t0
    toks = np.concatenate([np.arange(b * 128, min(N, b * 128 + 128)) for b in blocks])
    t0 = time.perf_counter()
    h = z = None
    if not w.dense:
        h, z = oracle.linear_states(kb, vb, 0, nthreads)
    t_states = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.sparse_rows(*quant[:4], vb, 0, toks, kh, want=("decl",), nthreads=nthreads)
    if not w.dense:
        oracle.linear_rows(qb, h, z, 0, toks, kh, nthreads)
    t_rows = time.perf_counter() - t0
    frac = nqb / len(blocks)
    t_head = t_quant + t_states + (t_mask + t_rows) * frac
    t_full = t_head * B * H
    ops_full, _ = effective_ops(kidx_np, N, nqb, nkb, w.dense)
    sample_s = t_quant + t_mask + t_states + t_rows
    return {
        "value": ops_full / t_full / 1e12,
        "unit": "TOPS",
        "cores": nthreads,
        "kind": "oracle",
        "sample": (f"head 0 of {B * H}: full quantization and linear states, {len(blocks)} of "
                   f"{nqb} query blocks of mask + attention rows ({sample_s:.1f} s of CPU work), "
                   f"extrapolated x{frac:.1f} over blocks and x{B * H} over heads; "
                   f"full-workload oracle time {t_full:.0f} s"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stages", action="store_true", help="also time each ABI call on its own")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the SageSLA path is "
              "per-head independent and this build measures one GPU's share; no multi-GPU "
              "figure is produced.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_sparse_attention_amd as ssa
    from bit_sparse_attention_amd.workloads import BENCH_WORKLOAD, WORKLOADS, make_workload

    w = WORKLOADS[args.workload or BENCH_WORKLOAD]
    dev = torch.device("cuda:0")
    print(f"# generating {w.name}", file=sys.stderr, flush=True)
    q, k, v = make_workload(w)
    plan = ssa.SageSLAPlan(w.B, w.H, w.N, w.topk, linear=True, device=dev)
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

    stages = None
    if args.stages:
        stages = {}
        for name, fn in (("sage_quant_qk", plan.quant), ("sla_block_mask", plan.mask),
                         ("sage_sla_attn_fwd", plan.attn)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(K):
                fn()
            e1.record()
            torch.cuda.synchronize()
            stages[name] = round(e0.elapsed_time(e1) / K, 4)

    kidx_np = None if plan.dense else plan.kidx.cpu().numpy()
    ops, _ = effective_ops(kidx_np, w.N, plan.nqb, plan.nkb, plan.dense)
    k_ms = float(np.mean(kern_ms)) if kern_ms else float("nan")
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
                   if plan.branches == 3 else "sparse", "spikes": w.spikes},
        "attn_kernel_ms": k_ms,
        "attn_kernel_tops": k_tops,
        "effective_ops": ops,
        "roofline": {"bound": "mfma", "achieved": k_tops, "peak": INT8_PEAK_TOPS,
                     "unit": "TOP/s", "frac": k_tops / INT8_PEAK_TOPS, "traffic": None},
    }
    if stages is not None:
        line["stages_ms"] = stages
    if not args.no_cpu_baseline:
        print("# timing the oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(q, k, v, w, plan.keep, kidx_np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
