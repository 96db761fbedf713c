#!/usr/bin/env python3
"""Benchmark of the SpargeAttn hot path on one MI355X.

Workload: 128K-token GQA causal prefill (B=1, 32 query heads, 8 kv heads,
N=131072, d=128, bf16; AR(1)+sink synthetic Q/K, N(0,1) V; tau=0.9,
theta=0.5, lambda=-6).  One step = stage 1 (sparge_predict_mask: pooling,
self-similarity, compressed map, TopCdf, forcing, row lists) + stage 2
(sparge_attn: block-sparse attention with the lambda rule) over the resident
inputs.  The int8 variant (sparge_quant_qk_int8 + int8-QK / fp16-PV attention)
is timed after it and reported beside the headline.

Prints one JSON line (rank 0).  The metric is dense-equivalent attention
TFLOPS = (4 N^2 d H / 2 for causal) / step time, with the achieved sparsity
and the mask-prediction share of the step; ``roofline`` is the attention
kernel's executed MFMA flops per second against the bf16 dense peak.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-int8", action="store_true", help="skip the int8 variant")
    ap.add_argument("--no-fp8pv", action="store_true", help="skip the fp8 P~V variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=150,
                    help="query blocks of head 0 the CPU oracle attends (sample size)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"))
    return ap.parse_args()


def dense_equiv_flops(N, d, H, causal):
    f = 4.0 * N * N * d * H
    return f / 2 if causal else f


def executed_flops(c, d, bq=128, bk=64, rows=32):
    return c["qk_exec"] * 2.0 * bq * bk * d + c["pv_exec"] * 2.0 * rows * bk * d


def attn_source_digest() -> str:
    """sha256 over the attention kernel's sources: HBM counters taken on an
    older kernel no longer describe this one."""
    import hashlib
    h = hashlib.sha256()
    for name in ("k_attn.hip", "common.hpp"):
        with open(os.path.join(ROOT, "free_block_sparse_mask_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def cpu_baseline(w, q, k, v, nblocks):
    """The float64 oracle on a bounded sample: stage 1 for query head 0 (its
    kv head pooled in full) and stage 2 for ``nblocks`` evenly spaced query
    blocks of head 0.  Returns a dict with dense-equivalent TFLOPS of the
    sampled work."""
    from oracle import sparge_oracle as O
    try:
        import threadpoolctl
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        threads = 1
    t0 = time.perf_counter()
    Q0 = O.widen(q[0, 0], w.dtype)
    K0 = O.widen(k[0, 0], w.dtype)
    V0 = O.widen(v[0, 0], w.dtype)
    pred = O.predict_mask_head(Q0, K0, w.tau, w.theta, w.causal)
    Tm = O.num_blocks(w.N, O.BQ)
    blocks = sorted(set(np.linspace(0, Tm - 1, nblocks).round().astype(int).tolist()))
    dense = 0.0
    for i in blocks:
        O.attend_row_block(Q0, K0, V0, pred["mg"][i], i, w.lam, w.causal)
        r = O.block_rows(w.N, O.BQ, i)
        if w.causal:
            pairs = sum(q_ + 1 for q_ in range(r.start, r.stop))
        else:
            pairs = len(r) * w.N
        dense += 4.0 * pairs * w.d
    dt = time.perf_counter() - t0
    return {"value": dense / dt / 1e12, "unit": "TFLOPS (dense-equivalent)", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 oracle: stage 1 for query head 0 of the workload (its kv head pooled "
                      f"over all {w.N} tokens) + stage 2 for {len(blocks)} evenly spaced query blocks "
                      f"of head 0; {dt:.1f} s wall; dense-equivalent flops of the sampled blocks / time"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus "
              f"{args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    import free_block_sparse_mask_amd as fb
    from free_block_sparse_mask_amd import inputs as I

    w = I.workload(4)
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    q, k, v = I.make_qkv(w, workers=16)
    log(f"[bench] generated inputs in {time.perf_counter() - t0:.1f} s")

    def up(bits, dtype):
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16 if dtype == "bf16" else torch.float16)
        return t.to(dev)

    qd, kd, vd = up(q, "bf16"), up(k, "bf16"), up(v, "bf16")
    vd16 = vd.float().to(torch.float16) if not args.no_int8 else None
    ws = fb.workspace(qd, kd)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal, ws=ws)
        if ev is not None:
            ev[1].record()
        o, counts, _ = fb.attn(qd, kd, vd, mask, w.lam, w.causal)
        if ev is not None:
            ev[2].record()
        return o, counts, mask

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for s in range(args.steps):
        o, counts, mask = step(evs[s])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    pred_ms = [e[0].elapsed_time(e[1]) for e in evs]
    attn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    c = fb.counts_dict(counts)
    log(f"[bench] bf16 step: wall {wall_ms:.3f} ms, predict {np.mean(pred_ms):.3f} ms, "
        f"attn {np.mean(attn_ms):.3f} ms, counts {c}")

    dense = dense_equiv_flops(w.N, w.d, w.H, w.causal)
    step_ms = float(np.mean(pred_ms) + np.mean(attn_ms))
    live_flops = c["live_tiles"] * 4.0 * 128 * 64 * w.d
    exe = executed_flops(c, w.d)
    attn_avg = float(np.mean(attn_ms))
    achieved = exe / (attn_avg * 1e-3) / 1e12
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            if tj.get("kernel_source_sha256") == attn_source_digest():
                traffic = tj.get("attn_fwd_bytes_per_launch")
        except Exception:
            traffic = None
    result = {
        "metric": "dense-equiv attn TFLOPS + sparsity @128K GQA prefill; mask-pred % of time",
        "value": dense / (wall_ms * 1e-3) / 1e12,
        "unit": "TFLOPS (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded AR(1)+sink Q/K, N(0,1) V; no trained weights)",
        "config": {"workload": "gqa_128k_causal_prefill", "B": w.B, "H": w.H, "H_kv": w.H_kv,
                   "N": w.N, "d": w.d, "causal": w.causal, "tau": w.tau, "theta": w.theta,
                   "lambda": w.lam, "bq": 128, "bk": 64},
        "sparsity": {
            "headline": 1.0 - exe / live_flops,
            "mg_block": 1.0 - c["qk_exec"] / c["live_tiles"],
            "lambda_skip_of_executed_groups": c["pv_skip"] / max(1, c["pv_exec"] + c["pv_skip"]),
        },
        "mask_pred_share": float(np.mean(pred_ms)) / step_ms,
        "predict_ms": float(np.mean(pred_ms)),
        "predict_ms_median_min": [float(np.median(pred_ms)), float(np.min(pred_ms))],
        "attn_ms": attn_avg,
        "attn_ms_median_min": [float(np.median(attn_ms)), float(np.min(attn_ms))],
        "event_step_ms": step_ms,
        "counts": c,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "transpose_v + build_packs + attn_stats (packed, then single) + sum_counts + attn_pv "
                               "<128, bf16, causal> (one sparge_attn call)",
                     "flops_per_launch": exe},
    }

    if not args.no_int8:
        del o, mask
        torch.cuda.synchronize()

        def step8(ev=None):
            if ev is not None:
                ev[0].record()
            q8, k8, qs, ks = fb.quant_qk_int8(qd, kd, ws=ws)
            if ev is not None:
                ev[1].record()
            mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal, ws=ws)
            if ev is not None:
                ev[2].record()
            o, counts, _ = fb.attn(q8, k8, vd16, mask, w.lam, w.causal, q_scale=qs, k_scale=ks)
            if ev is not None:
                ev[3].record()
            return counts

        for _ in range(args.warmup):
            step8()
        torch.cuda.synchronize()
        evs8 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        t8 = time.perf_counter()
        for s in range(args.steps):
            counts8 = step8(evs8[s])
        torch.cuda.synchronize()
        wall8 = (time.perf_counter() - t8) * 1e3 / args.steps
        quant_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs8]))
        pred8 = float(np.mean([e[1].elapsed_time(e[2]) for e in evs8]))
        attn8 = float(np.mean([e[2].elapsed_time(e[3]) for e in evs8]))
        c8 = fb.counts_dict(counts8)
        qk_f = c8["qk_exec"] * 2.0 * 128 * 64 * w.d
        pv_f = c8["pv_exec"] * 2.0 * 32 * 64 * w.d
        result["int8"] = {
            "ms_per_step": wall8, "quant_ms": quant_ms, "predict_ms": pred8, "attn_ms": attn8,
            "dense_equiv_tflops": dense / (wall8 * 1e-3) / 1e12,
            "mfma_frac_executed": (qk_f / (PEAK_INT8_TOPS * 1e12) + pv_f / (PEAK_BF16_TFLOPS * 1e12))
                                  / (attn8 * 1e-3),
            "counts": c8,
        }
        log(f"[bench] int8 step: wall {wall8:.3f} ms, quant {quant_ms:.3f}, predict {pred8:.3f}, attn {attn8:.3f}")

    if not args.no_fp8pv:
        # the fp8 P~V variant (sparge_attn_fp8pv) on the same bf16 inputs
        torch.cuda.synchronize()

        def step_f8(ev=None):
            if ev is not None:
                ev[0].record()
            mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal, ws=ws)
            if ev is not None:
                ev[1].record()
            o, counts, _ = fb.attn(qd, kd, vd, mask, w.lam, w.causal, ws=ws, fp8_pv=True)
            if ev is not None:
                ev[2].record()
            return counts

        for _ in range(args.warmup):
            step_f8()
        torch.cuda.synchronize()
        evsf = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        tf = time.perf_counter()
        for s in range(args.steps):
            countsf = step_f8(evsf[s])
        torch.cuda.synchronize()
        wallf = (time.perf_counter() - tf) * 1e3 / args.steps
        predf = float(np.mean([e[0].elapsed_time(e[1]) for e in evsf]))
        attnf = float(np.mean([e[1].elapsed_time(e[2]) for e in evsf]))
        cf = fb.counts_dict(countsf)
        result["fp8pv"] = {
            "ms_per_step": wallf, "predict_ms": predf, "attn_ms": attnf,
            "dense_equiv_tflops": dense / (wallf * 1e-3) / 1e12, "counts": cf,
        }
        log(f"[bench] fp8 P~V step: wall {wallf:.3f} ms, predict {predf:.3f}, attn {attnf:.3f}")

    if args.copy_calib_mb:
        n = args.copy_calib_mb * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calib_bytes_each_way"] = n * 4

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_blocks)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
