"""Token-order comparison on a video workload: the analogue of the
permutation table of [Review] (Table 4: random, row-major, time-major and
HilbertCurve orders, with Sim-q, Sim-k, L1 and sparsity).

Pages: [Review] "SpargeAttn: Accurate and Training-free Sparse Attention
Accelerating Any Model Inference" (xllm-io paper-review blog), Table 4 and
"HilbertCurve Permutation"; [Rebuttal] reply "Weaknesses3.2".

For each order the HIP path gathers Q, K, V into that order
(sparge_hilbert_permute), predicts M_g (whose block self-similarities give
Sim-q and Sim-k: the mean CosSim over the query / key blocks), runs sparse
attention and full attention (M_g all ones, lambda off), and measures the
relative L1 of the two (sparge_l1_sums) and the skipped share of the MFMA
work (kernel counters).  Full attention commutes with a token order, so each
order's L1 compares like with like.

Run: python -m free_block_sparse_mask_amd.permutation_report [--heads H] [--theta T] [--tau T]
"""
from __future__ import annotations

import argparse
import json
import math

import numpy as np

from . import (BK, BQ, ORDER_HILBERT, ORDER_ROWMAJOR, ORDER_TIMEMAJOR, attn, counts_dict, grid_order,
               hilbert_permute, l1_error, num_blocks, predict_mask)
from .tune import sparsity_from_counts

ORDERS = ("random", "rowmajor", "timemajor", "hilbert")


def order_perm(name: str, grid, seed: int = 0) -> np.ndarray:
    T, Hg, Wg = grid
    if name == "random":
        from .inputs import random_order
        return random_order(T * Hg * Wg, seed)
    code = {"rowmajor": ORDER_ROWMAJOR, "timemajor": ORDER_TIMEMAJOR, "hilbert": ORDER_HILBERT}[name]
    return grid_order(T, Hg, Wg, code)[0]


def measure(q, k, v, grid, tau: float, theta: float, lam: float, orders=ORDERS, seed: int = 0):
    """q [B, H, N, d], k/v [B, H_kv, N, d] on the device, tokens in raster
    order of ``grid`` (non-causal).  Returns one dict per order."""
    import torch
    B, H, N, d = q.shape
    rows = []
    for name in orders:
        perm = torch.from_numpy(order_perm(name, grid, seed)).to(q.device)
        qp, kp, vp = (hilbert_permute(x, perm) for x in (q, k, v))
        mask = predict_mask(qp, kp, tau, theta, False)
        o, counts, _ = attn(qp, kp, vp, mask, lam, False, out_f32=True)
        ones = torch.ones((B, H, num_blocks(N, BQ), num_blocks(N, BK)), dtype=torch.uint8, device=q.device)
        o_ref, _, _ = attn(qp, kp, vp, ones, -math.inf, False, out_f32=True)
        c = counts_dict(counts)
        rows.append({
            "order": name,
            "sim_q": float(mask.s_q.mean().item()),
            "sim_k": float(mask.s_k.mean().item()),
            "l1": l1_error(o, o_ref),
            "sparsity": sparsity_from_counts(c, d),
            "mg_density": c["qk_exec"] / max(1, c["live_tiles"]),
        })
        del qp, kp, vp, o, o_ref, mask
    return rows


def markdown(rows) -> str:
    out = ["| order | Sim-q | Sim-k | L1 | sparsity | M_g density |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| {r['order']} | {r['sim_q']:.3f} | {r['sim_k']:.3f} | {r['l1']:.4f} | "
                   f"{r['sparsity']:.3f} | {r['mg_density']:.3f} |")
    return "\n".join(out)


def main(argv=None):
    import torch
    from . import inputs as I
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--heads", type=int, default=0, help="query heads (0: the workload's 24)")
    ap.add_argument("--seed", type=int, default=0, help="seed of the random order")
    ap.add_argument("--theta", type=float, default=None, help="theta (default: the workload's 0.5)")
    ap.add_argument("--tau", type=float, default=None, help="tau (default: the workload's 0.9)")
    args = ap.parse_args(argv)
    w = I.workload(3)
    if args.heads:
        w = w.with_sizes(H=args.heads, H_kv=args.heads)
    if args.theta is not None:
        w = w.with_sizes(theta=args.theta)
    if args.tau is not None:
        w = w.with_sizes(tau=args.tau)
    q, k, v = I.make_qkv(w, workers=16)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")

    rows = measure(up(q), up(k), up(v), w.grid, w.tau, w.theta, w.lam, seed=args.seed)
    print(markdown(rows))
    print(json.dumps({"workload": w.name, "grid": w.grid, "H": w.H, "N": w.N, "tau": w.tau, "theta": w.theta,
                      "lambda": w.lam, "rows": rows}))


if __name__ == "__main__":
    main()
