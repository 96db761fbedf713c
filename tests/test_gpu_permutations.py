"""GPU check of the token-order comparison (the analogue of [Review] Table 4).

On a small video grid, for every order (random, row-major, time-major,
Hilbert) the report's Sim-q and Sim-k must equal the oracle's mean block
self-similarity of the permuted Q and K, and its L1 must equal the oracle's
relative L1 of sparse against full attention given the GPU's mask.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from free_block_sparse_mask_amd import permutation_report as R
from oracle import sparge_oracle as O

from gpu_common import DEV, log, to_dev

pytestmark = pytest.mark.gpu


def test_permutation_report_matches_oracle():
    grid = (4, 16, 16)
    w = I.workload(3, grid=grid, N=4 * 16 * 16, H=2, H_kv=2)
    q, k, v = I.make_qkv(w)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    rows = R.measure(qd, kd, vd, grid, w.tau, w.theta, w.lam)
    log("\n" + R.markdown(rows))
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    for r in rows:
        perm = R.order_perm(r["order"], grid)
        ref_perm = {"rowmajor": O.raster_order(*grid), "timemajor": O.time_major_order(*grid),
                    "hilbert": O.hilbert_permutation(*grid)[0], "random": perm}[r["order"]]
        assert np.array_equal(perm, ref_perm)
        Qp, Kp, Vp = (O.permute_tokens(x, perm) for x in (Q, K, V))
        sim_q = np.mean([O.block_self_similarity(Qp[0, h], O.BQ) for h in range(w.H)])
        sim_k = np.mean([O.block_self_similarity(Kp[0, h], O.BK) for h in range(w.H_kv)])
        assert abs(sim_q - r["sim_q"]) <= 1e-5 and abs(sim_k - r["sim_k"]) <= 1e-5, (r, sim_q, sim_k)
        # L1 given the GPU's mask for this order (the same call the report made)
        pd = torch.from_numpy(perm).to(DEV)
        mask = fb.predict_mask(*(fb.hilbert_permute(x, pd) for x in (qd, kd)), w.tau, w.theta, False)
        mg = mask.mg.cpu().numpy().astype(bool)
        dense = O.dense_attention(Qp, Kp, Vp, False)
        sparse, _, _ = O.sparse_attention(Qp, Kp, Vp, mg, w.lam, False)
        e = O.rel_l1(dense, sparse)
        log(f"   {r['order']}: oracle Sim-q {sim_q:.4f} Sim-k {sim_k:.4f} L1 {e:.5f} (GPU {r['l1']:.5f})")
        assert abs(e - r["l1"]) <= 3e-3
