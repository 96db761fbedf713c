"""GPU checks of the hyper-parameter search and its L1 measure.

* sparge_l1_sums against float64 numpy sums of the same elements (dtypes,
  strided head slices, a ragged N, an empty tensor), and the same bits on a
  second call.
* The tau/theta/lambda search run on the HIP path for a small workload,
  checked with the oracle: at the parameters it returns, the oracle's own
  mask matches the GPU's, the oracle's relative L1 of sparse against full
  attention matches the L1 the search measured, and it lies within l2.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from free_block_sparse_mask_amd import tune as T
from oracle import sparge_oracle as O

from gpu_common import DEV, check_mask, log, to_dev

pytestmark = pytest.mark.gpu

L1_TOL = 3e-3     # |L1 measured on the GPU - L1 of the oracle| (16-bit P~ and operands)


@pytest.mark.parametrize("dt_o,dt_r", [(torch.float32, torch.float32), (torch.bfloat16, torch.float32),
                                       (torch.float16, torch.float16)])
def test_l1_sums_match_numpy(dt_o, dt_r):
    g = torch.Generator().manual_seed(5)
    a = torch.randn(2, 3, 1000, 64, generator=g)
    b = a + 0.05 * torch.randn(2, 3, 1000, 64, generator=g)
    # strided views: every other head of a wider tensor
    wa = torch.zeros(2, 6, 1000, 64, dtype=dt_o)
    wa[:, ::2] = a.to(dt_o)
    o = wa.to(DEV)[:, ::2]
    ref = b.to(dt_r).to(DEV)
    s1 = fb.l1_sums(o, ref)
    s2 = fb.l1_sums(o, ref)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)                     # same bits on every call
    an = a.to(dt_o).double().numpy()
    bn = b.to(dt_r).double().numpy()
    want = np.array([np.abs(an - bn).sum(), np.abs(bn).sum()])
    got = s1.cpu().numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=0), (got, want)
    log(f"l1 sums {dt_o}/{dt_r}: {got} vs {want}")
    z = torch.empty(1, 2, 0, 64, dtype=dt_o, device=DEV)
    assert fb.l1_sums(z, z.to(dt_r)).cpu().tolist() == [0.0, 0.0]


def _oracle_l1(w, q, k, v, tau, theta, lam, mg_gpu):
    Q, K, V = O.widen(q, w.dtype), O.widen(k, w.dtype), O.widen(v, w.dtype)
    dense = O.dense_attention(Q, K, V, w.causal)
    sparse, _, _ = O.sparse_attention(Q, K, V, mg_gpu, lam, w.causal)
    return O.rel_l1(dense, sparse), (Q, K)


@pytest.mark.parametrize("wid", [0, 2], ids=["tiny", "llm_small"])
def test_search_result_is_pinned_by_the_oracle(wid):
    w = I.workload(0) if wid == 0 else I.workload(2, N=2048, H=2, H_kv=2)
    q, k, v = I.make_qkv(w)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    l1, l2 = 0.02, 0.03
    res = T.tune(qd, kd, vd, w.causal, l1, l2, thetas=(0.3, 0.6, 0.9), iters=6)
    log(f"[tune] {w.name}: tau={res.tau:.4f} theta={res.theta} lam={res.lam:.3f} L1={res.l1:.4f} "
        f"sparsity={res.sparsity:.3f} feasible={res.feasible} evals={len(res.trace)}")
    assert res.feasible and res.l1 <= l2
    # the rule's bookkeeping: the reported point is one of the evaluations
    assert any(e.tau == res.tau and e.theta == res.theta and e.lam == res.lam and e.l1 == res.l1
               for e in res.trace)
    # oracle: the GPU's mask at the returned (tau, theta), then L1 given that mask
    mask = fb.predict_mask(qd, kd, res.tau, res.theta, w.causal)
    torch.cuda.synchronize()
    e_or, (Q, K) = _oracle_l1(w, q, k, v, res.tau, res.theta, res.lam, mask.mg.cpu().numpy().astype(bool))
    rep = check_mask(mask, Q, K, res.tau, res.theta, w.causal)
    log(f"   oracle L1 {e_or:.5f} vs measured {res.l1:.5f}; mask ambiguous={rep['ambiguous']}")
    assert abs(e_or - res.l1) <= L1_TOL
    assert e_or <= l2 + L1_TOL
    # every mask the search measured, the tau = 1 dense ends included, is the oracle's
    pairs = sorted({(e.tau, e.theta) for e in res.trace})
    assert any(t == 1.0 for t, _ in pairs)
    for tau, theta in pairs:
        m = fb.predict_mask(qd, kd, tau, theta, w.causal)
        torch.cuda.synchronize()
        r = check_mask(m, Q, K, tau, theta, w.causal)
        log(f"   trace mask tau={tau:.4f} theta={theta}: ambiguous={r['ambiguous']} near_theta={r['near_theta']}")
