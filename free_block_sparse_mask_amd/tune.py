"""L1-bounded search of tau, theta and lambda on calibration inputs.

Pages: [Review] "SpargeAttn: Accurate and Training-free Sparse Attention
Accelerating Any Model Inference" (xllm-io paper-review blog), the
hyper-parameter determination paragraph and its per-model (l1, l2) list;
[Rebuttal] the reply on tuning cost (5-10 inference passes per layer, and the
fixed fallback tau = 0.5, theta = 0.95, lambda = -25).

The pages give one rule: with L1 = sum|O - O'| / sum|O| (O full attention,
O' sparse attention) and two bounds l1 < l2, an L1 under l1 means the
parameters may be made sparser, an L1 over l2 means they must be made
denser, and an L1 in [l1, l2] keeps them.  Read against TopCdf (eq. 8), a
larger tau keeps more blocks, so "sparser" means a smaller tau; a lambda
nearer 0 skips more P~V groups, so "sparser" means a larger lambda.

The search below applies that rule as a bisection, in the pages' order:
first tau with lambda off (lambda = -inf), for each theta of a small grid,
keeping the theta that gives the highest sparsity within l2; then lambda with
the chosen (tau, theta), under the same bounds on the final L1.  Every
evaluation runs the HIP path: the sparse output and the dense reference (M_g
all ones, lambda = -inf) come from sparge_attn, the L1 sums from
sparge_l1_sums, and sparsity is the fraction of the live tiles' QK^T and P~V
MFMA work that the two stages skipped (from the kernel counters).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, List, Optional, Sequence, Tuple

from . import BK, BQ, attn, counts_dict, l1_error, num_blocks, predict_mask

LAMBDA_OFF = -math.inf


@dataclasses.dataclass
class Eval:
    tau: float
    theta: float
    lam: float
    l1: float
    sparsity: float


@dataclasses.dataclass
class TuneResult:
    tau: float
    theta: float
    lam: float
    l1: float
    sparsity: float
    feasible: bool               # the final L1 is within l2
    trace: List[Eval]            # every evaluation, in order


def sparsity_from_counts(c: dict, d: int, bq: int = BQ, bk: int = BK, rows: int = 32) -> float:
    """1 - executed / live MFMA work: QK^T on executed tiles plus P~V on
    executed row groups, against both on every live tile."""
    live = c["live_tiles"] * 4.0 * bq * bk * d
    if live <= 0:
        return 0.0
    exe = c["qk_exec"] * 2.0 * bq * bk * d + c["pv_exec"] * 2.0 * rows * bk * d
    return 1.0 - exe / live


def two_level_search(evaluate: Callable[[float], Tuple[float, float]], dense_end: float,
                     sparse_end: float, l1: float, l2: float, iters: int = 8):
    """The two-level rule as a bisection on one parameter x.

    ``evaluate(x) -> (L1, sparsity)``; moving x from ``dense_end`` towards
    ``sparse_end`` is assumed to raise both.  Returns (x, L1, sparsity,
    feasible, [(x, L1, sparsity), ...]): the sparsest evaluated point with
    L1 <= l2 (stopping at the first one with l1 <= L1 <= l2), or the dense
    end, flagged infeasible, when even that exceeds l2."""
    if not (0.0 <= l1 <= l2):
        raise ValueError("need 0 <= l1 <= l2")
    trace = []

    def ev(x):
        e, s = evaluate(x)
        trace.append((x, e, s))
        return e, s

    e, s = ev(dense_end)
    if e > l2:
        return dense_end, e, s, False, trace
    best = (dense_end, e, s)
    if e >= l1:
        return dense_end, e, s, True, trace
    e, s = ev(sparse_end)
    if e <= l2:
        return sparse_end, e, s, True, trace
    safe, risky = dense_end, sparse_end      # L1(safe) < l1, L1(risky) > l2
    for _ in range(iters):
        mid = 0.5 * (safe + risky)
        e, s = ev(mid)
        if e < l1:
            safe = mid
            if s >= best[2]:
                best = (mid, e, s)
        elif e > l2:
            risky = mid
        else:
            return mid, e, s, True, trace
    return best[0], best[1], best[2], True, trace


class _Problem:
    """One calibration problem on the device: q, k, v and its dense reference."""

    def __init__(self, q, k, v, causal: bool):
        import torch
        self.q, self.k, self.v, self.causal = q, k, v, causal
        B, H, N, _ = q.shape
        ones = torch.ones((B, H, num_blocks(N, BQ), num_blocks(N, BK)), dtype=torch.uint8, device=q.device)
        self.o_ref, _, _ = attn(q, k, v, ones, LAMBDA_OFF, causal, out_f32=True)
        self.d = q.shape[3]
        self.trace: List[Eval] = []
        self._masks = {}

    def evaluate(self, tau: float, theta: float, lam: float) -> Tuple[float, float]:
        key = (tau, theta)
        mask = self._masks.get(key)
        if mask is None:
            mask = predict_mask(self.q, self.k, tau, theta, self.causal)
            self._masks = {key: mask}          # keep one: the searches revisit the last
        o, counts, _ = attn(self.q, self.k, self.v, mask, lam, self.causal, out_f32=True)
        e = l1_error(o, self.o_ref)
        s = sparsity_from_counts(counts_dict(counts), self.d)
        self.trace.append(Eval(tau, theta, lam, e, s))
        return e, s


def tune(q, k, v, causal: bool, l1: float, l2: float,
         thetas: Sequence[float] = (0.3, 0.5, 0.7, 0.9), tau_range: Tuple[float, float] = (0.05, 1.0),
         lam_range: Tuple[float, float] = (-40.0, -0.5), iters: int = 8) -> TuneResult:
    """Search (tau, theta, lambda) for one layer's calibration Q, K, V (device
    tensors [B, H, N, d], H a multiple of K's heads) so that the relative L1
    of the sparse output against full attention stays within [l1, l2] where
    it can, with the highest sparsity the bisection finds."""
    P = _Problem(q, k, v, causal)
    tau_lo, tau_hi = tau_range
    best = None
    for theta in thetas:
        tau, e, s, ok, _ = two_level_search(lambda t: P.evaluate(t, theta, LAMBDA_OFF), tau_hi, tau_lo,
                                            l1, l2, iters)
        cand = (ok, s if ok else -e, tau, theta, e)
        if best is None or cand[:2] > best[:2]:
            best = cand
    ok, _, tau, theta, e_tau = best
    if not ok:
        s = P.evaluate(tau, theta, LAMBDA_OFF)[1]
        return TuneResult(tau, theta, LAMBDA_OFF, e_tau, s, False, P.trace)
    lam_lo, lam_hi = lam_range
    lam, e, s, ok, _ = two_level_search(lambda x: P.evaluate(tau, theta, x), lam_lo, lam_hi, l1, l2, iters)
    if not ok:
        # even the most negative lambda of the range adds too much error: keep P~V whole
        e, s = P.evaluate(tau, theta, LAMBDA_OFF)
        lam, ok = LAMBDA_OFF, e <= l2
    return TuneResult(tau, theta, lam, e, s, ok, P.trace)


def tune_per_head(q, k, v, causal: bool, l1: float, l2: float, **kw) -> List[TuneResult]:
    """:func:`tune` on each query head alone (with its kv head).  The kernels
    take one (tau, theta, lambda) per call, so per-head parameters are used
    with one call per head."""
    H, Hkv = q.shape[1], k.shape[1]
    g = H // Hkv
    out = []
    for h in range(H):
        hk = h // g
        out.append(tune(q[:, h:h + 1], k[:, hk:hk + 1], v[:, hk:hk + 1], causal, l1, l2, **kw))
    return out
