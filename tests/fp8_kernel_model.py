"""A model of the fp8 P~V kernel's own rounding schedule.  NOT the oracle and
not a parity reference: the GPU's fp8 variant is scored against the oracle's
``sparse_attention(..., pv8=True)``, which follows Algorithm 1's order.

The kernel differs from that order in one place: its second pass forms
P~ = exp(S - m_final) at the row's final running max (the two-pass order of
the attention kernel) and rounds that to E4M3, where Algorithm 1 rounds
exp(S - m_ij) at the running max of each step and rescales afterwards.  It
also floors the per-channel V scale at 2^-100 (its scales are float32 and
it multiplies by their reciprocals).

This model restates that schedule in float64 so that a test can check the
kernel tightly against what it is built to compute; it catches arithmetic
slips (a wrong key order in the fp8 V^T copy, a wrong scale) that the
looser bound against the oracle would let through.  Its extra room for
float32 scores near an E4M3 rounding boundary, and for the matrix cores'
truncated 64-product sums, comes from probes of the kernel, which is why it
lives with the tests and not in oracle/.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from oracle import sparge_oracle as O

P_SCALE = 256.0
V_SCALE_FLOOR_LOG2 = -100


def kernel_channel_scales(Vh: np.ndarray) -> np.ndarray:
    """The oracle's per-channel power-of-two scales, floored at 2^-100 as the
    kernel's float32 scales are."""
    d = O.v_channel_scales(Vh)
    nz = np.abs(Vh).max(axis=0) > 0
    return np.where(nz, np.maximum(d, 2.0 ** V_SCALE_FLOOR_LOG2), 1.0)


def attend_row_block_final_max(Qh, Kh, Vh, mg_row, i, causal, decisions, score_fn=None,
                               amb_window: Optional[float] = None, sum_rel: float = 0.0):
    """O_i under the kernel's schedule for one query block, given the (tile,
    group) decisions ([Tn, c_w], 1 = P~V runs).  With ``amb_window`` w, also
    returns per element the most it can move when a P~ within relative
    distance w of an E4M3 rounding boundary rounds the other way, plus
    ``sum_rel`` times the sum of the absolute products of every tile."""
    N, d = Qh.shape
    bq, bk, R = O.BQ, O.BK, O.ROWS_PER_GROUP
    Tn = O.num_blocks(N, bk)
    rows = O.block_rows(N, bq, i)
    n = len(rows)
    q_idx = np.arange(rows.start, rows.stop)
    Qi = Qh[rows.start:rows.stop]
    live = O.tile_live(N, bq, bk, causal)[i]
    todo = [j for j in range(Tn) if mg_row[j] and live[j]]
    S_of = {}
    m = np.full(n, -np.inf)
    for j in todo:
        keys = O.block_rows(N, bk, j)
        k_idx = np.arange(keys.start, keys.stop)
        S = Qi @ Kh[keys.start:keys.stop].T / math.sqrt(d) if score_fn is None else score_fn(rows, keys)
        if causal:
            S = np.where(k_idx[None, :] > q_idx[:, None], -np.inf, S)
        S_of[j] = S
        m = np.maximum(m, S.max(axis=1))
    m_sub = np.where(np.isfinite(m), m, 0.0)
    l = np.zeros(n)
    delta = kernel_channel_scales(Vh)
    Vq = O.e4m3_round(Vh / delta[None, :])
    acc = np.zeros((n, Vh.shape[1]))
    amb = np.zeros_like(acc)
    for j in todo:
        keys = O.block_rows(N, bk, j)
        with np.errstate(invalid="ignore"):
            P = np.exp(S_of[j] - m_sub[:, None])
        l += P.sum(axis=1)
        Pq = O.e4m3_round(P_SCALE * P)
        if amb_window is not None:
            step = np.abs(O.e4m3_round(P_SCALE * P * (1 + amb_window)) -
                          O.e4m3_round(P_SCALE * P * (1 - amb_window)))
        for g in range(decisions.shape[1]):
            if decisions[j, g] != 1:
                continue
            gi = np.arange(g * R, min(n, g * R + R))
            acc[gi] += Pq[gi] @ Vq[keys.start:keys.stop]
            if amb_window is not None:
                amb[gi] += (step[gi] + sum_rel * np.abs(Pq[gi])) @ np.abs(Vq[keys.start:keys.stop])
    out = np.zeros_like(acc)
    nz = l > 0
    out[nz] = acc[nz] * delta[None, :] / P_SCALE / l[nz, None]
    if amb_window is None:
        return out
    amb_out = np.zeros_like(amb)
    amb_out[nz] = amb[nz] * delta[None, :] / P_SCALE / l[nz, None]
    return out, amb_out


def sparse_attention_final_max(Q, K, V, mg, causal, decisions, blocks=None, quant=None,
                               amb_window: Optional[float] = None, sum_rel: float = 0.0):
    """The model over Q [B, H, N, d], K/V [B, H_kv, N, d], with the lambda
    decisions [B, H, Tm, Tn, c_w] given (the GPU's).  ``blocks`` restricts the
    work to (b, h, i); other rows stay 0.  With ``amb_window``, returns (O, room)."""
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    Tm = O.num_blocks(N, O.BQ)
    out = np.zeros((B, H, N, V.shape[3]))
    room = np.zeros_like(out)
    todo = blocks if blocks is not None else [(b, h, i) for b in range(B) for h in range(H) for i in range(Tm)]
    for b, h, i in todo:
        hk = O.kv_head(h, H, H_kv)
        score_fn = None
        if quant is not None:
            qc, kc = quant["q_codes"][b, h], quant["k_codes"][b, hk]
            dq, dk = quant["q_scale"][b, h], quant["k_scale"][b, hk]

            def score_fn(rows, keys, qc=qc, kc=kc, dq=dq, dk=dk, i=i):
                j = keys.start // O.BK
                return (qc[rows.start:rows.stop] @ kc[keys.start:keys.stop].T) * (dq[i] * dk[j]) / math.sqrt(d)
        r = O.block_rows(N, O.BQ, i)
        res = attend_row_block_final_max(Q[b, h], K[b, hk], V[b, hk], mg[b, h, i], i, causal, decisions[b, h, i],
                                         score_fn=score_fn, amb_window=amb_window, sum_rel=sum_rel)
        if amb_window is None:
            out[b, h, r.start:r.stop] = res
        else:
            out[b, h, r.start:r.stop], room[b, h, r.start:r.stop] = res
    return out if amb_window is None else (out, room)
