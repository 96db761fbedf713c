"""Shared helpers of the GPU parity tests: moving the seeded inputs to the
device, running the oracle beside the HIP path, and the acceptance rules.

Acceptance (per component):
* M_g: bit-exact, except entries the oracle marks ambiguous (exclusive prefix
  within 1e-4 of tau*sum, or a near-tie at the cut); blocks whose similarity
  lies within 1e-4 of theta are replayed with the GPU's fix bit.  Both sides
  decide in float64, so the counts of such entries are reported and expected
  to be zero in practice.
* Attention given the same mask (fp16/bf16): max-abs <= 1e-2 and relative L1
  <= 5e-3 against the oracle replaying the GPU's lambda decisions; every
  decision that differs from the oracle's own rule must lie within 1e-3 nats
  of lambda.
* int8 attention: relative L1 <= 3e-2 and cosine >= 0.999 against the oracle
  on the same codes and mask.
"""
from __future__ import annotations

import contextlib
import math
import sys
from typing import Optional

import numpy as np
import torch

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from oracle import sparge_oracle as O

DEV = "cuda:0"
ATTN_MAX_ABS = 1e-2
ATTN_REL_L1 = 5e-3
INT8_REL_L1 = 3e-2
INT8_COS = 0.999
LAMBDA_WINDOW = 1e-3
THETA_WINDOW = 1e-4


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype: str):
    return {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).to(DEV)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def widen_dev(t: torch.Tensor, dtype: str) -> np.ndarray:
    return O.widen(to_bits(t), dtype)


def rel_l1(ref: np.ndarray, x: np.ndarray) -> float:
    return O.rel_l1(ref, x)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.ravel()
    b = b.ravel()
    den = float(np.linalg.norm(a) * np.linalg.norm(b))
    return float(a @ b) / den if den > 0 else 1.0


def check_mask(gpu_mask: fb.Mask, Q: np.ndarray, K: np.ndarray, tau: float, theta: float, causal: bool,
               heads=None) -> dict:
    """Compares the GPU's M_g (and lists, s_q, s_k) with the oracle's on the
    (b, h) pairs in ``heads`` (all if None).  Returns the report dict."""
    B, H, N, d = Q.shape
    Hkv = K.shape[1]
    s_q = gpu_mask.s_q.cpu().numpy()
    s_k = gpu_mask.s_k.cpu().numpy()
    mg = gpu_mask.mg.cpu().numpy().astype(bool)
    cnt = gpu_mask.row_cnt.cpu().numpy()
    idx = gpu_mask.row_idx.cpu().numpy().view(np.uint16)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    ref = O.predict_mask(Q, K, tau, theta, causal, heads=todo)
    rep = {"near_theta": 0, "ambiguous": 0, "mismatch": 0, "checked_rows": 0, "max_s_err": 0.0}
    kv_todo = sorted({(b, O.kv_head(h, H, Hkv)) for b, h in todo})
    for b, h in todo:
        rep["max_s_err"] = max(rep["max_s_err"], float(np.max(np.abs(s_q[b, h] - ref["s_q"][b, h]))))
    for b, hk in kv_todo:
        rep["max_s_err"] = max(rep["max_s_err"], float(np.max(np.abs(s_k[b, hk] - ref["s_k"][b, hk]))))
    assert rep["max_s_err"] <= 1e-5, rep
    # replay the GPU's fix/selective bit for blocks next to theta
    gfix_q = s_q < theta
    gfix_k = s_k < theta
    near_q = np.abs(ref["s_q"] - theta) <= THETA_WINDOW
    near_k = np.abs(ref["s_k"] - theta) <= THETA_WINDOW
    for b, h in todo:
        assert np.array_equal(gfix_q[b, h] & ~near_q[b, h], (ref["s_q"][b, h] < theta) & ~near_q[b, h])
    for b, hk in kv_todo:
        assert np.array_equal(gfix_k[b, hk] & ~near_k[b, hk], (ref["s_k"][b, hk] < theta) & ~near_k[b, hk])
    rep["near_theta"] = int(sum(near_q[b, h].sum() for b, h in todo) + sum(near_k[b, hk].sum() for b, hk in kv_todo))
    if rep["near_theta"]:
        ref = O.predict_mask(Q, K, tau, theta, causal, heads=todo, fix_q=gfix_q, fix_k=gfix_k)
    for b, h in todo:
        amb = ref["ambiguous"][b, h]
        diff = (mg[b, h] != ref["mg"][b, h])
        rep["ambiguous"] += int(amb.sum())
        rep["mismatch"] += int((diff & ~amb).sum())
        rep["checked_rows"] += mg.shape[2]
        # the lists hold the ascending ones of the GPU's own M_g row
        for i in range(mg.shape[2]):
            ones = np.nonzero(mg[b, h, i])[0]
            assert cnt[b, h, i] == ones.size
            assert np.array_equal(idx[b, h, i, :ones.size].astype(np.int64), ones)
    assert rep["mismatch"] == 0, rep
    rep["ref_mg"] = ref["mg"]
    return rep


def run_attn(q, k, v, mask, lam: float, causal: bool, **kw):
    """sparge_attn twice: storing O in V's type (the product configuration) and
    in float32.  The 16-bit output must be exactly the float32 output rounded
    to nearest even, so the float32 one carries the arithmetic error alone.
    Returns (o_native, o_f32, counts, pv_dbg)."""
    o, counts, dbg = fb.attn(q, k, v, mask, lam, causal, dbg=True, **kw)
    o32, counts32, dbg32 = fb.attn(q, k, v, mask, lam, causal, dbg=True, out_f32=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o32.to(o.dtype)), "16-bit output is not the rounded float32 output"
    assert torch.equal(counts, counts32) and torch.equal(dbg, dbg32)
    return o, o32, counts, dbg


def check_attention(o_gpu: torch.Tensor, counts: torch.Tensor, dbg: torch.Tensor, Q, K, V,
                    mg: np.ndarray, lam: float, causal: bool, out_dtype: str, blocks=None,
                    quant=None, int8: bool = False, o16: Optional[torch.Tensor] = None,
                    o16_dtype: Optional[str] = None) -> dict:
    """Compares the GPU output (and counters, decisions) with the oracle given
    the same mask, replaying the GPU's lambda decisions.  ``o_gpu`` is the
    float32 output (``out_dtype`` "f32") or a 16-bit one.  ``o16`` (of type
    ``o16_dtype``), the product's 16-bit output, is scored too: its relative
    L1 must meet the same bound (its max-abs is logged, not bounded: bf16
    storage alone moves a value near 4 by up to 2^-7)."""
    B, H, N, d = Q.shape
    Tm, Tn = O.num_blocks(N, O.BQ), O.num_blocks(N, O.BK)
    cw = O.BQ // O.ROWS_PER_GROUP
    gdec = dbg.cpu().numpy().astype(np.int8)
    margins = np.full((B, H, Tm, Tn, cw), np.nan)
    o_ref, cnt_ref, dec_ref = O.sparse_attention(Q, K, V, mg, lam, causal, blocks=blocks,
                                                 skip_override=gdec, quant=quant, margins=margins)
    todo = blocks if blocks is not None else [(b, h, i) for b in range(B) for h in range(H) for i in range(Tm)]
    o_g = o_gpu.detach().cpu().double().numpy() if out_dtype == "f32" else O.widen(to_bits(o_gpu), out_dtype)
    rep = {"blocks": len(todo), "lambda_flips": 0, "max_flip_margin": 0.0}
    # decisions: GPU vs the oracle's own rule (replayed flips must be near lambda)
    sel_g, sel_o = [], []
    for b, h, i in todo:
        g = gdec[b, h, i]
        rule = np.where(np.isnan(margins[b, h, i]), 0, np.where(margins[b, h, i] < 0, 2, 1))
        visited = g != 0
        assert np.array_equal(visited, dec_ref[b, h, i] != 0)
        void_g = g == 3
        assert np.array_equal(void_g, dec_ref[b, h, i] == 3)
        flip = visited & ~void_g & (g != rule)
        rep["lambda_flips"] += int(flip.sum())
        if flip.any():
            rep["max_flip_margin"] = max(rep["max_flip_margin"], float(np.max(np.abs(margins[b, h, i][flip]))))
        r = O.block_rows(N, O.BQ, i)
        sel_g.append(o_g[b, h, r.start:r.stop])
        sel_o.append(o_ref[b, h, r.start:r.stop])
    assert rep["max_flip_margin"] <= LAMBDA_WINDOW, rep
    og = np.concatenate(sel_g)
    orf = np.concatenate(sel_o)
    rep["max_abs"] = float(np.max(np.abs(og - orf))) if og.size else 0.0
    rep["rel_l1"] = rel_l1(orf, og)
    rep["cos"] = cosine(orf, og)
    if int8:
        assert rep["rel_l1"] <= INT8_REL_L1 and rep["cos"] >= INT8_COS, rep
    else:
        assert rep["max_abs"] <= ATTN_MAX_ABS and rep["rel_l1"] <= ATTN_REL_L1, rep
    if o16 is not None:
        o_n = O.widen(to_bits(o16), o16_dtype)
        g16 = np.concatenate([o_n[b, h, O.block_rows(N, O.BQ, i).start:O.block_rows(N, O.BQ, i).stop]
                              for b, h, i in todo])
        rep["max_abs_16"] = float(np.max(np.abs(g16 - orf))) if g16.size else 0.0
        rep["rel_l1_16"] = rel_l1(orf, g16)
        assert rep["rel_l1_16"] <= (INT8_REL_L1 if int8 else ATTN_REL_L1), rep
        log(f"   {o16_dtype} output: rel_l1={rep['rel_l1_16']:.2e} max_abs={rep['max_abs_16']:.2e}")
    if blocks is None:
        c = fb.counts_dict(counts)
        for k in O.COUNT_NAMES:
            assert c[k] == cnt_ref[k], (k, c, cnt_ref)
        rep["counts"] = c
    return rep


# ---------------------------------------------------------------------------
# fp8 P~V acceptance against the oracle (Algorithm 1's order)
# ---------------------------------------------------------------------------
# The oracle rounds P~ = exp(S - m_ij) to E4M3 at each step's running max and
# rescales exactly; the kernel rounds exp(S - m_final) once, in its second
# pass.  V's 8-bit values are the same on both sides.  One E4M3 rounding of
# x = 2^8 p moves it by at most 2^-4 x in the normal range and by at most
# 2^-10 (half the subnormal step) below it, and never by more than x itself,
# so either side's weight lies within min(p, max(2^-4 p, 2^-18)) of the
# exact p = exp(S - m_final) (the later rescalings of the oracle's order
# only shrink both terms).  The kernel adds float32 scores, exponentials and
# sums: 2^-7 p covers them (sums of up to 2^13 products lose at most
# 2^13 * 2^-23 of their absolute size), and 2^-10 |O| covers its float32 l.
# Hence, per output element, the room
#   sum over voted keys of (2 min(p, max(2^-4 p, 2^-18)) + 2^-7 p) |V8 delta|
#   / l + 2^-10 |O|.
# Beside it, two whole-output statistics: relative L1 <= 2^-4 (the largest
# relative move of one rounding) and cosine >= 0.998 (= 1 - (2^-4)^2 / 2).
FP8_REL_L1 = 2.0 ** -4
FP8_COS = 0.998


def fp8_room(Q, K, V, mg, causal, decisions, blocks, quant=None, ref=None):
    """The element-wise room above for the (b, h, i) blocks in ``blocks``
    (other rows 0), given the GPU's lambda decisions [B, H, Tm, Tn, c_w]."""
    B, H, N, d = Q.shape
    Hkv = K.shape[1]
    R = O.ROWS_PER_GROUP
    room = np.zeros((B, H, N, V.shape[3]))
    v8 = {}
    for b, h, i in blocks:
        hk = O.kv_head(h, H, Hkv)
        if (b, hk) not in v8:
            delta = O.v_channel_scales(V[b, hk])
            v8[b, hk] = np.abs(O.e4m3_round(V[b, hk] / delta[None, :]) * delta[None, :])
        av = v8[b, hk]
        rows = O.block_rows(N, O.BQ, i)
        q_idx = np.arange(rows.start, rows.stop)
        live = O.tile_live(N, O.BQ, O.BK, causal)[i]
        todo = [j for j in range(O.num_blocks(N, O.BK)) if mg[b, h, i, j] and live[j]]
        S_of = {}
        m = np.full(len(rows), -np.inf)
        for j in todo:
            keys = O.block_rows(N, O.BK, j)
            if quant is None:
                S = Q[b, h, rows.start:rows.stop] @ K[b, hk, keys.start:keys.stop].T / math.sqrt(d)
            else:
                S = (quant["q_codes"][b, h, rows.start:rows.stop] @ quant["k_codes"][b, hk, keys.start:keys.stop].T
                     * (quant["q_scale"][b, h, i] * quant["k_scale"][b, hk, j]) / math.sqrt(d))
            if causal:
                S = np.where(np.arange(keys.start, keys.stop)[None, :] > q_idx[:, None], -np.inf, S)
            S_of[j] = S
            m = np.maximum(m, S.max(axis=1))
        msub = np.where(np.isfinite(m), m, 0.0)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), V.shape[3]))
        for j in todo:
            keys = O.block_rows(N, O.BK, j)
            with np.errstate(invalid="ignore"):
                P = np.exp(S_of[j] - msub[:, None])
            l += P.sum(axis=1)
            e = 2.0 * np.minimum(P, np.maximum(2.0 ** -4 * P, 2.0 ** -18)) + 2.0 ** -7 * P
            for g in range(decisions.shape[-1]):
                if decisions[b, h, i, j, g] == 1:
                    gi = np.arange(g * R, min(len(rows), g * R + R))
                    acc[gi] += e[gi] @ av[keys.start:keys.stop]
        nz = l > 0
        room[b, h, rows.start:rows.stop][nz] = acc[nz] / l[nz, None]
    if ref is not None:
        room += 2.0 ** -10 * np.abs(ref)
    return room


def check_fp8(og: np.ndarray, ref: np.ndarray, room: np.ndarray, rows=None) -> dict:
    """The fp8 acceptance on the selected rows (an index array over N, all if
    None): every element within the room, relative L1 and cosine bounds."""
    if rows is not None:
        og, ref, room = og[..., rows, :], ref[..., rows, :], room[..., rows, :]
    over = np.abs(og - ref) - room
    rep = {"rel_l1": rel_l1(ref, og), "cos": cosine(ref, og), "max_abs": float(np.max(np.abs(og - ref))),
           "max_over_room": float(over.max()), "room_max": float(room.max())}
    assert rep["max_over_room"] <= 0.0, rep
    assert rep["rel_l1"] <= FP8_REL_L1 and rep["cos"] >= FP8_COS, rep
    return rep


@contextlib.contextmanager
def attn_path(path: int):
    """Runs the body with the stage-2 path forced process-wide, then restores it."""
    old = fb.attn_path(path)
    try:
        yield
    finally:
        fb.attn_path(old)
