"""Float64 CPU oracle for the SpargeAttn hot path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or run this module.  The product path (the HIP
library and its Python binding) never calls it, and this module imports
nothing from the product package: the two share no code.

It is a plain, slow restatement of the method, step by step, in float64:

Pages cited (by title and section):

* [Review]   "SpargeAttn: Accurate and Training-free Sparse Attention
             Accelerating Any Model Inference", xllm-io paper-review blog:
             section "Core formulas" (eqs. 1-9), the sparse warp online softmax
             rule, "Algorithm 1", the components table and "HilbertCurve
             Permutation".
* [Rebuttal] "SpargeAttention: Accurate and Training-free Sparse Attention
             Accelerating Any Model Inference", OpenReview author rebuttal:
             replies "Weaknesses1", "Weaknesses3.1" and "Weaknesses3.2".

Readings taken where the pages are open:

* CosSim (eq. 6) is the mean of the b x b cosine-similarity matrix of the
  block's tokens, diagonal included; a zero row has cosine 0 with everything
  ([Review] eq. 6 with [Rebuttal] Weaknesses3.1, which calls the printed
  matrix a typo and asks for one mean cosine similarity per block).
* The compressed map uses the same 1/sqrt(d) scale as S in eq. 1.
* TopCdf (eq. 8) orders entries by probability, descending, ties to the lower
  column, and keeps the shortest prefix whose inclusive cumulative sum reaches
  tau * sum(P): entry r is kept iff the exclusive prefix c_{r-1} < tau * sum.
  The sum is the last value of the same sequential cumulative sum.
* Causal prediction: key blocks that lie wholly in the future of a query block
  are -inf in the compressed map and 0 in M_g; eq. 9 only forces live tiles.
* The lambda vote is taken per group of R consecutive query rows (one GPU
  wavefront) in natural-log units of S; rows whose local max is -inf take no
  part, and a group with no such row skips.  l still takes rowsum(P~) when PV
  is skipped (Algorithm 1 computes m and P~ before testing M_pv).
* A query row with l = 0 at the end (no visible key executed) outputs 0.
* int8 (Algorithm 1 step 2, SageAttention-style): symmetric per-block scale
  delta = max|x| / 127 (1 for an all-zero block), code = clamp(rint(x/delta),
  -127, 127) with ties to even; K first has its per-(b, kv-head) mean over all
  tokens subtracted; S = (codes_q . codes_k) * delta_q * delta_k / sqrt(d).
  The garbled "delta Bias" term is dropped: it is constant along a row, and
  softmax and the lambda vote are invariant to a per-row constant.
* GQA: query head h reads kv head h // (H / H_kv).
* 3D Hilbert order: Skilling's transpose algorithm ("Programming the Hilbert
  curve", AIP Conf. Proc. 707, 2004) on the enclosing 2^b cube with axes
  (t, h, w), then tokens are sorted by curve index.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
closed forms, special cases, brute force on tiny inputs, hand-built rows and
the rebuttal's worked sparsity example.  Parity unpinned: the sparsity values
the method reaches on the synthetic workloads (only GPU-vs-oracle agreement
covers them; the pages' sparsities come from real models).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

BQ = 128          # query block rows (b_q)
BK = 64           # key/value block rows (b_k)
ROWS_PER_GROUP = 32   # rows that vote together in the lambda rule (b_q / c_w)

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# storage widening
# ---------------------------------------------------------------------------

def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of bfloat16 / float16 bit patterns (uint16) to float64."""
    bits = np.asarray(bits)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "f64":
        return np.asarray(bits, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# blocks and causal liveness
# ---------------------------------------------------------------------------

def num_blocks(N: int, b: int) -> int:
    return (N + b - 1) // b


def block_rows(N: int, b: int, i: int) -> range:
    """Rows of block i: [b*i, min(N, b*i + b)) ([Review] Algorithm 1 step 1)."""
    return range(b * i, min(N, b * i + b))


def tile_live(N: int, bq: int, bk: int, causal: bool) -> np.ndarray:
    """[Tm, Tn] bool: tile (i, j) holds at least one visible (query, key) pair.

    Non-causal: every tile.  Causal: the first key of block j is not after the
    last query of block i.
    """
    Tm, Tn = num_blocks(N, bq), num_blocks(N, bk)
    live = np.ones((Tm, Tn), dtype=bool)
    if causal:
        for i in range(Tm):
            last_q = min(N, bq * i + bq) - 1
            for j in range(Tn):
                live[i, j] = bk * j <= last_q
    return live


# ---------------------------------------------------------------------------
# Stage 1: selective token compression ([Review] eqs. 4-9, Algorithm 1 steps 3-5)
# ---------------------------------------------------------------------------

def mean_pool(X: np.ndarray, b: int) -> np.ndarray:
    """Eqs. 4-5: the mean token of every block of b rows.  X [N, d] -> [T, d]."""
    N = X.shape[0]
    return np.stack([X[block_rows(N, b, t)].mean(axis=0) for t in range(num_blocks(N, b))])


def cossim(Xb: np.ndarray) -> float:
    """Eq. 6 (as corrected in [Rebuttal] Weaknesses3.1): one block's mean cosine
    similarity, the mean of the b x b matrix of cos(x_a, x_c), diagonal included.
    """
    norms = np.sqrt((Xb * Xb).sum(axis=1))
    xhat = np.zeros_like(Xb)
    nz = norms > 0
    xhat[nz] = Xb[nz] / norms[nz, None]
    G = xhat @ xhat.T
    return float(G.mean())


def block_cossim(X: np.ndarray, b: int) -> np.ndarray:
    N = X.shape[0]
    return np.array([cossim(X[block_rows(N, b, t)]) for t in range(num_blocks(N, b))])


def topcdf(p: np.ndarray, tau: float) -> Tuple[np.ndarray, Dict[str, np.ndarray]]:
    """Eq. 8: TopCdf over one row of probabilities p [n] (all finite, >= 0).

    Entries are ordered by p descending with ties going to the lower index; the
    entry at sorted position r is kept iff the exclusive prefix sum
    c_{r-1} (c_{-1} = 0) is below tau * sum(p).  Returns (keep [n] bool, info)
    where info holds, per original index, the exclusive prefix and the order.
    """
    n = p.shape[0]
    order = np.lexsort((np.arange(n), -p))          # primary: -p ascending; secondary: index
    ps = p[order]
    c = np.cumsum(ps)                               # sequential, hence non-decreasing
    total = c[-1] if n else 0.0
    excl = np.concatenate([[0.0], c[:-1]]) if n else c
    keep_sorted = excl < tau * total
    keep = np.zeros(n, dtype=bool)
    keep[order] = keep_sorted
    excl_by_idx = np.empty(n)
    excl_by_idx[order] = excl
    return keep, {"excl": excl_by_idx, "order": order, "thresh": tau * total, "p": p}


def topcdf_ambiguous(p: np.ndarray, keep: np.ndarray, info: Dict[str, np.ndarray],
                     near_cdf: float = 1e-4, near_tie: float = 1e-6) -> np.ndarray:
    """Entries of one TopCdf row (eq. 8) whose selection another correct
    implementation may take the other way through rounding alone: the
    exclusive prefix lies within ``near_cdf`` of tau * sum, or the
    probability is tied (relatively within ``near_tie``) with the last kept
    entry while at least one other entry shares that tie (a tie that may
    straddle the cut).  Acceptance bookkeeping for comparisons, not part of
    the method.  ``keep`` and ``info`` are :func:`topcdf`'s results."""
    amb = np.abs(info["excl"] - info["thresh"]) <= near_cdf
    if keep.any():
        last_kept = info["order"][int(keep.sum()) - 1]
        tied = np.abs(p - p[last_kept]) <= near_tie * p[last_kept]
        if tied.sum() > 1:
            amb |= tied
    return amb


def predict_mask_head(Qh: np.ndarray, Kh: np.ndarray, tau: float, theta: float, causal: bool,
                      bq: int = BQ, bk: int = BK, fix_q: Optional[np.ndarray] = None,
                      fix_k: Optional[np.ndarray] = None, scale_in_map: bool = True,
                      near_cdf: float = 1e-4, near_tie: float = 1e-6) -> Dict[str, np.ndarray]:
    """Stage 1 for one (batch, query head): M_g [Tm, Tn] from Q [N, d] and K [N, d].

    Algorithm 1 steps 3-5 of [Review]: pool (eqs. 4-5), self-similarity
    (eq. 6), compressed map with -inf on fix key blocks (eq. 7), row softmax and
    TopCdf (eq. 8), then force fix rows and columns (eq. 9).  ``fix_q`` /
    ``fix_k`` override the (s < theta) classification, so a run can replay
    another implementation's decision for blocks whose similarity lies next to
    theta.  The returned ``ambiguous`` marks entries whose selection depends on
    rounding: exclusive prefix within ``near_cdf`` of tau*sum, or probability
    tied (relative ``near_tie``) with the last kept entry of its row.
    """
    N, d = Qh.shape
    Tm, Tn = num_blocks(N, bq), num_blocks(N, bk)
    qbar = mean_pool(Qh, bq)
    kbar = mean_pool(Kh, bk)
    s_q = block_cossim(Qh, bq)
    s_k = block_cossim(Kh, bk)
    fq = (s_q < theta) if fix_q is None else np.asarray(fix_q, dtype=bool)
    fk = (s_k < theta) if fix_k is None else np.asarray(fix_k, dtype=bool)
    live = tile_live(N, bq, bk, causal)

    shat = qbar @ kbar.T
    if scale_in_map:
        shat = shat / math.sqrt(d)
    shat[:, fk] = NEG_INF                           # eq. 7
    shat[~live] = NEG_INF                           # future key blocks (causal)

    mg = np.zeros((Tm, Tn), dtype=bool)
    ambiguous = np.zeros((Tm, Tn), dtype=bool)
    for i in range(Tm):
        cols = np.nonzero(np.isfinite(shat[i]))[0]
        if cols.size == 0:
            continue
        z = shat[i, cols]
        e = np.exp(z - z.max())
        p = e / e.sum()                              # P^[i] = softmax(S^[i])
        keep, info = topcdf(p, tau)
        mg[i, cols[keep]] = True
        ambiguous[i, cols[topcdf_ambiguous(p, keep, info, near_cdf, near_tie)]] = True
    mg[fq, :] = True                                 # eq. 9, rows
    mg[:, fk] = True                                 # eq. 9, columns
    mg &= live
    ambiguous &= live & ~fq[:, None] & ~fk[None, :]
    return {"mg": mg, "s_q": s_q, "s_k": s_k, "qbar": qbar, "kbar": kbar, "fix_q": fq,
            "fix_k": fk, "live": live, "ambiguous": ambiguous, "shat": shat}


def kv_head(h: int, H: int, H_kv: int) -> int:
    """GQA grouping: contiguous groups of H / H_kv query heads share a kv head."""
    return h // (H // H_kv)


def predict_mask(Q: np.ndarray, K: np.ndarray, tau: float, theta: float, causal: bool,
                 bq: int = BQ, bk: int = BK, fix_q=None, fix_k=None, heads=None, **kw):
    """Stage 1 for Q [B, H, N, d], K [B, H_kv, N, d].

    Returns M_g [B, H, Tm, Tn] (bool), s_q [B, H, Tm], s_k [B, H_kv, Tn],
    ambiguous [B, H, Tm, Tn].  ``heads`` restricts the work to a list of
    (b, h) pairs (other rows stay zero).  ``fix_q`` [B, H, Tm] / ``fix_k``
    [B, H_kv, Tn] override the fix classification.
    """
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    Tm, Tn = num_blocks(N, bq), num_blocks(N, bk)
    mg = np.zeros((B, H, Tm, Tn), dtype=bool)
    amb = np.zeros((B, H, Tm, Tn), dtype=bool)
    s_q = np.zeros((B, H, Tm))
    s_k = np.zeros((B, H_kv, Tn))
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        hk = kv_head(h, H, H_kv)
        r = predict_mask_head(Q[b, h], K[b, hk], tau, theta, causal, bq, bk,
                              None if fix_q is None else fix_q[b, h],
                              None if fix_k is None else fix_k[b, hk], **kw)
        mg[b, h] = r["mg"]
        amb[b, h] = r["ambiguous"]
        s_q[b, h] = r["s_q"]
        s_k[b, hk] = r["s_k"]
    return {"mg": mg, "s_q": s_q, "s_k": s_k, "ambiguous": amb}


# ---------------------------------------------------------------------------
# Stage 2: block-sparse FlashAttention with the lambda rule
# ([Review] eqs. 1-3, sparse warp online softmax, Algorithm 1 steps 6-17)
# ---------------------------------------------------------------------------

# Counters, in this order: live tiles; tiles whose QK^T ran (M_g = 1) and were
# skipped; row groups whose PV ran, were skipped by the lambda vote, or had no
# visible key in the tile at all (void: nothing to add); rows that saw no key;
# rows.
COUNT_NAMES = ("live_tiles", "qk_exec", "qk_skip", "pv_exec", "pv_skip", "pv_void",
               "empty_rows", "rows")


def _scores_float(Qi: np.ndarray, Kj: np.ndarray) -> np.ndarray:
    return Qi @ Kj.T / math.sqrt(Qi.shape[1])


def attend_row_block(Qh: np.ndarray, Kh: np.ndarray, Vh: np.ndarray, mg_row: np.ndarray, i: int,
                     lam: float, causal: bool, bq: int = BQ, bk: int = BK,
                     R: int = ROWS_PER_GROUP, skip_override: Optional[np.ndarray] = None,
                     score_fn=None, vote_info: Optional[list] = None,
                     margins: Optional[np.ndarray] = None,
                     pv8: Optional[Tuple[np.ndarray, np.ndarray]] = None):
    """O_i for one query block i of one head, visiting key blocks j with
    M_g[i, j] = 1 in ascending j (eq. 1 with eqs. 2-3 and the lambda rule).

    ``skip_override`` [Tn, c_w] (int8: 1 execute, 2 skip, anything else = use
    the rule) replays another implementation's PV decisions.
    ``score_fn(rows, keys)`` replaces Q_i K_j^T / sqrt(d) (used by the int8
    path).  ``pv8`` = (V8, delta) switches the P~V product to 8-bit floats
    ([Review] Fig. 9, "SpargeAttn + Sage2"): V8 [N, d_v] holds the E4M3
    values of V / delta (delta [d_v] per channel, :func:`v_channel_scales`),
    and each tile adds e4m3(P8_SCALE P~) V8 delta / P8_SCALE, with P~ =
    exp(S - m_new) taken at the running max of that step, in Algorithm 1's
    order; the rescaling by exp(m - m_new) and l are exact.
    ``margins`` [Tn, c_w], if given, receives max(m_loc - m_new) - lambda
    of every voting group (the rule skips iff it is negative).  Returns
    (O_i [n, d_v], counts dict, decisions [Tn, c_w] int8 with 1 = PV executed,
    2 = skipped by the lambda vote, 3 = void group (no visible key in the
    tile), 0 = tile not visited).
    """
    N, d = Qh.shape
    Tn = num_blocks(N, bk)
    rows = block_rows(N, bq, i)
    n = len(rows)
    q_idx = np.arange(rows.start, rows.stop)
    Qi = Qh[rows.start:rows.stop]
    m = np.full(n, NEG_INF)
    l = np.zeros(n)
    O = np.zeros((n, Vh.shape[1]))
    cw = (bq + R - 1) // R
    groups = [np.arange(g * R, min(n, g * R + R)) for g in range(cw) if g * R < n]
    live = tile_live(N, bq, bk, causal)[i]
    decisions = np.zeros((Tn, cw), dtype=np.int8)
    cnt = dict.fromkeys(COUNT_NAMES, 0)
    cnt["live_tiles"] = int(live.sum())
    for j in range(Tn):                               # ascending j
        if not (mg_row[j] and live[j]):
            continue
        cnt["qk_exec"] += 1
        keys = block_rows(N, bk, j)
        k_idx = np.arange(keys.start, keys.stop)
        if score_fn is None:
            S = _scores_float(Qi, Kh[keys.start:keys.stop])
        else:
            S = score_fn(rows, keys)
        if causal:
            S = np.where(k_idx[None, :] > q_idx[:, None], NEG_INF, S)
        m_loc = S.max(axis=1)
        m_new = np.maximum(m, m_loc)
        with np.errstate(invalid="ignore"):
            m_sub = np.where(np.isfinite(m_new), m_new, 0.0)
            Pt = np.exp(S - m_sub[:, None])           # exp(-inf) = 0
            alpha = np.where(np.isfinite(m), np.exp(m - m_sub), 0.0)
        l = alpha * l + Pt.sum(axis=1)
        for g, gi in enumerate(groups):
            fin = np.isfinite(m_loc[gi])
            rule_skip = (not fin.any()) or (np.max(m_loc[gi][fin] - m_new[gi][fin]) < lam)
            if margins is not None and fin.any():
                margins[j, g] = np.max(m_loc[gi][fin] - m_new[gi][fin]) - lam
            if vote_info is not None and fin.any():
                vote_info.append((j, g, float(np.max(m_loc[gi][fin] - m_new[gi][fin])),
                                  bool(np.any(m_new[gi] != m[gi]))))
            skip = rule_skip
            if skip_override is not None and fin.any() and skip_override[j, g] in (1, 2):
                skip = skip_override[j, g] == 2
            if not fin.any():
                cnt["pv_void"] += 1
                decisions[j, g] = 3
            elif skip:
                cnt["pv_skip"] += 1
                decisions[j, g] = 2                   # O_ij[I_w] = O_i,j-1[I_w]
            else:
                cnt["pv_exec"] += 1
                decisions[j, g] = 1
                if pv8 is None:
                    O[gi] = alpha[gi, None] * O[gi] + Pt[gi] @ Vh[keys.start:keys.stop]
                else:
                    V8, delta = pv8
                    P8 = e4m3_round(P8_SCALE * Pt[gi])
                    O[gi] = alpha[gi, None] * O[gi] + (P8 @ V8[keys.start:keys.stop]) * (delta / P8_SCALE)
        m = m_new
    out = np.zeros_like(O)
    nz = l > 0
    out[nz] = O[nz] / l[nz, None]
    cnt["qk_skip"] = cnt["live_tiles"] - cnt["qk_exec"]
    cnt["empty_rows"] = int((~nz).sum())
    cnt["rows"] = n
    return out, cnt, decisions


def sparse_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mg: np.ndarray, lam: float,
                     causal: bool, bq: int = BQ, bk: int = BK, R: int = ROWS_PER_GROUP,
                     blocks: Optional[Sequence[Tuple[int, int, int]]] = None,
                     skip_override: Optional[np.ndarray] = None, quant: Optional[dict] = None,
                     margins: Optional[np.ndarray] = None, pv8: bool = False):
    """Stage 2 for Q [B, H, N, d], K/V [B, H_kv, N, d] and M_g [B, H, Tm, Tn].

    ``blocks`` restricts the work to (b, h, i) query blocks; the other rows of
    the returned O stay 0.  ``skip_override`` [B, H, Tm, Tn, c_w] replays PV
    decisions.  ``quant`` (from :func:`quantize_qk`) switches S to the int8
    form.  ``pv8`` runs the P~V products on 8-bit floats (see
    :func:`attend_row_block`), with V scaled per channel of each kv head.
    ``margins`` [B, H, Tm, Tn, c_w] (NaN-filled by the caller) receives
    every vote's margin, as in :func:`attend_row_block`.  Returns (O [B, H, N, d_v], counts dict summed over the blocks,
    decisions [B, H, Tm, Tn, c_w]).
    """
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    Tm, Tn = num_blocks(N, bq), num_blocks(N, bk)
    cw = (bq + R - 1) // R
    O = np.zeros((B, H, N, V.shape[3]))
    dec = np.zeros((B, H, Tm, Tn, cw), dtype=np.int8)
    tot = dict.fromkeys(COUNT_NAMES, 0)
    todo = blocks if blocks is not None else [(b, h, i) for b in range(B) for h in range(H)
                                              for i in range(Tm)]
    v8 = {}
    for b, h, i in todo:
        hk = kv_head(h, H, H_kv)
        if pv8 and (b, hk) not in v8:
            delta = v_channel_scales(V[b, hk])
            v8[b, hk] = (e4m3_round(V[b, hk] / delta[None, :]), delta)
        score_fn = None
        if quant is not None:
            qc, kc = quant["q_codes"][b, h], quant["k_codes"][b, hk]
            dq, dk = quant["q_scale"][b, h], quant["k_scale"][b, hk]

            def score_fn(rows, keys, qc=qc, kc=kc, dq=dq, dk=dk, i=i):
                j = keys.start // bk
                acc = qc[rows.start:rows.stop] @ kc[keys.start:keys.stop].T   # exact integers
                return acc * (dq[i] * dk[j]) / math.sqrt(d)
        ov = None if skip_override is None else skip_override[b, h, i]
        o, c, decision = attend_row_block(Q[b, h], K[b, hk], V[b, hk], mg[b, h, i], i, lam, causal,
                                          bq, bk, R, ov, score_fn,
                                          margins=None if margins is None else margins[b, h, i],
                                          pv8=v8.get((b, hk)))
        rows = block_rows(N, bq, i)
        O[b, h, rows.start:rows.stop] = o
        dec[b, h, i] = decision
        for kname in COUNT_NAMES:
            tot[kname] += c[kname]
    return O, tot, dec


def dense_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, causal: bool) -> np.ndarray:
    """Brute force softmax(Q K^T / sqrt(d)) V (two-pass), Q [B,H,N,d], K/V [B,H_kv,N,d]."""
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    O = np.zeros((B, H, N, V.shape[3]))
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            S = Q[b, h] @ K[b, hk].T / math.sqrt(d)
            if causal:
                S = np.where(np.triu(np.ones((N, N), dtype=bool), 1), NEG_INF, S)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            O[b, h] = (P / P.sum(axis=1, keepdims=True)) @ V[b, hk]
    return O


def masked_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mg: np.ndarray, causal: bool,
                     bq: int = BQ, bk: int = BK) -> np.ndarray:
    """Closed form of eqs. 1-2 without the lambda rule: softmax(S + log M~) V, with
    M_g expanded to tokens (two-pass, per row); a row with no visible key gives 0."""
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    O = np.zeros((B, H, N, V.shape[3]))
    qb = np.arange(N) // bq
    kb = np.arange(N) // bk
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            S = Q[b, h] @ K[b, hk].T / math.sqrt(d)
            allow = mg[b, h][qb[:, None], kb[None, :]].astype(bool)
            if causal:
                allow &= ~np.triu(np.ones((N, N), dtype=bool), 1)
            S = np.where(allow, S, NEG_INF)
            for r in range(N):
                if not allow[r].any():
                    continue
                p = np.exp(S[r] - S[r].max())
                O[b, h, r] = (p / p.sum()) @ V[b, hk]
    return O


# ---------------------------------------------------------------------------
# fp8 P~V ([Review] Fig. 9, "SpargeAttn + Sage2": P~V on 8-bit floats)
# ---------------------------------------------------------------------------
# The pages name the variant and nothing more.  Format readings (the plainest
# ones the variant's name supports):
# * OCP E4M3: 4 exponent bits (bias 7), 3 mantissa bits, largest finite 448,
#   subnormal step 2^-9; round to nearest, ties to the even mantissa.
# * V per channel c of a kv head: delta_c = 2^e, e the least integer with
#   max_n |V[n, c]| <= 448 * 2^e (1 for an all-zero channel), so V / delta_c
#   is exact and fits the format before its one rounding.
# * P~ = exp(S - m_ij) lies in [0, 1] under the running max of Algorithm 1;
#   it is scaled by P8_SCALE = 2^8, the largest power of two that keeps 1
#   inside the format's range (2^8 <= 448 < 2^9), so the scaling is exact
#   and P~ keeps the format's full exponent range.
# * The products are summed, and l and the rescaling of eq. 1 are taken, as
#   in the unquantised recurrence (exactly, here).
# The recurrence itself is attend_row_block's, with its ``pv8`` argument.

E4M3_MAX = 448.0
P8_SCALE = 256.0


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value (ties to the even mantissa), saturating at +-448.
    Normal numbers (|x| >= 2^-6) keep 3 fraction bits; below, the step is 2^-9."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    q = 2.0 ** (e - 3)                                # spacing of the binade (2^-9 when subnormal)
    r = np.rint(a / q) * q                            # np.rint: ties to even
    r = np.minimum(r, E4M3_MAX)
    return np.sign(x) * r


def v_channel_scales(Vh: np.ndarray) -> np.ndarray:
    """delta_c = 2^e with e the least integer such that max|V[:, c]| <= 448 * 2^e;
    1 for an all-zero channel.  Vh [N, d_v]."""
    mx = np.abs(Vh).max(axis=0)
    e = np.zeros_like(mx)
    nz = mx > 0
    e[nz] = np.ceil(np.log2(mx[nz] / E4M3_MAX))
    # exact comparisons settle a log2 that lands next to an integer
    e = np.where(nz & (mx > E4M3_MAX * 2.0 ** e), e + 1, e)
    e = np.where(nz & (mx <= E4M3_MAX * 2.0 ** (e - 1)), e - 1, e)
    return np.where(nz, 2.0 ** e, 1.0)


# ---------------------------------------------------------------------------
# int8 per-block quantisation ([Review] Algorithm 1 step 2, components table)
# ---------------------------------------------------------------------------

def quantize_block(X: np.ndarray) -> Tuple[np.ndarray, float]:
    """Symmetric int8 codes of one block: delta = max|x| / 127, code = rint(x/delta)."""
    amax = float(np.abs(X).max()) if X.size else 0.0
    delta = amax / 127.0 if amax > 0 else 1.0
    codes = np.clip(np.rint(X / delta), -127, 127)
    return codes, delta


def quantize_qk(Q: np.ndarray, K: np.ndarray, bq: int = BQ, bk: int = BK) -> dict:
    """Per-block int8 codes and scales of Q [B,H,N,d] and of K - mean_t(K) [B,H_kv,N,d].

    Returns q_codes / k_codes (float64 holding integers), q_scale [B,H,Tm],
    k_scale [B,H_kv,Tn] (float64), k_mean [B,H_kv,d] and the per-element
    distance of x/delta from the nearest rounding tie (for near-tie accounting).
    """
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    Tm, Tn = num_blocks(N, bq), num_blocks(N, bk)
    k_mean = K.mean(axis=2)                                  # over all N tokens
    Kc = K - k_mean[:, :, None, :]
    q_codes = np.zeros_like(Q)
    k_codes = np.zeros_like(K)
    q_scale = np.zeros((B, H, Tm))
    k_scale = np.zeros((B, H_kv, Tn))
    q_tie = np.zeros_like(Q)
    k_tie = np.zeros_like(K)
    for b in range(B):
        for h in range(H):
            for i in range(Tm):
                r = block_rows(N, bq, i)
                c, dl = quantize_block(Q[b, h, r.start:r.stop])
                q_codes[b, h, r.start:r.stop] = c
                q_scale[b, h, i] = dl
                t = Q[b, h, r.start:r.stop] / dl
                q_tie[b, h, r.start:r.stop] = np.abs(t - np.floor(t) - 0.5)
        for h in range(H_kv):
            for j in range(Tn):
                r = block_rows(N, bk, j)
                c, dl = quantize_block(Kc[b, h, r.start:r.stop])
                k_codes[b, h, r.start:r.stop] = c
                k_scale[b, h, j] = dl
                t = Kc[b, h, r.start:r.stop] / dl
                k_tie[b, h, r.start:r.stop] = np.abs(t - np.floor(t) - 0.5)
    return {"q_codes": q_codes, "k_codes": k_codes, "q_scale": q_scale, "k_scale": k_scale,
            "k_mean": k_mean, "k_centered": Kc, "q_tie_dist": q_tie, "k_tie_dist": k_tie}


# ---------------------------------------------------------------------------
# 3D Hilbert-curve order ([Review] "HilbertCurve Permutation";
# [Rebuttal] Weaknesses3 / Weaknesses3.2)
# ---------------------------------------------------------------------------

def hilbert_index(coords: Sequence[int], bits: int) -> int:
    """Curve index of a point of the 2^bits cube, by Skilling's method: undo the
    excess work (inverse-undo pass), Gray-encode the transposed form, then
    interleave the transposed bits from the most significant level down."""
    x = [int(c) for c in coords]
    n = len(x)
    m = 1 << (bits - 1)
    q = m
    while q > 1:                                   # inverse undo
        p = q - 1
        for a in range(n):
            if x[a] & q:
                x[0] ^= p                          # invert low bits of axis 0
            else:
                t = (x[0] ^ x[a]) & p              # exchange low bits of axes 0 and a
                x[0] ^= t
                x[a] ^= t
        q >>= 1
    for a in range(1, n):                          # Gray encode
        x[a] ^= x[a - 1]
    t = 0
    q = m
    while q > 1:
        if x[n - 1] & q:
            t ^= q - 1
        q >>= 1
    for a in range(n):
        x[a] ^= t
    h = 0                                          # interleave: axis 0 is the most significant
    for level in range(bits - 1, -1, -1):
        for a in range(n):
            h = (h << 1) | ((x[a] >> level) & 1)
    return h


def hilbert_permutation(T: int, Hg: int, Wg: int) -> Tuple[np.ndarray, np.ndarray]:
    """perm[p] = raster token (t*Hg + h)*Wg + w whose curve rank is p; inv = perm^-1.

    Points are indexed on the enclosing 2^bits cube (bits = ceil(log2(max side)))
    and sorted by their index; indices are distinct, so the order is unique.
    """
    side = max(T, Hg, Wg, 1)
    bits = max(1, int(math.ceil(math.log2(side))))
    keys = np.empty(T * Hg * Wg, dtype=np.int64)
    for t in range(T):
        for h in range(Hg):
            for w in range(Wg):
                keys[(t * Hg + h) * Wg + w] = hilbert_index((t, h, w), bits)
    perm = np.argsort(keys, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return perm, inv


def raster_order(T: int, Hg: int, Wg: int) -> np.ndarray:
    """Row-major order of the permutation comparison ([Review] Table 4):
    tokens in (t, h, w) order with w fastest, i.e. the raster index itself."""
    return np.arange(T * Hg * Wg, dtype=np.int32)


def time_major_order(T: int, Hg: int, Wg: int) -> np.ndarray:
    """Time-major order ([Review] Table 4, read as: the frames of one pixel
    adjacent): position p = ((h * Wg) + w) * T + t holds raster token
    (t * Hg + h) * Wg + w."""
    perm = np.empty(T * Hg * Wg, dtype=np.int32)
    p = 0
    for h in range(Hg):
        for w in range(Wg):
            for t in range(T):
                perm[p] = (t * Hg + h) * Wg + w
                p += 1
    return perm


def block_self_similarity(X: np.ndarray, b: int) -> float:
    """Sim-q / Sim-k of [Review] Table 4: the mean CosSim (eq. 6) over the
    b-token blocks of X [N, d] (the last block may be ragged)."""
    return float(np.mean(block_cossim(X, b)))


def permute_tokens(X: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """X' [..., p, :] = X[..., perm[p], :] (gather along the token axis)."""
    return X[..., perm, :]


def unpermute_tokens(Xp: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Inverse of :func:`permute_tokens`: X[..., perm[p], :] = X'[..., p, :]."""
    out = np.empty_like(Xp)
    out[..., perm, :] = Xp
    return out


# ---------------------------------------------------------------------------
# relative L1 error ([Review] hyper-parameter section: L1 = sum|O - O'| / sum|O|)
# ---------------------------------------------------------------------------

def rel_l1(O_ref: np.ndarray, O: np.ndarray) -> float:
    den = float(np.abs(O_ref).sum())
    return float(np.abs(O_ref - O).sum()) / den if den > 0 else float(np.abs(O).sum())
