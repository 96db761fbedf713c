"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these tests re-types an oracle formula: each checks a closed form, a
special case, a brute force on a tiny input, a hand-built row or the worked
example printed in the authors' rebuttal.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import sparge_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# Whole pipeline: dense limit (theta > 1 forces every block, lambda = -inf)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,H,H_kv,d", [(300, 2, 1, 64), (256, 2, 2, 128), (70, 4, 2, 64)])
def test_dense_limit_equals_brute_force(causal, N, H, H_kv, d):
    Q = _rand((1, H, N, d), 1)
    K = _rand((1, H_kv, N, d), 2)
    V = _rand((1, H_kv, N, d), 3)
    pred = O.predict_mask(Q, K, tau=0.5, theta=2.0, causal=causal)
    live = O.tile_live(N, O.BQ, O.BK, causal)
    assert np.array_equal(pred["mg"][0, 0], live)
    out, cnt, _ = O.sparse_attention(Q, K, V, pred["mg"], -np.inf, causal)
    ref = O.dense_attention(Q, K, V, causal)
    assert np.max(np.abs(out - ref)) <= 1e-10
    assert cnt["pv_skip"] == 0 and cnt["qk_skip"] == 0 and cnt["empty_rows"] == 0
    if not causal:
        assert cnt["pv_void"] == 0


def test_dense_attention_matches_textbook_loop():
    """dense_attention itself against a per-element triple loop (tiny)."""
    Q, K, V = _rand((1, 1, 5, 3), 4), _rand((1, 1, 5, 3), 5), _rand((1, 1, 5, 2), 6)
    for causal in (False, True):
        ref = np.zeros((5, 2))
        for r in range(5):
            w = []
            for c in range(5):
                if causal and c > r:
                    w.append(0.0)
                    continue
                w.append(math.exp(sum(Q[0, 0, r, t] * K[0, 0, c, t] for t in range(3)) / math.sqrt(3)))
            z = sum(w)
            for e in range(2):
                ref[r, e] = sum(w[c] * V[0, 0, c, e] for c in range(5)) / z
        assert np.max(np.abs(O.dense_attention(Q, K, V, causal)[0, 0] - ref)) < 1e-12


# ---------------------------------------------------------------------------
# Attention given a mask: online recurrence (eq. 1) == two-pass masked softmax
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_equals_masked_closed_form(causal):
    N, d = 450, 64
    Q, K, V = _rand((1, 3, N, d), 7), _rand((1, 1, N, d), 8), _rand((1, 1, N, d), 9)
    Tm, Tn = O.num_blocks(N, O.BQ), O.num_blocks(N, O.BK)
    mg = np.random.default_rng(10).random((1, 3, Tm, Tn)) < 0.5
    mg[0, 0, 1, :] = False                         # a block row with no key at all
    out, cnt, _ = O.sparse_attention(Q, K, V, mg, -np.inf, causal)
    ref = O.masked_attention(Q, K, V, mg, causal)
    assert np.max(np.abs(out - ref)) <= 1e-10
    assert cnt["empty_rows"] >= 128                 # the empty block row outputs zeros
    assert np.all(out[0, 0, 128:256] == 0)


# ---------------------------------------------------------------------------
# Lambda rule on a hand-built two-block toy
# ---------------------------------------------------------------------------

def _lambda_toy():
    """N = 128, d = 64, one query block (four 32-row groups), two key blocks.

    Scores are S[r, key in block 0] = alpha_r and S[r, key in block 1] = beta_r:
    groups 0 and 1: alpha = 30, beta = 10 (block 1 is 20 nats below: skip);
    group 2: alpha = 30, beta = 10 except one row with beta = 29 (-1 nat: run);
    group 3: alpha = 0, beta = 5 (block 1 raises the max: run).
    """
    N, d = 128, 64
    Q = np.zeros((1, 1, N, d))
    K = np.zeros((1, 1, N, d))
    alpha = np.array([30.0] * 96 + [0.0] * 32)
    beta = np.array([10.0] * 96 + [5.0] * 32)
    beta[64 + 7] = 29.0
    Q[0, 0, :, 0] = alpha
    Q[0, 0, :, 1] = beta
    K[0, 0, :64, 0] = math.sqrt(d)                 # S = q . k / sqrt(d)
    K[0, 0, 64:, 1] = math.sqrt(d)
    V = _rand((1, 1, N, 16), 11)
    return Q, K, V, alpha, beta


def test_lambda_vote_toy_counts_and_values():
    Q, K, V, alpha, beta = _lambda_toy()
    mg = np.ones((1, 1, 1, 2), dtype=bool)
    out, cnt, dec = O.sparse_attention(Q, K, V, mg, -5.0, False)
    assert cnt["pv_exec"] == 6 and cnt["pv_skip"] == 2
    assert dec[0, 0, 0, 0].tolist() == [1, 1, 1, 1]
    assert dec[0, 0, 0, 1].tolist() == [2, 2, 1, 1]
    v0 = V[0, 0, :64].mean(axis=0)
    v1 = V[0, 0, 64:].mean(axis=0)
    # skipped rows: numerator keeps only block 0, the denominator still counts block 1
    e = math.exp(10.0 - 30.0)
    assert np.max(np.abs(out[0, 0, 0] - v0 / (1.0 + e))) < 1e-12
    # executed rows are exact attention over both blocks
    e3 = math.exp(5.0 - 0.0)
    assert np.max(np.abs(out[0, 0, 100] - (v0 + e3 * v1) / (1.0 + e3))) < 1e-12
    e2 = math.exp(29.0 - 30.0)
    assert np.max(np.abs(out[0, 0, 71] - (v0 + e2 * v1) / (1.0 + e2))) < 1e-12


def test_lambda_vote_threshold_and_ascending_order():
    """Block 1 sits 20 nats below block 0 for groups 0-1: they skip iff -20 < lambda.
    Visiting block 1 first would never skip (its max would be the running max),
    so two skips at lambda = -19 also pin the ascending j order."""
    Q, K, V, _, _ = _lambda_toy()
    mg = np.ones((1, 1, 1, 2), dtype=bool)
    for lam, skips in ((-25.0, 0), (-20.001, 0), (-19.999, 2), (-19.0, 2), (-0.5, 3)):
        _, cnt, _ = O.sparse_attention(Q, K, V, mg, lam, False)
        assert cnt["pv_skip"] == skips, lam
        assert cnt["pv_exec"] + cnt["pv_skip"] == 8 and cnt["pv_void"] == 0


def test_lambda_very_negative_equals_no_rule():
    N, d = 400, 64
    Q, K, V = _rand((1, 2, N, d), 12, 2.0), _rand((1, 2, N, d), 13, 2.0), _rand((1, 2, N, d), 14)
    mg = np.ones((1, 2, O.num_blocks(N, 128), O.num_blocks(N, 64)), dtype=bool)
    a, _, _ = O.sparse_attention(Q, K, V, mg, -1e9, True)
    b, _, _ = O.sparse_attention(Q, K, V, mg, -np.inf, True)
    assert np.array_equal(a, b)


def test_lambda_skip_leaves_running_max_unchanged():
    """Whenever a group skips, none of its rows' running max moved (so skipping
    the rescale of O is exact), and the output differs from the no-skip one."""
    N, d = 512, 64
    Q = _rand((1, 1, N, d), 15, 3.0)
    K = _rand((1, 1, N, d), 16, 3.0)
    V = _rand((1, 1, N, d), 17)
    Q[0, 0, :, 0] += 10.0                           # key block 0 dominates by about 12 nats
    K[0, 0, :64, 0] += 10.0
    info = []
    o, c, dec = O.attend_row_block(Q[0, 0], K[0, 0], V[0, 0], np.ones(8, bool), 2, -3.0, False,
                                   vote_info=info)
    assert c["pv_skip"] > 0 and c["pv_exec"] > 0
    for (j, g, worst, moved) in info:
        if dec[j, g] == 2:
            assert not moved and worst < -3.0
    full, _, _ = O.attend_row_block(Q[0, 0], K[0, 0], V[0, 0], np.ones(8, bool), 2, -np.inf, False)
    assert 0 < np.max(np.abs(o - full)) < 0.5


# ---------------------------------------------------------------------------
# CosSim (eq. 6 as the mean pairwise cosine)
# ---------------------------------------------------------------------------

def test_cossim_special_cases():
    x = _rand(64, 18)
    assert abs(O.cossim(np.tile(x, (128, 1))) - 1.0) < 1e-12          # identical rows
    assert abs(O.cossim(np.tile(x, (64, 1)) * np.arange(1, 65)[:, None]) - 1.0) < 1e-12
    assert abs(O.cossim(np.eye(64) * 3.0) - 1.0 / 64) < 1e-15          # orthogonal rows
    alt = np.tile(x, (64, 1)) * np.where(np.arange(64) % 2 == 0, 1.0, -1.0)[:, None]
    assert abs(O.cossim(alt)) < 1e-15                                  # x, -x, x, ...
    z = np.zeros((4, 8))
    z[0] = _rand(8, 19)
    assert abs(O.cossim(z) - 1.0 / 16) < 1e-15                         # zero rows count 0


def test_cossim_brute_force_pairs():
    X = _rand((7, 5), 20)
    tot = 0.0
    for a, c in itertools.product(range(7), repeat=2):
        dot = sum(X[a, t] * X[c, t] for t in range(5))
        na = math.sqrt(sum(v * v for v in X[a]))
        nc = math.sqrt(sum(v * v for v in X[c]))
        tot += dot / (na * nc)
    assert abs(O.cossim(X) - tot / 49) < 1e-13


def test_mean_pool_ragged_blocks():
    X = np.arange(10 * 3, dtype=np.float64).reshape(10, 3)
    m = O.mean_pool(X, 4)
    assert m.shape == (3, 3)
    assert np.array_equal(m[2], X[8:10].mean(axis=0))
    assert np.array_equal(m[0], np.array([4.5, 5.5, 6.5]))


# ---------------------------------------------------------------------------
# TopCdf (eq. 8) on hand-built dyadic rows
# ---------------------------------------------------------------------------

def test_topcdf_golden_rows():
    with open(os.path.join(GOLDEN, "topcdf_rows.json")) as f:
        rows = json.load(f)["rows"]
    for r in rows:
        keep, _ = O.topcdf(np.array(r["p"]), r["tau"])
        assert sorted(np.nonzero(keep)[0].tolist()) == r["keep"], r


# ---------------------------------------------------------------------------
# Stage 1 on constructed blocks
# ---------------------------------------------------------------------------

def _const_blocks(vectors, b):
    """Tokens: block t repeats vectors[t] b times (s = 1, mean = the vector)."""
    return np.concatenate([np.tile(v, (b, 1)) for v in vectors])


def _fix_block(u, b):
    """Alternating +u, -u: mean 0 and mean pairwise cosine 0 (a fix block)."""
    return np.tile(u, (b, 1)) * np.where(np.arange(b) % 2 == 0, 1.0, -1.0)[:, None]


def test_compressed_map_scale_is_one_over_sqrt_d():
    """Two selective key blocks with q.k = 8 ln 3 and 0 and d = 64: with the
    1/sqrt(d) scale P^ = [3/4, 1/4] and tau = 0.8 keeps both; without it
    P^ ~ [0.99985, 0.00015] would keep one."""
    d = 64
    e0 = np.eye(d)[0]
    N = 128
    Q = _const_blocks([e0], 128)
    K = _const_blocks([8 * math.log(3.0) * e0, 0 * e0], 64)
    K[64:, 1] = 1.0                                 # keep block 1 non-zero (its mean.q = 0)
    r = O.predict_mask_head(Q, K, tau=0.8, theta=0.5, causal=False)
    assert r["mg"].tolist() == [[True, True]]
    z = r["shat"][0]
    assert abs(z[0] - math.log(3.0)) < 1e-12 and abs(z[1]) < 1e-12
    r = O.predict_mask_head(Q, K, tau=0.74, theta=0.5, causal=False)
    assert r["mg"].tolist() == [[True, False]]


def test_fix_rows_and_columns_are_forced_and_future_is_zero():
    d = 64
    rng = np.random.default_rng(21)
    N = 64 * 8
    e0 = np.eye(d)[0]
    kvecs = [e0 * 10.0 if j == 0 else -e0 * 10.0 for j in range(8)]
    K = _const_blocks(kvecs, 64)
    K[3 * 64:4 * 64] = _fix_block(np.eye(d)[1], 64)     # key block 3 is fix
    Q = _const_blocks([e0, e0, e0, e0], 128)
    Q[128:256] = rng.standard_normal((128, d))           # query block 1 is fix (s ~ 1/128)
    r = O.predict_mask_head(Q, K, tau=0.5, theta=0.5, causal=True)
    live = O.tile_live(N, 128, 64, True)
    mg = r["mg"]
    assert r["fix_q"].tolist() == [False, True, False, False]
    assert r["fix_k"].tolist() == [False, False, False, True, False, False, False, False]
    assert not mg[~live].any()                           # wholly future tiles are 0
    assert mg[1][live[1]].all()                          # fix query row: every live tile
    assert mg[:, 3][live[:, 3]].all()                    # fix key column: every live tile
    # selective rows keep the dominant block 0 only (besides the forced column)
    assert np.nonzero(mg[0])[0].tolist() == [0]
    for i in (2, 3):
        assert np.nonzero(mg[i])[0].tolist() == [0, 3]


@pytest.mark.parametrize("case", [0, 1])
def test_rebuttal_worked_sparsity_example(case):
    """The rebuttal's arithmetic: sparsity = selective fraction x sparsity inside it,
    reproduced on a constructed toy: 100 key blocks, of which 80 (resp. 90) are
    selective; 30% of those carry negligible probability, so TopCdf drops them."""
    with open(os.path.join(GOLDEN, "rebuttal_worked_example.json")) as f:
        g = json.load(f)["cases"][case]
    d, Tn = 64, 100
    n_sel = int(round(g["selective_fraction"] * Tn))
    n_drop = int(round(g["sparsity_within_selective"] * n_sel))
    e0, e1 = np.eye(d)[0], np.eye(d)[1]
    fix_cols = set(range(0, Tn, Tn // (Tn - n_sel))) if n_sel < Tn else set()
    sel_cols = [j for j in range(Tn) if j not in fix_cols]
    drop_cols = set(sel_cols[1::2][:n_drop]) if n_drop <= len(sel_cols[1::2]) else set()
    assert len(fix_cols) == Tn - n_sel and len(drop_cols) == n_drop
    blocks = []
    for j in range(Tn):
        if j in fix_cols:
            blocks.append(_fix_block(e1, 64))
        else:
            blocks.append(np.tile(e0 * (-40.0 if j in drop_cols else 0.0) + np.eye(d)[2], (64, 1)))
    K = np.concatenate(blocks)[None, None]
    N = K.shape[2]
    Q = np.tile(e0 * 8.0 + np.eye(d)[3], (N, 1))[None, None]
    pred = O.predict_mask(Q, K, tau=0.99, theta=0.5, causal=False)
    mg = pred["mg"][0, 0]
    live = mg.size
    computed = mg.sum() / live
    assert abs((1 - computed) - g["effective_sparsity"]) < 1e-12
    assert abs(computed - g["blocks_computed"]) < 1e-12
    frac_sel = (pred["s_k"][0, 0] >= 0.5).mean()
    inside = 1 - mg[:, pred["s_k"][0, 0] >= 0.5].mean()
    assert abs(frac_sel - g["selective_fraction"]) < 1e-12
    assert abs(inside - g["sparsity_within_selective"]) < 1e-12


# ---------------------------------------------------------------------------
# int8 per-block quantisation
# ---------------------------------------------------------------------------

def test_quantize_block_hand_values():
    X = np.array([[127.0, 63.5, -0.5, 1.5], [2.5, -2.5, 0.0, -127.0]])
    codes, delta = O.quantize_block(X)
    assert delta == 1.0
    assert codes.tolist() == [[127, 64, 0, 2], [2, -2, 0, -127]]    # ties to even
    codes, delta = O.quantize_block(np.zeros((3, 3)))
    assert delta == 1.0 and not codes.any()


def test_quantize_error_bound_and_range():
    N, d = 333, 64
    Q = _rand((1, 2, N, d), 22, 3.0)
    K = _rand((1, 1, N, d), 23, 3.0) + 5.0
    qz = O.quantize_qk(Q, K)
    for X, codes, scale, b in ((Q, qz["q_codes"], qz["q_scale"], 128),
                               (qz["k_centered"], qz["k_codes"], qz["k_scale"], 64)):
        for t in range(scale.shape[2]):
            r = O.block_rows(N, b, t)
            blk = X[0, 0, r.start:r.stop]
            c = codes[0, 0, r.start:r.stop]
            dl = scale[0, 0, t]
            assert np.all(np.abs(blk - dl * c) <= dl / 2 * (1 + 1e-12))
            assert np.max(np.abs(c)) == 127
    assert np.allclose(qz["k_centered"].mean(axis=2), 0.0, atol=1e-12)


def test_key_mean_shift_leaves_attention_unchanged():
    """softmax is invariant to a per-row constant, so q.(k - mu) gives the same O."""
    N, d = 200, 64
    Q, K, V = _rand((1, 2, N, d), 24), _rand((1, 1, N, d), 25) + 2.0, _rand((1, 1, N, d), 26)
    for causal in (False, True):
        a = O.dense_attention(Q, K, V, causal)
        b = O.dense_attention(Q, K - K.mean(axis=2, keepdims=True), V, causal)
        assert np.max(np.abs(a - b)) < 1e-12


def test_int8_attention_is_close_to_float_attention():
    N, d = 256, 64
    Q, K, V = _rand((1, 1, N, d), 27), _rand((1, 1, N, d), 28), _rand((1, 1, N, d), 29)
    mg = np.ones((1, 1, 2, 4), dtype=bool)
    qz = O.quantize_qk(Q, K)
    oq, _, _ = O.sparse_attention(Q, K, V, mg, -np.inf, False, quant=qz)
    of = O.dense_attention(Q, K, V, False)
    assert O.rel_l1(of, oq) < 2e-2


@pytest.mark.parametrize("sq,sk", [(1.0, 1.0), (0.5, 0.25)])
def test_int8_scores_exact_on_representable_inputs(sq, sk):
    """Integer-valued blocks whose max is 127 (times sq, sk) have exact codes and
    scales delta = sq, sk; K has zero column means, so centring changes nothing.
    The int8 score (codes_q . codes_k) delta_q delta_k / sqrt(d) then equals the
    float score and the outputs agree to rounding."""
    N, d = 256, 64
    rng = np.random.default_rng(30)
    Qi = rng.integers(-100, 101, size=(N, d)).astype(np.float64)
    Qi[0, 0] = 127.0
    Qi[128, 5] = -127.0
    A = rng.integers(-100, 101, size=(128, d)).astype(np.float64)
    A[0, 1] = 127.0
    A[64, 2] = -127.0
    Ki = np.concatenate([A, -A])
    Q = (sq * Qi)[None, None]
    K = (sk * Ki)[None, None]
    V = _rand((1, 1, N, d), 31)
    qz = O.quantize_qk(Q, K)
    assert np.all(qz["q_scale"] == sq) and np.all(qz["k_scale"] == sk)
    assert np.array_equal(qz["q_codes"][0, 0], Qi) and np.array_equal(qz["k_codes"][0, 0], Ki)
    mg = np.ones((1, 1, 2, 4), dtype=bool)
    for causal in (False, True):
        oq, _, _ = O.sparse_attention(Q, K, V, mg, -np.inf, causal, quant=qz)
        assert np.max(np.abs(oq - O.dense_attention(Q, K, V, causal))) < 1e-12


# ---------------------------------------------------------------------------
# 3D Hilbert order
# ---------------------------------------------------------------------------

def _cube_order(n_axes, bits):
    side = 1 << bits
    pts = list(itertools.product(range(side), repeat=n_axes))
    idx = [O.hilbert_index(p, bits) for p in pts]
    order = [p for _, p in sorted(zip(idx, pts))]
    return idx, order


@pytest.mark.parametrize("n_axes,bits", [(2, 4), (3, 2), (3, 3)])
def test_hilbert_cube_is_a_face_adjacent_bijection(n_axes, bits):
    idx, order = _cube_order(n_axes, bits)
    assert sorted(idx) == list(range((1 << bits) ** n_axes))
    for a, b in zip(order, order[1:]):
        assert sum(abs(x - y) for x, y in zip(a, b)) == 1
    assert all(c == 0 for c in order[0])


@pytest.mark.parametrize("n_axes,bits", [(3, 3), (2, 4)])
def test_hilbert_aligned_subcubes_are_contiguous(n_axes, bits):
    idx, _ = _cube_order(n_axes, bits)
    side = 1 << bits
    pts = list(itertools.product(range(side), repeat=n_axes))
    for m in range(1, bits):
        groups = {}
        for p, h in zip(pts, idx):
            groups.setdefault(tuple(c >> m for c in p), []).append(h)
        for hs in groups.values():
            hs = sorted(hs)
            assert hs[-1] - hs[0] == len(hs) - 1 and hs[0] % len(hs) == 0


def test_hilbert_video_grid_runs_are_aligned_4_cubes():
    T, Hg, Wg = 12, 48, 80
    perm, inv = O.hilbert_permutation(T, Hg, Wg)
    assert np.array_equal(np.sort(perm), np.arange(T * Hg * Wg))
    assert np.array_equal(perm[inv], np.arange(T * Hg * Wg))
    t, rem = np.divmod(perm, Hg * Wg)
    h, w = np.divmod(rem, Wg)
    for s in range(0, perm.size, 64):
        sl = slice(s, s + 64)
        corner = (t[sl].min(), h[sl].min(), w[sl].min())
        assert all(c % 4 == 0 for c in corner)
        assert t[sl].max() - corner[0] == 3 and h[sl].max() - corner[1] == 3
        assert w[sl].max() - corner[2] == 3


def test_dense_attention_commutes_with_permutation():
    """Standard attention is token-permutation invariant (rebuttal, Weaknesses3.2)."""
    T, Hg, Wg = 2, 4, 8
    perm, _ = O.hilbert_permutation(T, Hg, Wg)
    N, d = T * Hg * Wg, 16
    Q, K, V = _rand((1, 2, N, d), 32), _rand((1, 2, N, d), 33), _rand((1, 2, N, d), 34)
    base = O.dense_attention(Q, K, V, False)
    Qp, Kp, Vp = (O.permute_tokens(x, perm) for x in (Q, K, V))
    back = O.unpermute_tokens(O.dense_attention(Qp, Kp, Vp, False), perm)
    assert np.max(np.abs(back - base)) < 1e-12


# ---------------------------------------------------------------------------
# relative L1 metric
# ---------------------------------------------------------------------------

def test_rel_l1():
    a = np.array([1.0, -2.0, 3.0])
    assert O.rel_l1(a, a) == 0.0
    assert abs(O.rel_l1(a, a * 1.1) - 0.1) < 1e-15


def test_gqa_grouping_is_contiguous():
    """Query heads 2g, 2g+1 share kv head g: same as repeating each kv head."""
    N, d = 200, 64
    Q, K, V = _rand((1, 4, N, d), 40), _rand((1, 2, N, d), 41), _rand((1, 2, N, d), 42)
    Krep, Vrep = np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1)
    for causal in (False, True):
        a = O.dense_attention(Q, K, V, causal)
        b = O.dense_attention(Q, Krep, Vrep, causal)
        assert np.max(np.abs(a - b)) == 0.0
        mg = np.ones((1, 4, 2, 4), dtype=bool)
        s, _, _ = O.sparse_attention(Q, K, V, mg, -np.inf, causal)
        assert np.max(np.abs(s - b)) < 1e-10
    pa = O.predict_mask(Q, K, 0.7, 0.0, True)
    pb = O.predict_mask(Q, Krep, 0.7, 0.0, True)
    assert np.array_equal(pa["mg"], pb["mg"])


# ---------------------------------------------------------------------------
# token orders and block self-similarity of the permutation comparison
# ([Review] Table 4)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("grid", [(1, 4, 6), (5, 1, 1), (3, 4, 5), (12, 6, 10)])
def test_time_major_order_closed_form(grid):
    T, Hg, Wg = grid
    perm = O.time_major_order(T, Hg, Wg)
    assert np.array_equal(np.sort(perm), np.arange(T * Hg * Wg))
    p = np.arange(perm.size)
    # run r = p // T is pixel (h, w) = divmod(r, Wg); inside it t = p % T
    t, pix = perm // (Hg * Wg), perm % (Hg * Wg)
    assert np.array_equal(t, p % T)
    assert np.array_equal(pix, p // T)
    if T == 1 or Hg * Wg == 1:
        assert np.array_equal(perm, O.raster_order(T, Hg, Wg))


def test_block_self_similarity_closed_forms():
    d, b = 16, 8
    same = np.tile(np.arange(1.0, d + 1.0), (2 * b, 1))
    assert abs(O.block_self_similarity(same, b) - 1.0) < 1e-15
    ortho = np.vstack([np.eye(d)[:b], np.eye(d)[:b]])
    # each block: cosine matrix = identity, mean 1/b
    assert abs(O.block_self_similarity(ortho, b) - 1.0 / b) < 1e-15
    # a ragged last block of 3 identical tokens averages in as 1
    X = np.vstack([np.eye(d)[:b], np.ones((3, d))])
    assert abs(O.block_self_similarity(X, b) - 0.5 * (1.0 / b + 1.0)) < 1e-15


# ---------------------------------------------------------------------------
# fp8 (E4M3) rounding and the fp8 P~V variant
# ---------------------------------------------------------------------------

def _e4m3_from_bits(code):
    """Value of an E4M3 code from its definition: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    return s * (m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))


def test_e4m3_round_fixes_every_finite_code_and_saturates():
    vals = np.array([v for v in (_e4m3_from_bits(c) for c in range(256)) if v is not None])
    assert vals.size == 254 and vals.max() == 448.0 and vals.min() == -448.0
    assert np.array_equal(O.e4m3_round(vals), vals)
    assert np.array_equal(O.e4m3_round(np.array([450.0, 463.9, 1e9, -1e9])), [448.0, 448.0, 448.0, -448.0])


def test_e4m3_round_is_nearest_with_ties_to_even():
    pos = np.unique(np.array([v for v in (_e4m3_from_bits(c) for c in range(128)) if v is not None]))
    mids = (pos[:-1] + pos[1:]) / 2
    got = O.e4m3_round(mids)
    # a midpoint goes to the neighbour whose mantissa is even
    for lo, hi, g in zip(pos[:-1], pos[1:], got):
        code_lo = [c for c in range(128) if _e4m3_from_bits(c) == lo][0]
        assert g == (lo if code_lo % 2 == 0 else hi), (lo, hi, g)
    rng = np.random.default_rng(3)
    x = rng.uniform(-448, 448, 5000)
    r = O.e4m3_round(x)
    # nearest: no representable value is strictly closer
    d = np.abs(x[:, None] - np.concatenate([pos, -pos])[None, :]).min(axis=1)
    assert np.allclose(np.abs(x - r), d, rtol=0, atol=1e-12)
    # closed form on [1, 2): steps of 1/8
    y = rng.uniform(1, 2, 1000)
    assert np.array_equal(O.e4m3_round(y), np.rint(8 * y) / 8)


def test_v_channel_scales_are_the_least_power_of_two():
    rng = np.random.default_rng(4)
    V = rng.standard_normal((50, 8)) * (10.0 ** rng.uniform(-3, 4, 8))
    V[:, 3] = 0.0
    V[0, 5] = 448.0 * 4          # exactly at a power of two
    V[:, 5] = np.clip(V[:, 5], -448.0 * 4, 448.0 * 4)
    dl = O.v_channel_scales(V)
    mx = np.abs(V).max(axis=0)
    assert np.all(np.log2(dl) == np.round(np.log2(dl)))
    assert dl[3] == 1.0 and dl[5] == 4.0
    nz = mx > 0
    assert np.all(mx[nz] <= 448.0 * dl[nz]) and np.all(mx[nz] > 224.0 * dl[nz])


def test_fp8pv_equals_exact_attention_when_nothing_rounds():
    """One-hot attention (each row sees one key far above the rest) and V on
    the E4M3 grid: the fp8 variant's roundings change nothing."""
    N, d = 128, 64
    rng = np.random.default_rng(6)
    Kh = rng.standard_normal((N, d)) * 0.01
    Qh = np.zeros((N, d))
    Qh[:, 0] = 1.0
    Kh[:, 0] = -200.0
    Kh[np.arange(0, N, 7), 0] = 200.0                # the keys every row attends to (S = +-25)
    Vh = O.e4m3_round(rng.uniform(-300, 300, (N, d)))
    Vh[0, :] = 448.0                                 # delta = 1 in every channel
    mg = np.ones((1, 1, 1, 2), dtype=bool)
    Q, K, V = Qh[None, None], Kh[None, None], Vh[None, None]
    exact, _, dec = O.sparse_attention(Q, K, V, mg, -np.inf, False)
    o8 = O.sparse_attention(Q, K, V, mg, -np.inf, False, pv8=True)[0][0, 0]
    # 19 attended keys per row with equal weight 1/19: P~ = 1 exactly at the
    # running max (25 from the first tile on), and the others underflow to 0
    # after scaling
    assert np.max(np.abs(o8 - exact[0, 0])) < 1e-12


def test_fp8pv_error_within_the_rounding_bound():
    N, d = 256, 64
    rng = np.random.default_rng(7)
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    V[..., 5] *= 1000.0
    mg = np.ones((1, 1, 2, 4), dtype=bool)
    for causal in (False, True):
        exact, _, dec = O.sparse_attention(Q, K, V, mg, -np.inf, causal)
        o8 = O.sparse_attention(Q, K, V, mg, -np.inf, causal, pv8=True)[0]
        # per element: |p^ - p| <= 2^-4 p + 2^-18 (P~ scaled by 2^8, step 2^-9
        # below 2^-6; in Algorithm 1's order p is rounded at the step's max
        # and then scaled down by the later rescalings, which only shrinks
        # both terms) and |v^ delta - v| <= 2^-4 |v| + 2^-10 delta
        S = Q[0, 0] @ K[0, 0].T / math.sqrt(d)
        if causal:
            S = np.where(np.triu(np.ones((N, N), dtype=bool), 1), -np.inf, S)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        l = P.sum(axis=1, keepdims=True)
        dl = O.v_channel_scales(V[0, 0])
        av = np.abs(V[0, 0])
        bound = ((2.0 ** -4 * P + 2.0 ** -18) @ (av * (1 + 2.0 ** -4) + 2.0 ** -10 * dl)
                 + P @ (2.0 ** -4 * av + 2.0 ** -10 * dl)) / l
        err = np.abs(o8[0, 0] - exact[0, 0])
        assert np.all(err <= bound + 1e-12), float(np.max(err - bound))
        assert O.rel_l1(exact, o8) < 0.05


def test_fp8pv_two_tile_worked_example():
    """tests/golden/fp8_two_tile.json: a row whose running max moves between
    its two tiles.  Algorithm 1's order rounds P~ = exp(S - m_ij) at each
    step's max, then rescales; the worked E4M3 roundings give O = (35/24,
    25/24) / l.  Rounding exp(S - m_final) instead (the two-pass order) gives
    (47/32, 17/16) / l: the orders round differently, and the oracle follows
    the pages'."""
    import json
    import os
    from fractions import Fraction
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_two_tile.json")))
    N, d = 128, 64
    S_row = np.full(N, -1000.0)
    S_row[0], S_row[1], S_row[64] = 0.0, -1.0, math.log(3.0)

    def score_fn(rows, keys):
        return np.tile(S_row[keys.start:keys.stop], (len(rows), 1))

    V = np.zeros((N, d))
    V[:, 0] = g["v_channel_0"]["all"]
    for key, val in g["v_channel_1"].items():
        V[int(key), 1] = val
    delta = O.v_channel_scales(V)
    assert delta[0] == 2.0 ** -8 and delta[1] == 2.0 ** -7 and delta[2] == 1.0
    V8 = O.e4m3_round(V / delta)
    assert np.array_equal(V8, V / delta)                 # exact on the grid
    # the worked roundings
    assert O.e4m3_round(256 * math.exp(-1.0)) == 96.0
    assert O.e4m3_round(256 / 3.0) == 88.0
    assert O.e4m3_round(256 * math.exp(-1.0) / 3.0) == 32.0
    dummy = np.zeros((N, d))
    out, cnt, dec = O.attend_row_block(dummy, dummy, V, np.array([True, True]), 0, -np.inf, False,
                                       score_fn=score_fn, pv8=(V8, delta))
    l = (1.0 + math.exp(-1.0)) / 3.0 + 1.0
    want = [float(Fraction(*g["running_max_numerators"][c])) / l for c in ("ch0", "ch1")]
    other = [float(Fraction(*g["final_max_numerators"][c])) / l for c in ("ch0", "ch1")]
    for r in range(N):
        assert abs(out[r, 0] - want[0]) < 1e-12 and abs(out[r, 1] - want[1]) < 1e-12
        assert np.all(out[r, 2:] == 0.0)
    assert min(abs(want[0] - other[0]), abs(want[1] - other[1])) > 5e-3
    assert cnt["pv_exec"] == 8 and np.all(dec == 1)
    # unquantised, channel 0 is exactly 1 (it averages ones)
    exact, _, _ = O.attend_row_block(dummy, dummy, V, np.array([True, True]), 0, -np.inf, False,
                                     score_fn=score_fn)
    assert np.allclose(exact[:, 0], 1.0, rtol=0, atol=1e-14)
    assert np.allclose(exact[:, 1], (2.0 / 3 - math.exp(-1.0) / 3 + 0.5) / l, rtol=0, atol=1e-14)


def test_fp8pv_keeps_the_lambda_decisions_and_counts():
    """The 8-bit operands enter only the P~V product: m, the votes, l and the
    counters are those of the unquantised recurrence."""
    rng = np.random.default_rng(9)
    N, d = 300, 64
    u = rng.standard_normal(d)
    Q = rng.standard_normal((1, 2, N, d)) + u
    K = rng.standard_normal((1, 1, N, d))
    K[0, 0, :64] += 2.0 * u                  # the first key tile dominates every row
    V = rng.standard_normal((1, 1, N, d))
    mg = rng.random((1, 2, 3, 5)) < 0.7
    for causal in (False, True):
        a, ca, da = O.sparse_attention(Q, K, V, mg, -0.5, causal)
        b, cb, db = O.sparse_attention(Q, K, V, mg, -0.5, causal, pv8=True)
        assert ca == cb and np.array_equal(da, db)
        assert ca["pv_skip"] > 0 and ca["pv_exec"] > 0
        assert 0 < O.rel_l1(a, b) < 0.05


# ---------------------------------------------------------------------------
# the TopCdf ambiguity window the GPU parity tests exclude
# ---------------------------------------------------------------------------
# Dyadic rows: every prefix sum is exact, so the distance of an exclusive
# prefix from tau * sum is the offset put into tau.  Each case lists, by
# hand, the entries that must be flagged (exclusive prefix within 1e-4 of
# tau * sum, or a relative near-tie within 1e-6 with the last kept entry
# shared by another entry).
AMBIGUITY_CASES = [
    # p = .5, .25, .125, .0625, .0625: exclusive prefixes 0, .5, .75, .875, .9375
    ("prefix .75 at tau*sum - 0.5e-4 (kept)", [.5, .25, .125, .0625, .0625], .75 + .5e-4, {2}, {0, 1, 2}),
    ("prefix .75 at tau*sum + 0.5e-4 (dropped)", [.5, .25, .125, .0625, .0625], .75 - .5e-4, {2}, {0, 1}),
    ("prefix .75 at tau*sum - 2e-4", [.5, .25, .125, .0625, .0625], .75 + 2e-4, set(), {0, 1, 2}),
    ("prefix .75 at tau*sum + 2e-4", [.5, .25, .125, .0625, .0625], .75 - 2e-4, set(), {0, 1}),
    # the two .0625 entries tie exactly and straddle the cut: 3 kept, 4 not
    ("exact tie across the cut", [.5, .25, .125, .0625, .0625], .9, {3, 4}, {0, 1, 2, 3}),
    # a near-tie (relative 2e-7) of the last kept entry and the first dropped one
    ("near-tie across the cut", [.5, .25, .125 * (1 + 1e-7), .125 * (1 - 1e-7)], .8, {2, 3}, {0, 1, 2}),
    # a near-tie well inside the kept set, not involving the last kept entry
    ("near-tie away from the cut", [.3 * (1 + 1e-7), .3 * (1 - 1e-7), .25, .15], .7, set(), {0, 1, 2}),
    # a near-tie of 2e-6 relative is not a tie
    ("no tie at 2e-6", [.5, .25, .125 * (1 + 2e-6), .125 * (1 - 2e-6)], .8, set(), {0, 1, 2}),
]


@pytest.mark.parametrize("label,p,tau,flagged,kept", AMBIGUITY_CASES, ids=[c[0] for c in AMBIGUITY_CASES])
def test_topcdf_ambiguity_marks_exactly_the_window(label, p, tau, flagged, kept):
    p = np.array(p)
    keep, info = O.topcdf(p, tau)
    assert set(np.nonzero(keep)[0]) == kept
    amb = O.topcdf_ambiguous(p, keep, info)
    assert set(np.nonzero(amb)[0]) == flagged


@pytest.mark.parametrize("label,p,tau,flagged,kept", AMBIGUITY_CASES, ids=[c[0] for c in AMBIGUITY_CASES])
def test_predict_mask_head_flags_the_same_entries(label, p, tau, flagged, kept):
    """The same rows end to end: query blocks whose mean is e_0 and key blocks
    whose mean is sqrt(d) ln(p_j) e_0 (every token of a block equal, so every
    block is selective) give the compressed row ln(p_j), whose softmax is p.
    predict_mask_head flags the same entries in every query block row."""
    p = np.array(p)
    d, n = 64, len(p)
    N = 64 * n
    Q = np.zeros((N, d))
    Q[:, 0] = 1.0
    K = np.zeros((N, d))
    for j in range(n):
        K[64 * j:64 * j + 64, 0] = math.sqrt(d) * math.log(p[j] / p.sum())
    r = O.predict_mask_head(Q, K, tau, 0.5, False)
    assert not r["fix_q"].any() and not r["fix_k"].any()
    for i in range(r["mg"].shape[0]):
        assert set(np.nonzero(r["mg"][i])[0]) == kept, i
        assert set(np.nonzero(r["ambiguous"][i])[0]) == flagged, i


# ---------------------------------------------------------------------------
# Monotone structure the definitions fix
# ---------------------------------------------------------------------------

def test_topcdf_keep_set_grows_with_tau():
    """[Review] eq. 8: TopCdf keeps the shortest prefix of the probabilities
    in descending order whose mass reaches tau of the row, so a larger tau
    keeps a prefix of the same order that is at least as long; the fix blocks
    of eq. 9 and the -inf key blocks of eq. 7 do not depend on tau.  M_g can
    only gain ones as tau grows (a reversed cut or comparison breaks this)."""
    Q = _rand((1, 2, 1100, 64), 41)
    K = _rand((1, 1, 1100, 64), 42)
    # smooth the tokens so that some blocks are self-similar and TopCdf acts
    Q += 2.0 * _rand((1, 2, 1, 64), 43)
    K += 2.0 * _rand((1, 1, 1, 64), 44)
    prev = None
    sizes = []
    for tau in (0.1, 0.3, 0.5, 0.7, 0.9, 0.99, 1.0):
        mg = O.predict_mask(Q, K, tau, 0.5, causal=True)["mg"]
        if prev is not None:
            assert not (prev & ~mg).any(), tau
        prev = mg
        sizes.append(int(mg.sum()))
    assert sizes[0] < sizes[-1], sizes


def test_lambda_decisions_nest_and_leave_the_row_sums_alone():
    """[Review] sparse warp online softmax: a group skips P~V on a tile when
    every row's tile maximum lies more than |lambda| below its running max.
    The running max and the row sum l never depend on lambda (P~ feeds l
    before the test), so lowering lambda can only turn skips into executions:
    the executed (tile, group) pairs nest, their total with the skipped ones
    stays fixed, and with V = 1 (every row of O is then l_exec / l) O grows
    toward 1 as lambda falls."""
    from free_block_sparse_mask_amd import inputs as I
    w = I.workload(2, N=700, H=1, H_kv=1)      # AR(1) tokens with sinks: skips at every lambda below
    q, k, _ = I.make_qkv(w)
    Q, K = (O.widen(x, w.dtype) for x in (q, k))
    V = np.ones((1, 1, w.N, w.d))
    mg = O.tile_live(w.N, O.BQ, O.BK, True)[None, None]
    prev_dec, prev_o, totals, execs = None, None, set(), []
    for lam in (-0.5, -1.0, -2.0, -4.0, -8.0, -16.0, -np.inf):
        o, cnt, dec = O.sparse_attention(Q, K, V, mg, lam, True)
        ran = dec == 1
        totals.add(cnt["pv_exec"] + cnt["pv_skip"])
        execs.append(cnt["pv_exec"])
        if prev_dec is not None:
            assert not (prev_dec & ~ran).any(), lam
            assert np.all(o >= prev_o - 1e-12), lam
        assert np.all(o <= 1.0 + 1e-12)
        prev_dec, prev_o = ran, o
    assert len(totals) == 1
    assert execs == sorted(execs) and execs[0] < execs[-1], execs
    assert np.allclose(prev_o, 1.0, atol=1e-12)
