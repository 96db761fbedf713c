"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the whole problem in one call per stage, bf16 or int8
inputs, the default workspace).

The oracle cannot redo a whole 128K problem in seconds, so these tests
compare what it can compute one by one: the mask rows of a few sampled query
heads (each head's stage 1 depends only on its own Q and its kv head's K),
and the output rows of a few sampled query blocks of those heads (stage 2 of
a block depends only on its row of M_g, its Q rows and its kv head's K, V),
with the same acceptance rules as the small parity tests.  Properties that
hold at any size are checked on the whole output: the counters against the
mask, finiteness, and the 16-bit output being the rounded float32 one.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from oracle import sparge_oracle as O

from gpu_common import DEV, attn_path, check_attention, check_mask, log

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _up(bits: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(DEV)


def _sample_blocks(Tm: int, n: int = 5):
    return sorted({0, 1, Tm // 2, Tm - 2, Tm - 1} if n >= 5 else {0, Tm - 1})


def _sub_mask(mask: fb.Mask, h: int, hk: int) -> fb.Mask:
    return fb.Mask(mask.mg[:, h:h + 1], mask.row_cnt[:, h:h + 1], mask.row_idx[:, h:h + 1],
                   mask.s_q[:, h:h + 1], mask.s_k[:, hk:hk + 1])


def _check_whole(w, mask, counts, o16, o32):
    """Properties of the whole output and counters."""
    c = fb.counts_dict(counts)
    Tm, Tn = O.num_blocks(w.N, O.BQ), O.num_blocks(w.N, O.BK)
    live = int(O.tile_live(w.N, O.BQ, O.BK, w.causal).sum()) * w.B * w.H
    assert c["live_tiles"] == live
    assert c["qk_exec"] == int(mask.mg.sum().item())
    assert c["qk_exec"] + c["qk_skip"] == c["live_tiles"]
    assert c["rows"] == w.B * w.H * w.N
    assert int(mask.row_cnt.sum().item()) == c["qk_exec"]
    assert bool(torch.isfinite(o32).all())
    assert torch.equal(o16, o32.to(o16.dtype))
    return c


def _run(w, q, k, v, int8=False, perm=None):
    qd, kd = _up(q, w.dtype), _up(k, w.dtype)
    vd = _up(v, "f16" if int8 else w.dtype)
    if perm is not None:
        qd, kd, vd = (fb.hilbert_permute(x, perm) for x in (qd, kd, vd))
    ws = fb.workspace(qd, kd)
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal, ws=ws)
    kw = {}
    qa, ka = qd, kd
    if int8:
        qa, ka, qs, ks = fb.quant_qk_int8(qd, kd, ws=ws)
        kw = dict(q_scale=qs, k_scale=ks)
    o16, counts, dbg = fb.attn(qa, ka, vd, mask, w.lam, w.causal, ws=ws, dbg=True, **kw)
    o32, counts32, _ = fb.attn(qa, ka, vd, mask, w.lam, w.causal, ws=ws, out_f32=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(counts, counts32)
    return mask, counts, dbg, o16, o32


def _random_blocks(w, n, seed, heads=None):
    """n distinct seeded-random (h, i) query blocks over ``heads`` (all by default)."""
    Tm = O.num_blocks(w.N, O.BQ)
    hs = list(range(w.H)) if heads is None else list(heads)
    rng = np.random.default_rng(seed)
    flat = rng.choice(len(hs) * Tm, size=min(n, len(hs) * Tm), replace=False)
    return [(hs[int(x) // Tm], int(x) % Tm) for x in flat]


def _check_heads(w, q, k, v, mask, dbg, o32, heads, int8=False, v_dtype=None, perm_np=None, o16=None,
                 extra_blocks=()):
    """Mask rows of every head in ``heads`` against the oracle, and the output
    of the fixed extreme blocks of those heads plus ``extra_blocks`` ((h, i)
    pairs on any head) given the GPU's mask."""
    group = w.H // w.H_kv
    Tm = O.num_blocks(w.N, O.BQ)
    blocks_of = {h: set(_sample_blocks(Tm)) for h in heads}
    for h, i in extra_blocks:
        blocks_of.setdefault(h, set()).add(i)
    n_blocks = 0
    for h in sorted(blocks_of):
        hk = h // group
        Qh = O.widen(q[:, h:h + 1], w.dtype)
        Kh = O.widen(k[:, hk:hk + 1], w.dtype)
        Vh = O.widen(v[:, hk:hk + 1], v_dtype or w.dtype)
        if perm_np is not None:
            Qh, Kh, Vh = (O.permute_tokens(x, perm_np) for x in (Qh, Kh, Vh))
        mtxt = ""
        if h in heads:
            rep = check_mask(_sub_mask(mask, h, hk), Qh, Kh, w.tau, w.theta, w.causal)
            mtxt = f"mask near_theta={rep['near_theta']} ambiguous={rep['ambiguous']} s_err={rep['max_s_err']:.1e}; "
        blocks = [(0, 0, i) for i in sorted(blocks_of[h])]
        n_blocks += len(blocks)
        # int8: the K mean is over all tokens of the kv head, which the slice holds whole
        quant = O.quantize_qk(Qh, Kh) if int8 else None
        # attention is compared given the mask the GPU used
        mg_h = mask.mg[:, h:h + 1].cpu().numpy().astype(bool)
        arep = check_attention(o32[:, h:h + 1], None, dbg[:, h:h + 1], Qh, Kh, Vh, mg_h, w.lam, w.causal,
                               "f32", blocks=blocks, quant=quant, int8=int8,
                               o16=None if o16 is None else o16[:, h:h + 1],
                               o16_dtype=v_dtype or w.dtype)
        log(f"   head {h}: {mtxt}blocks {[b[2] for b in blocks]}: max_abs={arep['max_abs']:.2e} "
            f"rel_l1={arep['rel_l1']:.2e} flips={arep['lambda_flips']}")
    log(f"   {len(heads)} heads' mask rows and {n_blocks} query blocks checked")


# 128K GQA: every query head of kv heads 0 and 7 for the mask rows, and 64
# seeded-random query blocks over all 32 heads beside the fixed extremes
GQA_MASK_HEADS = [0, 1, 2, 3, 28, 29, 30, 31]


@pytest.mark.parametrize("wid,heads,n_random", [(1, [0, 23], 16), (2, [0, 31], 32), (3, [0, 23], 16),
                                                (4, GQA_MASK_HEADS, 64)],
                         ids=["image_dit", "llm_32k", "video_dit_raster", "gqa_128k"])
def test_full_size_bf16(wid, heads, n_random):
    w = I.workload(wid)
    log(f"[full] {w.name}: B={w.B} H={w.H} Hkv={w.H_kv} N={w.N} d={w.d} causal={w.causal}")
    q, k, v = I.make_qkv(w, workers=16)
    mask, counts, dbg, o16, o32 = _run(w, q, k, v)
    c = _check_whole(w, mask, counts, o16, o32)
    log(f"   counts {c}")
    _check_heads(w, q, k, v, mask, dbg, o32, heads, o16=o16,
                 extra_blocks=_random_blocks(w, n_random, seed=100 + wid))


def test_full_size_video_hilbert():
    w = I.workload(3)
    T, Hg, Wg = w.grid
    log(f"[full] {w.name} in 3D Hilbert order: N={w.N} grid={w.grid}")
    q, k, v = I.make_qkv(w, workers=16)
    perm, _ = fb.hilbert_index(T, Hg, Wg)
    perm_np, _ = O.hilbert_permutation(T, Hg, Wg)
    assert np.array_equal(perm, perm_np)
    mask, counts, dbg, o16, o32 = _run(w, q, k, v, perm=torch.from_numpy(perm).to(DEV))
    c = _check_whole(w, mask, counts, o16, o32)
    log(f"   counts {c}")
    _check_heads(w, q, k, v, mask, dbg, o32, [0, 23], perm_np=perm_np, o16=o16,
                 extra_blocks=_random_blocks(w, 16, seed=131))


def test_full_size_gqa_int8():
    w = I.workload(4)
    log(f"[full] {w.name} int8 Q/K, fp16 P~V")
    q, k, _ = I.make_qkv(w, workers=16)
    v = I.make_tensor(w, I.TENSOR_V, dtype="f16", workers=16)
    mask, counts, dbg, o16, o32 = _run(w, q, k, v, int8=True)
    c = _check_whole(w, mask, counts, o16, o32)
    log(f"   counts {c}")
    _check_heads(w, q, k, v, mask, dbg, o32, [0, 31], int8=True, v_dtype="f16", o16=o16,
                 extra_blocks=_random_blocks(w, 32, seed=140))


def test_full_size_gqa_fp8pv():
    """The fp8 P~V variant at 128K GQA, in the bench's configuration: the
    fixed extreme blocks of two heads and 16 seeded-random blocks over all
    heads against the oracle's fp8 recurrence (Algorithm 1's order), with
    the acceptance of the small fp8 parity tests; whole-output properties
    on everything."""
    from gpu_common import check_fp8, fp8_room
    w = I.workload(4)
    log(f"[full] {w.name} fp8 P~V")
    q, k, v = I.make_qkv(w, workers=16)
    qd, kd, vd = _up(q, w.dtype), _up(k, w.dtype), _up(v, w.dtype)
    ws = fb.workspace(qd, kd)
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal, ws=ws)
    o16, counts, dbg = fb.attn(qd, kd, vd, mask, w.lam, w.causal, ws=ws, dbg=True, fp8_pv=True)
    o32, counts32, _ = fb.attn(qd, kd, vd, mask, w.lam, w.causal, ws=ws, out_f32=True, fp8_pv=True)
    torch.cuda.synchronize()
    assert torch.equal(counts, counts32)
    c = _check_whole(w, mask, counts, o16, o32)
    log(f"   counts {c}")
    group = w.H // w.H_kv
    Tm = O.num_blocks(w.N, O.BQ)
    blocks_of = {h: set(_sample_blocks(Tm)) for h in (0, 31)}
    for h, i in _random_blocks(w, 16, seed=160):
        blocks_of.setdefault(h, set()).add(i)
    for h in sorted(blocks_of):
        hk = h // group
        Qh = O.widen(q[:, h:h + 1], w.dtype)
        Kh = O.widen(k[:, hk:hk + 1], w.dtype)
        Vh = O.widen(v[:, hk:hk + 1], w.dtype)
        blocks = [(0, 0, i) for i in sorted(blocks_of[h])]
        mg_h = mask.mg[:, h:h + 1].cpu().numpy().astype(bool)
        gdec = dbg[:, h:h + 1].cpu().numpy().astype(np.int8)
        ref, _, _ = O.sparse_attention(Qh, Kh, Vh, mg_h, w.lam, w.causal, blocks=blocks, skip_override=gdec,
                                       pv8=True)
        room = fp8_room(Qh, Kh, Vh, mg_h, w.causal, gdec, blocks, ref=ref)
        og = o32[:, h:h + 1].cpu().double().numpy()
        sel = np.concatenate([np.arange(O.block_rows(w.N, O.BQ, i).start, O.block_rows(w.N, O.BQ, i).stop)
                              for _, _, i in blocks])
        rep = check_fp8(og, ref, room, rows=sel)
        log(f"   head {h}: blocks {[bl[2] for bl in blocks]}: rel_l1={rep['rel_l1']:.2e} cos={rep['cos']:.6f} "
            f"max_abs={rep['max_abs']:.2e}")


MAX_TN = 4096   # SPARGE_MAX_TN of include/sparge.h


@pytest.mark.parametrize("H,H_kv,causal,int8,fused", [(2, 1, True, False, False), (1, 1, False, False, False),
                                                    (2, 1, True, True, False), (2, 1, True, False, True),
                                                    (2, 1, True, True, True)],
                         ids=["causal_gqa", "noncausal", "causal_gqa_int8", "causal_gqa_fused",
                              "causal_gqa_int8_fused"])
def test_largest_supported_sequence(H, H_kv, causal, int8, fused):
    """N = 64 * SPARGE_MAX_TN = 262144, the longest sequence the library takes:
    Tn = 4096 key blocks, so the widest M_g rows and row lists, the largest
    LDS lists, vote arrays and (int8) K-scale arrays of both attention
    passes, and (causal) rows whose dense lists walk 4096 tiles; with the
    fused pass forced, its packs of two dense blocks of one kv head on those
    rows.  The llm_32k recipe at that length; mask rows of every head and
    sampled query blocks against the oracle."""
    from gpu_common import attn_path
    w = I.workload(2, N=64 * MAX_TN, H=H, H_kv=H_kv, causal=causal)
    assert O.num_blocks(w.N, O.BK) == MAX_TN
    log(f"[full] largest N: H={w.H} Hkv={w.H_kv} N={w.N} causal={w.causal} int8={int8} fused={fused}")
    q, k, v = I.make_qkv(w, workers=16)
    if int8:
        v = I.make_tensor(w, I.TENSOR_V, dtype="f16", workers=16)
    with attn_path(fb.PATH_FUSED if fused else fb.PATH_AUTO):
        mask, counts, dbg, o16, o32 = _run(w, q, k, v, int8=int8)
    c = _check_whole(w, mask, counts, o16, o32)
    log(f"   counts {c}")
    _check_heads(w, q, k, v, mask, dbg, o32, list(range(w.H)), int8=int8, v_dtype="f16" if int8 else None,
                 o16=o16, extra_blocks=_random_blocks(w, 8, seed=150 + w.H + (7 if int8 else 0) + (3 if fused else 0)))


def test_full_size_llm_32k_fused_path():
    """The fused stage-2 path on the llm_32k workload (causal, 32 heads,
    lists up to 512 tiles; the automatic choice takes it there too):
    sampled mask rows and blocks against the oracle, whole-output
    properties, and the same counters and decisions as the two-pass path."""
    from gpu_common import attn_path
    w = I.workload(2)
    log(f"[full] {w.name} on the fused path")
    q, k, v = I.make_qkv(w, workers=16)
    with attn_path(fb.PATH_FUSED):
        mask, counts, dbg, o16, o32 = _run(w, q, k, v)
    with attn_path(fb.PATH_TWO_PASS):
        _, counts2, dbg2, _, _ = _run(w, q, k, v)
    assert torch.equal(counts, counts2) and torch.equal(dbg, dbg2)
    c = _check_whole(w, mask, counts, o16, o32)
    log(f"   counts {c}")
    _check_heads(w, q, k, v, mask, dbg, o32, [0, 31], o16=o16, extra_blocks=_random_blocks(w, 24, seed=170))


def test_full_size_mask_and_decisions_are_monotone():
    """At 128K GQA, over every head, tile and wavefront (where the oracle
    cannot follow): eq. 8 keeps a longer prefix of one order as tau grows and
    eqs. 7 and 9 do not depend on tau, so M_g at tau 0.8 lies inside M_g at
    0.9; the running max and the row sums do not depend on lambda, so on one
    mask the (tile, wavefront) pairs that run P~V at lambda -4 lie inside
    those at -6, which lie inside those at -8, executed plus skipped stays
    fixed, and the fused pass takes the same decisions as the two passes."""
    w = I.workload(4)
    q, k, v = I.make_qkv(w)
    qd, kd, vd = _up(q, w.dtype), _up(k, w.dtype), _up(v, w.dtype)
    ws = fb.workspace(qd, kd)
    log(f"[monotone] {w.name}: tau 0.8 / 0.9, lambda -4 / -6 / -8")
    mg_lo = fb.predict_mask(qd, kd, 0.8, w.theta, w.causal, ws=ws).mg.clone()
    mask = fb.predict_mask(qd, kd, 0.9, w.theta, w.causal, ws=ws)
    torch.cuda.synchronize()
    assert not bool((mg_lo.bool() & ~mask.mg.bool()).any())
    n_lo, n_hi = int(mg_lo.sum().item()), int(mask.mg.sum().item())
    assert n_lo < n_hi
    prev, totals = None, set()
    for lam in (-4.0, -6.0, -8.0):
        with attn_path(fb.PATH_TWO_PASS):
            _, counts, dbg = fb.attn(qd, kd, vd, mask, lam, w.causal, ws=ws, dbg=True)
        torch.cuda.synchronize()
        ran = dbg == 1
        c = fb.counts_dict(counts)
        totals.add(c["pv_exec"] + c["pv_skip"])
        log(f"   lambda {lam}: pv_exec {c['pv_exec']} pv_skip {c['pv_skip']}")
        if prev is not None:
            assert not bool((prev & ~ran).any()), lam
        prev = ran
        if lam == -6.0:
            dbg6, counts6 = dbg, counts
    assert len(totals) == 1
    with attn_path(fb.PATH_FUSED):
        _, counts_f, dbg_f = fb.attn(qd, kd, vd, mask, -6.0, w.causal, ws=ws, dbg=True)
    torch.cuda.synchronize()
    assert torch.equal(dbg_f, dbg6) and torch.equal(counts_f, counts6)
    log(f"   M_g ones: {n_lo} at tau 0.8, {n_hi} at 0.9; fused decisions equal at lambda -6")


def test_full_size_rows_normalise():
    """With V = 1 every output element is the share of its row's softmax
    weight that ran P~V (eq. 1 divides by the row sum of all visited
    weights).  At lambda = -inf every listed tile runs, so each of the 4.2 M
    rows at 128K GQA gives 1 up to the rounding of P~ to bf16 (each weight
    within 2^-8 of itself, the row's largest, exp(0) = 1 at its tile,
    exactly; 1e-5 more for float32 sums and rescales), and exactly the empty
    rows give 0; at lambda -6 no element exceeds that bound above 1.  On
    both stage-2 paths."""
    w = I.workload(4)
    q, k, _ = I.make_qkv(w)
    qd, kd = _up(q, w.dtype), _up(k, w.dtype)
    vd = torch.ones((w.B, w.H_kv, w.N, w.d), dtype=torch.bfloat16, device=DEV)
    ws = fb.workspace(qd, kd)
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal, ws=ws)
    for path, pname in ((fb.PATH_TWO_PASS, "two_pass"), (fb.PATH_FUSED, "fused")):
        with attn_path(path):
            o_all, c_all, _ = fb.attn(qd, kd, vd, mask, -np.inf, w.causal, ws=ws, out_f32=True)
            o_lam, _, _ = fb.attn(qd, kd, vd, mask, w.lam, w.causal, ws=ws, out_f32=True)
        torch.cuda.synchronize()
        c = fb.counts_dict(c_all)
        empty = (o_all == 0).all(dim=-1)
        assert int(empty.sum().item()) == c["empty_rows"], (int(empty.sum().item()), c)
        dev = float((o_all[~empty] - 1.0).abs().max().item())
        top = float(o_lam.max().item())
        lo = float(o_lam.min().item())
        log(f"[normalise] {pname}: empty rows {c['empty_rows']}, max |O - 1| {dev:.2e} at lambda -inf; "
            f"O in [{lo:.3g}, {top:.6f}] at lambda {w.lam}")
        assert dev <= 2.0 ** -8 + 1e-5
        assert lo >= 0.0 and top <= 1.0 + 2.0 ** -8 + 1e-5
