"""GPU parity of every hot-path kernel against the float64 oracle, on inputs
the oracle finishes in seconds that still span several tiles and ragged tails.

Every call goes through the C ABI (libsparge.so) via the ctypes binding.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from oracle import sparge_oracle as O

from gpu_common import (DEV, check_attention, check_mask, log, run_attn, to_bits, to_dev, widen_dev)

pytestmark = pytest.mark.gpu


def _case(wid, **over):
    w = I.workload(wid, **over)
    q, k, v = I.make_qkv(w)
    return w, q, k, v


# (label, workload id, size overrides) -- all cover several tiles and a ragged tail
CASES = [
    ("tiny_full", 0, {}),
    ("tiny_ragged", 0, {"N": 1000}),
    ("llm_gqa_ragged", 2, {"N": 1000, "H": 4, "H_kv": 2}),
    ("llm_small_causal", 2, {"N": 2048, "H": 2, "H_kv": 2}),
    ("image_small", 1, {"N": 64 + 24 * 24, "H": 2, "H_kv": 2, "grid": (24, 24), "text_tokens": 64}),
    ("video_small", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}),
]


@pytest.mark.parametrize("label,wid,over", CASES, ids=[c[0] for c in CASES])
def test_predict_mask_matches_oracle(label, wid, over):
    w, q, k, v = _case(wid, **over)
    log(f"[predict] {label}: B={w.B} H={w.H} Hkv={w.H_kv} N={w.N} d={w.d} causal={w.causal}")
    qd, kd = to_dev(q, w.dtype), to_dev(k, w.dtype)
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    torch.cuda.synchronize()
    Q, K = O.widen(q, w.dtype), O.widen(k, w.dtype)
    rep = check_mask(mask, Q, K, w.tau, w.theta, w.causal)
    log(f"   near_theta={rep['near_theta']} ambiguous={rep['ambiguous']} s_err={rep['max_s_err']:.2e}")


@pytest.mark.parametrize("tau", [1.0, float(np.nextafter(1.0, 0.0)), 0.999])
@pytest.mark.parametrize("label,wid,over", [CASES[0], CASES[3]], ids=[CASES[0][0], CASES[3][0]])
def test_predict_mask_at_tau_near_one(label, wid, over, tau):
    """tau = 1 (the dense end of the hyper-parameter search) and the doubles
    just below it: the TopCdf threshold is ceil(tau * sum) in fixed point,
    at most the sum, so the radix select always finds its boundary.  At
    tau = 1 a selective row keeps every column whose probability reaches
    2^-61 (its fixed-point value is then non-zero)."""
    w, q, k, v = _case(wid, **over)
    log(f"[predict tau] {label}: tau={tau!r} N={w.N} causal={w.causal}")
    qd, kd = to_dev(q, w.dtype), to_dev(k, w.dtype)
    mask = fb.predict_mask(qd, kd, tau, w.theta, w.causal)
    torch.cuda.synchronize()
    Q, K = O.widen(q, w.dtype), O.widen(k, w.dtype)
    rep = check_mask(mask, Q, K, tau, w.theta, w.causal)
    log(f"   near_theta={rep['near_theta']} ambiguous={rep['ambiguous']}")
    if tau == 1.0:
        mg = mask.mg.cpu().numpy().astype(bool)
        kept_small = 0
        for b in range(w.B):
            for h in range(w.H):
                r = O.predict_mask_head(Q[b, h], K[b, O.kv_head(h, w.H, w.H_kv)], tau, w.theta, w.causal)
                for i in np.nonzero(~r["fix_q"])[0]:
                    z = r["shat"][i]
                    fin = np.isfinite(z)
                    if not fin.any():
                        continue
                    p = np.zeros_like(z)
                    p[fin] = np.exp(z[fin] - z[fin].max())
                    p /= p.sum()
                    big = p >= 2.0 ** -61
                    assert np.all(mg[b, h, i][big]), (b, h, i)
                    kept_small += int(np.sum(big & (p < 1e-6)))
        log(f"   every column with p >= 2^-61 kept ({kept_small} of them below 1e-6)")


@pytest.mark.parametrize("tau,theta", [(1e-9, 0.0), (1e-9, 2.0), (0.5, 0.0), (0.5, -1.0)],
                         ids=["tau0_no_fix", "tau0_all_fix", "half_no_fix", "half_theta_negative"])
@pytest.mark.parametrize("label,wid,over", [CASES[2], CASES[5]], ids=[CASES[2][0], CASES[5][0]])
def test_predict_mask_at_extreme_tau_and_theta(label, wid, over, tau, theta):
    """The ends of the hyper-parameters: tau -> 0+ keeps only each selective
    row's largest probability (its exclusive prefix 0 is below any positive
    tau * sum; ties go to the lower j); theta <= 0 leaves no fix block (a
    self-similarity is never negative) so TopCdf alone decides; theta > 1
    makes every block fix, so M_g is the live tiles."""
    w, q, k, v = _case(wid, **over)
    log(f"[predict ends] {label}: tau={tau} theta={theta} N={w.N} causal={w.causal}")
    qd, kd = to_dev(q, w.dtype), to_dev(k, w.dtype)
    mask = fb.predict_mask(qd, kd, tau, theta, w.causal)
    torch.cuda.synchronize()
    Q, K = O.widen(q, w.dtype), O.widen(k, w.dtype)
    rep = check_mask(mask, Q, K, tau, theta, w.causal)
    mg = mask.mg.cpu().numpy().astype(bool)
    live = O.tile_live(w.N, O.BQ, O.BK, w.causal)
    if theta > 1.0:
        assert np.array_equal(mg, np.broadcast_to(live, mg.shape))
    elif tau < 1e-6:
        # one block per row: the row's largest probability (no fix block forces
        # more).  The ambiguity window marks exactly that entry (its exclusive
        # prefix 0 lies within 1e-4 of tau * sum), so compare it directly: both
        # sides rank the same float64 map, and no other entry lies near a tie.
        assert np.all(mg.sum(axis=-1) == 1)
        assert rep["ambiguous"] == mg.shape[0] * mg.shape[1] * mg.shape[2]
        assert np.array_equal(mg, rep["ref_mg"])
    log(f"   ones per row {mg.sum(axis=-1).mean():.2f}; ambiguous={rep['ambiguous']}")


@pytest.mark.parametrize("label,wid,over", CASES, ids=[c[0] for c in CASES])
def test_attention_given_oracle_mask(label, wid, over):
    w, q, k, v = _case(wid, **over)
    log(f"[attn] {label}: B={w.B} H={w.H} Hkv={w.H_kv} N={w.N} d={w.d} causal={w.causal} lam={w.lam}")
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    ref = O.predict_mask(Q, K, w.tau, w.theta, w.causal)
    mg = torch.from_numpy(ref["mg"].astype(np.uint8)).to(DEV)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    o, o32, counts, dbg = run_attn(qd, kd, vd, mg, w.lam, w.causal)
    rep = check_attention(o32, counts, dbg, Q, K, V, ref["mg"], w.lam, w.causal, "f32", o16=o, o16_dtype=w.dtype)
    log(f"   max_abs={rep['max_abs']:.2e} rel_l1={rep['rel_l1']:.2e} flips={rep['lambda_flips']} "
        f"counts={rep['counts']}")


@pytest.mark.parametrize("dtype,d,causal", [("f16", 128, False), ("bf16", 64, True), ("bf16", 128, True),
                                            ("f16", 64, False)])
def test_attention_random_mask_edge_rows(dtype, d, causal):
    """A random mask with empty block rows, lambda strong enough to skip, and a
    ragged N; also lambda = -inf (plain block-sparse attention)."""
    N, H, Hkv = 777, 3, 1
    rng = np.random.default_rng(5)
    Qf = rng.standard_normal((1, H, N, d)) * 2.0
    Kf = rng.standard_normal((1, Hkv, N, d)) * 2.0
    Kf[0, 0, :64] += 3.0 * Qf[0, 0, :64].mean(axis=0)        # a dominant early block
    Vf = rng.standard_normal((1, Hkv, N, d))
    q, k, v = (I.to_bits(x, dtype) for x in (Qf, Kf, Vf))
    Q, K, V = (O.widen(x, dtype) for x in (q, k, v))
    Tm, Tn = O.num_blocks(N, 128), O.num_blocks(N, 64)
    mg_np = rng.random((1, H, Tm, Tn)) < 0.6
    mg_np[0, 0, 2] = False                                     # an empty row block
    mg_np[0, 1, :, 0] = True
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    mg = torch.from_numpy(mg_np.astype(np.uint8)).to(DEV)
    for lam in (-2.0, -math.inf):
        log(f"[attn-random] dtype={dtype} d={d} causal={causal} lam={lam}")
        o, o32, counts, dbg = run_attn(qd, kd, vd, mg, lam, causal)
        rep = check_attention(o32, counts, dbg, Q, K, V, mg_np, lam, causal, "f32", o16=o, o16_dtype=dtype)
        log(f"   max_abs={rep['max_abs']:.2e} rel_l1={rep['rel_l1']:.2e} counts={rep['counts']}")
        assert rep["counts"]["empty_rows"] >= 128
        if lam == -2.0:
            assert rep["counts"]["pv_skip"] > 0


@pytest.mark.parametrize("causal", [True, False])
def test_attention_dense_rows_in_packs(causal):
    """Query blocks that list every live tile share a pass-1 workgroup with
    another block of their kv head.  Two batches, two kv heads of two query
    heads each, and a ragged N.  The dense blocks per kv head number 7, 6, 5
    and 9, so three kv heads end on a pair with an empty slot.  Their i differ, so lists of different
    lengths share one K stream.  The remaining blocks are random and include
    an empty one."""
    B, H, Hkv, N, d = 2, 4, 2, 1100, 64
    rng = np.random.default_rng(17)
    Qf = rng.standard_normal((B, H, N, d)) * 1.5
    Kf = rng.standard_normal((B, Hkv, N, d)) * 1.5
    Vf = rng.standard_normal((B, Hkv, N, d))
    q, k, v = (I.to_bits(x, "bf16") for x in (Qf, Kf, Vf))
    Q, K, V = (O.widen(x, "bf16") for x in (q, k, v))
    Tm, Tn = O.num_blocks(N, 128), O.num_blocks(N, 64)
    live = O.tile_live(N, 128, 64, causal)
    mg_np = (rng.random((B, H, Tm, Tn)) < 0.5) & live
    n_dense = {(0, 0): 7, (0, 1): 6, (1, 0): 5, (1, 1): 9}
    empty = (1, 3, 1)
    chosen = set()
    for (b, hk), n in n_dense.items():
        cand = [(b, h, i) for h in (2 * hk, 2 * hk + 1) for i in range(Tm) if (b, h, i) != empty]
        chosen.update(cand[x] for x in rng.choice(len(cand), size=n, replace=False))
    for b in range(B):
        for h in range(H):
            for i in range(Tm):
                if (b, h, i) in chosen:
                    mg_np[b, h, i] = live[i]
                elif mg_np[b, h, i].sum() == live[i].sum():
                    mg_np[b, h, i, 0] = False           # only the chosen blocks are dense
    mg_np[empty] = False
    dense_rows = sum(int(mg_np[b, h, i].sum() == live[i].sum()) for b in range(B) for h in range(H)
                     for i in range(Tm))
    assert dense_rows == sum(n_dense.values())
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    mg = torch.from_numpy(mg_np.astype(np.uint8)).to(DEV)
    for lam in (-3.0, -math.inf):
        log(f"[attn-packs] causal={causal} lam={lam} dense blocks={dense_rows}")
        o, o32, counts, dbg = run_attn(qd, kd, vd, mg, lam, causal)
        rep = check_attention(o32, counts, dbg, Q, K, V, mg_np, lam, causal, "f32", o16=o, o16_dtype="bf16")
        log(f"   max_abs={rep['max_abs']:.2e} rel_l1={rep['rel_l1']:.2e} counts={rep['counts']}")


@pytest.mark.parametrize("N", [1, 17, 64, 65, 127, 129])
@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_short_sequences_whole_path(N, d, causal):
    """Sequences of one token up to just past one query block: a single
    ragged key tile, wavefronts whose 32 rows all lie beyond N, one-entry
    softmax rows in stage 1, and dense blocks paired with padding.  Three
    query heads on one kv head; stage 1 and stage 2 against the oracle on
    every block."""
    H, Hkv = 3, 1
    rng = np.random.default_rng(1000 + N + d)
    Qf = rng.standard_normal((1, H, N, d))
    Kf = rng.standard_normal((1, Hkv, N, d))
    Vf = rng.standard_normal((1, Hkv, N, d))
    # one self-similar query head (selective blocks) and self-similar keys (no
    # forced columns); the other heads' blocks are fix, so dense
    Qf[0, 1] = Qf[0, 1, :1] + 0.05 * Qf[0, 1]
    Kf[0, 0] = Kf[0, 0, :1] + 0.05 * Kf[0, 0]
    q, k, v = (I.to_bits(x, "bf16") for x in (Qf, Kf, Vf))
    Q, K, V = (O.widen(x, "bf16") for x in (q, k, v))
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    tau, theta, lam = 0.1, 0.9, -1.0
    log(f"[short] N={N} d={d} causal={causal}")
    mask = fb.predict_mask(qd, kd, tau, theta, causal)
    torch.cuda.synchronize()
    rep = check_mask(mask, Q, K, tau, theta, causal)
    mg_np = mask.mg.cpu().numpy().astype(bool)
    o, o32, counts, dbg = run_attn(qd, kd, vd, mask.mg, lam, causal)
    arep = check_attention(o32, counts, dbg, Q, K, V, mg_np, lam, causal, "f32", o16=o, o16_dtype="bf16")
    log(f"   mask ambiguous={rep['ambiguous']}; max_abs={arep['max_abs']:.2e} counts={arep['counts']}")
    assert arep["counts"]["rows"] == H * N
    if O.num_blocks(N, 64) >= 2:
        assert arep["counts"]["qk_skip"] > 0            # the selective head keeps only its top tile


@pytest.mark.parametrize("causal", [True, False])
def test_strided_layouts_and_batches(causal):
    """Q, K, V and O in the [B, N, H, d] layout (token stride H*d, head stride
    d), two batches, GQA and a ragged N: both stages give the same bits as on
    contiguous [B, H, N, d] copies, and match the oracle."""
    w = I.workload(2, N=700, H=4, H_kv=2, B=2, causal=causal)
    q, k, v = I.make_qkv(w)
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))

    def bshd(x):       # the same values with the strides of a [B, N, H, d] tensor
        return x.transpose(1, 2).contiguous().transpose(1, 2)

    qs, ks, vs = bshd(qd), bshd(kd), bshd(vd)
    assert qs.stride(2) == w.H * w.d and ks.stride(1) == w.d
    log(f"[strided] B={w.B} H={w.H} Hkv={w.H_kv} N={w.N} causal={causal}")
    m1 = fb.predict_mask(qd, kd, w.tau, w.theta, causal)
    m2 = fb.predict_mask(qs, ks, w.tau, w.theta, causal)
    torch.cuda.synchronize()
    assert torch.equal(m1.mg, m2.mg) and torch.equal(m1.row_cnt, m2.row_cnt)
    assert torch.equal(m1.s_q, m2.s_q) and torch.equal(m1.s_k, m2.s_k)
    cnt = m1.row_cnt.cpu().numpy()
    valid = np.arange(m1.row_idx.shape[-1]) < cnt[..., None]
    assert np.array_equal(m1.row_idx.cpu().numpy()[valid], m2.row_idx.cpu().numpy()[valid])
    o1, c1, _ = fb.attn(qd, kd, vd, m1, w.lam, causal)
    out = torch.empty(w.B, w.N, w.H, w.d, dtype=vd.dtype, device=DEV).transpose(1, 2)
    o2, c2, _ = fb.attn(qs, ks, vs, m2, w.lam, causal, out=out)
    torch.cuda.synchronize()
    assert o2.data_ptr() == out.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(c1, c2)
    # int8 quantisation reads the same strides
    a8 = fb.quant_qk_int8(qd, kd)
    b8 = fb.quant_qk_int8(qs, ks)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a8, b8))
    rep = check_mask(m2, Q, K, w.tau, w.theta, causal)
    o, o32, counts, dbg = run_attn(qs, ks, vs, m2, w.lam, causal)
    arep = check_attention(o32, counts, dbg, Q, K, V, m2.mg.cpu().numpy().astype(bool), w.lam, causal, "f32",
                           o16=o, o16_dtype=w.dtype)
    log(f"   mask ambiguous={rep['ambiguous']}; max_abs={arep['max_abs']:.2e} rel_l1={arep['rel_l1']:.2e} "
        f"counts={arep['counts']}")


def test_repeat_calls_bit_identical():
    """Pass 1 hands its pairs of dense blocks out from atomic per-kv-head
    queues, so which workgroup runs which pair changes from call to call;
    every block's result must not.  The llm_32k recipe at N = 16384 with
    GQA, where pairs carry most tiles: three calls, each with a workspace of
    its own, give the same O, counters and decision map bit for bit.  Stage
    1 likewise: its only atomics are integer histogram counts and
    fixed-point sums, so three predictions agree in every output."""
    w, q, k, v = _case(2, N=16384, H=8, H_kv=2)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    masks = [fb.predict_mask(qd, kd, w.tau, w.theta, w.causal, ws=torch.empty_like(fb.workspace(qd, kd)))
             for _ in range(3)]
    torch.cuda.synchronize()
    mask = masks[0]
    # a row list holds row_cnt entries; the rest of its storage is unwritten
    listed = torch.arange(mask.row_idx.shape[-1], device=qd.device) < mask.row_cnt[..., None].long()
    for m in masks[1:]:
        for f in ("mg", "row_cnt", "s_q", "s_k"):
            assert torch.equal(getattr(m, f), getattr(mask, f)), f
        assert torch.equal(m.row_idx[listed], mask.row_idx[listed])
    runs = []
    for r in range(3):
        ws = torch.empty_like(fb.workspace(qd, kd))
        runs.append(fb.attn(qd, kd, vd, mask, w.lam, w.causal, dbg=True, ws=ws))
    torch.cuda.synchronize()
    o0, c0, d0 = runs[0]
    log(f"[repeat] counts {fb.counts_dict(c0)}")
    assert fb.counts_dict(c0)["qk_exec"] > 0
    for o, c, d in runs[1:]:
        assert torch.equal(o, o0) and torch.equal(c, c0) and torch.equal(d, d0)


def test_attention_with_predicted_lists_equals_mask_path():
    """The row lists written by predict_mask and the lists built from M_g give
    bit-identical outputs."""
    w, q, k, v = _case(2, N=1500, H=4, H_kv=2)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    o1, c1, _ = fb.attn(qd, kd, vd, mask, w.lam, w.causal)
    o2, c2, _ = fb.attn(qd, kd, vd, mask.mg, w.lam, w.causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(c1, c2)


def test_dense_limit_matches_brute_force():
    """theta > 1 and lambda = -inf: the whole GPU path is dense attention."""
    w, q, k, v = _case(2, N=900, H=2, H_kv=1)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    o, mask, counts = fb.sparge_attention(qd, kd, vd, 0.5, 2.0, -math.inf, True)
    torch.cuda.synchronize()
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    ref = O.dense_attention(Q, K, V, True)
    o32, _, _ = fb.attn(qd, kd, vd, mask, -math.inf, True, out_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o32.to(o.dtype))
    og = o32.cpu().double().numpy()
    assert np.max(np.abs(og - ref)) <= 1e-2 and O.rel_l1(ref, og) <= 5e-3
    c = fb.counts_dict(counts)
    assert c["qk_skip"] == 0 and c["pv_skip"] == 0


def test_quant_codes_match_oracle():
    for wid, over in ((4, {"N": 1100, "H": 4, "H_kv": 2}), (0, {"N": 700})):
        w, q, k, v = _case(wid, **over)
        log(f"[quant] wid={wid} N={w.N} H={w.H} Hkv={w.H_kv} d={w.d}")
        qd, kd = to_dev(q, w.dtype), to_dev(k, w.dtype)
        q8, k8, qs, ks = fb.quant_qk_int8(qd, kd)
        torch.cuda.synchronize()
        Q, K = O.widen(q, w.dtype), O.widen(k, w.dtype)
        ref = O.quantize_qk(Q, K)
        near_q = ref["q_tie_dist"] < 1e-6
        near_k = ref["k_tie_dist"] < 1e-6
        gq = q8.cpu().numpy().astype(np.float64)
        gk = k8.cpu().numpy().astype(np.float64)
        assert np.array_equal(gq[~near_q], ref["q_codes"][~near_q])
        assert np.array_equal(gk[~near_k], ref["k_codes"][~near_k])
        assert np.array_equal(qs.cpu().numpy(), ref["q_scale"].astype(np.float32))
        assert np.array_equal(ks.cpu().numpy(), ref["k_scale"].astype(np.float32))
        log(f"   near-tie codes: q={int(near_q.sum())} k={int(near_k.sum())}")


def test_quant_codes_at_rounding_ties():
    """An fp16 query block whose maximum is 60000 (delta = 60000 / 127) and
    whose other entries are the fp16 values nearest (k + 1/2) delta, k = -127
    .. 126: x / delta falls on or next to half-integers, and for some entries
    x * (1 / delta) rounds to a different integer than the quotient does.
    The codes must be those of the rounded quotient, entry for entry; no
    entry is excluded here."""
    d, N, m = 64, 128, 60000.0
    delta = m / 127.0
    near = ((np.arange(-127, 127) + 0.5) * delta).astype(np.float16).astype(np.float64)
    vals = np.resize(near, N * d)
    vals[0] = m
    Qf = vals.reshape(1, 1, N, d)
    qbits = Qf.astype(np.float16).view(np.uint16)
    assert np.array_equal(qbits.view(np.float16).astype(np.float64), Qf)   # exact in fp16
    # the case separates the two routes: a product alone would get some codes wrong
    assert np.any(np.rint(near * (1.0 / delta)) != np.rint(near / delta))
    kbits = np.random.default_rng(5).standard_normal((1, 1, N, d)).astype(np.float16).view(np.uint16)
    q8, k8, qs, ks = fb.quant_qk_int8(to_dev(qbits, "f16"), to_dev(kbits, "f16"))
    torch.cuda.synchronize()
    ref = O.quantize_qk(Qf, O.widen(kbits, "f16"))
    assert np.array_equal(q8.cpu().numpy().astype(np.float64), ref["q_codes"])
    assert np.array_equal(qs.cpu().numpy(), ref["q_scale"].astype(np.float32))
    log(f"[quant ties] {int(np.sum(ref['q_tie_dist'] < 1e-9))} entries within 1e-9 of a tie, codes equal")


@pytest.mark.parametrize("v_dtype,d,causal", [("f16", 128, True), ("bf16", 128, True), ("f16", 64, False),
                                               ("bf16", 64, True)])
def test_int8_attention_matches_oracle(v_dtype, d, causal):
    """int8 Q/K with fp16 or bf16 P~V (both pairs the ABI takes), d 64 and 128,
    causal and not."""
    w, q, k, _ = _case(4, N=1100, H=4, H_kv=2, d=d, causal=causal)
    v = I.make_tensor(w, I.TENSOR_V, dtype=v_dtype)
    log(f"[int8] V {v_dtype} d={d} causal={causal}")
    Q, K = O.widen(q, w.dtype), O.widen(k, w.dtype)
    V = O.widen(v, v_dtype)
    qd, kd = to_dev(q, w.dtype), to_dev(k, w.dtype)
    vd = to_dev(v, v_dtype)
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    q8, k8, qs, ks = fb.quant_qk_int8(qd, kd)
    o, o32, counts, dbg = run_attn(q8, k8, vd, mask, w.lam, w.causal, q_scale=qs, k_scale=ks)
    ref_mask = O.predict_mask(Q, K, w.tau, w.theta, w.causal)["mg"]
    assert np.array_equal(mask.mg.cpu().numpy().astype(bool), ref_mask)
    quant = O.quantize_qk(Q, K)
    rep = check_attention(o32, counts, dbg, Q, K, V, ref_mask, w.lam, w.causal, "f32", quant=quant, o16=o,
                          o16_dtype=v_dtype,
                          int8=True)
    log(f"[int8] rel_l1={rep['rel_l1']:.2e} cos={rep['cos']:.6f} max_abs={rep['max_abs']:.2e} "
        f"flips={rep['lambda_flips']}")
    # against the unquantised oracle the error is the quantisation error
    o_float, _, _ = O.sparse_attention(Q, K, V, ref_mask, w.lam, w.causal)
    og = O.widen(to_bits(o), v_dtype)
    log(f"   vs float path: rel_l1={O.rel_l1(o_float, og):.2e}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_hilbert_permute_roundtrip(dtype, d):
    T, Hg, Wg = 4, 16, 12
    N = T * Hg * Wg
    rng = np.random.default_rng(3)
    x = I.to_bits(rng.standard_normal((2, 3, N, d)), dtype)
    perm, inv = fb.hilbert_index(T, Hg, Wg)
    perm_d = torch.from_numpy(perm).to(DEV)
    xd = to_dev(x, dtype)
    y = fb.hilbert_permute(xd, perm_d)
    z = fb.hilbert_permute(y, perm_d, inverse=True)
    torch.cuda.synchronize()
    p_ref, _ = O.hilbert_permutation(T, Hg, Wg)
    assert np.array_equal(to_bits(y), O.permute_tokens(x, p_ref))
    assert np.array_equal(to_bits(z), x)
    # a strided (non-contiguous heads) input
    big = torch.zeros((2, 3, N, d + 8), dtype=xd.dtype, device=DEV)
    big[..., :d] = xd
    ys = fb.hilbert_permute(big[..., :d], perm_d)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(ys), O.permute_tokens(x, p_ref))


def test_hilbert_permute_skips_out_of_range_entries():
    """A malformed order (entries -1, N, N + 5 and 2^31 - 1) moves nothing for
    those entries: the gather leaves their rows of y as they were, the
    scatter writes nothing from them, and every other row moves as usual."""
    N, d, H = 300, 64, 2
    rng = np.random.default_rng(21)
    x = I.to_bits(rng.standard_normal((1, H, N, d)), "bf16")
    perm = rng.permutation(N).astype(np.int32)
    bad = np.array([0, 7, 150, N - 1])
    perm[bad] = np.array([-1, N, N + 5, 2**31 - 1], dtype=np.int32)
    ok = np.setdiff1d(np.arange(N), bad)
    xd = to_dev(x, "bf16")
    perm_d = torch.from_numpy(perm).to(DEV)
    sentinel = torch.full((1, H, N, d), 7.0, dtype=torch.bfloat16, device=DEV)
    y = fb.hilbert_permute(xd, perm_d, out=sentinel.clone())
    z = fb.hilbert_permute(xd, perm_d, inverse=True, out=sentinel.clone())
    torch.cuda.synchronize()
    yb, zb, sb = to_bits(y), to_bits(z), to_bits(sentinel)
    assert np.array_equal(yb[:, :, ok], x[:, :, perm[ok]])
    assert np.array_equal(yb[:, :, bad], sb[:, :, bad])
    written = perm[ok]
    assert np.array_equal(zb[:, :, written], x[:, :, ok])
    untouched = np.setdiff1d(np.arange(N), written)
    assert untouched.size == bad.size and np.array_equal(zb[:, :, untouched], sb[:, :, untouched])
    log(f"[permute bad entries] {bad.size} skipped, {ok.size} rows moved")


def test_video_pipeline_with_hilbert_order():
    """Gather -> predict -> attend -> scatter on the GPU vs the oracle doing the
    same steps with its own Hilbert order."""
    w, q, k, v = _case(3, N=4 * 16 * 12, H=2, H_kv=2, grid=(4, 16, 12))
    T, Hg, Wg = w.grid
    perm, _ = fb.hilbert_index(T, Hg, Wg)
    perm_d = torch.from_numpy(perm).to(DEV)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    o, mask, counts = fb.sparge_attention(qd, kd, vd, w.tau, w.theta, w.lam, w.causal, perm=perm_d)
    torch.cuda.synchronize()
    p_ref, _ = O.hilbert_permutation(T, Hg, Wg)
    Qp, Kp, Vp = (O.permute_tokens(O.widen(x, w.dtype), p_ref) for x in (q, k, v))
    rep = check_mask(mask, Qp, Kp, w.tau, w.theta, w.causal)
    o_ref, _, _ = O.sparse_attention(Qp, Kp, Vp, rep["ref_mg"], w.lam, w.causal)
    o_ref = O.unpermute_tokens(o_ref, p_ref)
    # the float32 result of the same attention, scattered back on the GPU
    qp, kp, vp = (fb.hilbert_permute(x, perm_d) for x in (qd, kd, vd))
    o32, _, _ = fb.attn(qp, kp, vp, mask, w.lam, w.causal, out_f32=True)
    o32 = fb.hilbert_permute(o32, perm_d, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o32.to(o.dtype))
    og = o32.cpu().double().numpy()
    log(f"[video] rel_l1={O.rel_l1(o_ref, og):.2e} max_abs={np.max(np.abs(o_ref - og)):.2e}")
    assert np.max(np.abs(o_ref - og)) <= 1e-2 and O.rel_l1(o_ref, og) <= 5e-3


def test_empty_sequence_is_a_no_op():
    qd = torch.zeros((1, 2, 0, 64), dtype=torch.float16, device=DEV)
    mask = fb.predict_mask(qd, qd, 0.9, 0.5, True)
    o, counts, _ = fb.attn(qd, qd, qd, mask, -5.0, True)
    torch.cuda.synchronize()
    assert o.numel() == 0 and int(counts.sum()) == 0
