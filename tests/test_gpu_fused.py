"""GPU parity of the fused stage-2 path (one pass in Algorithm 1's order,
sparge_attn_path(SPARGE_PATH_FUSED)) against the float64 oracle, on the same
inputs and acceptance as the two-pass parity tests, and of the automatic
choice between the two paths.

The fused path rounds P~ at the running max of each step (the oracle's
order) where the two-pass path rounds it at the final max, so the two give
different bits within the same tolerance; their lambda decisions, decision
maps and counters are identical.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from oracle import sparge_oracle as O

from gpu_common import DEV, attn_path, check_attention, check_mask, log, run_attn, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_full", 0, {}),
    ("tiny_ragged", 0, {"N": 1000}),
    ("llm_gqa_ragged", 2, {"N": 1000, "H": 4, "H_kv": 2}),
    ("llm_small_causal", 2, {"N": 2048, "H": 2, "H_kv": 2}),
    ("image_small", 1, {"N": 64 + 24 * 24, "H": 2, "H_kv": 2, "grid": (24, 24), "text_tokens": 64}),
    ("video_small", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}),
]


def _both_paths(qd, kd, vd, mask, lam, causal, **kw):
    """The call on each forced path: (o16, o32, counts, dbg) per path."""
    out = {}
    for path in (fb.PATH_TWO_PASS, fb.PATH_FUSED):
        with attn_path(path):
            out[path] = run_attn(qd, kd, vd, mask, lam, causal, **kw)
    return out


@pytest.mark.parametrize("label,wid,over", CASES, ids=[c[0] for c in CASES])
def test_fused_matches_oracle(label, wid, over):
    w = I.workload(wid, **over)
    q, k, v = I.make_qkv(w)
    log(f"[fused] {label}: B={w.B} H={w.H} Hkv={w.H_kv} N={w.N} d={w.d} causal={w.causal} lam={w.lam}")
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    res = _both_paths(qd, kd, vd, mask, w.lam, w.causal)
    o16, o32, counts, dbg = res[fb.PATH_FUSED]
    _, _, counts2, dbg2 = res[fb.PATH_TWO_PASS]
    assert torch.equal(counts, counts2) and torch.equal(dbg, dbg2)
    mg = mask.mg.cpu().numpy().astype(bool)
    rep = check_attention(o32, counts, dbg, Q, K, V, mg, w.lam, w.causal, "f32", o16=o16, o16_dtype=w.dtype)
    log(f"   max_abs={rep['max_abs']:.2e} rel_l1={rep['rel_l1']:.2e} flips={rep['lambda_flips']} counts={rep['counts']}")


@pytest.mark.parametrize("dtype,d,causal", [("f16", 128, False), ("bf16", 64, True), ("bf16", 128, True),
                                            ("f16", 64, False)])
def test_fused_random_mask_edge_rows(dtype, d, causal):
    """The random mask of the two-pass edge-row test (empty block rows, a
    dominant early block that makes lambda skip, a ragged N), lambda finite
    and -inf, on the fused path."""
    N, H, Hkv = 777, 3, 1
    rng = np.random.default_rng(5)
    Qf = rng.standard_normal((1, H, N, d)) * 2.0
    Kf = rng.standard_normal((1, Hkv, N, d)) * 2.0
    Kf[0, 0, :64] += 3.0 * Qf[0, 0, :64].mean(axis=0)
    Vf = rng.standard_normal((1, Hkv, N, d))
    q, k, v = (I.to_bits(x, dtype) for x in (Qf, Kf, Vf))
    Q, K, V = (O.widen(x, dtype) for x in (q, k, v))
    Tm, Tn = O.num_blocks(N, 128), O.num_blocks(N, 64)
    mg_np = rng.random((1, H, Tm, Tn)) < 0.6
    mg_np[0, 0, 2] = False
    mg_np[0, 1, :, 0] = True
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    mg = torch.from_numpy(mg_np.astype(np.uint8)).to(DEV)
    for lam in (-2.0, -math.inf):
        with attn_path(fb.PATH_FUSED):
            o, o32, counts, dbg = run_attn(qd, kd, vd, mg, lam, causal)
        rep = check_attention(o32, counts, dbg, Q, K, V, mg_np, lam, causal, "f32", o16=o, o16_dtype=dtype)
        log(f"[fused random] {dtype} d={d} causal={causal} lam={lam}: max_abs={rep['max_abs']:.2e} "
            f"rel_l1={rep['rel_l1']:.2e} counts={rep['counts']}")
        assert rep["counts"]["empty_rows"] >= 128
        if lam == -2.0:
            assert rep["counts"]["pv_skip"] > 0


@pytest.mark.parametrize("N", [1, 17, 64, 65, 127, 129])
@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_fused_short_sequences(N, d, causal):
    """One token up to just past one query block, on the fused path: a single
    ragged tile, wavefronts whose rows all lie beyond N, empty lists."""
    H, Hkv = 3, 1
    rng = np.random.default_rng(1000 + N + d)
    Qf = rng.standard_normal((1, H, N, d))
    Kf = rng.standard_normal((1, Hkv, N, d))
    Vf = rng.standard_normal((1, Hkv, N, d))
    Qf[0, 1] = Qf[0, 1, :1] + 0.05 * Qf[0, 1]
    Kf[0, 0] = Kf[0, 0, :1] + 0.05 * Kf[0, 0]
    q, k, v = (I.to_bits(x, "bf16") for x in (Qf, Kf, Vf))
    Q, K, V = (O.widen(x, "bf16") for x in (q, k, v))
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    mask = fb.predict_mask(qd, kd, 0.1, 0.9, causal)
    with attn_path(fb.PATH_FUSED):
        o, o32, counts, dbg = run_attn(qd, kd, vd, mask.mg, -1.0, causal)
    rep = check_attention(o32, counts, dbg, Q, K, V, mask.mg.cpu().numpy().astype(bool), -1.0, causal, "f32",
                          o16=o, o16_dtype="bf16")
    log(f"[fused short] N={N} d={d} causal={causal}: max_abs={rep['max_abs']:.2e} counts={rep['counts']}")
    assert rep["counts"]["rows"] == H * N


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,N", [(False, 16384 - 37), (True, 32768 - 100)])
def test_fused_packs_of_dense_blocks(d, causal, N):
    """Rows of at least 192 live tiles (192 x 2 on a causal call), where the
    fused path runs the dense query blocks of a kv head in pairs on one K and
    V stream: a mask in which an odd number of block rows per kv head list
    every live tile (so one pair has a single member) and the rest about half
    of them, ragged N.  Both paths give the same decisions and counters, and
    sampled blocks (paired, unpaired, the ragged last one) match the oracle."""
    H, Hkv = 2, 1
    w = I.workload(2, N=N, H=H, H_kv=Hkv, d=d, causal=causal)
    q, k, v = I.make_qkv(w)
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    Tm, Tn = O.num_blocks(N, O.BQ), O.num_blocks(N, O.BK)
    rng = np.random.default_rng(31 + d + (1 if causal else 0))
    mg_np = rng.random((1, H, Tm, Tn)) < 0.5
    dense = rng.random((H, Tm)) < 0.4
    if dense.sum() % 2 == 0:
        dense[0, Tm - 1] = not dense[0, Tm - 1]
    mg_np[0][dense] = True
    mg = torch.from_numpy(mg_np.astype(np.uint8)).to(DEV)
    log(f"[fused packs] d={d} causal={causal} N={N}: Tn={Tn}, {int(dense.sum())} dense block rows")
    res = _both_paths(qd, kd, vd, mg, w.lam, causal)
    o16, o32, counts, dbg = res[fb.PATH_FUSED]
    _, _, counts2, dbg2 = res[fb.PATH_TWO_PASS]
    assert torch.equal(counts, counts2) and torch.equal(dbg, dbg2)
    picks = [(h, i) for h in range(H) for i in (0, Tm - 1)]
    picks += [(h, int(i)) for h in range(H) for i in np.flatnonzero(dense[h])[-3:]]
    picks += [(h, int(i)) for h in range(H) for i in np.flatnonzero(~dense[h])[-2:]]
    blocks = sorted({(0, h, i) for h, i in picks})
    rep = check_attention(o32, counts, dbg, Q, K, V, mg_np, w.lam, causal, "f32", blocks=blocks,
                          o16=o16, o16_dtype=w.dtype)
    log(f"   {len(blocks)} blocks: max_abs={rep['max_abs']:.2e} rel_l1={rep['rel_l1']:.2e} "
        f"flips={rep['lambda_flips']} counts={fb.counts_dict(counts)}")


@pytest.mark.parametrize("causal", [True, False])
def test_fused_strided_layouts_and_batches(causal):
    """[B, N, H, d] strides, two batches, GQA, ragged N on the fused path: the
    same bits as contiguous inputs, and the oracle's result."""
    w = I.workload(2, N=700, H=4, H_kv=2, B=2, causal=causal)
    q, k, v = I.make_qkv(w)
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))

    def bshd(x):
        return x.transpose(1, 2).contiguous().transpose(1, 2)

    qs, ks, vs = bshd(qd), bshd(kd), bshd(vd)
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, causal)
    with attn_path(fb.PATH_FUSED):
        o1, c1, _ = fb.attn(qd, kd, vd, mask, w.lam, causal)
        out = torch.empty(w.B, w.N, w.H, w.d, dtype=vd.dtype, device=DEV).transpose(1, 2)
        o2, c2, _ = fb.attn(qs, ks, vs, mask, w.lam, causal, out=out)
        o, o32, counts, dbg = run_attn(qs, ks, vs, mask, w.lam, causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(c1, c2) and torch.equal(o1, o)
    rep = check_attention(o32, counts, dbg, Q, K, V, mask.mg.cpu().numpy().astype(bool), w.lam, causal, "f32",
                          o16=o, o16_dtype=w.dtype)
    log(f"[fused strided] causal={causal}: rel_l1={rep['rel_l1']:.2e} counts={rep['counts']}")


def test_fused_repeat_calls_bit_identical():
    w = I.workload(3, N=4 * 16 * 12, H=4, H_kv=2, grid=(4, 16, 12))
    q, k, v = I.make_qkv(w)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    with attn_path(fb.PATH_FUSED):
        runs = [fb.attn(qd, kd, vd, mask, w.lam, w.causal, dbg=True, ws=torch.empty_like(fb.workspace(qd, kd)))
                for _ in range(3)]
    torch.cuda.synchronize()
    for o, c, d in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(c, runs[0][1]) and torch.equal(d, runs[0][2])


@pytest.mark.parametrize("label,wid,over,expect", [
    ("image_small", 1, {"N": 64 + 24 * 24, "H": 2, "H_kv": 2, "grid": (24, 24), "text_tokens": 64}, "fused"),
    ("video_small", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}, "fused"),
    ("llm_16k_causal", 2, {"N": 16384, "H": 4, "H_kv": 2}, "fused"),
    ("llm_64k_causal", 2, {"N": 65536, "H": 2, "H_kv": 1}, "two_pass"),
], ids=["image_small", "video_small", "llm_16k_causal", "llm_64k_causal"])
def test_auto_path_follows_the_vote_rate(label, wid, over, expect):
    """With SPARGE_PATH_AUTO the pilot takes the fused path where nearly every
    (tile, wavefront) votes (image and video recipes) or rows are short (the
    LLM recipe at N 16384: some 80 listed tiles per block), and two passes on
    long rows where few vote (the LLM recipe at N 65536): the automatic
    call's bits equal those of the forced path it chose, and its counters
    both paths'."""
    w = I.workload(wid, **over)
    q, k, v = I.make_qkv(w)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    outs = {}
    for path in (fb.PATH_AUTO, fb.PATH_TWO_PASS, fb.PATH_FUSED):
        with attn_path(path):
            outs[path] = fb.attn(qd, kd, vd, mask, w.lam, w.causal, out_f32=True)
    torch.cuda.synchronize()
    c = fb.counts_dict(outs[fb.PATH_AUTO][1])
    rate = c["pv_exec"] / max(1, c["pv_exec"] + c["pv_skip"])
    want = fb.PATH_FUSED if expect == "fused" else fb.PATH_TWO_PASS
    other = fb.PATH_TWO_PASS if expect == "fused" else fb.PATH_FUSED
    log(f"[auto] {label}: vote rate {rate:.3f}, expected {expect}")
    assert torch.equal(outs[fb.PATH_AUTO][0], outs[want][0])
    assert not torch.equal(outs[fb.PATH_AUTO][0], outs[other][0])
    for path in (fb.PATH_TWO_PASS, fb.PATH_FUSED):
        assert torch.equal(outs[path][1], outs[fb.PATH_AUTO][1])


@pytest.mark.parametrize("label,wid,over,expect", [
    ("video_small", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}, "fused"),
    ("llm_64k_causal", 2, {"N": 65536, "H": 2, "H_kv": 1}, "fused"),
    ("llm_128k_causal", 2, {"N": 131072, "H": 2, "H_kv": 1}, "two_pass"),
], ids=["video_small", "llm_64k_causal", "llm_128k_causal"])
def test_fp8pv_paths_and_automatic_choice(label, wid, over, expect):
    """fp8 P~V on each path: the same decisions, decision map and counters
    (the oracle comparison of both is in test_gpu_fp8pv.py), different bits
    (the fused pass rounds P~ at the running max, the second pass at the
    final one), and the automatic choice: fused on the LLM recipe up to N
    65536 (fp8's bound of 448 listed tiles), two passes at 131072."""
    w = I.workload(wid, **over)
    q, k, v = I.make_qkv(w)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    res = {}
    for path in (fb.PATH_TWO_PASS, fb.PATH_FUSED, fb.PATH_AUTO):
        with attn_path(path):
            res[path] = fb.attn(qd, kd, vd, mask, w.lam, w.causal, fp8_pv=True, dbg=True, out_f32=True)
    torch.cuda.synchronize()
    two, fused, auto = res[fb.PATH_TWO_PASS], res[fb.PATH_FUSED], res[fb.PATH_AUTO]
    assert torch.equal(two[1], fused[1]) and torch.equal(two[2], fused[2])
    assert not torch.equal(two[0], fused[0])
    assert torch.equal(auto[0], fused[0] if expect == "fused" else two[0])
    log(f"[fp8pv paths] {label}: counts {fb.counts_dict(two[1])}")


@pytest.mark.parametrize("N,expect", [(8192, "fused"), (16384, "two_pass")])
def test_int8_fp8pv_automatic_choice(N, expect):
    """int8 Q/K with fp8 P~V: both paths give the same decisions and
    counters, and the automatic choice takes the fused pass on the LLM
    recipe at N 8192 (some 40 listed tiles per block, under that pair's bound
    of 64) and two passes at 16384 (some 80)."""
    w = I.workload(2, N=N, H=2, H_kv=1)
    q, k, _ = I.make_qkv(w)
    v = I.make_tensor(w, I.TENSOR_V, dtype="f16")
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, "f16")
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    q8, k8, qs, ks = fb.quant_qk_int8(qd, kd)
    res = {}
    for path in (fb.PATH_TWO_PASS, fb.PATH_FUSED, fb.PATH_AUTO):
        with attn_path(path):
            res[path] = fb.attn(q8, k8, vd, mask, w.lam, w.causal, q_scale=qs, k_scale=ks, fp8_pv=True, dbg=True,
                                out_f32=True)
    torch.cuda.synchronize()
    two, fused, auto = res[fb.PATH_TWO_PASS], res[fb.PATH_FUSED], res[fb.PATH_AUTO]
    assert torch.equal(two[1], fused[1]) and torch.equal(two[2], fused[2])
    assert not torch.equal(two[0], fused[0])
    assert torch.equal(auto[0], fused[0] if expect == "fused" else two[0])
    log(f"[int8 fp8pv paths] N={N}: counts {fb.counts_dict(two[1])}")


INT8_CASES = [
    # label, workload, overrides, V type, sampled blocks (None: every block), automatic path
    ("llm_gqa_ragged_causal_f16", 2, {"N": 1100, "H": 4, "H_kv": 2}, "f16", None, "fused"),
    ("llm_ragged_d64_bf16", 2, {"N": 1100, "H": 4, "H_kv": 2, "d": 64, "causal": False}, "bf16", None, "fused"),
    ("image_small_bf16", 1, {"N": 64 + 24 * 24, "H": 2, "H_kv": 2, "grid": (24, 24), "text_tokens": 64}, "bf16",
     None, "fused"),
    ("video_small_f16", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}, "f16", None, "fused"),
    ("llm_32k_pairs_causal_f16", 2, {"N": 32768 - 100, "H": 2, "H_kv": 1}, "f16", 10, "two_pass"),
    ("llm_64k_causal_f16", 2, {"N": 65536, "H": 2, "H_kv": 1}, "f16", 6, "two_pass"),
    ("llm_16k_d64_pairs_bf16", 2, {"N": 16384 - 37, "H": 2, "H_kv": 1, "d": 64, "causal": False}, "bf16", 8, None),
]


@pytest.mark.parametrize("label,wid,over,v_dtype,n_blocks,auto", INT8_CASES, ids=[c[0] for c in INT8_CASES])
def test_int8_both_paths_match_oracle(label, wid, over, v_dtype, n_blocks, auto):
    """int8 Q/K (with fp16 or bf16 P~V) on each stage-2 path: the same lambda
    decisions, decision map and counters on both, each output within the
    int8 bar of the oracle (codes and scales of the oracle's quantisation),
    and the automatic choice: fused where nearly every wavefront votes or
    rows are short (for int8 at most 112 listed tiles per block on average,
    half the 16-bit bound), two passes on the LLM recipe from N 32768 on.
    The long rows (causal at N 32668, and d 64 non-causal at 16347) run the
    fused pass's pairs of dense blocks; there the oracle checks sampled
    blocks (the last, the first and seeded random ones)."""
    w = I.workload(wid, **over)
    q, k, _ = I.make_qkv(w)
    v = I.make_tensor(w, I.TENSOR_V, dtype=v_dtype)
    Q, K, V = O.widen(q, w.dtype), O.widen(k, w.dtype), O.widen(v, v_dtype)
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, v_dtype)
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    q8, k8, qs, ks = fb.quant_qk_int8(qd, kd)
    kw = dict(q_scale=qs, k_scale=ks)
    res = _both_paths(q8, k8, vd, mask, w.lam, w.causal, **kw)
    with attn_path(fb.PATH_AUTO):
        o_auto = fb.attn(q8, k8, vd, mask, w.lam, w.causal, out_f32=True, **kw)[0]
    torch.cuda.synchronize()
    _, o32_two, counts, dbg = res[fb.PATH_TWO_PASS]
    _, o32_fused, counts_f, dbg_f = res[fb.PATH_FUSED]
    assert torch.equal(counts, counts_f) and torch.equal(dbg, dbg_f)
    if auto is None:
        assert torch.equal(o_auto, o32_fused) or torch.equal(o_auto, o32_two)
    else:
        assert torch.equal(o_auto, o32_fused if auto == "fused" else o32_two)
    assert not torch.equal(o32_two, o32_fused)
    mg = mask.mg.cpu().numpy().astype(bool)
    quant = O.quantize_qk(Q, K)
    Tm = O.num_blocks(w.N, O.BQ)
    blocks = None
    if n_blocks is not None:
        rng = np.random.default_rng(300 + w.N % 997)
        picks = {(h, Tm - 1) for h in range(w.H)} | {(0, 0)}
        picks |= {(int(rng.integers(w.H)), int(i)) for i in rng.choice(Tm, size=n_blocks, replace=False)}
        blocks = sorted((0, h, i) for h, i in picks)
    for path in (fb.PATH_TWO_PASS, fb.PATH_FUSED):
        o16, o32 = res[path][0], res[path][1]
        rep = check_attention(o32, counts, dbg, Q, K, V, mg, w.lam, w.causal, "f32", blocks=blocks, quant=quant,
                              int8=True, o16=o16, o16_dtype=v_dtype)
        log(f"[int8 {label}] {'fused' if path == fb.PATH_FUSED else 'two-pass'}: rel_l1={rep['rel_l1']:.2e} "
            f"cos={rep['cos']:.6f} flips={rep['lambda_flips']}")
    log(f"   counts {fb.counts_dict(counts)}")
