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

from gpu_common import DEV, check_attention, check_mask, log

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


def _check_heads(w, q, k, v, mask, dbg, o32, heads, int8=False, v_dtype=None, perm_np=None):
    group = w.H // w.H_kv
    Tm = O.num_blocks(w.N, O.BQ)
    for h in heads:
        hk = h // group
        Qh = O.widen(q[:, h:h + 1], w.dtype)
        Kh = O.widen(k[:, hk:hk + 1], w.dtype)
        Vh = O.widen(v[:, hk:hk + 1], v_dtype or w.dtype)
        if perm_np is not None:
            Qh, Kh, Vh = (O.permute_tokens(x, perm_np) for x in (Qh, Kh, Vh))
        rep = check_mask(_sub_mask(mask, h, hk), Qh, Kh, w.tau, w.theta, w.causal)
        blocks = [(0, 0, i) for i in _sample_blocks(Tm)]
        # int8: the K mean is over all tokens of the kv head, which the slice holds whole
        quant = O.quantize_qk(Qh, Kh) if int8 else None
        # attention is compared given the mask the GPU used
        mg_h = mask.mg[:, h:h + 1].cpu().numpy().astype(bool)
        arep = check_attention(o32[:, h:h + 1], None, dbg[:, h:h + 1], Qh, Kh, Vh, mg_h, w.lam, w.causal,
                               "f32", blocks=blocks, quant=quant, int8=int8)
        log(f"   head {h}: mask near_theta={rep['near_theta']} ambiguous={rep['ambiguous']} "
            f"s_err={rep['max_s_err']:.1e}; blocks {[b[2] for b in blocks]}: max_abs={arep['max_abs']:.2e} "
            f"rel_l1={arep['rel_l1']:.2e} flips={arep['lambda_flips']}")


@pytest.mark.parametrize("wid,heads", [(1, [0, 23]), (2, [0, 31]), (3, [0, 23]), (4, [0, 17, 31])],
                         ids=["image_dit", "llm_32k", "video_dit_raster", "gqa_128k"])
def test_full_size_bf16(wid, heads):
    w = I.workload(wid)
    log(f"[full] {w.name}: B={w.B} H={w.H} Hkv={w.H_kv} N={w.N} d={w.d} causal={w.causal}")
    q, k, v = I.make_qkv(w, workers=16)
    mask, counts, dbg, o16, o32 = _run(w, q, k, v)
    c = _check_whole(w, mask, counts, o16, o32)
    log(f"   counts {c}")
    _check_heads(w, q, k, v, mask, dbg, o32, heads)


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
    _check_heads(w, q, k, v, mask, dbg, o32, [0, 23], perm_np=perm_np)


def test_full_size_gqa_int8():
    w = I.workload(4)
    log(f"[full] {w.name} int8 Q/K, fp16 P~V")
    q, k, _ = I.make_qkv(w, workers=16)
    v = I.make_tensor(w, I.TENSOR_V, dtype="f16", workers=16)
    mask, counts, dbg, o16, o32 = _run(w, q, k, v, int8=True)
    c = _check_whole(w, mask, counts, o16, o32)
    log(f"   counts {c}")
    _check_heads(w, q, k, v, mask, dbg, o32, [0, 31], int8=True, v_dtype="f16")


def test_full_size_gqa_fp8pv():
    """The fp8 P~V variant at 128K GQA, in the bench's configuration: sampled
    blocks of two heads against the oracle's fp8 restatement (same rules as
    the small fp8 parity tests), whole-output properties on everything."""
    from test_gpu_fp8pv import FP8_ABS_SLACK, FP8_AMB_WINDOW, FP8_REL_L1, FP8_SUM_REL
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
    for h in (0, 31):
        hk = h // group
        Qh = O.widen(q[:, h:h + 1], w.dtype)
        Kh = O.widen(k[:, hk:hk + 1], w.dtype)
        Vh = O.widen(v[:, hk:hk + 1], w.dtype)
        blocks = [(0, 0, i) for i in _sample_blocks(Tm)]
        mg_h = mask.mg[:, h:h + 1].cpu().numpy().astype(bool)
        gdec = dbg[:, h:h + 1].cpu().numpy().astype(np.int8)
        ref, room = O.sparse_attention_fp8pv(Qh, Kh, Vh, mg_h, w.lam, w.causal, blocks=blocks, skip_override=gdec,
                                             amb_window=FP8_AMB_WINDOW, sum_rel=FP8_SUM_REL)
        og = o32[:, h:h + 1].cpu().double().numpy()
        sel = np.concatenate([np.arange(O.block_rows(w.N, O.BQ, i).start, O.block_rows(w.N, O.BQ, i).stop)
                              for _, _, i in blocks])
        r, g, rm = ref[0, 0, sel], og[0, 0, sel], room[0, 0, sel]
        e_rel = O.rel_l1(r, g)
        over = float(np.max(np.abs(r - g) - rm))
        log(f"   head {h}: blocks {[bl[2] for bl in blocks]}: rel_l1={e_rel:.2e} max over room={over:.2e}")
        assert e_rel <= FP8_REL_L1 and over <= FP8_ABS_SLACK


MAX_TN = 4096   # SPARGE_MAX_TN of include/sparge.h


@pytest.mark.parametrize("H,H_kv,causal", [(2, 1, True), (1, 1, False)], ids=["causal_gqa", "noncausal"])
def test_largest_supported_sequence(H, H_kv, causal):
    """N = 64 * SPARGE_MAX_TN = 262144, the longest sequence the library takes:
    Tn = 4096 key blocks, so the widest M_g rows and row lists, the largest
    LDS lists and vote arrays of both attention passes, and (causal) rows
    whose dense lists walk 4096 tiles.  The llm_32k recipe at that length;
    mask rows of every head and sampled query blocks against the oracle."""
    w = I.workload(2, N=64 * MAX_TN, H=H, H_kv=H_kv, causal=causal)
    assert O.num_blocks(w.N, O.BK) == MAX_TN
    log(f"[full] largest N: H={w.H} Hkv={w.H_kv} N={w.N} causal={w.causal}")
    q, k, v = I.make_qkv(w, workers=16)
    mask, counts, dbg, o16, o32 = _run(w, q, k, v)
    c = _check_whole(w, mask, counts, o16, o32)
    log(f"   counts {c}")
    _check_heads(w, q, k, v, mask, dbg, o32, list(range(w.H)))
