"""GPU parity of the fp8 P~V variant (sparge_attn_fp8pv) against the oracle's
restatement of the same arithmetic (oracle.sparge_attention_fp8pv: E4M3 codes
of V / delta_c with power-of-two channel scales, P~ * 2^8 at the final row
max rounded to E4M3, exact sums).

The V codes are exact on both sides (a power-of-two scaling, then one
rounding), so the only differences are: P~ from float32 scores and exp2
against float64 ones, which can move a P~ that lies near an E4M3 rounding
boundary across it, each such flip changing one product by one E4M3 step
(1/16 of it); the sums of the f8f6f4 MFMA, which truncate (a probe of
64-product sums with one product far above the rest measured errors up to
2^-12.8 of the sum of the absolute products; FP8_SUM_REL allows 2^-11); l in
float32.  A float32
score is a sum of d products of up to a few hundred in size, so it can be
off by ~1e-3, about 1e-4 in the log2 exponent, and P~ by ~1e-4 relative:
the window below is 2^-12.  Hence the acceptance, against the oracle on the
same mask and the GPU's lambda decisions: relative L1 <= 5e-3, and every
element within the room the oracle reports for P~ values closer than the
window to an E4M3 rounding boundary, plus 1e-3.  Against the exact
(unrounded) attention the variant's own error is reported and bounded by
5e-2 relative L1.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from oracle import sparge_oracle as O

from gpu_common import DEV, log, rel_l1, to_dev

pytestmark = pytest.mark.gpu

FP8_REL_L1 = 5e-3
FP8_ABS_SLACK = 1e-3
FP8_AMB_WINDOW = 2.0 ** -12
FP8_SUM_REL = 2.0 ** -11
FP8_VS_EXACT_REL_L1 = 5e-2


def _check(ref, room, og):
    e_rel = rel_l1(ref, og)
    over = np.abs(ref - og) - room
    assert e_rel <= FP8_REL_L1, e_rel
    assert np.all(over <= FP8_ABS_SLACK), float(over.max())
    return e_rel, float(np.max(np.abs(ref - og))), float(room.max())

CASES = [
    ("tiny_f16_d64", 0, {}),
    ("llm_gqa_ragged", 2, {"N": 1000, "H": 4, "H_kv": 2}),
    ("llm_small_causal", 2, {"N": 2048, "H": 2, "H_kv": 2}),
    ("video_small", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}),
]


def _run(w, q, k, v, int8=False):
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    kw = {}
    qa, ka = qd, kd
    quant = None
    if int8:
        qa, ka, qs, ks = fb.quant_qk_int8(qd, kd)
        kw = dict(q_scale=qs, k_scale=ks)
    o16, c16, dbg = fb.attn(qa, ka, vd, mask, w.lam, w.causal, dbg=True, fp8_pv=True, **kw)
    o32, c32, dbg32 = fb.attn(qa, ka, vd, mask, w.lam, w.causal, dbg=True, out_f32=True, fp8_pv=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(c16, c32) and torch.equal(dbg, dbg32)
    assert torch.equal(o16, o32.to(o16.dtype))
    return mask, o32, c32, dbg


@pytest.mark.parametrize("label,wid,over", CASES, ids=[c[0] for c in CASES])
def test_fp8pv_matches_oracle(label, wid, over):
    w = I.workload(wid, **over)
    log(f"[fp8pv] {label}: H={w.H} Hkv={w.H_kv} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    q, k, v = I.make_qkv(w)
    mask, o32, counts, dbg = _run(w, q, k, v)
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    mg = mask.mg.cpu().numpy().astype(bool)
    gdec = dbg.cpu().numpy().astype(np.int8)
    ref, room = O.sparse_attention_fp8pv(Q, K, V, mg, w.lam, w.causal, skip_override=gdec,
                                         amb_window=FP8_AMB_WINDOW, sum_rel=FP8_SUM_REL)
    og = o32.cpu().double().numpy()
    e_rel, e_abs, r_max = _check(ref, room, og)
    exact, cnt, _ = O.sparse_attention(Q, K, V, mg, w.lam, w.causal, skip_override=gdec)
    e_exact = rel_l1(exact, og)
    c = fb.counts_dict(counts)
    for key in O.COUNT_NAMES:
        assert c[key] == cnt[key], (key, c, cnt)
    log(f"   vs fp8 oracle: rel_l1={e_rel:.2e} max_abs={e_abs:.2e} (largest rounding room {r_max:.2e}); "
        f"vs exact: rel_l1={e_exact:.2e}")
    assert e_exact <= FP8_VS_EXACT_REL_L1


def test_fp8pv_int8_qk_matches_oracle():
    w = I.workload(2, N=1000, H=2, H_kv=1)
    q, k, _ = I.make_qkv(w)
    v = I.make_tensor(w, I.TENSOR_V, dtype="f16")
    log(f"[fp8pv int8] N={w.N}")
    qd = to_dev(q, w.dtype)
    kd = to_dev(k, w.dtype)
    vd = to_dev(v, "f16")
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    q8, k8, qs, ks = fb.quant_qk_int8(qd, kd)
    o32, counts, dbg = fb.attn(q8, k8, vd, mask, w.lam, w.causal, q_scale=qs, k_scale=ks, dbg=True,
                               out_f32=True, fp8_pv=True)
    torch.cuda.synchronize()
    Q, K = O.widen(q, w.dtype), O.widen(k, w.dtype)
    V = O.widen(v, "f16")
    quant = O.quantize_qk(Q, K)
    mg = mask.mg.cpu().numpy().astype(bool)
    gdec = dbg.cpu().numpy().astype(np.int8)
    ref, room = O.sparse_attention_fp8pv(Q, K, V, mg, w.lam, w.causal, skip_override=gdec, quant=quant,
                                         amb_window=FP8_AMB_WINDOW, sum_rel=FP8_SUM_REL)
    og = o32.cpu().double().numpy()
    e_rel, e_abs, r_max = _check(ref, room, og)
    log(f"   vs fp8 oracle (int8 codes): rel_l1={e_rel:.2e} max_abs={e_abs:.2e} (room {r_max:.2e})")


def test_fp8pv_channel_scales_and_extreme_channels():
    """Channels of very different ranges (one all zero, one near the bf16 top,
    one tiny) keep their relative accuracy: the scale is per channel."""
    N, d, H = 300, 64, 1
    rng = np.random.default_rng(11)
    Qf = rng.standard_normal((1, H, N, d))
    Kf = rng.standard_normal((1, H, N, d))
    Vf = rng.standard_normal((1, H, N, d))
    Vf[..., 1] = 0.0
    Vf[..., 2] *= 1e30
    Vf[..., 3] *= 1e-20
    q, k, v = (I.to_bits(x, "bf16") for x in (Qf, Kf, Vf))
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    Q, K, V = (O.widen(x, "bf16") for x in (q, k, v))
    mg_np = np.ones((1, H, O.num_blocks(N, 128), O.num_blocks(N, 64)), dtype=bool)
    mg = torch.from_numpy(mg_np.astype(np.uint8)).to(DEV)
    o32, counts, dbg = fb.attn(qd, kd, vd, mg, -np.inf, False, dbg=True, out_f32=True, fp8_pv=True)
    torch.cuda.synchronize()
    gdec = dbg.cpu().numpy().astype(np.int8)
    ref, room = O.sparse_attention_fp8pv(Q, K, V, mg_np, -np.inf, False, skip_override=gdec,
                                         amb_window=FP8_AMB_WINDOW, sum_rel=FP8_SUM_REL)
    og = o32.cpu().double().numpy()
    assert np.all(og[..., 1] == 0.0)
    for c in (0, 2, 3, 10):
        e = rel_l1(ref[..., c], og[..., c])
        log(f"   channel {c}: rel_l1 vs fp8 oracle {e:.2e}")
        assert e <= FP8_REL_L1
        # relative room: the channel's own scale
        scale = np.abs(ref[..., c]).max()
        assert np.all(np.abs(ref[..., c] - og[..., c]) <= room[..., c] + FP8_ABS_SLACK * scale)
