"""GPU parity of the fp8 P~V variant (sparge_attn_fp8pv, [Review] Fig. 9
"SpargeAttn + Sage2") against the oracle's fp8 recurrence in Algorithm 1's
order (oracle.sparse_attention(..., pv8=True)): E4M3 operands, P~ rounded at
the running max of each step and rescaled exactly.

The fused pass rounds at the running max too, in float32; the two-pass path
rounds exp(S - m_final) in its second pass instead.  Either way every output
element must lie within the room that E4M3's rounding error allows both
schedules (tests/gpu_common.py, fp8_room), and the whole output within
relative L1 2^-4 and cosine 0.998 of the oracle's.  Decisions and counters
are those of the unquantised rule, on both paths.

A second, tighter check compares the two-pass path with a model of its own
schedule (tests/fp8_kernel_model.py).  It is a diagnostic for arithmetic
slips, not parity: its constants come from probes of the kernel.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from oracle import sparge_oracle as O

import fp8_kernel_model as KM
from gpu_common import DEV, FP8_REL_L1, attn_path, check_fp8, fp8_room, log, rel_l1, to_bits, to_dev

pytestmark = pytest.mark.gpu

# kernel-schedule model (diagnostic): float32 P~ next to an E4M3 rounding
# boundary may round the other way (window 2^-12 relative), and the f8f6f4
# matrix cores truncate their 64-product sums (measured below 2^-12.8 of the
# sum of absolute products; 2^-11 allowed)
MODEL_REL_L1 = 5e-3
MODEL_ABS_SLACK = 1e-3
MODEL_AMB_WINDOW = 2.0 ** -12
MODEL_SUM_REL = 2.0 ** -11

CASES = [
    ("tiny_f16_d64", 0, {}),
    ("llm_gqa_ragged", 2, {"N": 1000, "H": 4, "H_kv": 2}),
    ("llm_small_causal", 2, {"N": 2048, "H": 2, "H_kv": 2}),
    ("video_small", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}),
    ("image_small", 1, {"N": 64 + 24 * 24, "H": 2, "H_kv": 2, "grid": (24, 24), "text_tokens": 64}),
]


def _run(w, q, k, v, v_dtype=None, int8=False):
    qd, kd = to_dev(q, w.dtype), to_dev(k, w.dtype)
    vd = to_dev(v, v_dtype or w.dtype)
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    kw = {}
    qa, ka = qd, kd
    if int8:
        qa, ka, qs, ks = fb.quant_qk_int8(qd, kd)
        kw = dict(q_scale=qs, k_scale=ks)
    o16, c16, dbg = fb.attn(qa, ka, vd, mask, w.lam, w.causal, dbg=True, fp8_pv=True, **kw)
    o32, c32, dbg32 = fb.attn(qa, ka, vd, mask, w.lam, w.causal, dbg=True, out_f32=True, fp8_pv=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(c16, c32) and torch.equal(dbg, dbg32)
    assert torch.equal(o16, o32.to(o16.dtype))
    return mask, o16, o32, c32, dbg


def _all_blocks(w):
    return [(b, h, i) for b in range(w.B) for h in range(w.H) for i in range(O.num_blocks(w.N, O.BQ))]


PATHS = [(fb.PATH_TWO_PASS, "two_pass"), (fb.PATH_FUSED, "fused")]


@pytest.mark.parametrize("path,pname", PATHS, ids=[p[1] for p in PATHS])
@pytest.mark.parametrize("label,wid,over", CASES, ids=[c[0] for c in CASES])
def test_fp8pv_matches_oracle(label, wid, over, path, pname):
    w = I.workload(wid, **over)
    log(f"[fp8pv {pname}] {label}: H={w.H} Hkv={w.H_kv} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    q, k, v = I.make_qkv(w)
    with attn_path(path):
        mask, o16, o32, counts, dbg = _run(w, q, k, v)
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    mg = mask.mg.cpu().numpy().astype(bool)
    gdec = dbg.cpu().numpy().astype(np.int8)
    ref, cnt, dec = O.sparse_attention(Q, K, V, mg, w.lam, w.causal, skip_override=gdec, pv8=True)
    room = fp8_room(Q, K, V, mg, w.causal, gdec, _all_blocks(w), ref=ref)
    og = o32.cpu().double().numpy()
    rep = check_fp8(og, ref, room)
    c = fb.counts_dict(counts)
    for key in O.COUNT_NAMES:
        assert c[key] == cnt[key], (key, c, cnt)
    e16 = rel_l1(ref, O.widen(to_bits(o16), w.dtype))
    assert e16 <= FP8_REL_L1
    exact, _, _ = O.sparse_attention(Q, K, V, mg, w.lam, w.causal, skip_override=gdec)
    e_exact = rel_l1(exact, og)
    log(f"   vs oracle: rel_l1={rep['rel_l1']:.2e} cos={rep['cos']:.6f} max_abs={rep['max_abs']:.2e} "
        f"(room up to {rep['room_max']:.2e}); {w.dtype} output rel_l1={e16:.2e}; vs exact: rel_l1={e_exact:.2e}")
    assert e_exact <= FP8_REL_L1


@pytest.mark.parametrize("path,pname", PATHS, ids=[p[1] for p in PATHS])
def test_fp8pv_int8_qk_matches_oracle(path, pname):
    w = I.workload(2, N=1000, H=2, H_kv=1)
    q, k, _ = I.make_qkv(w)
    v = I.make_tensor(w, I.TENSOR_V, dtype="f16")
    log(f"[fp8pv int8 {pname}] N={w.N}")
    with attn_path(path):
        mask, o16, o32, counts, dbg = _run(w, q, k, v, v_dtype="f16", int8=True)
    Q, K = O.widen(q, w.dtype), O.widen(k, w.dtype)
    V = O.widen(v, "f16")
    quant = O.quantize_qk(Q, K)
    mg = mask.mg.cpu().numpy().astype(bool)
    gdec = dbg.cpu().numpy().astype(np.int8)
    ref, cnt, _ = O.sparse_attention(Q, K, V, mg, w.lam, w.causal, skip_override=gdec, quant=quant, pv8=True)
    room = fp8_room(Q, K, V, mg, w.causal, gdec, _all_blocks(w), quant=quant, ref=ref)
    rep = check_fp8(o32.cpu().double().numpy(), ref, room)
    assert fb.counts_dict(counts) == {k_: cnt[k_] for k_ in O.COUNT_NAMES}
    log(f"   vs oracle (int8 codes): rel_l1={rep['rel_l1']:.2e} cos={rep['cos']:.6f} max_abs={rep['max_abs']:.2e}")


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
    with attn_path(fb.PATH_TWO_PASS):
        o32, counts, dbg = fb.attn(qd, kd, vd, mg, -np.inf, False, dbg=True, out_f32=True, fp8_pv=True)
    with attn_path(fb.PATH_FUSED):
        o32f, counts_f, dbg_f = fb.attn(qd, kd, vd, mg, -np.inf, False, dbg=True, out_f32=True, fp8_pv=True)
    torch.cuda.synchronize()
    assert torch.equal(counts, counts_f) and torch.equal(dbg, dbg_f)
    gdec = dbg.cpu().numpy().astype(np.int8)
    ref, _, _ = O.sparse_attention(Q, K, V, mg_np, -np.inf, False, skip_override=gdec, pv8=True)
    blocks = [(0, 0, i) for i in range(mg_np.shape[2])]
    room = fp8_room(Q, K, V, mg_np, False, gdec, blocks, ref=ref)
    for o in (o32, o32f):
        og = o.cpu().double().numpy()
        assert np.all(og[..., 1] == 0.0)
        assert np.all(np.abs(og - ref) <= room)
        for c in (0, 2, 3, 10):
            e = rel_l1(ref[..., c], og[..., c])
            log(f"   channel {c}: rel_l1 vs oracle {e:.2e}")
            assert e <= FP8_REL_L1


@pytest.mark.parametrize("label,wid,over", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_fp8pv_kernel_schedule_model(label, wid, over):
    """Diagnostic, not parity: the two-pass path against a float64 model of
    its own schedule (P~ at the final max, V scales floored at 2^-100)."""
    w = I.workload(wid, **over)
    q, k, v = I.make_qkv(w)
    with attn_path(fb.PATH_TWO_PASS):
        mask, o16, o32, counts, dbg = _run(w, q, k, v)
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    mg = mask.mg.cpu().numpy().astype(bool)
    gdec = dbg.cpu().numpy().astype(np.int8)
    model, room = KM.sparse_attention_final_max(Q, K, V, mg, w.causal, gdec, amb_window=MODEL_AMB_WINDOW,
                                                sum_rel=MODEL_SUM_REL)
    og = o32.cpu().double().numpy()
    e = rel_l1(model, og)
    over_ = float(np.max(np.abs(model - og) - room))
    log(f"[fp8pv model] {label}: rel_l1={e:.2e} max over room={over_:.2e}")
    assert e <= MODEL_REL_L1 and over_ <= MODEL_ABS_SLACK
