"""Seeded random configurations of the whole path against the oracle.

Each case draws, from its own seed, one point of the space the fixed cases
cover a few at a time: the input recipe (segments, 2-D or 3-D Gaussian
fields, AR(1) with sinks), B, H, H_kv and the GQA group, a ragged N (down to
a single token), d, the storage type, causal or not, tau, theta, lambda
(down to -inf, where every visited tile runs P~V), the stage-2 path (forced
or automatic), the Q/K and P~V types (16-bit, int8 Q/K, fp8 P~V, both) and
the layout of Q, K and V ([B, H, N, d], or the strides of [B, N, H, d]).
Every case runs stage 1 and stage 2 through the C ABI and meets the same
acceptance as the fixed cases: M_g and the lists bit-exact outside the
oracle's ambiguous entries, the output and the counters against the oracle
replaying the GPU's lambda decisions (the fp8 room where P~V is fp8).
"""
from __future__ import annotations

import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from oracle import sparge_oracle as O

from gpu_common import (FP8_REL_L1, attn_path, check_attention, check_fp8, check_mask, fp8_room, log, rel_l1,
                        run_attn, to_bits, to_dev)

pytestmark = pytest.mark.gpu

SWEEP_SEED = 7321
N_CASES = 64
PATHS = {"auto": fb.PATH_AUTO, "two_pass": fb.PATH_TWO_PASS, "fused": fb.PATH_FUSED}


def draw_case(n: int):
    """Case n: (workload, path name, variant, V's type, input layout)."""
    rng = np.random.default_rng([SWEEP_SEED, n])
    recipe = str(rng.choice(["segments", "grf2d", "grf3d", "ar1"]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    B = int(rng.choice([1, 1, 2]))
    H_kv = int(rng.choice([1, 2]))
    H = H_kv * int(rng.choice([1, 2, 4]))
    grid, text = None, 0
    if recipe == "grf2d":
        hg, wg = (int(x) for x in rng.integers(6, 41, 2))
        text = int(rng.choice([0, 17, 64]))
        grid, N = (hg, wg), text + hg * wg
    elif recipe == "grf3d":
        t = int(rng.integers(2, 7))
        hg, wg = (int(x) for x in rng.integers(6, 20, 2))
        grid, N = (t, hg, wg), t * hg * wg
    else:
        # half near a multiple of the 64-key tile, half anywhere
        if rng.random() < 0.5:
            N = max(1, int(rng.integers(1, 65)) * 64 + int(rng.integers(-2, 3)))
        else:
            N = int(rng.integers(1, 2600))
    causal = bool(rng.integers(2))
    tau = float(np.round(rng.uniform(0.5, 0.99), 3))
    theta = float(np.round(rng.uniform(0.2, 0.9), 2))
    lam = float(rng.choice([-0.25, -0.5, -1.0, -2.0, -4.0, -6.0, -10.0, -20.0, -math.inf]))
    path = str(rng.choice(list(PATHS)))
    variant = str(rng.choice(["", "", "int8", "fp8", "int8fp8"]))
    v_dtype = str(rng.choice(["f16", "bf16"])) if variant.startswith("int8") else dtype
    # a third of the cases pass Q, K and V with the strides of [B, N, H, d]
    layout = str(rng.choice(["bhnd", "bhnd", "bnhd"]))
    w = I.Workload(900 + n, f"sweep{n}", B, H, H_kv, N, d, dtype, causal, tau, theta, lam, recipe,
                   grid=grid, text_tokens=text)
    return w, path, variant, v_dtype, layout


def _label(n: int) -> str:
    w, path, variant, v_dtype, layout = draw_case(n)
    return (f"{n:02d}-{w.recipe}-B{w.B}H{w.H}kv{w.H_kv}-N{w.N}-d{w.d}-{w.dtype}{'-causal' if w.causal else ''}"
            f"-{path}{'-' + variant if variant else ''}{'-' + layout if layout != 'bhnd' else ''}")


@pytest.mark.parametrize("n", range(N_CASES), ids=[_label(n) for n in range(N_CASES)])
def test_random_configuration_matches_oracle(n):
    w, path, variant, v_dtype, layout = draw_case(n)
    int8 = variant.startswith("int8")
    fp8 = variant.endswith("fp8")
    log(f"[sweep {n}] {_label(n)} tau={w.tau} theta={w.theta} lam={w.lam} V {v_dtype}")
    q, k, v = I.make_qkv(w, v_dtype=v_dtype)
    Q, K = O.widen(q, w.dtype), O.widen(k, w.dtype)
    V = O.widen(v, v_dtype)
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, v_dtype)
    if layout == "bnhd":     # the same values, token stride H * d, head stride d
        qd, kd, vd = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (qd, kd, vd))

    with attn_path(PATHS[path]):
        mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
        kw, quant = {}, None
        qa, ka = qd, kd
        if int8:
            qa, ka, qs, ks = fb.quant_qk_int8(qd, kd)
            kw = dict(q_scale=qs, k_scale=ks)
            quant = O.quantize_qk(Q, K)
        if fp8:
            kw["fp8_pv"] = True
        o, o32, counts, dbg = run_attn(qa, ka, vd, mask, w.lam, w.causal, **kw)

    mrep = check_mask(mask, Q, K, w.tau, w.theta, w.causal)
    mg = mask.mg.cpu().numpy().astype(bool)
    if fp8:
        gdec = dbg.cpu().numpy().astype(np.int8)
        ref, cnt, _ = O.sparse_attention(Q, K, V, mg, w.lam, w.causal, skip_override=gdec, quant=quant, pv8=True)
        blocks = [(b, h, i) for b in range(w.B) for h in range(w.H) for i in range(O.num_blocks(w.N, O.BQ))]
        room = fp8_room(Q, K, V, mg, w.causal, gdec, blocks, quant=quant, ref=ref)
        rep = check_fp8(o32.cpu().double().numpy(), ref, room)
        c = fb.counts_dict(counts)
        for key in O.COUNT_NAMES:
            assert c[key] == cnt[key], (key, c, cnt)
        assert rel_l1(ref, O.widen(to_bits(o), v_dtype)) <= FP8_REL_L1
    else:
        rep = check_attention(o32, counts, dbg, Q, K, V, mg, w.lam, w.causal, "f32", quant=quant, int8=int8,
                              o16=o, o16_dtype=v_dtype)
    log(f"   mask: ambiguous={mrep['ambiguous']} near_theta={mrep['near_theta']}; "
        f"attn: rel_l1={rep['rel_l1']:.2e} cos={rep['cos']:.6f} max_abs={rep['max_abs']:.2e}; "
        f"counts {fb.counts_dict(counts)}")
