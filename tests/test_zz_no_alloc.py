"""GPU check of sparge_attn_noalloc, the attention entry point that allocates
nothing (its scratch is the library's static device array): two calls in a
row through the C ABI, the second on a smaller problem, each against
sparge_attn with a workspace of its own (the same bits, counters and
decisions) and against the float64 oracle (the parity bar of sparge_attn).
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from oracle import sparge_oracle as O

from gpu_common import check_attention, log, to_dev

pytestmark = pytest.mark.gpu


def _one(w, lists):
    q, k, v = I.make_qkv(w)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (q, k, v))
    mask = fb.predict_mask(qd, kd, w.tau, w.theta, w.causal)
    m = mask if lists else mask.mg
    o_ws, c_ws, d_ws = fb.attn(qd, kd, vd, m, w.lam, w.causal, dbg=True, out_f32=True)
    o_na, c_na, d_na = fb.attn(qd, kd, vd, m, w.lam, w.causal, dbg=True, out_f32=True, noalloc=True)
    o16_na, _, _ = fb.attn(qd, kd, vd, m, w.lam, w.causal, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws), "sparge_attn_noalloc differs from sparge_attn"
    assert torch.equal(c_na, c_ws) and torch.equal(d_na, d_ws)
    assert torch.equal(o16_na, o_na.to(o16_na.dtype))
    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    rep = check_attention(o_na, c_na, d_na, Q, K, V, mask.mg.cpu().numpy().astype(bool), w.lam, w.causal, "f32",
                          o16=o16_na, o16_dtype=w.dtype)
    log(f"[noalloc] N={w.N} H={w.H} Hkv={w.H_kv} lists={lists}: equal to sparge_attn; vs oracle "
        f"max_abs={rep['max_abs']:.2e} rel_l1={rep['rel_l1']:.2e} counts={rep['counts']}")


def test_noalloc_equals_workspace_entry_point_twice():
    # the second call is smaller, so the array still holds the first call's larger contents
    _one(I.workload(2, N=3000, H=4, H_kv=2), lists=True)
    _one(I.workload(2, N=700, H=2, H_kv=1), lists=False)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    w = I.workload(2, N=70000, H=8, H_kv=2)
    qd = torch.zeros((1, 8, w.N, 128), dtype=torch.bfloat16, device="cuda:0")
    kd = torch.zeros((1, 2, w.N, 128), dtype=torch.bfloat16, device="cuda:0")
    mg = torch.ones((1, 8, O.num_blocks(w.N, 128), O.num_blocks(w.N, 64)), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(fb.SpargeError) as e:
        fb.attn(qd, kd, kd, mg, -5.0, True, noalloc=True)
    assert e.value.code == fb.SPARGE_EWORKSPACE
