"""The whole path driven from C alone: tests/c/attn_from_c.c (built by
__graft_entry__.build()) allocates device memory with the HIP runtime and
calls sparge_predict_mask and sparge_attn through include/sparge.h, with no
Python or torch in its process.  Its mask, decisions, output and counters
meet the same acceptance against the oracle as the Python-driven cases."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I
from oracle import sparge_oracle as O

from gpu_common import check_attention, log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = os.path.join(ROOT, "tests", "c", "_bin", "attn_from_c")

CASES = [
    # label, workload, overrides
    ("llm_gqa_ragged_causal", 2, {"N": 1500, "H": 4, "H_kv": 2}),
    ("video_small", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}),
]


@pytest.mark.parametrize("label,wid,over", CASES, ids=[c[0] for c in CASES])
def test_c_program_matches_oracle(label, wid, over, tmp_path):
    if not os.path.exists(PROGRAM):
        pytest.skip(f"{PROGRAM} is not built: __graft_entry__.build() builds it")
    w = I.workload(wid, dtype="bf16", **over)
    q, k, v = I.make_qkv(w)
    for name, x in (("q", q), ("k", k), ("v", v)):
        np.ascontiguousarray(x).tofile(str(tmp_path / f"{name}.bin"))
    args = [PROGRAM, str(tmp_path), str(w.B), str(w.H), str(w.H_kv), str(w.N), str(w.d), str(int(w.causal)),
            repr(w.tau), repr(w.theta), repr(w.lam)]
    log(f"[c program] {label}: {' '.join(args[2:])}")
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr

    Tm, Tn = O.num_blocks(w.N, O.BQ), O.num_blocks(w.N, O.BK)
    groups = O.BQ // fb.rows_per_wave()
    mg = np.fromfile(str(tmp_path / "mg.bin"), dtype=np.uint8).reshape(w.B, w.H, Tm, Tn).astype(bool)
    o = np.fromfile(str(tmp_path / "o.bin"), dtype=np.float32).reshape(w.B, w.H, w.N, w.d)
    counts = np.fromfile(str(tmp_path / "counts.bin"), dtype=np.int64)
    dbg = np.fromfile(str(tmp_path / "dbg.bin"), dtype=np.uint8).reshape(w.B, w.H, Tm, Tn, groups)

    Q, K, V = (O.widen(x, w.dtype) for x in (q, k, v))
    ref = O.predict_mask(Q, K, w.tau, w.theta, w.causal)
    assert not ((mg != ref["mg"]) & ~ref["ambiguous"]).any()
    rep = check_attention(torch.from_numpy(o), torch.from_numpy(counts), torch.from_numpy(dbg), Q, K, V, mg,
                          w.lam, w.causal, "f32")
    log(f"   rel_l1={rep['rel_l1']:.2e} max_abs={rep['max_abs']:.2e} counts {rep['counts']}")
