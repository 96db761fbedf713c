"""The whole hot path (sparge_predict_mask, then sparge_attn) captured in one
HIP graph and replayed.  The library issues no allocation, memset or
synchronisation, and every call rewrites whatever scratch it later reads
(packs, queues, partial counters, the path flag, the pilot's counts), so a
graph of its launches replays like the eager calls: every replay must give
the eager bits, with other eager work and synchronisations between the
replays, and again after the inputs are rewritten in place.
"""
from __future__ import annotations

import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import free_block_sparse_mask_amd as fb
from free_block_sparse_mask_amd import inputs as I

from gpu_common import attn_path, log, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", 0, {}),
    ("llm_gqa_ragged_causal", 2, {"N": 3000, "H": 4, "H_kv": 2}),
    ("video_small", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}),
]
PATHS = [(fb.PATH_AUTO, "auto"), (fb.PATH_TWO_PASS, "two_pass"), (fb.PATH_FUSED, "fused")]


def _inputs(w, seed_wid):
    q, k, v = I.make_qkv(w.with_sizes(wid=seed_wid))
    return tuple(to_dev(x, w.dtype) for x in (q, k, v))


def _outputs(mask, o, counts):
    return [mask.mg, mask.row_cnt, mask.row_idx, o, counts]


def _same(got, ref):
    """Equal M_g, counts, output and counters, and equal lists: a row's list
    holds row_cnt entries, and the rest of its slots are never written."""
    mg, cnt, idx, o, counts = got
    rmg, rcnt, ridx, ro, rcounts = ref
    if not (torch.equal(mg, rmg) and torch.equal(cnt, rcnt) and torch.equal(o, ro) and torch.equal(counts, rcounts)):
        return False
    valid = torch.arange(idx.shape[-1], device=idx.device) < cnt.unsqueeze(-1).to(torch.int64)
    return torch.equal(idx[valid], ridx[valid])


@pytest.mark.parametrize("path,pname", PATHS, ids=[p[1] for p in PATHS])
@pytest.mark.parametrize("label,wid,over,variant", [c + (None,) for c in CASES] + [
    ("llm_gqa_ragged_causal_int8", 2, {"N": 3000, "H": 4, "H_kv": 2}, "int8"),
    ("video_small_fp8", 3, {"N": 4 * 16 * 12, "H": 2, "H_kv": 1, "grid": (4, 16, 12)}, "fp8"),
], ids=[c[0] for c in CASES] + ["llm_gqa_ragged_causal_int8", "video_small_fp8"])
def test_graph_replay_matches_eager(label, wid, over, variant, path, pname):
    """Also with int8 Q/K (quantisation inside the graph) and with fp8 P~V."""
    w = I.workload(wid, **over)
    qd, kd, vd = _inputs(w, w.wid)
    if variant == "int8":
        vd = vd.float().to(torch.float16)
    ws = torch.empty_like(fb.workspace(qd, kd))

    def run(q, k, v):
        if variant == "int8":
            v = v.float().to(torch.float16) if v.dtype != torch.float16 else v
        mask = fb.predict_mask(q, k, w.tau, w.theta, w.causal, ws=ws)
        kw = {}
        if variant == "int8":
            q, k, qs, ks = fb.quant_qk_int8(q, k, ws=ws)
            kw = dict(q_scale=qs, k_scale=ks)
        elif variant == "fp8":
            kw = dict(fp8_pv=True)
        o, counts, _ = fb.attn(q, k, v, mask, w.lam, w.causal, ws=ws, **kw)
        return mask, o, counts

    with attn_path(path):
        ref = [t.clone() for t in _outputs(*run(qd, kd, vd))]
        torch.cuda.synchronize()
        # the first calls on a side stream, as torch asks before a capture
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run(qd, kd, vd)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            captured = _outputs(*run(qd, kd, vd))

        # other data for the eager work between replays and for the rewrite
        q2, k2, v2 = _inputs(w, w.wid + 90)
        ref2 = [t.clone() for t in _outputs(*run(q2, k2, v2))]
        torch.cuda.synchronize()
        assert not _same(ref2, ref)

        for rep in range(3):
            graph.replay()
            torch.cuda.synchronize()
            assert _same(captured, ref), f"replay {rep} differs from the eager call"
            # eager work on the same workspace between replays
            assert _same([t.clone() for t in _outputs(*run(q2, k2, v2))], ref2)
            torch.cuda.synchronize()

        # the inputs rewritten in place: the replay computes on the new data
        qd.copy_(q2)
        kd.copy_(k2)
        vd.copy_(v2)
        for rep in range(2):
            graph.replay()
            torch.cuda.synchronize()
            assert _same(captured, ref2), f"replay {rep} on rewritten inputs differs"

        # launch cost: eager calls against replays, same stream, same work
        n = 20
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            run(qd, kd, vd)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(n):
            graph.replay()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
    log(f"[graph] {label} {pname}: eager {1e3 * (t1 - t0) / n:.3f} ms/call, replay {1e3 * (t2 - t1) / n:.3f} ms/call, "
        f"counts {fb.counts_dict(ref[4])}")
