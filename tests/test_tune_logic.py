"""CPU checks of the hyper-parameter search logic (free_block_sparse_mask_amd.tune):
the two-level rule as a bisection, on synthetic monotone error curves, and the
sparsity measure from the kernel counters.  No GPU: the evaluations are plain
functions here; the GPU test runs the same search on the HIP path and checks
its result with the oracle."""
import math

import pytest

from free_block_sparse_mask_amd.tune import sparsity_from_counts, two_level_search


def _curve(err_of_x, spars_of_x, log):
    def f(x):
        log.append(x)
        return err_of_x(x), spars_of_x(x)
    return f


def test_rule_moves_towards_sparsity_while_error_is_below_l1():
    # tau-like: x from 1 (dense) to 0.05 (sparse); L1 = (1 - x)^2 / 4
    log = []
    f = _curve(lambda x: (1 - x) ** 2 / 4, lambda x: 1 - x, log)
    x, e, s, ok, trace = two_level_search(f, 1.0, 0.05, 0.05, 0.06, iters=20)
    assert ok and 0.05 <= e <= 0.06
    # the answer solves (1 - x)^2 / 4 in [0.05, 0.06]
    assert 1 - math.sqrt(0.24) <= x <= 1 - math.sqrt(0.20)
    # every step after the two ends follows the rule: below l1 -> sparser next
    pts = [t[0] for t in trace]
    assert pts[0] == 1.0 and pts[1] == 0.05
    for (x0, e0, _), x1 in zip(trace[2:], pts[3:]):
        if e0 < 0.05:
            assert x1 < x0          # moved towards the sparse end
        elif e0 > 0.06:
            assert x1 > x0          # moved back towards the dense end


def test_sparse_end_accepted_when_within_l2():
    f = _curve(lambda x: 0.01 * (1 - x), lambda x: 1 - x, [])
    x, e, s, ok, trace = two_level_search(f, 1.0, 0.0, 0.05, 0.06)
    assert ok and x == 0.0 and len(trace) == 2


def test_dense_end_kept_when_its_error_is_already_in_band():
    f = _curve(lambda x: 0.055, lambda x: 0.0, [])
    x, e, s, ok, trace = two_level_search(f, -40.0, -0.5, 0.05, 0.06)
    assert ok and x == -40.0 and len(trace) == 1


def test_infeasible_when_even_the_dense_end_exceeds_l2():
    f = _curve(lambda x: 0.5, lambda x: 0.0, [])
    x, e, s, ok, trace = two_level_search(f, 1.0, 0.05, 0.05, 0.06)
    assert not ok and x == 1.0 and e == 0.5


def test_lambda_direction_and_best_feasible_point():
    # lambda-like: x from -40 (dense) to -0.5 (sparse), a step in the error at -3
    f = _curve(lambda x: 0.01 if x < -3.0 else 0.2, lambda x: (x + 40) / 39.5, [])
    x, e, s, ok, trace = two_level_search(f, -40.0, -0.5, 0.05, 0.06, iters=12)
    # the band [l1, l2] is never hit: the sparsest point below l1 is returned
    assert ok and e == 0.01 and -3.2 < x < -3.0
    assert all(t[1] <= 0.06 or t[0] >= -3.0 for t in trace)


def test_bad_bounds_are_rejected():
    with pytest.raises(ValueError):
        two_level_search(lambda x: (0.0, 0.0), 1.0, 0.0, 0.1, 0.05)


def test_sparsity_from_counts_closed_forms():
    d = 128
    dense = dict(live_tiles=10, qk_exec=10, pv_exec=40)      # 4 row groups per 128-row block
    assert abs(sparsity_from_counts(dense, d)) < 1e-15
    none = dict(live_tiles=10, qk_exec=0, pv_exec=0)
    assert sparsity_from_counts(none, d) == 1.0
    # QK on every tile, P~V skipped everywhere: half the work
    half = dict(live_tiles=10, qk_exec=10, pv_exec=0)
    assert abs(sparsity_from_counts(half, d) - 0.5) < 1e-15
    assert sparsity_from_counts(dict(live_tiles=0, qk_exec=0, pv_exec=0), d) == 0.0
