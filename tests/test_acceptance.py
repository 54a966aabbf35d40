"""The routing acceptance rule (tests/moe_check.py) on hand-made logits, on
the CPU: exact ids pass; a different selected set passes only on a boundary
near tie (k-th and (k+1)-th oracle logits within 1e-3 relative) and only if
it is a valid top-k; a slot-order swap passes only between near-equal
logits; anything else fails."""
import numpy as np
import pytest

from moe_check import check_routing

L = np.array([[5.0, 4.0, 3.0, 1.0],          # clear margins everywhere
              [5.0, 4.0, 3.9999, 1.0],       # 2nd/3rd near tie: the k = 2 boundary
              [5.0, 4.9999, 3.0, 1.0]])      # 1st/2nd near tie: inside the top 2


def weights(ids):
    import oracle
    return oracle.gate_weights(L, np.asarray(ids, np.int64))


def test_exact_ids_pass():
    ids = [[0, 1], [0, 1], [0, 1]]
    assert check_routing(np.array(ids), weights(ids), L, 2) == (0, 0)


def test_boundary_swap_on_near_tie_is_excused():
    ids = [[0, 1], [0, 2], [0, 1]]
    assert check_routing(np.array(ids), weights(ids), L, 2) == (1, 0)


def test_within_swap_between_near_equal_slots_is_excused():
    ids = [[0, 1], [0, 1], [1, 0]]
    assert check_routing(np.array(ids), weights(ids), L, 2) == (0, 1)


@pytest.mark.parametrize("ids", [
    [[0, 2], [0, 1], [0, 1]],     # set change without a near tie
    [[1, 0], [0, 1], [0, 1]],     # slot swap of clearly different logits
    [[0, 1], [0, 3], [0, 1]],     # near tie at the boundary, but 3 is not a valid 2nd
    [[0, 1], [2, 1], [0, 1]],     # a near tie elsewhere does not excuse dropping expert 0
])
def test_other_mismatches_fail(ids):
    with pytest.raises(AssertionError):
        check_routing(np.array(ids), weights(ids), L, 2)


def test_gate_weights_are_checked():
    ids = [[0, 1], [0, 1], [0, 1]]
    w = weights(ids)
    w[0, 0] += 2e-3
    with pytest.raises(AssertionError):
        check_routing(np.array(ids), w, L, 2)


@pytest.mark.parametrize("ids,kinds", [
    ([[0, 1], [0, 1], [0, 1]], (0, 0, 0)),
    ([[0, 1], [0, 2], [0, 1]], (1, 0, 0)),     # boundary near tie
    ([[0, 1], [0, 1], [1, 0]], (0, 1, 0)),     # near-equal slots swapped
    ([[0, 2], [0, 1], [0, 1]], (0, 0, 1)),     # set change without a near tie
    ([[1, 0], [0, 1], [0, 1]], (0, 0, 1)),     # slot swap of clearly different logits
])
def test_bench_counts_follow_the_rule(ids, kinds):
    """bench.py's near-tie counts (its oracle check) sort mismatches the way
    the rule above does: what the rule excuses is counted as boundary or
    within, what it fails as other."""
    import bench
    import oracle
    ref = oracle.topk_ids(L, 2)
    got = bench.classify_ids(np.array(ids), ref, L, oracle.boundary_near_tie(L, 2))
    assert (got["boundary"], got["within"], got["other"]) == kinds


def test_bench_shape_option():
    """bench.py --shape builds a layer of the given shape (bf16 by default)."""
    import argparse

    import bench
    cfg = bench.workload(argparse.Namespace(shape="64,4096,8,2,14336", config="mixtral_bf16"))
    assert (cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.dtype) == (64, 4096, 8, 2, 14336, "bf16")
    cfg = bench.workload(argparse.Namespace(shape="70,72,6,3,40,f32", config="mixtral_bf16"))
    assert (cfg.T, cfg.dtype) == (70, "f32")
    assert bench.workload(argparse.Namespace(shape=None, config="skewed_bf16")).bias0 == 3.0
    with pytest.raises(SystemExit):
        bench.workload(argparse.Namespace(shape="1,2,3", config="mixtral_bf16"))
