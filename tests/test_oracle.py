"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics:
hand-worked fixtures, closed forms, library routines for special cases, brute
force on tiny inputs and invariants.  CPU only."""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _rand_layer(T, H, E, F, seed=0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((T, H)), g.standard_normal((H, E)) / math.sqrt(H),
            g.standard_normal((E, H, F)) / math.sqrt(H), g.standard_normal((E, F, H)) / math.sqrt(F))


# --- GELU ---------------------------------------------------------------------

def test_gelu_matches_torch_tanh_gelu():
    z = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(z), ref, rtol=1e-14, atol=1e-15)


def test_gelu_is_tanh_form_not_erf_form():
    # the tanh form differs from the erf form by at most ~4.7e-4 (near |z| 2.7),
    # and by more than 1e-4 somewhere: pins the form, not just "a GELU"
    z = np.linspace(-6, 6, 24001)
    erf_form = 0.5 * z * (1 + scipy.special.erf(z / math.sqrt(2)))
    d = np.abs(oracle.gelu_tanh(z) - erf_form)
    assert 3e-4 < d.max() < 5e-4


def test_gelu_closed_forms():
    z = np.linspace(-5, 5, 1001)
    g = oracle.gelu_tanh(z)
    # g(z) - g(-z) = z exactly in the tanh form (tanh is odd)
    np.testing.assert_allclose(g - oracle.gelu_tanh(-z), z, atol=1e-14)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert oracle.gelu_tanh(np.array([20.0]))[0] == 20.0
    assert oracle.gelu_tanh(np.array([-20.0]))[0] == 0.0
    # slope 1/2 at the origin
    h = 1e-6
    assert abs((oracle.gelu_tanh(np.array([h]))[0] - oracle.gelu_tanh(np.array([-h]))[0]) / (2 * h) - 0.5) < 1e-9


# --- routing ------------------------------------------------------------------

def _read_route_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "route_tiny.txt")):
        if line.startswith("#") or not line.strip():
            continue
        t, l, ids, w = [p.split() for p in line.split("|")]
        rows.append(([float(v) for v in l], [int(v) for v in ids], [float(v) for v in w]))
    return rows


def test_route_golden_hand_worked():
    rows = _read_route_golden()
    logits = np.array([r[0] for r in rows])
    x = np.eye(len(rows))
    ids, w, l = oracle.route(x, logits, None, 2)
    np.testing.assert_array_equal(l, logits)
    np.testing.assert_array_equal(ids, np.array([r[1] for r in rows]))
    np.testing.assert_allclose(w, np.array([r[2] for r in rows]), rtol=0, atol=2e-16)


def _rank_bruteforce(l, k):
    """ids by counting: rank(e) = #{e': l[e'] > l[e]} + #{e' < e: l[e'] == l[e]}."""
    E = len(l)
    rank = [sum(l[f] > l[e] for f in range(E)) + sum(l[f] == l[e] for f in range(e)) for e in range(E)]
    inv = {r: e for e, r in enumerate(rank)}
    return [inv[j] for j in range(k)]


@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (8, 8), (16, 5), (33, 8)])
def test_topk_matches_rank_counting_with_ties(E, k):
    l = RNG.integers(-3, 4, size=(40, E)).astype(np.float64)   # many exact ties
    ids = oracle.topk_ids(l, k)
    for t in range(l.shape[0]):
        assert list(ids[t]) == _rank_bruteforce(l[t], k)


def test_topk_set_maximises_the_sum():
    # the selected set is a maximum-sum k-subset, and the lexicographically
    # smallest such subset when several tie (brute force over all subsets)
    E, k = 7, 3
    l = RNG.integers(-2, 3, size=(25, E)).astype(np.float64)
    ids = oracle.topk_ids(l, k)
    for t in range(l.shape[0]):
        best = max(sum(l[t, list(c)]) for c in itertools.combinations(range(E), k))
        cands = sorted(c for c in itertools.combinations(range(E), k) if sum(l[t, list(c)]) == best)
        assert sum(l[t, ids[t]]) == best
        # lowest-index tie-break: the chosen set equals the sorted candidate that
        # prefers lower indices among the elements at the boundary value
        assert tuple(sorted(ids[t])) in cands


def test_gate_k1_is_exactly_one():
    l = RNG.standard_normal((50, 8))
    ids = oracle.topk_ids(l, 1)
    assert np.all(oracle.gate_weights(l, ids) == 1.0)


def test_gate_k2_is_logistic():
    l = RNG.standard_normal((50, 8)) * 3
    ids = oracle.topk_ids(l, 2)
    w = oracle.gate_weights(l, ids)
    d = l[np.arange(50), ids[:, 0]] - l[np.arange(50), ids[:, 1]]
    np.testing.assert_allclose(w[:, 0], scipy.special.expit(d), rtol=1e-14)
    np.testing.assert_allclose(w[:, 1], scipy.special.expit(-d), rtol=1e-13)


def test_gate_kE_is_full_softmax():
    l = RNG.standard_normal((30, 16)) * 4
    ids = oracle.topk_ids(l, 16)
    w = oracle.gate_weights(l, ids)
    full = scipy.special.softmax(l, axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids, 1), rtol=1e-13)


def test_gate_invariants():
    l = RNG.standard_normal((64, 128)) * 2
    for k in (1, 2, 8, 128):
        ids = oracle.topk_ids(l, k)
        w = oracle.gate_weights(l, ids)
        assert np.all(np.abs(w.sum(1) - 1) < 1e-15 * k + 1e-16)
        assert all(len(set(r)) == k for r in ids)          # distinct
        assert np.all((ids >= 0) & (ids < 128))
        sel = np.take_along_axis(l, ids, 1)
        assert np.all(np.diff(sel, axis=1) <= 0)           # descending
        assert np.all(np.diff(w, axis=1) <= 1e-17)


def test_router_bias_adds_to_logits():
    x = np.zeros((3, 5))
    b = np.array([3.0, 0.0, -1.0, 0.5])
    l = oracle.router_logits(x, RNG.standard_normal((5, 4)), b)
    np.testing.assert_array_equal(l, np.tile(b, (3, 1)))
    ids = oracle.topk_ids(l, 2)
    np.testing.assert_array_equal(ids, [[0, 3]] * 3)


def test_router_logits_is_the_matrix_product():
    x, w_r = RNG.standard_normal((6, 9)), RNG.standard_normal((9, 4))
    l = oracle.router_logits(x, w_r)
    for t in range(6):
        for e in range(4):
            assert abs(l[t, e] - sum(x[t, h] * w_r[h, e] for h in range(9))) < 1e-12


# --- dispatch -----------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 8, 2), (64, 8, 8), (200, 128, 8), (37, 256, 3)])
def test_dispatch_invariants(T, E, k):
    l = RNG.standard_normal((T, E))
    ids = oracle.topk_ids(l, k)
    off, st, ss, inv = oracle.dispatch(ids, E)
    R = T * k
    assert off[0] == 0 and off[-1] == R
    np.testing.assert_array_equal(np.diff(off), np.bincount(ids.ravel(), minlength=E))
    assert sorted(inv.ravel().tolist()) == list(range(R))        # bijection
    for e in range(E):
        blk = st[off[e]:off[e + 1]]
        assert np.all(np.diff(blk) > 0)                          # ascending tokens
        assert np.all(ids[blk, ss[off[e]:off[e + 1]]] == e)
    t_idx = np.repeat(np.arange(T), k)
    np.testing.assert_array_equal(st[inv.ravel()], t_idx)
    np.testing.assert_array_equal(ss[inv.ravel()], np.tile(np.arange(k), T))


def test_dispatch_hand_example():
    ids = np.array([[1, 0], [0, 2], [1, 2]])
    off, st, ss, inv = oracle.dispatch(ids, 4)
    np.testing.assert_array_equal(off, [0, 2, 4, 6, 6])
    np.testing.assert_array_equal(st, [0, 1, 0, 2, 1, 2])
    np.testing.assert_array_equal(ss, [1, 0, 0, 0, 1, 1])
    np.testing.assert_array_equal(inv, [[2, 0], [1, 4], [3, 5]])


# --- experts and the whole layer ----------------------------------------------

def _torch_mlp(x, w1, w2):
    xt, a, b = (torch.from_numpy(np.asarray(v, np.float64)) for v in (x, w1, w2))
    return (torch.nn.functional.gelu(xt @ a, approximate="tanh") @ b).numpy()


def test_single_expert_top1_is_the_dense_mlp():
    x, w_r, w1, w2 = _rand_layer(7, 12, 1, 20)
    out = oracle.forward(x, w_r, None, w1, w2, 1)
    np.testing.assert_allclose(out["y"], _torch_mlp(x, w1[0], w2[0]), rtol=1e-12, atol=1e-13)


def test_topE_is_the_dense_softmax_mixture():
    T, H, E, F = 9, 10, 5, 14
    x, w_r, w1, w2 = _rand_layer(T, H, E, F, seed=3)
    out = oracle.forward(x, w_r, None, w1, w2, E)
    p = scipy.special.softmax(x @ w_r, axis=1)
    ref = sum(p[:, e:e + 1] * _torch_mlp(x, w1[e], w2[e]) for e in range(E))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T,H,E,k,F", [(6, 8, 4, 2, 12), (16, 16, 8, 3, 24), (3, 5, 8, 8, 7), (1, 4, 6, 1, 3)])
def test_forward_equals_dense_bruteforce(T, H, E, k, F):
    x, w_r, w1, w2 = _rand_layer(T, H, E, F, seed=T + E)
    out = oracle.forward(x, w_r, None, w1, w2, k)
    y_bf = oracle.dense_bruteforce(x, w1, w2, out["ids"], out["w"], E)
    np.testing.assert_allclose(out["y"], y_bf, rtol=1e-12, atol=1e-12 * np.abs(y_bf).max())


def test_stagewise_pipeline_equals_forward():
    T, H, E, k, F = 20, 16, 8, 2, 24
    x, w_r, w1, w2 = _rand_layer(T, H, E, F, seed=7)
    ids, w, _ = oracle.route(x, w_r, None, k)
    off, st, ss, inv = oracle.dispatch(ids, E)
    yp = oracle.expert_ffn(oracle.gather_rows(x, st), off, w1, w2)
    y = oracle.combine(yp, inv, w)
    np.testing.assert_allclose(y, oracle.forward(x, w_r, None, w1, w2, k)["y"], rtol=1e-13, atol=1e-13)


def test_forward_golden_hand_worked():
    vals = {}
    for line in open(os.path.join(GOLDEN, "forward_tiny.txt")):
        if line.startswith("#") or ":" not in line:
            continue
        name, rest = line.split(":")
        vals[name.strip()] = np.array([float(v) for v in rest.split()])
    x = np.array([[1.0, 0], [0, 1]])
    w_r = np.array([[2.0, 1, 0], [0, 0, 3]])
    w1 = np.array([[[20.0, -20], [0, 0]], [[-20.0, 20], [20, 20]], [[20.0, 20], [20, -20]]])
    w2 = np.array([[[1.0, 2], [3, 4]], [[1.0, 1], [0.5, -1]], [[-1.0, 0.25], [7, 7]]])
    out = oracle.forward(x, w_r, None, w1, w2, 2)
    np.testing.assert_array_equal(out["ids"].ravel(), vals["ids"])
    np.testing.assert_allclose(out["w"].ravel(), vals["w"], rtol=0, atol=2e-16)
    np.testing.assert_allclose(out["y"].ravel(), vals["y"], rtol=0, atol=1e-13)


def test_token_permutation_equivariance():
    T, H, E, k, F = 17, 8, 6, 2, 10
    x, w_r, w1, w2 = _rand_layer(T, H, E, F, seed=11)
    perm = RNG.permutation(T)
    y = oracle.forward(x, w_r, None, w1, w2, k)["y"]
    yp = oracle.forward(x[perm], w_r, None, w1, w2, k)["y"]
    np.testing.assert_allclose(yp, y[perm], rtol=1e-13, atol=1e-14)


def test_expert_relabelling_invariance():
    T, H, E, k, F = 15, 8, 6, 3, 10
    x, w_r, w1, w2 = _rand_layer(T, H, E, F, seed=13)
    b = RNG.standard_normal(E)
    p = RNG.permutation(E)
    a = oracle.forward(x, w_r, b, w1, w2, k)
    c = oracle.forward(x, w_r[:, p], b[p], w1[p], w2[p], k)
    np.testing.assert_array_equal(p[c["ids"]], a["ids"])
    np.testing.assert_allclose(c["y"], a["y"], rtol=1e-13, atol=1e-14)


def test_forward_tokens_matches_forward():
    T, H, E, k, F = 12, 8, 8, 2, 6
    x, w_r, w1, w2 = _rand_layer(T, H, E, F, seed=5)
    out = oracle.forward(x, w_r, None, w1, w2, k)
    sel = np.array([0, 5, 11])
    ys = oracle.forward_tokens(x[sel], out["ids"][sel], out["w"][sel], lambda e: w1[e], lambda e: w2[e])
    np.testing.assert_allclose(ys, out["y"][sel], rtol=1e-13, atol=1e-14)


def test_boundary_near_tie():
    l = np.array([[5.0, 4.0, 3.9999, 0.0], [5.0, 4.0, 3.0, 0.0]])
    np.testing.assert_array_equal(oracle.boundary_near_tie(l, 2), [True, False])
    np.testing.assert_array_equal(oracle.boundary_near_tie(l, 4), [False, False])


def test_integer_inputs_give_exact_logits_in_bf16():
    inp = mi.integer_inputs(8, 64, 8, 16, -2, 2, seed=1, dtype=torch.bfloat16)
    x = inp["x"].float().numpy().astype(np.float64)
    l = oracle.router_logits(x, inp["w_r"].float().numpy().astype(np.float64))
    # fp32 accumulation of the same products is exact: |l| <= 4*64 = 256
    l32 = (inp["x"].float() @ inp["w_r"].float()).numpy()
    np.testing.assert_array_equal(l, l32.astype(np.float64))


# --- gating variant: softmax over all experts, then top-k (not renormalised) --

def _read_gating_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "gating_softmax_topk.txt")):
        if line.startswith("#") or not line.strip():
            continue
        t, l, ids, w = [p.strip() for p in line.split("|")]
        rows.append((np.array([float(v) for v in l.split()]), [int(v) for v in ids.split()],
                     np.array([float(v) for v in w.split()])))
    return rows


def test_softmax_topk_golden():
    rows = _read_gating_golden()
    W_r = np.stack([r[0] for r in rows])
    x = np.eye(4)
    ids, w, _ = oracle.route(x, W_r, None, 2, gating="softmax_topk")
    for t, (_, ids_ref, w_ref) in enumerate(rows):
        assert list(ids[t]) == ids_ref
        np.testing.assert_allclose(w[t], w_ref, rtol=1e-14)


def test_gating_variants_agree_on_selection_and_ratios():
    l = RNG.standard_normal((50, 16)) * 3
    ids = oracle.topk_ids(l, 4)
    a = oracle.gate_weights(l, ids, "topk_softmax")
    b = oracle.gate_weights(l, ids, "softmax_topk")
    # both are proportional to exp(l) of the selected experts: equal ratios
    np.testing.assert_allclose(a[:, 1:] / a[:, :1], b[:, 1:] / b[:, :1], rtol=1e-12)
    # the top-k softmax sums to one; the full softmax's top-k share is less
    np.testing.assert_allclose(a.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(b.sum(axis=1) < 1.0)
    # b is a times the selected experts' share of the full softmax
    share = np.exp(np.take_along_axis(l, ids, 1)).sum(1) / np.exp(l).sum(1)
    np.testing.assert_allclose(b, a * share[:, None], rtol=1e-12)


def test_softmax_topk_full_k_is_full_softmax():
    l = RNG.standard_normal((20, 6))
    ids = oracle.topk_ids(l, 6)
    b = oracle.gate_weights(l, ids, "softmax_topk")
    full = scipy.special.softmax(l, axis=1)
    np.testing.assert_allclose(b, np.take_along_axis(full, ids, 1), rtol=1e-13)
    np.testing.assert_allclose(b.sum(axis=1), 1.0, rtol=1e-13)


def test_softmax_topk_shift_invariant():
    l = RNG.standard_normal((10, 8))
    ids = oracle.topk_ids(l, 2)
    np.testing.assert_allclose(oracle.gate_weights(l + 100.0, ids, "softmax_topk"),
                               oracle.gate_weights(l, ids, "softmax_topk"), rtol=1e-12)


def test_unknown_gating_rejected():
    with pytest.raises(ValueError):
        oracle.gate_weights(np.zeros((1, 2)), np.zeros((1, 1), dtype=np.int64), "softmax")


# --- capacity-limited dispatch ---------------------------------------------------

def _read_capacity_golden():
    d = {}
    for line in open(os.path.join(GOLDEN, "dispatch_capacity_tiny.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, rest = line.split(None, 1)
        if "/" in rest:
            d[key] = np.array([[int(v) for v in r.split()] for r in rest.split("/")])
        elif key == "factor":
            d[key] = float(rest)
        else:
            vals = [int(v) for v in rest.split()]
            d[key] = vals[0] if len(vals) == 1 and key in ("T", "k", "E", "capacity") else np.array(vals)
    return d


def test_capacity_golden():
    g = _read_capacity_golden()
    assert oracle.expert_capacity(g["T"], g["k"], g["E"], g["factor"]) == g["capacity"]
    off, st, ss, inv = oracle.dispatch(g["ids"], g["E"], g["capacity"])
    np.testing.assert_array_equal(off, g["offsets"])
    np.testing.assert_array_equal(st, g["sorted_token"])
    np.testing.assert_array_equal(ss, g["sorted_slot"])
    np.testing.assert_array_equal(inv, g["inv_pos"])


def test_expert_capacity_values():
    # ceil(factor * T * k / E), exact: the pages' factor 1.2 at the layer shapes
    assert oracle.expert_capacity(2048, 2, 8, 1.2) == 615      # 614.4
    assert oracle.expert_capacity(4096, 8, 128, 1.2) == 308    # 307.2
    assert oracle.expert_capacity(64, 2, 8, 1.0) == 16         # exactly 16
    assert oracle.expert_capacity(64, 8, 256, 1.2) == 3        # 2.4
    assert oracle.expert_capacity(64, 2, 8, 0.0) == 0          # no limit
    assert oracle.expert_capacity(7, 1, 7, 0.5) == 1           # 0.5


def _brute_dispatch(ids, E, cap):
    """Pure-Python brute force: walk all pairs in (t, j) order, count per
    expert, keep while under the cap."""
    T, k = ids.shape
    kept = {e: [] for e in range(E)}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if cap <= 0 or len(kept[e]) < cap:
                kept[e].append((t, j))
    return kept


@pytest.mark.parametrize("cap", [0, 1, 2, 3, 5, 1000])
def test_capacity_dispatch_bruteforce(cap):
    g = np.random.default_rng(cap)
    T, k, E = 23, 3, 5
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)])
    off, st, ss, inv = oracle.dispatch(ids, E, cap)
    kept = _brute_dispatch(ids, E, cap)
    pos = 0
    for e in range(E):
        assert off[e] == pos
        for (t, j) in kept[e]:
            assert st[pos] == t and ss[pos] == j and inv[t, j] == pos
            pos += 1
    assert off[E] == pos == len(st)
    assert (inv >= 0).sum() == pos
    if cap == 0 or cap >= T:
        full = oracle.dispatch(ids, E)
        for a, b in zip(full, (off, st, ss, inv)):
            np.testing.assert_array_equal(a, b)


def test_capacity_forward_matches_dense_with_dropped_weights_zeroed():
    T, H, E, F, k = 12, 16, 4, 24, 2
    x, W_r, W1, W2 = _rand_layer(T, H, E, F, seed=7)
    cap = 3
    out = oracle.forward(x, W_r, None, W1, W2, k, capacity=cap)
    ids, w = out["ids"], out["w"]
    _, _, _, inv = oracle.dispatch(ids, E, cap)
    assert (inv < 0).any()                       # the cap really drops pairs
    w_kept = np.where(inv >= 0, w, 0.0)
    ref = oracle.dense_bruteforce(x, W1, W2, ids, w_kept, E)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    # the staged pipeline (dispatch, expert FFN, combine) agrees
    off, st, _, inv = oracle.dispatch(ids, E, cap)
    yp = oracle.expert_ffn(oracle.gather_rows(x, st), off, W1, W2)
    np.testing.assert_allclose(oracle.combine(yp, inv, w), ref, rtol=1e-12, atol=1e-12)


def test_capacity_all_dropped_token_is_zero():
    # every token on expert 0 with cap 1: only token 0 keeps its slot
    ids = np.zeros((4, 1), dtype=np.int64)
    off, st, _, inv = oracle.dispatch(ids, 2, 1)
    np.testing.assert_array_equal(off, [0, 1, 1])
    np.testing.assert_array_equal(inv[:, 0], [0, -1, -1, -1])
    y = oracle.combine(np.ones((1, 3)), inv, np.ones((4, 1)))
    np.testing.assert_array_equal(y, [[1, 1, 1], [0, 0, 0], [0, 0, 0], [0, 0, 0]])
