"""Pins of the oracle's backward (CPU only).

The backward is pinned to things other than its own arithmetic:
  * central finite differences of the oracle's forward (which shares none of
    the backward's formulas) for every entry of every gradient, on tiny
    layers whose routing margins keep the top-k choice fixed under the step;
  * torch autograd of the dense MLP (E = 1, top_k = 1, where the layer is
    GELU(x W1) W2 and the gate is constant 1);
  * torch autograd of torch's tanh-GELU for the GELU derivative;
  * the softmax invariant: each token's logit gradients sum to zero.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle


def _layer(T, H, E, F, seed, bias):
    g = np.random.default_rng(seed)
    return {
        "x": g.standard_normal((T, H)),
        "w_r": g.standard_normal((H, E)),
        "b_r": g.standard_normal(E) if bias else None,
        "w1": g.standard_normal((E, H, F)) / np.sqrt(H),
        "w2": g.standard_normal((E, F, H)) / np.sqrt(F),
    }


def _margin_ok(L, k, rel=1e-3):
    """No near tie at the top-k boundary (the choice is fixed under a small step)."""
    E = L["w_r"].shape[1]
    if k >= E:
        return True
    logits = oracle.router_logits(L["x"], L["w_r"], L["b_r"])
    s = -np.sort(-logits, axis=1)
    return bool(np.all(s[:, k - 1] - s[:, k] > rel))


def _loss(L, k, dy, gating, capacity):
    y = oracle.forward(L["x"], L["w_r"], L["b_r"], L["w1"], L["w2"], k, gating=gating,
                       capacity=capacity)["y"]
    return float((dy * y).sum())


def _fd_grad(L, name, k, dy, gating, capacity, eps=1e-6):
    a = L[name]
    grad = np.zeros_like(a)
    it = np.nditer(a, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        keep = a[idx]
        a[idx] = keep + eps
        lp = _loss(L, k, dy, gating, capacity)
        a[idx] = keep - eps
        lm = _loss(L, k, dy, gating, capacity)
        a[idx] = keep
        grad[idx] = (lp - lm) / (2 * eps)
    return grad


CASES = [
    # (T, H, E, k, F, gating, capacity, bias, seed)
    (5, 6, 4, 2, 7, "topk_softmax", 0, False, 1),
    (5, 6, 4, 2, 7, "topk_softmax", 0, True, 2),
    (6, 5, 4, 2, 6, "softmax_topk", 0, True, 3),
    (8, 4, 3, 2, 5, "topk_softmax", 3, False, 4),     # capacity drops pairs
    (8, 4, 3, 2, 5, "softmax_topk", 3, True, 5),
    (4, 5, 5, 3, 4, "topk_softmax", 0, False, 6),     # k = 3
    (4, 3, 3, 1, 4, "topk_softmax", 0, True, 7),      # k = 1: no router gradient
]


@pytest.mark.parametrize("T,H,E,k,F,gating,capacity,bias,seed", CASES)
def test_backward_matches_finite_differences(T, H, E, k, F, gating, capacity, bias, seed):
    for s in range(seed, seed + 50):
        L = _layer(T, H, E, F, s, bias)
        if _margin_ok(L, k):
            break
    else:
        pytest.fail("no draw with clear routing margins")
    dy = np.random.default_rng(100 + seed).standard_normal((T, H))
    if capacity:
        _, _, _, inv = oracle.dispatch(oracle.topk_ids(
            oracle.router_logits(L["x"], L["w_r"], L["b_r"]), k), E, capacity)
        assert (inv < 0).any(), "case meant to drop pairs drops none"
    g = oracle.backward(L["x"], L["w_r"], L["b_r"], L["w1"], L["w2"], k, dy, gating=gating,
                        capacity=capacity)
    names = [("x", "dx"), ("w_r", "dw_r"), ("w1", "dw1"), ("w2", "dw2")]
    if bias:
        names.append(("b_r", "db_r"))
    for name, gname in names:
        fd = _fd_grad(L, name, k, dy, gating, capacity)
        scale = max(1.0, np.abs(fd).max())
        err = np.abs(g[gname] - fd).max()
        assert err <= 1e-6 * scale, f"{gname}: max|analytic - fd| = {err:.3e}"


def test_backward_k1_has_no_router_gradient():
    L = _layer(6, 5, 4, 3, 11, True)
    dy = np.random.default_rng(0).standard_normal((6, 5))
    g = oracle.backward(L["x"], L["w_r"], L["b_r"], L["w1"], L["w2"], 1, dy)
    assert np.all(g["w"] == 1.0)
    assert np.abs(g["dlogits"]).max() == 0.0
    assert np.abs(g["dw_r"]).max() == 0.0 and np.abs(g["db_r"]).max() == 0.0


def test_backward_dense_mlp_matches_autograd():
    """E = 1, k = 1: the layer is GELU(x W1) W2 and every gate weight is 1."""
    T, H, F = 7, 6, 9
    L = _layer(T, H, 1, F, 21, False)
    dy = np.random.default_rng(3).standard_normal((T, H))
    g = oracle.backward(L["x"], L["w_r"], None, L["w1"], L["w2"], 1, dy)
    x = torch.tensor(L["x"], requires_grad=True)
    w1 = torch.tensor(L["w1"][0], requires_grad=True)
    w2 = torch.tensor(L["w2"][0], requires_grad=True)
    y = torch.nn.functional.gelu(x @ w1, approximate="tanh") @ w2
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(g["dx"], x.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw1"][0], w1.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw2"][0], w2.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_gelu_grad_matches_autograd():
    z = torch.linspace(-9.0, 9.0, 2001, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(z, approximate="tanh").sum().backward()
    np.testing.assert_allclose(oracle.gelu_tanh_grad(z.detach().numpy()), z.grad.numpy(),
                               rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("gating", ["topk_softmax", "softmax_topk"])
def test_logit_gradients_sum_to_zero(gating):
    """Softmax outputs are invariant to adding one constant to every logit of a
    token, so each token's logit gradients sum to zero (both gatings)."""
    g = np.random.default_rng(5)
    logits = g.standard_normal((40, 16))
    ids = oracle.topk_ids(logits, 4)
    dw = g.standard_normal((40, 4))
    dl = oracle.gate_weights_grad(logits, ids, dw, gating)
    assert np.abs(dl.sum(axis=1)).max() < 1e-14
    if gating == "topk_softmax":
        mask = np.zeros_like(dl, dtype=bool)
        mask[np.arange(40)[:, None], ids] = True
        assert np.abs(dl[~mask]).max() == 0.0


def test_logit_gradient_is_linear_in_dw():
    g = np.random.default_rng(6)
    logits = g.standard_normal((10, 8))
    ids = oracle.topk_ids(logits, 2)
    a, b = g.standard_normal((10, 2)), g.standard_normal((10, 2))
    for gating in ("topk_softmax", "softmax_topk"):
        lhs = oracle.gate_weights_grad(logits, ids, 2 * a - b, gating)
        rhs = 2 * oracle.gate_weights_grad(logits, ids, a, gating) - \
            oracle.gate_weights_grad(logits, ids, b, gating)
        assert np.abs(lhs - rhs).max() < 1e-13


def test_expert_ffn_backward_matches_finite_differences():
    """The dispatched-rows form: L = sum(dyp * expert_ffn(xp, offsets, W1, W2)),
    with an expert that has no rows (zero weight gradients)."""
    g = np.random.default_rng(8)
    E, H, F = 4, 5, 6
    offsets = np.array([0, 3, 3, 7, 9])
    xp = g.standard_normal((9, H))
    w1 = g.standard_normal((E, H, F)) / np.sqrt(H)
    w2 = g.standard_normal((E, F, H)) / np.sqrt(F)
    dyp = g.standard_normal((9, H))
    dxp, dw1, dw2 = oracle.expert_ffn_backward(xp, offsets, w1, w2, dyp)
    arrays = {"xp": xp, "w1": w1, "w2": w2}

    def loss():
        return float((dyp * oracle.expert_ffn(arrays["xp"], offsets, arrays["w1"],
                                              arrays["w2"])).sum())

    for name, grad in (("xp", dxp), ("w1", dw1), ("w2", dw2)):
        a = arrays[name]
        fd = np.zeros_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            keep = a[i]
            a[i] = keep + 1e-6
            lp = loss()
            a[i] = keep - 1e-6
            lm = loss()
            a[i] = keep
            fd[i] = (lp - lm) / 2e-6
        assert np.abs(grad - fd).max() <= 1e-6 * max(1.0, np.abs(fd).max()), name
    assert np.abs(dw1[1]).max() == 0.0 and np.abs(dw2[1]).max() == 0.0
