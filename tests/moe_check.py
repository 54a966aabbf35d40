"""Acceptance checks of the HIP path against the fp64 oracle (test helpers).

Routing acceptance: the GPU's expert ids must equal the oracle's bit for bit,
except on tokens where the oracle's own logits make another answer equally
correct within a relative gap of 1e-3 (a "near tie").  Such a token is
excused only if the GPU's choice is itself a valid top-k under that gap:
its k ids are distinct, their oracle logits are in descending slot order up
to the gap, and no unselected expert beats the last selected one by more
than the gap.  Excused tokens are counted and reported, split into
"boundary" (the selected set differs) and "within" (same set, two
near-equal slots swapped).

Gate weights are compared with the oracle's fp64 softmax over the GPU's ids,
and y with the oracle's layer driven by the GPU's ids (so a legitimate
near-tie choice does not count as an output error).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

REL_GAP = 1e-3
W_ATOL = 1e-3
TOL = {"bf16": 2e-2, "f32": 1e-4}


def f64(t):
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def _gap(a, b):
    return REL_GAP * max(abs(a), abs(b))


def valid_topk(l_row: np.ndarray, ids_row: np.ndarray) -> bool:
    k = len(ids_row)
    if len(set(ids_row.tolist())) != k or ids_row.min() < 0 or ids_row.max() >= len(l_row):
        return False
    s = l_row[ids_row]
    for j in range(k - 1):
        if s[j] < s[j + 1] - _gap(s[j], s[j + 1]):
            return False
    rest = np.setdiff1d(np.arange(len(l_row)), ids_row)
    if rest.size and l_row[rest].max() > s[-1] + _gap(l_row[rest].max(), s[-1]):
        return False
    return True


def check_routing(ids_gpu: np.ndarray, w_gpu: np.ndarray, logits_ref: np.ndarray, k: int,
                  gating: str = "topk_softmax"):
    """Assert the routing acceptance rule; return (n_boundary, n_within)."""
    ids_ref = oracle.topk_ids(logits_ref, k)
    ids_gpu = np.asarray(ids_gpu, np.int64)
    bad = np.nonzero((ids_gpu != ids_ref).any(axis=1))[0]
    n_boundary = n_within = 0
    for t in bad:
        assert valid_topk(logits_ref[t], ids_gpu[t]), (
            f"token {t}: ids {ids_gpu[t].tolist()} vs oracle {ids_ref[t].tolist()}, logits "
            f"{np.sort(logits_ref[t])[::-1][:k + 1].tolist()}")
        if set(ids_gpu[t].tolist()) == set(ids_ref[t].tolist()):
            n_within += 1
        else:
            n_boundary += 1
    w_ref = oracle.gate_weights(logits_ref, ids_gpu, gating)
    err = np.abs(np.asarray(w_gpu, np.float64) - w_ref).max()
    assert err <= W_ATOL, f"gate weights differ by {err}"
    return n_boundary, n_within


def assert_close_rel(got: np.ndarray, ref: np.ndarray, tol: float, what: str):
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= tol * scale, f"{what}: max|err| {err:.3e} > {tol} * max|ref| {scale:.3e}"
    return err / scale if scale else err


def gpu_layer(cfg, device="cuda"):
    import moe_inputs as mi
    return mi.make_inputs(cfg, device)


def expert_getters(layer):
    """Callables e -> fp64 numpy weights of one expert (converted on demand)."""
    return (lambda e: f64(layer["w1"][e])), (lambda e: f64(layer["w2"][e]))


def sample_tokens(T: int, extra=(), n_random: int = 24, seed: int = 0) -> np.ndarray:
    g = np.random.default_rng(seed)
    base = set(range(min(T, 8))) | set(range(max(0, T - 8), T))
    base |= set(g.choice(T, size=min(T, n_random), replace=False).tolist())
    base |= set(int(t) for t in extra)
    return np.array(sorted(base), dtype=np.int64)
