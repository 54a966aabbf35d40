"""Acceptance checks of the HIP path against the fp64 oracle (test helpers).

Routing acceptance: the GPU's expert ids must equal the oracle's bit for bit,
except on two kinds of token, each counted and reported:
  * "boundary": the selected set differs.  Excused only on a token whose k-th
    and (k+1)-th largest oracle logits differ by less than 1e-3 relative
    (oracle.boundary_near_tie, the stated acceptance rule), and only if the
    GPU's choice is itself a valid top-k under that gap: its k ids are
    distinct, their oracle logits are in descending slot order up to the gap,
    and no unselected expert beats the last selected one by more than it.
  * "within": the same set in another slot order.  Excused only if the GPU's
    order is descending up to the same gap (two near-equal slots swapped).
Any other mismatch fails.

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


def f64g(t):
    """f64 for large device tensors: the (exact) upcast runs on the device,
    then the fp64 copy comes to the host; the values are those of f64(t)."""
    if t is None:
        return None
    return t.detach().to(torch.float64).cpu().numpy()


def _gap(a, b):
    return REL_GAP * max(abs(a), abs(b))


def _descending_up_to_gap(s: np.ndarray) -> bool:
    return all(s[j] >= s[j + 1] - _gap(s[j], s[j + 1]) for j in range(len(s) - 1))


def valid_topk(l_row: np.ndarray, ids_row: np.ndarray) -> bool:
    k = len(ids_row)
    if len(set(ids_row.tolist())) != k or ids_row.min() < 0 or ids_row.max() >= len(l_row):
        return False
    s = l_row[ids_row]
    if not _descending_up_to_gap(s):
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
    near = oracle.boundary_near_tie(logits_ref, k, REL_GAP)
    n_boundary = n_within = 0
    for t in bad:
        what = (f"token {t}: ids {ids_gpu[t].tolist()} vs oracle {ids_ref[t].tolist()}, "
                f"logits {np.sort(logits_ref[t])[::-1][:k + 1].tolist()}")
        if set(ids_gpu[t].tolist()) == set(ids_ref[t].tolist()):
            assert _descending_up_to_gap(logits_ref[t][ids_gpu[t]]), "slot order: " + what
            n_within += 1
        else:
            assert near[t], "not a boundary near tie: " + what
            assert valid_topk(logits_ref[t], ids_gpu[t]), "not a valid top-k: " + what
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
    return (lambda e: f64g(layer["w1"][e])), (lambda e: f64g(layer["w2"][e]))


def assert_close_rel_blocks(pairs, tol: float, what: str):
    """assert_close_rel over a tensor compared block by block: pairs yields
    (got, ref) blocks; the bound is tol times the largest |ref| of all."""
    err = scale = 0.0
    for got, ref in pairs:
        err = max(err, float(np.abs(got - ref).max()))
        scale = max(scale, float(np.abs(ref).max()))
    assert err <= tol * scale, f"{what}: max|err| {err:.3e} > {tol} * max|ref| {scale:.3e}"
    return err / scale if scale else err


def sample_tokens(T: int, extra=(), n_random: int = 24, seed: int = 0) -> np.ndarray:
    g = np.random.default_rng(seed)
    base = set(range(min(T, 8))) | set(range(max(0, T - 8), T))
    base |= set(g.choice(T, size=min(T, n_random), replace=False).tolist())
    base |= set(int(t) for t in extra)
    return np.array(sorted(base), dtype=np.int64)
