"""Plain, slow, fp64 CPU oracle for the MoE layer forward and its backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links this module; only the tests, the
smoke check and the bench's CPU-baseline leg do.  It shares no code, tables or
constants with the HIP path.

Every function follows a passage of the pages ("Writing a fused MoE operator
in Ascend C" = the fused-operator article; "MoE routing operator: load
balancing strategy" = the routing article) and is written for a reader to
check by eye: numpy fp64 throughout, one library call per step, no blocking,
fusion or reordering beyond what the passage states.

Readings taken where the pages are silent or ambiguous (each is listed with
its reason in the design notes):
  * gating is top-k first, then softmax over the k selected logits (fused
    article, "MoE computation flow" steps 1-2 and the router kernel's step 3);
  * ties in the top-k go to the lower expert index, and the k slots are in
    descending logit order (routing article, local top-k scan: strict ">"
    keeps the first maximum);
  * GELU is the tanh form 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
    (Hendrycks & Gimpel 2016), for every workload;
  * experts have no biases; the router has an optional bias b_r[E];
  * dispatch is dropless by default: every (token, slot) pair is computed
    (the gather routine has no capacity limit).

Variants (the CANN MoE operator-optimization article, "the CANN article"):
  * gating "softmax_topk": softmax over all E logits first, then the k
    largest probabilities kept as they are, not renormalised (section 2.1,
    Softmax -> Top-k -> mask);
  * a router weight in fp32 while the experts are half precision (section
    4.2) needs nothing here: every input is upcast to fp64 exactly;
  * capacity-limited dispatch: each expert keeps at most `capacity` rows,
    capacity = ceil(capacity_factor * T * k / E) (section 4.3 gives the
    factor 1.2; the fused-operator article's dispatch makes blocks of
    [num_experts, expert_capacity]).  The kept rows of an expert are its
    first `capacity` (token, slot) pairs in the gather's scan order; a dropped
    pair contributes nothing to y and the other weights are not renormalised
    (the routing article names token dropping for overloaded experts).

Backward (the CANN article's training setting: section 3 names the backward
pass's gradient aggregation, section 4.2 keeps the router in fp32, section 5
times whole training steps).  The pages print no gradient formulas; the
reading taken is the exact derivative of the forward above for a loss whose
gradient with respect to y is dy.  The top-k choice and the capacity drop are
piecewise constant in the logits, so no gradient flows through them: the
gradient reaches the logits only through the gate weights of the selected
experts, and a dropped pair's weight gets none (it does not reach y).
"""
from __future__ import annotations

import math

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)


# --- activation ------------------------------------------------------------

def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation, in fp64.

    Fused article, expert kernel step 3: Activation(hidden, GELU) between the
    two matrix multiplies; the tanh form is the reading taken for "GELU".
    """
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(SQRT_2_OVER_PI * (z + 0.044715 * z ** 3)))


# --- routing + gating (fused article, section 1; routing article) ----------

def gelu_tanh_grad(z: np.ndarray) -> np.ndarray:
    """d GELU / dz for the tanh form, in fp64.

    With u = sqrt(2/pi) (z + 0.044715 z^3) and GELU = 0.5 z (1 + tanh u):
    0.5 (1 + tanh u) + 0.5 z (1 - tanh(u)^2) sqrt(2/pi) (1 + 3 * 0.044715 z^2).
    """
    z = np.asarray(z, dtype=np.float64)
    th = np.tanh(SQRT_2_OVER_PI * (z + 0.044715 * z ** 3))
    du = SQRT_2_OVER_PI * (1.0 + 3.0 * 0.044715 * z ** 2)
    return 0.5 * (1.0 + th) + 0.5 * z * (1.0 - th ** 2) * du


def router_logits(x: np.ndarray, w_r: np.ndarray, b_r: np.ndarray | None = None) -> np.ndarray:
    """logits[T,E] = x[T,H] . W_r[H,E] (+ b_r[E]), fp64.

    Fused article, router kernel step 1 (x x W_router on the matrix unit);
    routing article: the router is a linear layer W_r producing logits.
    """
    l = np.asarray(x, np.float64) @ np.asarray(w_r, np.float64)
    if b_r is not None:
        l = l + np.asarray(b_r, np.float64)[None, :]
    return l


def topk_ids(logits: np.ndarray, k: int) -> np.ndarray:
    """ids[T,k]: the k largest logits per token, in descending order, ties to
    the lower expert index.

    Fused article, router kernel step 2 (TopK per sample); the tie rule is the
    routing article's scan, which replaces the running maximum only on a
    strictly greater value.  np.lexsort with keys (e, -l) is a stable sort by
    (-l, e): the primary key is the last one.
    """
    logits = np.asarray(logits, np.float64)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("top_k must be in [1, E]")
    ids = np.empty((T, k), dtype=np.int64)
    e_idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((e_idx, -logits[t]))
        ids[t] = order[:k]
    return ids


GATINGS = ("topk_softmax", "softmax_topk")


def gate_weights(logits: np.ndarray, ids: np.ndarray, gating: str = "topk_softmax") -> np.ndarray:
    """w[T,k] in slot order.

    "topk_softmax" (default): softmax over the k selected logits only (fused
    article, router kernel step 3).
    "softmax_topk": softmax over all E logits, then the probabilities of the
    k selected experts, not renormalised (CANN article, section 2.1).  Softmax
    is monotone, so the selected experts are the same either way.
    The max is subtracted first (softmax is invariant to the shift).
    """
    logits = np.asarray(logits, np.float64)
    sel = np.take_along_axis(logits, ids, axis=1)
    if gating == "topk_softmax":
        m = sel.max(axis=1, keepdims=True)
        ex = np.exp(sel - m)
        return ex / ex.sum(axis=1, keepdims=True)
    if gating == "softmax_topk":
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        p = p / p.sum(axis=1, keepdims=True)
        return np.take_along_axis(p, ids, axis=1)
    raise ValueError(f"unknown gating {gating!r}")


def gate_weights_grad(logits: np.ndarray, ids: np.ndarray, dw: np.ndarray,
                      gating: str = "topk_softmax") -> np.ndarray:
    """dlogits[T,E] from dw[T,k], the gradient with respect to the gate
    weights, by the softmax's Jacobian (no gradient through the choice of ids).

    "topk_softmax": w = softmax of the k selected logits, so the selected
    logit of slot j gets w_j (dw_j - sum_j' w_j' dw_j') and the other logits 0.
    "softmax_topk": p = softmax of all E logits and w_j = p[ids_j]; with
    g_e = dw_j where e = ids_j (0 for unselected e), logit e gets
    p_e (g_e - sum_e' p_e' g_e').
    """
    logits = np.asarray(logits, np.float64)
    dw = np.asarray(dw, np.float64)
    T, E = logits.shape
    dl = np.zeros((T, E), dtype=np.float64)
    if gating == "topk_softmax":
        w = gate_weights(logits, ids, gating)
        s = (w * dw).sum(axis=1, keepdims=True)
        dsel = w * (dw - s)
        for j in range(ids.shape[1]):
            dl[np.arange(T), ids[:, j]] += dsel[:, j]
        return dl
    if gating == "softmax_topk":
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        p = p / p.sum(axis=1, keepdims=True)
        g = np.zeros((T, E), dtype=np.float64)
        for j in range(ids.shape[1]):
            g[np.arange(T), ids[:, j]] += dw[:, j]
        return p * (g - (p * g).sum(axis=1, keepdims=True))
    raise ValueError(f"unknown gating {gating!r}")


def route(x, w_r, b_r, k: int, gating: str = "topk_softmax"):
    """(ids[T,k] int64, w[T,k] fp64, logits[T,E] fp64) for one MoE layer."""
    l = router_logits(x, w_r, b_r)
    ids = topk_ids(l, k)
    return ids, gate_weights(l, ids, gating), l


# --- dispatch (fused article, GatherTokensByExpert) -----------------------

def expert_capacity(T: int, k: int, E: int, capacity_factor: float) -> int:
    """Rows each expert may keep: ceil(capacity_factor * T * k / E); 0 means
    no limit (capacity_factor <= 0).  CANN article, section 4.3 (factor);
    fused article, MoE computation flow ([num_experts, expert_capacity]).
    Computed in exact rational arithmetic from the factor's decimal value."""
    from fractions import Fraction
    if capacity_factor <= 0:
        return 0
    q = Fraction(str(capacity_factor)) * T * k / E
    return int(-((-q.numerator) // q.denominator))


def dispatch(ids: np.ndarray, E: int, capacity: int = 0):
    """Group the (token, slot) pairs by expert, as the gather routine does.

    For each expert e in ascending order, scan tokens b in ascending order and
    slots k in ascending order, appending (b, k) whenever ids[b,k] == e.  The
    appended rows of expert e form the contiguous block
    [offsets[e], offsets[e+1]) of the dispatched order.  np.nonzero on the
    [T,k] mask returns exactly that (row-major, i.e. b then k) order.
    With capacity > 0 only the first `capacity` pairs of each expert in that
    order are appended; the others are dropped (inv_pos = -1).

    Returns offsets[E+1], sorted_token[R'] (token of each dispatched row),
    sorted_slot[R'] (slot k of each row) and inv_pos[T,k] (dispatched row of
    each (token, slot), -1 if dropped); R' = offsets[E].
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    offsets = np.zeros(E + 1, dtype=np.int64)
    sorted_token, sorted_slot = [], []
    for e in range(E):
        b, s = np.nonzero(ids == e)
        if capacity > 0:
            b, s = b[:capacity], s[:capacity]
        sorted_token.append(b)
        sorted_slot.append(s)
        offsets[e + 1] = offsets[e] + b.size
    sorted_token = np.concatenate(sorted_token).astype(np.int64)
    sorted_slot = np.concatenate(sorted_slot).astype(np.int64)
    inv_pos = np.full((T, k), -1, dtype=np.int64)
    inv_pos[sorted_token, sorted_slot] = np.arange(offsets[E])
    return offsets, sorted_token, sorted_slot, inv_pos


def gather_rows(x: np.ndarray, sorted_token: np.ndarray) -> np.ndarray:
    """xp[R,H]: the token rows in dispatched order (the gather's Copy)."""
    return np.asarray(x, np.float64)[sorted_token]


# --- experts (fused article, expert kernel step 3) --------------------------

def expert_ffn_block(x_e: np.ndarray, w1_e: np.ndarray, w2_e: np.ndarray) -> np.ndarray:
    """y_e = GELU(x_e . W1_e) . W2_e for one expert's rows; no biases.

    First matrix multiply M=rows, N=F, K=H; GELU; second M=rows, N=H, K=F.
    """
    h = gelu_tanh(np.asarray(x_e, np.float64) @ np.asarray(w1_e, np.float64))
    return h @ np.asarray(w2_e, np.float64)


def expert_ffn(xp: np.ndarray, offsets: np.ndarray, w1, w2) -> np.ndarray:
    """yp[R,H]: every dispatched row through its expert's FFN.

    w1/w2 are either [E,H,F]/[E,F,H] arrays or callables e -> [H,F]/[F,H]
    arrays (so a large layer can be processed one expert at a time).  Experts
    with no rows are skipped, as the expert kernel skips unselected experts.
    """
    xp = np.asarray(xp, np.float64)
    E = len(offsets) - 1
    H = xp.shape[1]
    yp = np.zeros((xp.shape[0], H), dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        yp[a:b] = expert_ffn_block(xp[a:b], _get(w1, e), _get(w2, e))
    return yp


def combine(yp: np.ndarray, inv_pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[T,H] = sum over slots j of w[t,j] * yp[inv_pos[t,j]], over the slots
    that were not dropped (inv_pos >= 0).

    Fused article, ScatterWithWeights: every dispatched row is scaled by its
    gate weight and accumulated (not overwritten) into its token's output.
    """
    yp = np.asarray(yp, np.float64)
    T, k = inv_pos.shape
    y = np.zeros((T, yp.shape[1]), dtype=np.float64)
    for j in range(k):
        kept = inv_pos[:, j] >= 0
        y[kept] += np.asarray(w, np.float64)[kept, j:j + 1] * yp[inv_pos[kept, j]]
    return y


# --- the whole layer --------------------------------------------------------

def forward(x, w_r, b_r, w1, w2, k: int, ids=None, w=None, gating: str = "topk_softmax",
            capacity: int = 0):
    """One MoE layer forward, as the fused article's flow states it.

    Routing (TopK of x.W_r), gating (softmax of the k scores, or the gating
    variant), then for each expert: gather its tokens (its first `capacity`
    ones when capacity > 0), skip it if it has none, run GELU(x_e W1) W2, and
    scatter the rows back into y weighted by their gate weights, with "+=".

    ids/w may be given to drive the expert and combine steps with a chosen
    routing (used when a near-tie lets two routings both be correct); by
    default they are the oracle's own.
    Returns dict(y, ids, w, logits).
    """
    x = np.asarray(x, np.float64)
    logits = router_logits(x, w_r, b_r)
    if ids is None:
        ids = topk_ids(logits, k)
    if w is None:
        w = gate_weights(logits, ids, gating)
    E = np.asarray(w_r).shape[1]
    T = x.shape[0]
    y = np.zeros((T, x.shape[1]), dtype=np.float64)
    for e in range(E):
        b_idx, s_idx = np.nonzero(ids == e)
        if capacity > 0:
            b_idx, s_idx = b_idx[:capacity], s_idx[:capacity]
        if b_idx.size == 0:
            continue
        y_e = expert_ffn_block(x[b_idx], _get(w1, e), _get(w2, e))
        np.add.at(y, b_idx, w[b_idx, s_idx][:, None] * y_e)
    return {"y": y, "ids": ids, "w": w, "logits": logits}


def expert_block_backward(x_e, w1_e, w2_e, dy_e, weights: bool = True):
    """Gradients through one expert's FFN y_e = GELU(x_e W1_e) W2_e for the
    gradient dy_e of its rows: (dx_e, dW1_e, dW2_e).
      dW2_e = h^T dy_e,  dz = (dy_e W2_e^T) * GELU'(z),  dW1_e = x_e^T dz,
      dx_e = dz W1_e^T,  with z = x_e W1_e and h = GELU(z).
    weights=False skips the two weight gradients (returned as None)."""
    x_e = np.asarray(x_e, np.float64)
    w1_e = np.asarray(w1_e, np.float64)
    w2_e = np.asarray(w2_e, np.float64)
    dy_e = np.asarray(dy_e, np.float64)
    z = x_e @ w1_e
    dz = (dy_e @ w2_e.T) * gelu_tanh_grad(z)
    if not weights:
        return dz @ w1_e.T, None, None
    return dz @ w1_e.T, x_e.T @ dz, gelu_tanh(z).T @ dy_e


def expert_ffn_backward(xp, offsets, w1, w2, dyp):
    """(dxp[R,H], dW1[E,H,F], dW2[E,F,H]) for the dispatched rows: every
    expert's block of rows through expert_block_backward; experts with no rows
    get zero weight gradients."""
    xp = np.asarray(xp, np.float64)
    dyp = np.asarray(dyp, np.float64)
    E = len(offsets) - 1
    H = xp.shape[1]
    F = np.asarray(_get(w1, 0)).shape[1]
    dxp = np.zeros_like(dyp)
    dw1 = np.zeros((E, H, F), dtype=np.float64)
    dw2 = np.zeros((E, F, H), dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        dxp[a:b], dw1[e], dw2[e] = expert_block_backward(xp[a:b], _get(w1, e), _get(w2, e),
                                                          dyp[a:b])
    return dxp, dw1, dw2


def backward(x, w_r, b_r, w1, w2, k: int, dy, ids=None, gating: str = "topk_softmax",
             capacity: int = 0):
    """Gradients of the layer forward for an output gradient dy[T,H].

    Each step is the chain rule through one step of forward(), taken in the
    reverse order:
      combine      y[t] += w[t,j] yp[p]   ->  dw[t,j] = dy[t] . yp[p],
                                              dyp[p] = w[t,j] dy[t]
      expert GEMM2 yp = h W2_e            ->  dW2_e = h^T dyp,  dh = dyp W2_e^T
      GELU         h = GELU(z)            ->  dz = dh * GELU'(z)
      expert GEMM1 z = x_e W1_e           ->  dW1_e = x_e^T dz, dx_e = dz W1_e^T
      dispatch     x_e = x[tokens of e]   ->  dx[t] += dx_e rows of token t
      gating       w = gate(logits)       ->  dlogits (gate_weights_grad)
      router       logits = x W_r + b_r   ->  dx += dlogits W_r^T,
                                              dW_r = x^T dlogits, db_r = sum_t dlogits
    ids may be given (a routing chosen on a near tie); the gate weights are
    then recomputed from the oracle's logits for those ids.
    Returns dict(dx, dw_r, db_r, dw1, dw2, dw, dlogits, ids, w).
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    w_r64 = np.asarray(w_r, np.float64)
    T, H = x.shape
    E = w_r64.shape[1]
    logits = router_logits(x, w_r, b_r)
    if ids is None:
        ids = topk_ids(logits, k)
    ids = np.asarray(ids, np.int64)
    w = gate_weights(logits, ids, gating)
    offsets, sorted_token, sorted_slot, _ = dispatch(ids, E, capacity)
    w1_0 = np.asarray(_get(w1, 0))
    F = w1_0.shape[1]
    dx = np.zeros((T, H), dtype=np.float64)
    dw1 = np.zeros((E, H, F), dtype=np.float64)
    dw2 = np.zeros((E, F, H), dtype=np.float64)
    dw = np.zeros(ids.shape, dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        tok, slot = sorted_token[a:b], sorted_slot[a:b]
        w1_e = np.asarray(_get(w1, e), np.float64)
        w2_e = np.asarray(_get(w2, e), np.float64)
        x_e = x[tok]
        y_e = gelu_tanh(x_e @ w1_e) @ w2_e
        g = dy[tok]
        dw[tok, slot] = (g * y_e).sum(axis=1)
        dy_e = w[tok, slot][:, None] * g
        dx_e, dw1[e], dw2[e] = expert_block_backward(x_e, w1_e, w2_e, dy_e)
        np.add.at(dx, tok, dx_e)
    dl = gate_weights_grad(logits, ids, dw, gating)
    dx += dl @ w_r64.T
    return {"dx": dx, "dw_r": x.T @ dl, "db_r": dl.sum(axis=0), "dw1": dw1, "dw2": dw2,
            "dw": dw, "dlogits": dl, "ids": ids, "w": w}


def forward_tokens(x_rows, ids_rows, w_rows, w1, w2) -> np.ndarray:
    """y for a chosen subset of tokens, one token at a time: y[t] = sum_j
    w[t,j] * FFN_{ids[t,j]}(x[t]).  Used to check sampled outputs of a layer
    too large for the full oracle."""
    x_rows = np.asarray(x_rows, np.float64)
    out = np.zeros(x_rows.shape, dtype=np.float64)
    for i in range(x_rows.shape[0]):
        for j in range(ids_rows.shape[1]):
            e = int(ids_rows[i, j])
            out[i] += float(w_rows[i, j]) * expert_ffn_block(x_rows[i:i + 1], _get(w1, e), _get(w2, e))[0]
    return out


def dense_bruteforce(x, w1, w2, ids, w, E: int) -> np.ndarray:
    """Independent formulation for tiny shapes: run every expert on every
    token, then mix with a dense [T,E] gate matrix that is w[t,j] at
    (t, ids[t,j]) and zero elsewhere."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    M = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            M[t, ids[t, j]] += w[t, j]
    y = 0.0
    for e in range(E):
        Z = expert_ffn_block(x, _get(w1, e), _get(w2, e))
        y = y + M[:, e:e + 1] * Z
    return np.asarray(y)


# --- near ties (reading of the "1e-3 relative" acceptance rule) -------------

def boundary_near_tie(logits: np.ndarray, k: int, rel: float = 1e-3) -> np.ndarray:
    """bool[T]: the k-th and (k+1)-th largest logits differ by less than rel
    times the larger magnitude, so either expert is a correct k-th choice."""
    T, E = logits.shape
    if k >= E:
        return np.zeros(T, dtype=bool)
    s = -np.sort(-np.asarray(logits, np.float64), axis=1)
    a, b = s[:, k - 1], s[:, k]
    return np.abs(a - b) < rel * np.maximum(np.abs(a), np.abs(b))


def _get(w, e):
    return w(e) if callable(w) else w[e]

