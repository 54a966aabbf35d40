"""Backward parity at the full workload sizes, in the configuration bench.py
--pass train runs (moe_forward_train + moe_backward), every element:

  * mixtral_bf16, skewed_bf16, many_experts_bf16 and the mid-size hand-off
    layer (both expert GEMMs run whole rounds, then split leftover tiles):
    oracle.backward over the whole batch; dx, the gate weights' gradient dw,
    dW_r, db_r, dW1 and dW2 compared on every element (the weight gradients
    expert by expert, to bound host memory);
  * weight_bound_bf16 (15 GB of expert weights; the oracle's dense [E,H,F]
    gradients would take 60 GB of host memory): the same quantities from the
    oracle's per-expert pieces over every token (expert_ffn_block for dw,
    expert_block_backward for dx and the weight gradients of every expert
    that received rows, gate_weights_grad for the router), compared expert
    by expert; experts without rows must have exactly zero weight gradients.

Routing passes the acceptance rule first, and the oracle is driven by the
GPU's ids (as in the forward's full-size test).  Tolerance: 2e-2 of the
largest magnitude of each compared gradient (bf16 workloads)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_check import TOL, assert_close_rel, assert_close_rel_blocks, check_routing, f64, f64g

pytestmark = pytest.mark.gpu

import mixture_experts_layer_21_amd as moe  # fails loudly if the library is missing

HANDOFF = mi.MoEConfig("handoff_bf16", T=2048, H=2048, E=8, k=4, F=8192, dtype="bf16")
CFGS = {**{n: mi.CONFIGS[n] for n in ("mixtral_bf16", "skewed_bf16", "many_experts_bf16",
                                       "weight_bound_bf16")}, HANDOFF.name: HANDOFF}


def run(cfg):
    print(f"\n[gen] {cfg.name}", flush=True)
    L = mi.make_inputs(cfg, "cuda")
    dy = mi.make_dy(cfg, "cuda")
    bias = L["router_bias"] is not None
    y, ids, w, saved = moe.moe_forward_train(L["x"], L["w_r"], L["router_bias"], L["w1"],
                                             L["w2"], cfg.k)
    g = moe.moe_backward(dy, L["x"], L["w_r"], L["w1"], L["w2"], cfg.k, ids, w, saved,
                         with_bias_grad=bias)
    torch.cuda.synchronize()
    print(f"[{cfg.name}] GPU done", flush=True)
    return L, dy, ids, w, g


@pytest.mark.parametrize("name", ["mixtral_bf16", "skewed_bf16", "many_experts_bf16",
                                  "handoff_bf16"])
def test_backward_full(name):
    cfg = CFGS[name]
    L, dy, ids, w, g = run(cfg)
    tol = TOL["bf16"]
    x64, wr64 = f64(L["x"]), f64(L["w_r"])
    b64 = f64(L["router_bias"])
    logits = oracle.router_logits(x64, wr64, b64)
    ids_np = ids.cpu().numpy().astype(np.int64)
    check_routing(ids_np, w.cpu().numpy(), logits, cfg.k)
    ref = oracle.backward(x64, wr64, b64, lambda e: f64g(L["w1"][e]),
                          lambda e: f64g(L["w2"][e]), cfg.k, f64(dy), ids=ids_np)
    print(f"[{name}] oracle done", flush=True)
    errs = {}
    for n in ("dx", "dw", "dw_r"):
        errs[n] = assert_close_rel(f64(g[n]), ref[n], tol, f"{name} {n}")
    if b64 is not None:
        errs["db_r"] = assert_close_rel(f64(g["db_r"]), ref["db_r"], tol, f"{name} db_r")
    for n in ("dw1", "dw2"):
        errs[n] = assert_close_rel_blocks(((f64g(g[n][e]), ref[n][e]) for e in range(cfg.E)),
                                          tol, f"{name} {n}")
    print(f"[{name}] max|err|/max|ref|: " +
          ", ".join(f"{n} {v:.2e}" for n, v in errs.items()), flush=True)


def test_backward_full_weight_bound():
    cfg = CFGS["weight_bound_bf16"]
    L, dy, ids, w, g = run(cfg)
    tol = TOL["bf16"]
    x64, wr64, dy64 = f64(L["x"]), f64(L["w_r"]), f64(dy)
    logits = oracle.router_logits(x64, wr64, None)
    ids_np = ids.cpu().numpy().astype(np.int64)
    check_routing(ids_np, w.cpu().numpy(), logits, cfg.k)
    w_ref = oracle.gate_weights(logits, ids_np)
    offsets, sorted_token, sorted_slot, _ = oracle.dispatch(ids_np, cfg.E)
    dw_ref = np.zeros(ids_np.shape)
    dx_exp = np.zeros((cfg.T, cfg.H))
    e1 = e2 = s1 = s2 = 0.0
    empty = []
    for e in range(cfg.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            empty.append(e)
            continue
        tok, slot = sorted_token[a:b], sorted_slot[a:b]
        W1e, W2e = f64g(L["w1"][e]), f64g(L["w2"][e])
        x_e = x64[tok]
        dw_ref[tok, slot] = (dy64[tok] * oracle.expert_ffn_block(x_e, W1e, W2e)).sum(axis=1)
        dx_e, dW1e, dW2e = oracle.expert_block_backward(x_e, W1e, W2e,
                                                        w_ref[tok, slot][:, None] * dy64[tok])
        np.add.at(dx_exp, tok, dx_e)
        got1, got2 = f64g(g["dw1"][e]), f64g(g["dw2"][e])
        e1, s1 = max(e1, np.abs(got1 - dW1e).max()), max(s1, np.abs(dW1e).max())
        e2, s2 = max(e2, np.abs(got2 - dW2e).max()), max(s2, np.abs(dW2e).max())
    assert e1 <= tol * s1, f"dW1: max|err| {e1:.3e} > {tol} * {s1:.3e}"
    assert e2 <= tol * s2, f"dW2: max|err| {e2:.3e} > {tol} * {s2:.3e}"
    if empty:
        sel = torch.tensor(empty, device="cuda")
        assert torch.count_nonzero(g["dw1"][sel]) == 0 and torch.count_nonzero(g["dw2"][sel]) == 0
    print(f"[weight_bound_bf16] {cfg.E - len(empty)} experts with rows, {len(empty)} without",
          flush=True)
    assert_close_rel(f64(g["dw"]), dw_ref, tol, "dw")
    dl = oracle.gate_weights_grad(logits, ids_np, dw_ref)
    assert_close_rel(f64(g["dx"]), dx_exp + dl @ wr64.T, tol, "dx")
    assert_close_rel(f64(g["dw_r"]), x64.T @ dl, tol, "dw_r")
    print(f"[weight_bound_bf16] dx, dw, dW_r, dW1, dW2 ok over all {cfg.T} tokens", flush=True)
