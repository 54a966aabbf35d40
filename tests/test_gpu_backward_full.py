"""Backward parity at the full workload sizes, in the configuration bench.py
--pass train runs (moe_forward_train + moe_backward), on outputs the fp64
oracle can compute a piece at a time:

  * dw (the gate weights' gradient) and dx on sampled tokens: each sampled
    token's expert outputs and input gradient through the oracle's per-expert
    forward and backward, plus the router term from its logit gradient;
  * dW1[e] on sampled columns f and dW2[e] on the same sampled rows f, for a
    few experts (first, last, the largest, one more): the sampled part of the
    oracle's expert backward over all of that expert's rows;
  * dW_r and db_r in full: the oracle's x^T dl and sum_t dl with dl from the
    oracle's softmax Jacobian applied to the GPU's dw (dw itself is checked on
    the sampled tokens above; the full dw would need every expert output).

Routing passes the acceptance rule first, and the oracle is driven by the
GPU's ids (as in the forward's full-size test).  Tolerance: 2e-2 of the
largest magnitude of each compared block (bf16 workloads)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_check import TOL, assert_close_rel, check_routing, f64, sample_tokens

pytestmark = pytest.mark.gpu

import mixture_experts_layer_21_amd as moe  # fails loudly if the library is missing

FULL = ["mixtral_bf16", "skewed_bf16", "many_experts_bf16", "weight_bound_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_backward_full_sampled(name):
    cfg = mi.CONFIGS[name]
    print(f"\n[gen] {name}", flush=True)
    L = mi.make_inputs(cfg, "cuda")
    dy = mi.make_dy(cfg, "cuda")
    bias = L["router_bias"] is not None
    y, ids, w, saved = moe.moe_forward_train(L["x"], L["w_r"], L["router_bias"], L["w1"],
                                             L["w2"], cfg.k)
    g = moe.moe_backward(dy, L["x"], L["w_r"], L["w1"], L["w2"], cfg.k, ids, w, saved,
                         with_bias_grad=bias)
    torch.cuda.synchronize()
    print(f"[{name}] GPU done", flush=True)
    tol = TOL["bf16"]
    x64, wr64, dy64 = f64(L["x"]), f64(L["w_r"]), f64(dy)
    b64 = f64(L["router_bias"]) if bias else None
    logits = oracle.router_logits(x64, wr64, b64)
    ids_np = ids.cpu().numpy().astype(np.int64)
    check_routing(ids_np, w.cpu().numpy(), logits, cfg.k)
    w_ref = oracle.gate_weights(logits, ids_np)
    dw_gpu = g["dw"].cpu().numpy().astype(np.float64)
    w1 = lambda e: f64(L["w1"][e])  # noqa: E731
    w2 = lambda e: f64(L["w2"][e])  # noqa: E731

    # --- dw and dx on sampled tokens, expert by expert ---------------------------
    sel = sample_tokens(cfg.T, n_random=12, seed=3)
    dw_ref = np.zeros((len(sel), cfg.k))
    dx_exp = np.zeros((len(sel), cfg.H))
    for e in np.unique(ids_np[sel]):
        W1e, W2e = w1(e), w2(e)
        for a, t in enumerate(sel):
            for j in np.nonzero(ids_np[t] == e)[0]:
                x_t = x64[t:t + 1]
                y_e = oracle.expert_ffn_block(x_t, W1e, W2e)[0]
                dw_ref[a, j] = float(dy64[t] @ y_e)
                dx_e, _, _ = oracle.expert_block_backward(x_t, W1e, W2e,
                                                          w_ref[t, j] * dy64[t:t + 1],
                                                          weights=False)
                dx_exp[a] += dx_e[0]
    assert_close_rel(dw_gpu[sel], dw_ref, tol, f"{name} dw (sampled)")
    dl_sel = oracle.gate_weights_grad(logits[sel], ids_np[sel], dw_ref)
    dx_ref = dx_exp + dl_sel @ wr64.T
    assert_close_rel(f64(g["dx"])[sel], dx_ref, tol, f"{name} dx (sampled)")
    print(f"[{name}] dw, dx ok on {len(sel)} tokens", flush=True)

    # --- dW1 / dW2 on sampled columns of a few experts --------------------------
    offsets, sorted_token, sorted_slot, _ = oracle.dispatch(ids_np, cfg.E)
    counts = np.diff(offsets)
    rng = np.random.default_rng(4)
    experts = sorted({0, cfg.E - 1, int(np.argmax(counts)), int(rng.integers(cfg.E))})
    fs = np.unique(np.concatenate([rng.choice(cfg.F, 6, replace=False), [0, cfg.F - 1]]))
    dw1_gpu, dw2_gpu = g["dw1"], g["dw2"]
    for e in experts:
        a, b = int(offsets[e]), int(offsets[e + 1])
        got1 = f64(dw1_gpu[e][:, torch.from_numpy(fs).cuda()])
        got2 = f64(dw2_gpu[e][torch.from_numpy(fs).cuda(), :])
        if a == b:
            assert np.abs(got1).max() == 0.0 and np.abs(got2).max() == 0.0
            continue
        tok, slot = sorted_token[a:b], sorted_slot[a:b]
        x_e = x64[tok]
        dy_e = w_ref[tok, slot][:, None] * dy64[tok]
        W1s = w1(e)[:, fs]
        W2s = w2(e)[fs, :]
        z = x_e @ W1s
        dz = (dy_e @ W2s.T) * oracle.gelu_tanh_grad(z)
        assert_close_rel(got1, x_e.T @ dz, tol, f"{name} dW1[{e}] (sampled columns)")
        assert_close_rel(got2, oracle.gelu_tanh(z).T @ dy_e, tol,
                         f"{name} dW2[{e}] (sampled rows)")
    print(f"[{name}] dW1, dW2 ok for experts {experts}", flush=True)

    # --- dW_r, db_r in full, from the GPU's (sample-checked) dw ------------------
    dl = oracle.gate_weights_grad(logits, ids_np, dw_gpu)
    assert_close_rel(f64(g["dw_r"]), x64.T @ dl, tol, f"{name} dW_r")
    if bias:
        assert_close_rel(g["db_r"].cpu().numpy().astype(np.float64), dl.sum(axis=0), tol,
                         f"{name} db_r")
    print(f"[{name}] dW_r ok", flush=True)
