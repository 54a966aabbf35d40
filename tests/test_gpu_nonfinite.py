"""Tokens whose router logits are all NaN (a NaN in the token's activations).

The selection ranks a NaN logit as -inf, so such a token goes to experts
0 .. k-1 (equal values: the lower index first), with NaN gate weights, and
its y row is written (NaN), so no row of y keeps what it held before the
call.  Every other token is unaffected: its ids, gate weights and y match
the oracle's as in the parity tests.  That includes the tokens dispatched
next to a NaN token: the expert GEMMs read whole 64-element K stages and
zero the part past K, which would otherwise hold the next row's elements
(NaN times the zero weight rows past K is NaN).  The cases take each router
and combine path: the two-kernel router (one token per wave, and one per
16-lane row), the one-launch router, top-1 with the combine inside the
second expert GEMM, top-k with the combine kernel, K tails in both expert
GEMMs (H = 200, F = 136; H = 224, F = 96), tiles split along K, and fp32."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_check import TOL, assert_close_rel, check_routing, f64, gpu_layer

pytestmark = pytest.mark.gpu

import mixture_experts_layer_21_amd as moe  # fails loudly if the library is missing

C = mi.MoEConfig
CASES = {
    "top1_bf16": C("nf_top1_bf16", T=50, H=128, E=16, k=1, F=64, dtype="bf16"),
    "top1_fused_router_bf16": C("nf_top1_fr_bf16", T=1025, H=448, E=8, k=1, F=64, dtype="bf16"),
    "top2_fused_router_bf16": C("nf_top2_fr_bf16", T=1035, H=2048, E=16, k=2, F=64,
                                dtype="bf16"),
    "rows_bf16": C("nf_rows_bf16", T=1100, H=128, E=40, k=6, F=64, dtype="bf16"),
    "topE_bf16": C("nf_topE_bf16", T=33, H=64, E=4, k=4, F=64, dtype="bf16"),
    "ragged_bf16": C("nf_ragged_bf16", T=75, H=200, E=5, k=2, F=136, dtype="bf16"),
    # K = 224 and 96: each expert GEMM's last stage half past K
    "ktail32_bf16": C("nf_ktail32_bf16", T=600, H=224, E=4, k=2, F=96, dtype="bf16"),
    # few tiles with a long K: the first GEMM's tiles split in 8 pieces of
    # K = 4160 (130 steps of 32: even piece bounds 0, 16, .., 112)
    "ksplit_bf16": C("nf_ksplit_bf16", T=300, H=4160, E=2, k=2, F=512, dtype="bf16"),
    "ragged_f32": C("nf_ragged_f32", T=70, H=72, E=6, k=3, F=40, dtype="f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_nan_tokens(name):
    cfg = CASES[name]
    L = gpu_layer(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    bad = sorted({0, 17 % T, T // 2, T - 1})
    x = L["x"].clone()
    x[bad, 3] = float("nan")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, cfg.H), 7.0, dtype=x.dtype, device="cuda")
    print(f"[nonfinite] {name} NaN tokens {bad}", flush=True)
    moe.moe_forward(x, L["w_r"], L["router_bias"], L["w1"], L["w2"], k, y=y,
                    topk_ids_out=ids, topk_w_out=w)
    torch.cuda.synchronize()
    ids_np = ids.cpu().numpy().astype(np.int64)
    w_np = w.cpu().numpy()
    for t in bad:
        np.testing.assert_array_equal(ids_np[t], np.arange(k), err_msg=f"token {t}")
        assert np.isnan(w_np[t]).all(), f"token {t}: gate weights {w_np[t]}"
        assert torch.isnan(y[t].float()).all(), f"token {t}: y row not written"
    good = np.setdiff1d(np.arange(T), bad)
    xg = f64(x)[good]
    logits = oracle.router_logits(xg, f64(L["w_r"]), f64(L["router_bias"]))
    check_routing(ids_np[good], w_np[good], logits, k)
    ref = oracle.forward_tokens(xg, ids_np[good], oracle.gate_weights(logits, ids_np[good]),
                                f64(L["w1"]), f64(L["w2"]))
    assert_close_rel(f64(y)[good], ref, TOL[cfg.dtype], f"{name} y")


@pytest.mark.parametrize("name", ["top1_bf16", "ragged_bf16", "ktail32_bf16",
                                  "top2_fused_router_bf16", "ragged_f32"])
def test_nan_tokens_backward(name):
    """The training step with NaN tokens in the batch: the other tokens' dx
    and the weight gradients of the experts no NaN token reached (experts
    k .. E-1) match the oracle's backward over the finite tokens alone."""
    cfg = CASES[name]
    L = gpu_layer(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    bad = sorted({0, 17 % T, T // 2, T - 1})
    x = L["x"].clone()
    x[bad, 3] = float("nan")
    dy = mi.make_dy(cfg, "cuda")
    print(f"[nonfinite] backward {name} NaN tokens {bad}", flush=True)
    y, ids, w, saved = moe.moe_forward_train(x, L["w_r"], L["router_bias"], L["w1"], L["w2"], k)
    out = moe.moe_backward(dy, x, L["w_r"], L["w1"], L["w2"], k, ids, w, saved)
    torch.cuda.synchronize()
    ids_np = ids.cpu().numpy().astype(np.int64)
    good = np.setdiff1d(np.arange(T), bad)
    dx = f64(out["dx"])
    assert np.isnan(dx[bad]).all()
    ref = oracle.backward(f64(x)[good], f64(L["w_r"]), f64(L["router_bias"]), f64(L["w1"]),
                          f64(L["w2"]), k, f64(dy)[good], ids=ids_np[good])
    tol = TOL[cfg.dtype]
    assert_close_rel(dx[good], ref["dx"], tol, f"{name} dx")
    assert_close_rel(f64(out["dw1"])[k:], ref["dw1"][k:], tol, f"{name} dW1 of experts >= k")
    assert_close_rel(f64(out["dw2"])[k:], ref["dw2"][k:], tol, f"{name} dW2 of experts >= k")
