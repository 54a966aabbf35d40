"""The whole forward on seeded random layer shapes (bf16 and fp32; any T, H
and F that are multiples of 8, 1 to 300 experts, top-k up to 16), against
the oracle driven by the GPU's ids: the routing acceptance rule and the
output tolerance of the fixed shapes.  The shapes land on every path the
forward chooses between: the one-launch and two-kernel routers, the one-
and three-launch dispatches, both wave layouts of the expert GEMM, split and
whole last rounds, the top-1 combine in the second GEMM and the separate
combine pass; and twelve decode-sized layers (1 to 16 tokens) that take the
router-side dispatch and the split sums formed in the combine launch,
checked bit for bit against the training forward's separate launches."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_check import TOL, assert_close_rel, check_routing, f64, gpu_layer

pytestmark = pytest.mark.gpu

import mixture_experts_layer_21_amd as moe  # fails loudly if the library is missing


def shapes(n=24, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(g.choice([1, 2, 5, 8, 16, 24, 40, 64, 128, 200, 300]))
        k = int(min(E, g.choice([1, 1, 2, 2, 4, 6, 8, 16])))
        T = int(g.choice([1, 3, 17, 64, 200, 700, 1024, 1100, 2100, 3000]))
        H = int(8 * g.integers(1, 128 if T * E < 200000 else 64))
        F = int(8 * g.integers(1, 64))
        dt = "f32" if g.random() < 0.2 else "bf16"
        bias0 = float(g.choice([0.0, 0.0, 1.0]))
        out.append(mi.MoEConfig(f"rand{i}_T{T}_H{H}_E{E}_k{k}_F{F}_{dt}", T=T, H=H, E=E, k=k,
                                F=F, dtype=dt, bias0=bias0, seed=100 + i))
    return out


SHAPES = shapes()


@pytest.mark.parametrize("cfg", SHAPES, ids=[c.name for c in SHAPES])
def test_forward_random_shape(cfg):
    L = gpu_layer(cfg)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    print(f"[rand] {cfg.name}", flush=True)
    y = moe.moe_forward(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k,
                        topk_ids_out=ids, topk_w_out=w)
    torch.cuda.synchronize()
    logits = oracle.router_logits(f64(L["x"]), f64(L["w_r"]), f64(L["router_bias"]))
    ids_np = ids.cpu().numpy().astype(np.int64)
    check_routing(ids_np, w.cpu().numpy(), logits, cfg.k)
    ref = oracle.forward(f64(L["x"]), f64(L["w_r"]), f64(L["router_bias"]), f64(L["w1"]),
                         f64(L["w2"]), cfg.k, ids=ids_np,
                         w=oracle.gate_weights(logits, ids_np))["y"]
    assert_close_rel(f64(y), ref, TOL[cfg.dtype], f"{cfg.name} y")


def decode_shapes(n=12, seed=77):
    """Decode-sized bf16 layers: 1 to 16 tokens, up to 128 dispatched rows
    (the router-side dispatch for E <= 16, the split sums formed inside the
    combine launch), H up to 4096 so that the second GEMM splits its tiles."""
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(g.choice([8, 16, 24, 64]))
        T = int(g.integers(1, 17))
        k = int(min(E, g.choice([2, 3, 4, 8])))
        while T * k > 128:
            k //= 2
        H = int(8 * g.integers(16, 513))
        F = int(8 * g.integers(4, 257))
        out.append(mi.MoEConfig(f"dec{i}_T{T}_H{H}_E{E}_k{k}_F{F}", T=T, H=H, E=E, k=k, F=F,
                                dtype="bf16", bias0=float(g.choice([0.0, 1.0])), seed=300 + i))
    return out


DECODE = decode_shapes()


@pytest.mark.parametrize("cfg", DECODE, ids=[c.name for c in DECODE])
def test_decode_random_shape(cfg):
    """Against the oracle, and bit for bit against the training forward
    (which runs the separate dispatch, split reduce and combine launches)."""
    L = gpu_layer(cfg)
    print(f"[decode] {cfg.name}", flush=True)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    y = moe.moe_forward(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k,
                        topk_ids_out=ids, topk_w_out=w)
    y2, ids2, w2, _ = moe.moe_forward_train(L["x"], L["w_r"], L["router_bias"], L["w1"],
                                            L["w2"], cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(y, y2)
    logits = oracle.router_logits(f64(L["x"]), f64(L["w_r"]), f64(L["router_bias"]))
    ids_np = ids.cpu().numpy().astype(np.int64)
    check_routing(ids_np, w.cpu().numpy(), logits, cfg.k)
    ref = oracle.forward(f64(L["x"]), f64(L["w_r"]), f64(L["router_bias"]), f64(L["w1"]),
                         f64(L["w2"]), cfg.k, ids=ids_np,
                         w=oracle.gate_weights(logits, ids_np))["y"]
    assert_close_rel(f64(y), ref, TOL[cfg.dtype], f"{cfg.name} y")
