"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Small shapes are checked element by element on every output, at sizes that
span several 256x256 GEMM tiles with ragged row, column and K tails, plus the
degenerate cases (T=1, k=1, k=E, E=1, empty experts, skewed routing, exact
ties).  The five full-size workloads, in the launch configuration the bench
times, are checked on every routing decision and dispatch index and on every
element of y and of the dispatched expert outputs yp, against the oracle run
one expert at a time over the whole batch.  So is a mid-size layer whose two
expert GEMMs both run whole rounds of 256x256 tiles on every CU and then
split the leftover tiles along K (the persistent kernel's hand-off from whole
tiles to split pieces), with expert row counts that leave 10- to 32-row
tiles."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_check import (TOL, assert_close_rel, check_routing, expert_getters, f64, f64g,
                       gpu_layer)

pytestmark = pytest.mark.gpu

import mixture_experts_layer_21_amd as moe  # fails loudly if the library is missing

C = mi.MoEConfig
SMALL = {
    "tiny_fp32": mi.CONFIGS["tiny_fp32"],
    "ragged_bf16": C("ragged_bf16", T=75, H=200, E=5, k=2, F=136, dtype="bf16"),
    "multitile_bf16": C("multitile_bf16", T=1000, H=256, E=3, k=2, F=392, dtype="bf16"),
    "ragged_f32": C("ragged_f32", T=70, H=72, E=6, k=3, F=40, dtype="f32"),
    "multitile_f32": C("multitile_f32", T=300, H=136, E=3, k=2, F=200, dtype="f32"),
    "topE_bf16": C("topE_bf16", T=33, H=64, E=4, k=4, F=64, dtype="bf16"),
    "top1_bf16": C("top1_bf16", T=50, H=128, E=16, k=1, F=64, dtype="bf16"),
    "one_expert_bf16": C("one_expert_bf16", T=40, H=64, E=1, k=1, F=128, dtype="bf16"),
    "one_token_bf16": C("one_token_bf16", T=1, H=128, E=8, k=2, F=256, dtype="bf16"),
    "many_small_bf16": C("many_small_bf16", T=128, H=128, E=128, k=8, F=64, dtype="bf16"),
    "wide_E_bf16": C("wide_E_bf16", T=20, H=64, E=1000, k=16, F=32, dtype="bf16"),
    "skewed_small_bf16": C("skewed_small_bf16", T=256, H=128, E=8, k=2, F=256, dtype="bf16",
                           bias0=3.0),
    # T >= 1024 and E <= 256: the selection runs one token per 16-lane row
    "rows_bf16": C("rows_bf16", T=1100, H=128, E=40, k=6, F=64, dtype="bf16"),
    # the one-launch dispatch over 36 workgroups (the last one partly full)
    "long_dispatch_bf16": C("long_dispatch_bf16", T=4500, H=64, E=64, k=8, F=64, dtype="bf16"),
    # more pairs than the one-launch dispatch takes (T*k > 65536): the count /
    # scan / place kernels
    "huge_dispatch_bf16": C("huge_dispatch_bf16", T=9000, H=64, E=96, k=8, F=64, dtype="bf16"),
    # the one-launch dispatch at E = 1000 (LDS tables of 19 E ints)
    "wide_E_dispatch_bf16": C("wide_E_dispatch_bf16", T=3000, H=64, E=1000, k=4, F=32,
                              dtype="bf16"),
    # few tiles with a long K: the expert GEMM splits tiles along K (partials
    # summed by the last piece), checked here on every element
    "ksplit_bf16": C("ksplit_bf16", T=300, H=4096, E=2, k=1, F=512, dtype="bf16"),
    # the one-launch router for E <= 16 at few tokens (8-token tiles, the last
    # one partly or, at T = 1, mostly empty)
    "fused_T1_E8_bf16": C("fused_T1_E8_bf16", T=1, H=4096, E=8, k=2, F=64, dtype="bf16"),
    "fused_T37_E16_bf16": C("fused_T37_E16_bf16", T=37, H=1000, E=16, k=3, F=64,
                            dtype="bf16", bias0=0.5),
    "fused_T200_E8_bf16": C("fused_T200_E8_bf16", T=200, H=448, E=8, k=1, F=64, dtype="bf16"),
    # up to 16 tokens with E <= 16: the router's one workgroup (8-token tile
    # up to 8 tokens, else 16) also does the dispatch (no separate dispatch
    # launch in moe_forward)
    "route_dispatch_T5_bf16": C("route_dispatch_T5_bf16", T=5, H=256, E=16, k=4, F=64,
                                dtype="bf16"),
    "route_dispatch_T8_kE_bf16": C("route_dispatch_T8_kE_bf16", T=8, H=512, E=8, k=8, F=64,
                                   dtype="bf16"),
    "route_dispatch_top1_T3_bf16": C("route_dispatch_top1_T3_bf16", T=3, H=128, E=8, k=1,
                                     F=64, dtype="bf16"),
    "route_dispatch_T13_bf16": C("route_dispatch_T13_bf16", T=13, H=1000, E=16, k=5, F=64,
                                 dtype="bf16"),
    "route_dispatch_T16_kE_bf16": C("route_dispatch_T16_kE_bf16", T=16, H=4096, E=8, k=8,
                                    F=64, dtype="bf16"),
    # more experts (or H > 4096) at up to 4 tokens: the two-kernel router's
    # selection launch (one workgroup) does the dispatch
    "select_dispatch_E256_bf16": C("select_dispatch_E256_bf16", T=4, H=512, E=256, k=8,
                                   F=64, dtype="bf16", bias0=1.0),
    "select_dispatch_E1000_bf16": C("select_dispatch_E1000_bf16", T=3, H=64, E=1000, k=16,
                                    F=32, dtype="bf16"),
    "select_dispatch_H8192_bf16": C("select_dispatch_H8192_bf16", T=4, H=8192, E=8, k=2,
                                    F=64, dtype="bf16"),
    # the one-launch router (E <= 128 in multiples of 8, H <= 4096; E > 16 at
    # T >= 1024 only):
    # each of the 8 waves takes NS = 1, 2, 4, 8, 16 steps of 32 rows of H
    # (H = 40 .. 4096: waves with partly and wholly empty ranges), in both
    # kernels (E <= 16, and E = 24 .. 128 read in whole rows), a last token
    # tile of 1 to 15 tokens; E <= 16 in 8-token tiles (fewer than 256 tiles
    # of 16) and, at T = 4100, in 16-token tiles; and one layer with H > 4096
    # that takes the two-kernel router at T >= 1024
    "fused_E8_bf16": C("fused_E8_bf16", T=1031, H=4096, E=8, k=2, F=64, dtype="bf16"),
    "fused_E8_H448_bf16": C("fused_E8_H448_bf16", T=1025, H=448, E=8, k=1, F=64, dtype="bf16"),
    "fused_E16_H2048_bf16": C("fused_E16_H2048_bf16", T=1035, H=2048, E=16, k=4, F=64,
                              dtype="bf16", bias0=0.5),
    "fused_E16_H1000_bf16": C("fused_E16_H1000_bf16", T=1100, H=1000, E=16, k=3, F=64,
                              dtype="bf16"),
    "fused_E128_bf16": C("fused_E128_bf16", T=1027, H=2048, E=128, k=8, F=64, dtype="bf16"),
    "fused_E64_H4096_bf16": C("fused_E64_H4096_bf16", T=1040, H=4096, E=64, k=6, F=64,
                              dtype="bf16"),
    "fused_H1000_bf16": C("fused_H1000_bf16", T=1033, H=1000, E=64, k=8, F=64, dtype="bf16",
                          bias0=1.0),
    "fused_H448_bf16": C("fused_H448_bf16", T=1049, H=448, E=24, k=3, F=64, dtype="bf16"),
    "fused_H40_bf16": C("fused_H40_bf16", T=1300, H=40, E=16, k=4, F=64, dtype="bf16"),
    "fused_H40_E32_bf16": C("fused_H40_E32_bf16", T=1024, H=40, E=32, k=5, F=64, dtype="bf16"),
    "fused_E16_T4100_bf16": C("fused_E16_T4100_bf16", T=4100, H=256, E=16, k=2, F=64,
                              dtype="bf16"),
    "route2_H7168_bf16": C("route2_H7168_bf16", T=1039, H=7168, E=64, k=8, F=64, dtype="bf16",
                           bias0=1.0),
    # the two-kernel router with a split longer than one staged W_r chunk
    # (16 splits of 384 rows: chunks of 256 + 128 rows; with an fp32 W_r,
    # six chunks of 64)
    "route2_chunks_bf16": C("route2_chunks_bf16", T=2100, H=6144, E=256, k=8, F=64,
                            dtype="bf16"),
}
FULL = [n for n in mi.CONFIG_ORDER]
# both expert GEMMs: 4 whole rounds + 96 tiles split in 2 (GEMM1, 1120 tiles),
# 1 whole round + 24 tiles split in 10 (GEMM2, 280 tiles); expert rows
# [1007, 1000, 1043, 1008, 1020, 1056, 1034, 1024]
HANDOFF = C("handoff_bf16", T=2048, H=2048, E=8, k=4, F=8192, dtype="bf16")
FULL_CFG = {**{n: mi.CONFIGS[n] for n in FULL}, HANDOFF.name: HANDOFF}

_cache = {}


def layer(cfg):
    if cfg.name not in _cache:
        if len(_cache) > 2:          # keep at most a few layers resident
            _cache.pop(next(iter(_cache)))
            torch.cuda.empty_cache()
        print(f"\n[gen] {cfg.name}", flush=True)
        _cache[cfg.name] = gpu_layer(cfg)
    return _cache[cfg.name]


def ref_logits(cfg, L):
    return oracle.router_logits(f64(L["x"]), f64(L["w_r"]), f64(L["router_bias"]))


def dt(cfg):
    return cfg.dtype


# --- small shapes: every stage, every element ---------------------------------

@pytest.mark.parametrize("name", list(SMALL))
def test_route_small(name):
    cfg = SMALL[name]
    L = layer(cfg)
    ids, w = moe.moe_route(L["x"], L["w_r"], L["router_bias"], cfg.k)
    torch.cuda.synchronize()
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref_logits(cfg, L), cfg.k)
    assert np.all(np.abs(w.cpu().numpy().sum(1) - 1) < 1e-5)


@pytest.mark.parametrize("name", list(SMALL))
def test_permute_small(name):
    cfg = SMALL[name]
    L = layer(cfg)
    ids, _ = moe.moe_route(L["x"], L["w_r"], L["router_bias"], cfg.k)
    off, st, inv, xp = moe.moe_permute(L["x"], ids, cfg.E)
    torch.cuda.synchronize()
    o_off, o_st, _, o_inv = oracle.dispatch(ids.cpu().numpy().astype(np.int64), cfg.E)
    np.testing.assert_array_equal(off.cpu().numpy(), o_off)
    np.testing.assert_array_equal(st.cpu().numpy(), o_st)
    np.testing.assert_array_equal(inv.cpu().numpy(), o_inv.ravel())
    assert torch.equal(xp.cpu(), L["x"].cpu()[torch.from_numpy(o_st)])


@pytest.mark.parametrize("name", list(SMALL))
def test_expert_ffn_small(name):
    cfg = SMALL[name]
    L = layer(cfg)
    ids, _ = moe.moe_route(L["x"], L["w_r"], L["router_bias"], cfg.k)
    off, st, inv, xp = moe.moe_permute(L["x"], ids, cfg.E)
    yp = moe.moe_expert_ffn(xp, off, L["w1"], L["w2"])
    torch.cuda.synchronize()
    ref = oracle.expert_ffn(f64(xp), off.cpu().numpy(), f64(L["w1"]), f64(L["w2"]))
    assert_close_rel(f64(yp), ref, TOL[dt(cfg)], f"{name} yp")


@pytest.mark.parametrize("name", list(SMALL))
def test_combine_small(name):
    cfg = SMALL[name]
    L = layer(cfg)
    ids, w = moe.moe_route(L["x"], L["w_r"], L["router_bias"], cfg.k)
    off, st, inv, xp = moe.moe_permute(L["x"], ids, cfg.E)
    yp = moe.moe_expert_ffn(xp, off, L["w1"], L["w2"])
    y = moe.moe_combine(yp, inv, w)
    torch.cuda.synchronize()
    ref = oracle.combine(f64(yp), inv.cpu().numpy().reshape(cfg.T, cfg.k), f64(w))
    # only the final rounding of y to the storage dtype separates the two
    assert_close_rel(f64(y), ref, 4e-3 if cfg.dtype == "bf16" else 1e-6, f"{name} y")


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    cfg = SMALL[name]
    L = layer(cfg)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    y = moe.moe_forward(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k,
                        topk_ids_out=ids, topk_w_out=w)
    torch.cuda.synchronize()
    logits = ref_logits(cfg, L)
    ids_np = ids.cpu().numpy().astype(np.int64)
    check_routing(ids_np, w.cpu().numpy(), logits, cfg.k)
    ref = oracle.forward(f64(L["x"]), f64(L["w_r"]), f64(L["router_bias"]), f64(L["w1"]),
                         f64(L["w2"]), cfg.k, ids=ids_np,
                         w=oracle.gate_weights(logits, ids_np))["y"]
    assert_close_rel(f64(y), ref, TOL[dt(cfg)], f"{name} y")


# --- exact ties: integer-valued inputs make every logit exact ---------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (64, 8), (128, 8), (256, 8), (33, 5)])
@pytest.mark.parametrize("T", [96, 1100])   # one token per wave / per 16-lane row
def test_route_exact_ties(dtype, E, k, T):
    inp = mi.integer_inputs(T, 64, E, 8, -2, 2, seed=E * 31 + k, dtype=dtype, device="cuda")
    ids, w = moe.moe_route(inp["x"], inp["w_r"], None, k)
    torch.cuda.synchronize()
    l = oracle.router_logits(f64(inp["x"]), f64(inp["w_r"]))
    assert (l == np.round(l)).all()
    np.testing.assert_array_equal(ids.cpu().numpy(), oracle.topk_ids(l, k))
    w_np = w.cpu().numpy()
    if k == 1:
        assert np.all(w_np == 1.0)
    np.testing.assert_allclose(w_np, oracle.gate_weights(l, oracle.topk_ids(l, k)), atol=1e-6)


def test_generator_is_bit_identical_on_cpu_and_gpu():
    cfg = mi.CONFIGS["tiny_fp32"]
    a, b = mi.make_inputs(cfg, "cpu"), mi.make_inputs(cfg, "cuda")
    for key in ("x", "w_r", "w1", "w2"):
        assert torch.equal(a[key], b[key].cpu()), key
    c1 = mi.CONFIGS["many_experts_bf16"]
    assert torch.equal(mi.make_x(c1, "cpu"), mi.make_x(c1, "cuda").cpu())
    assert torch.equal(mi.make_w2_expert(c1, 77, "cpu"), mi.make_w2_expert(c1, 77, "cuda").cpu())


# --- full-size workloads: every element ---------------------------------------

@pytest.mark.parametrize("name", list(FULL_CFG))
def test_forward_full(name):
    cfg = FULL_CFG[name]
    L = layer(cfg)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    y = moe.moe_forward(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k,
                        topk_ids_out=ids, topk_w_out=w)
    torch.cuda.synchronize()
    logits = ref_logits(cfg, L)
    ids_np = ids.cpu().numpy().astype(np.int64)
    nb, nw = check_routing(ids_np, w.cpu().numpy(), logits, cfg.k)
    print(f"[{name}] near ties: boundary {nb}, within-set {nw}", flush=True)
    g1, g2 = expert_getters(L)
    y_ref = oracle.forward(f64(L["x"]), f64(L["w_r"]), f64(L["router_bias"]), g1, g2, cfg.k,
                           ids=ids_np, w=oracle.gate_weights(logits, ids_np))["y"]
    rel = assert_close_rel(f64(y), y_ref, TOL[dt(cfg)], f"{name} y")
    print(f"[{name}] y: max|err|/max|y_ref| = {rel:.3e} over all {cfg.T} tokens", flush=True)


@pytest.mark.parametrize("name", list(FULL_CFG))
def test_dispatch_full(name):
    cfg = FULL_CFG[name]
    L = layer(cfg)
    ids, w = moe.moe_route(L["x"], L["w_r"], L["router_bias"], cfg.k)
    off, st, inv, xp = moe.moe_permute(L["x"], ids, cfg.E)
    torch.cuda.synchronize()
    o_off, o_st, _, o_inv = oracle.dispatch(ids.cpu().numpy().astype(np.int64), cfg.E)
    np.testing.assert_array_equal(off.cpu().numpy(), o_off)
    np.testing.assert_array_equal(st.cpu().numpy(), o_st)
    np.testing.assert_array_equal(inv.cpu().numpy(), o_inv.ravel())
    assert torch.equal(xp, L["x"][st.long()])
    # every dispatched row of the expert FFN, on the real shapes
    yp = moe.moe_expert_ffn(xp, off, L["w1"], L["w2"])
    torch.cuda.synchronize()
    g1, g2 = expert_getters(L)
    ref = oracle.expert_ffn(f64g(xp), o_off, g1, g2)
    rel = assert_close_rel(f64g(yp), ref, TOL[dt(cfg)], f"{name} yp")
    print(f"[{name}] yp: max|err|/max|yp_ref| = {rel:.3e} over all {cfg.R} rows", flush=True)


# top_k = 1, bf16, dropless: the second expert GEMM writes each token's row
# of y itself (its dispatched row, weighted); the result must be bit for bit
# the staged path's (dispatched rows stored, then the combine pass) and agree
# with the oracle on every token.  The last two shapes run that epilogue in
# the split reduce: every second-GEMM tile split along K (24 tiles, K = 4096),
# and one whole round of 256 tiles followed by split leftover tiles.
TOP1 = {
    **{n: SMALL[n] for n in ("top1_bf16", "one_expert_bf16", "ksplit_bf16",
                             "fused_E8_H448_bf16", "route_dispatch_top1_T3_bf16")},
    "top1_split_bf16": C("top1_split_bf16", T=2100, H=512, E=4, k=1, F=4096, dtype="bf16"),
    "top1_rounds_bf16": C("top1_rounds_bf16", T=4096, H=4096, E=16, k=1, F=2048,
                          dtype="bf16"),
}


@pytest.mark.parametrize("name", list(TOP1))
def test_top1_fused_combine(name):
    cfg = TOP1[name]
    L = layer(cfg)
    ids = torch.empty((cfg.T, 1), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, 1), dtype=torch.float32, device="cuda")
    y = moe.moe_forward(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], 1,
                        topk_ids_out=ids, topk_w_out=w)
    assert torch.all(w == 1.0)          # top-1 then softmax: a weight of exactly 1
    off, st, inv, xp = moe.moe_permute(L["x"], ids, cfg.E)
    yp = moe.moe_expert_ffn(xp, off, L["w1"], L["w2"])
    y_staged = moe.moe_combine(yp, inv, w)
    torch.cuda.synchronize()
    assert torch.equal(y, y_staged)
    logits = ref_logits(cfg, L)
    ids_np = ids.cpu().numpy().astype(np.int64)
    check_routing(ids_np, w.cpu().numpy(), logits, 1)
    g1, g2 = expert_getters(L)
    y_ref = oracle.forward(f64(L["x"]), f64(L["w_r"]), f64(L["router_bias"]), g1, g2, 1,
                           ids=ids_np, w=oracle.gate_weights(logits, ids_np))["y"]
    rel = assert_close_rel(f64(y), y_ref, TOL[dt(cfg)], f"{name} y")
    print(f"[{name}] y: max|err|/max|y_ref| = {rel:.3e} over all {cfg.T} tokens", flush=True)


@pytest.mark.parametrize("name", ["top1_bf16", "top1_split_bf16"])
def test_top1_fused_combine_softmax_first(name):
    """Softmax over all experts, then the top 1 (gate weight below 1): the
    second GEMM's epilogue applies the weight as the combine pass does."""
    cfg = TOP1[name]
    L = layer(cfg)
    gs = moe.MOE_GATE_SOFTMAX_TOPK
    ids = torch.empty((cfg.T, 1), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, 1), dtype=torch.float32, device="cuda")
    y = moe.moe_forward_ex(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], 1, gating=gs,
                           topk_ids_out=ids, topk_w_out=w)
    ids2, w2 = moe.moe_route_ex(L["x"], L["w_r"], L["router_bias"], 1, gating=gs)
    off, st, inv, xp = moe.moe_permute(L["x"], ids2, cfg.E)
    yp = moe.moe_expert_ffn(xp, off, L["w1"], L["w2"])
    y_staged = moe.moe_combine(yp, inv, w2)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2)
    assert bool(torch.all(w < 1.0))
    assert torch.equal(y, y_staged)


@pytest.mark.parametrize("name", ["mixtral_bf16", "many_experts_bf16"])
def test_forward_is_deterministic(name):
    cfg = mi.CONFIGS[name]
    L = layer(cfg)
    ws = torch.empty(moe.moe_workspace_bytes(cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.torch_dtype),
                     dtype=torch.uint8, device="cuda")
    a = moe.moe_forward(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k, ws=ws)
    ws.fill_(0x5A)
    b = moe.moe_forward(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
