"""Parity of the training forward and the backward (moe_forward_train,
moe_backward) with the fp64 oracle's backward.

The oracle is driven by the GPU's expert ids (a near tie may legitimately
choose either expert; the ids themselves pass the routing acceptance rule
first).  Every gradient (dx, dW_r, dW1, dW2, the gate weights' gradient and,
where asked, db_r) must lie within the forward's tolerance of the oracle's,
relative to the largest magnitude of that gradient: 2e-2 for the bf16 path
(whose intermediates dyp, z, h, dz are bf16 like its forward's h), 1e-4 for
fp32.  Shapes cover several tiles with ragged tails, K tails that are not a
multiple of 64 (H = 200, F = 136), K step counts that leave 9 and 11 steps
after the transposed-weight GEMM's 12-step period, the split-K path (H or
F = 4096), experts
with no rows, k = 1, and the variants (softmax-first gating, capacity drops,
an fp32 router, a router bias)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_check import TOL, assert_close_rel, check_routing, f64

pytestmark = pytest.mark.gpu

import mixture_experts_layer_21_amd as moe  # fails loudly if the library is missing

C = mi.MoEConfig
GS, GT = moe.MOE_GATE_SOFTMAX_TOPK, moe.MOE_GATE_TOPK_SOFTMAX
GNAME = {GT: "topk_softmax", GS: "softmax_topk"}
CASES = {
    "tiny_fp32": mi.CONFIGS["tiny_fp32"],
    "ragged_bf16": C("ragged_bf16", T=75, H=200, E=5, k=2, F=136, dtype="bf16"),
    "multitile_bf16": C("multitile_bf16", T=1000, H=256, E=3, k=2, F=392, dtype="bf16"),
    "ragged_f32": C("ragged_f32", T=70, H=72, E=6, k=3, F=40, dtype="f32"),
    "top1_bf16": C("top1_bf16", T=50, H=128, E=16, k=1, F=64, dtype="bf16"),
    "one_token_bf16": C("one_token_bf16", T=1, H=128, E=8, k=2, F=256, dtype="bf16"),
    # the router's one workgroup dispatching a decode-sized batch (saved indices)
    "decode_T7_bf16": C("decode_T7_bf16", T=7, H=256, E=16, k=3, F=128, dtype="bf16"),
    "decode_T12_bf16": C("decode_T12_bf16", T=12, H=512, E=8, k=2, F=128, dtype="bf16"),
    "many_small_bf16": C("many_small_bf16", T=128, H=128, E=128, k=8, F=64, dtype="bf16"),
    "skewed_small_bf16": C("skewed_small_bf16", T=256, H=128, E=8, k=2, F=256, dtype="bf16",
                           bias0=3.0),
    "longH_bf16": C("longH_bf16", T=40, H=4096, E=24, k=3, F=64, dtype="bf16"),
    "longF_bf16": C("longF_bf16", T=64, H=128, E=4, k=2, F=4096, dtype="bf16"),
    # K step counts 21 (H = 672) and 11 (F = 352): remainders of 9 and 11 steps
    # after the transposed-weight GEMM's 12-step period
    "period_tail_bf16": C("period_tail_bf16", T=96, H=672, E=4, k=2, F=352, dtype="bf16"),
    # 33..64 experts (the router weight gradient's 64-expert tile, 40 of them
    # real), h blocks of 64 with a ragged last one, ragged token splits
    "midE_bf16": C("midE_bf16", T=300, H=200, E=40, k=4, F=96, dtype="bf16"),
}
_cache = {}


def layer(cfg):
    if cfg.name not in _cache:
        if len(_cache) > 3:
            _cache.pop(next(iter(_cache)))
            torch.cuda.empty_cache()
        print(f"\n[gen] {cfg.name}", flush=True)
        L = mi.make_inputs(cfg, "cuda")
        L["dy"] = mi.make_dy(cfg, "cuda")
        if cfg.dtype == "bf16":
            L["w_r32"] = mi.make_w_r_f32(cfg, "cuda")
        _cache[cfg.name] = L
    return _cache[cfg.name]


def run(cfg, gating=GT, capacity=0, wf32=False, with_bias=False):
    L = layer(cfg)
    w_r = L["w_r32"] if wf32 else L["w_r"]
    print(f"[case] {cfg.name} gating={GNAME[gating]} capacity={capacity} wf32={wf32}", flush=True)
    y, ids, w, saved = moe.moe_forward_train(L["x"], w_r, L["router_bias"], L["w1"], L["w2"],
                                             cfg.k, gating, capacity)
    out = moe.moe_backward(L["dy"], L["x"], w_r, L["w1"], L["w2"], cfg.k, ids, w, saved, gating,
                           with_bias_grad=with_bias)
    torch.cuda.synchronize()
    return L, w_r, y, ids, w, saved, out


def check(cfg, L, w_r, ids, w, out, gating, capacity, with_bias):
    tol = TOL[cfg.dtype]
    x64, wr64 = f64(L["x"]), f64(w_r)
    logits = oracle.router_logits(x64, wr64, f64(L["router_bias"]))
    ids_np = ids.cpu().numpy().astype(np.int64)
    check_routing(ids_np, w.cpu().numpy(), logits, cfg.k, GNAME[gating])
    ref = oracle.backward(x64, wr64, f64(L["router_bias"]), f64(L["w1"]), f64(L["w2"]), cfg.k,
                          f64(L["dy"]), ids=ids_np, gating=GNAME[gating], capacity=capacity)
    for name in ("dx", "dw_r", "dw1", "dw2", "dw"):
        assert_close_rel(f64(out[name]), ref[name], tol, name)
    if with_bias:
        assert_close_rel(f64(out["db_r"]), ref["db_r"], tol, "db_r")
    return ref


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    cfg = CASES[name]
    bias = cfg.bias0 != 0.0
    L, w_r, y, ids, w, saved, out = run(cfg, with_bias=bias)
    check(cfg, L, w_r, ids, w, out, GT, 0, bias)


@pytest.mark.parametrize("name,gating,cap_factor,wf32", [
    ("ragged_bf16", GS, 0.0, False),
    ("tiny_fp32", GS, 1.2, False),
    ("skewed_small_bf16", GT, 1.2, False),
    ("skewed_small_bf16", GS, 0.6, False),
    ("multitile_bf16", GT, 0.0, True),
    ("many_small_bf16", GS, 1.2, True),
    ("ragged_f32", GT, 0.6, False),
])
def test_backward_variants_match_oracle(name, gating, cap_factor, wf32):
    cfg = CASES[name]
    cap = oracle.expert_capacity(cfg.T, cfg.k, cfg.E, cap_factor)
    L, w_r, y, ids, w, saved, out = run(cfg, gating, cap, wf32, with_bias=True)
    check(cfg, L, w_r, ids, w, out, gating, cap, True)
    if cap:
        # dropped pairs get a zero gate-weight gradient
        _, _, _, inv = oracle.dispatch(ids.cpu().numpy().astype(np.int64), cfg.E, cap)
        assert np.all(out["dw"].cpu().numpy()[inv < 0] == 0.0)


# (one_token and decode_T12: moe_forward sums the split tiles inside its
# combine launch, moe_forward_train runs the split reduce and the combine)
@pytest.mark.parametrize("name", ["ragged_bf16", "tiny_fp32", "longH_bf16", "top1_bf16",
                                  "one_token_bf16", "decode_T12_bf16"])
def test_forward_train_equals_forward(name):
    """The training forward's y, ids and w are the plain forward's, bit for bit
    (top1_bf16: the plain forward combines inside its second expert GEMM, the
    training forward keeps yp and runs the combine pass)."""
    cfg = CASES[name]
    L = layer(cfg)
    y, ids, w, _ = moe.moe_forward_train(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"],
                                         cfg.k)
    ids2 = torch.empty_like(ids)
    w2 = torch.empty_like(w)
    y2 = moe.moe_forward_ex(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k,
                            topk_ids_out=ids2, topk_w_out=w2)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(y, y2)


def test_backward_is_deterministic():
    cfg = CASES["longH_bf16"]        # split-K partials included
    L, w_r, y, ids, w, saved, a = run(cfg)
    b = moe.moe_backward(L["dy"], L["x"], w_r, L["w1"], L["w2"], cfg.k, ids, w, saved)
    torch.cuda.synchronize()
    for name in ("dx", "dw_r", "dw1", "dw2", "dw"):
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_empty_batch_zeroes_weight_gradients(dtype):
    cfg = C("empty", T=0, H=64, E=4, k=2, F=32, dtype=dtype)
    L = mi.make_inputs(cfg, "cuda")
    dy = mi.make_dy(cfg, "cuda")
    y, ids, w, saved = moe.moe_forward_train(L["x"], L["w_r"], None, L["w1"], L["w2"], cfg.k)
    out = {n: torch.full(s, float("nan"), dtype=cfg.torch_dtype, device="cuda")
           for n, s in (("dw_r", (64, 4)), ("dw1", (4, 64, 32)), ("dw2", (4, 32, 64)))}
    out["db_r"] = torch.full((4,), float("nan"), device="cuda")
    g = moe.moe_backward(dy, L["x"], L["w_r"], L["w1"], L["w2"], cfg.k, ids, w, saved,
                         with_bias_grad=True, out=out)
    torch.cuda.synchronize()
    for name in ("dw_r", "dw1", "dw2", "db_r"):
        assert torch.count_nonzero(g[name]).item() == 0, name
    assert g["dx"].shape == (0, 64)


@pytest.mark.parametrize("name", ["ragged_bf16", "multitile_bf16", "ragged_f32", "longF_bf16",
                                  "period_tail_bf16"])
def test_expert_ffn_backward_stage_matches_oracle(name):
    """The expert stage alone, on seeded dispatched rows: an offsets table with
    an empty expert, dyp and xp from the seeded generator, and z, h computed by
    the oracle and rounded once to the layer's type (inputs of both sides)."""
    cfg = CASES[name]
    L = layer(cfg)
    R = cfg.R
    g = torch.Generator().manual_seed(7)
    cuts = torch.sort(torch.randint(0, R + 1, (cfg.E - 1,), generator=g)).values
    off = torch.cat([torch.zeros(1, dtype=torch.int64), cuts, torch.tensor([R])])
    off[2] = off[1]                                   # expert 1 has no rows
    off = torch.maximum(off, torch.cat([torch.zeros(1, dtype=torch.int64), off[:-1]]))
    offsets = off.to(torch.int32)
    big = mi.MoEConfig(cfg.name + "_rows", T=R, H=cfg.H, E=cfg.E, k=1, F=cfg.F, dtype=cfg.dtype,
                       seed=cfg.seed + 1)
    xp = mi.make_x(big, "cuda")
    dyp = mi.make_dy(big, "cuda")
    xp64, dyp64 = f64(xp), f64(dyp)
    w1_64, w2_64 = f64(L["w1"]), f64(L["w2"])
    z64 = np.zeros((R, cfg.F))
    for e in range(cfg.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        z64[a:b] = xp64[a:b] @ w1_64[e]
    td = cfg.torch_dtype
    z = torch.tensor(z64).to(td).cuda()
    h = torch.tensor(oracle.gelu_tanh(z64)).to(td).cuda()
    dxp, dw1, dw2 = moe.moe_expert_ffn_backward(dyp, xp, offsets.cuda(), z, h, L["w1"], L["w2"])
    torch.cuda.synchronize()
    ref_dxp, ref_dw1, ref_dw2 = oracle.expert_ffn_backward(xp64, offsets.numpy(), w1_64, w2_64,
                                                           dyp64)
    tol = TOL[cfg.dtype]
    assert_close_rel(f64(dxp), ref_dxp, tol, "dxp")
    assert_close_rel(f64(dw1), ref_dw1, tol, "dw1")
    assert_close_rel(f64(dw2), ref_dw2, tol, "dw2")
    assert torch.count_nonzero(dw1[1]).item() == 0 and torch.count_nonzero(dw2[1]).item() == 0


@pytest.mark.parametrize("name,gating", [("ragged_bf16", GT), ("ragged_bf16", GS),
                                         ("many_small_bf16", GT), ("tiny_fp32", GT)])
def test_backward_skips_out_of_range_ids(name, gating):
    """Expert ids handed back to the backward that lie outside [0, E) (-1 and
    E; not ids the training forward produced).  Such a slot is left out of the
    router gradient; the expert side and the gate-weight gradient follow the
    dispatch kept in `saved`.  Reference: the oracle's backward for the
    forward's own ids, with the softmax Jacobian redone after zeroing those
    slots' gate-weight gradient (a dropped pair's), and (top-k then softmax)
    no gradient for the logit an out-of-range id no longer names."""
    cfg = CASES[name]
    L, w_r, y, ids, w, saved, clean = run(cfg, gating, with_bias=True)
    T, k = cfg.T, cfg.k
    rng = np.random.default_rng(7)
    flat = rng.choice(T * k, size=max(2, T * k // 10), replace=False)
    vals = np.where(np.arange(len(flat)) % 2 == 0, -1, cfg.E).astype(np.int32)
    ids_bad = ids.clone()
    ids_bad.view(-1)[torch.from_numpy(flat).long().cuda()] = torch.from_numpy(vals).cuda()
    out = moe.moe_backward(L["dy"], L["x"], w_r, L["w1"], L["w2"], k, ids_bad, w, saved, gating,
                           with_bias_grad=True)
    torch.cuda.synchronize()
    for n in ("dw1", "dw2", "dw"):
        assert torch.equal(out[n], clean[n]), n
    tol = TOL[cfg.dtype]
    x64, wr64 = f64(L["x"]), f64(w_r)
    logits = oracle.router_logits(x64, wr64, f64(L["router_bias"]))
    ids_np = ids.cpu().numpy().astype(np.int64)
    bad = np.zeros(T * k, dtype=bool)
    bad[flat] = True
    bad = bad.reshape(T, k)
    ref = oracle.backward(x64, wr64, f64(L["router_bias"]), f64(L["w1"]), f64(L["w2"]), k,
                          f64(L["dy"]), ids=ids_np, gating=GNAME[gating])
    dl = oracle.gate_weights_grad(logits, ids_np, np.where(bad, 0.0, ref["dw"]), GNAME[gating])
    if gating == GT:
        tb, jb = np.nonzero(bad)
        dl[tb, ids_np[tb, jb]] = 0.0
    dx_ref = ref["dx"] - ref["dlogits"] @ wr64.T + dl @ wr64.T
    assert_close_rel(f64(out["dx"]), dx_ref, tol, "dx")
    assert_close_rel(f64(out["dw_r"]), x64.T @ dl, tol, "dw_r")
    assert_close_rel(f64(out["db_r"]), dl.sum(axis=0), tol, "db_r")


def random_cases(n=12, seed=77):
    """Seeded random training shapes (both gatings, with and without a
    capacity, bf16 and fp32), small enough for the oracle's dense backward."""
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(g.choice([1, 3, 8, 16, 40, 64, 130]))
        k = int(min(E, g.choice([1, 2, 2, 4, 8])))
        T = int(g.choice([1, 5, 48, 200, 600, 1100]))
        H = int(8 * g.integers(1, 48))
        F = int(8 * g.integers(1, 48))
        dt = "f32" if g.random() < 0.25 else "bf16"
        gating = GS if g.random() < 0.3 else GT
        capf = float(g.choice([0.0, 0.0, 0.6, 1.2]))
        cap = oracle.expert_capacity(T, k, E, capf) if capf else 0
        cfg = C(f"rb{i}_T{T}_H{H}_E{E}_k{k}_F{F}_{dt}", T=T, H=H, E=E, k=k, F=F, dtype=dt,
                bias0=float(g.choice([0.0, 1.0])), seed=300 + i)
        out.append((cfg, gating, cap))
    return out


RANDOM = random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=[c[0].name for c in RANDOM])
def test_backward_random_shape(case):
    cfg, gating, cap = case
    bias = cfg.bias0 != 0.0
    L, w_r, y, ids, w, saved, out = run(cfg, gating=gating, capacity=cap, with_bias=bias)
    check(cfg, L, w_r, ids, w, out, gating, cap, bias)
