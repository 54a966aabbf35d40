"""The layer's launches captured in a HIP graph (torch.cuda.CUDAGraph over the
binding, which enqueues on torch's current stream).  The library makes no
allocation, synchronisation, copy or memset call on its launch paths (zero
fills are kernels), so moe_forward, moe_forward_noalloc and a training step
(moe_forward_train then moe_backward) can be captured once and replayed.

Each graph is replayed for several token matrices: eager work between the
replays copies new tokens into the captured x and overwrites every output
with a fill value, and each replay must give the eager call's results on the
same tokens bit for bit (ids, gate weights, y, and for the training step
every gradient)."""
import dataclasses

import pytest
import torch

import moe_inputs as mi
from moe_check import gpu_layer

pytestmark = pytest.mark.gpu

import mixture_experts_layer_21_amd as moe  # fails loudly if the library is missing

C = mi.MoEConfig
CASES = {
    "ragged_bf16": C("g_ragged_bf16", T=75, H=200, E=5, k=2, F=136, dtype="bf16"),
    # one-launch router, top-1 (the combine inside the second GEMM)
    "top1_bf16": C("g_top1_bf16", T=1025, H=448, E=8, k=1, F=64, dtype="bf16"),
    # one token (decode): the one-launch router's single, mostly empty tile
    "decode_bf16": C("g_decode_bf16", T=1, H=4096, E=8, k=2, F=512, dtype="bf16"),
    # few tiles with a long K: split tiles and their reduce launch
    "ksplit_bf16": C("g_ksplit_bf16", T=300, H=4096, E=2, k=2, F=512, dtype="bf16"),
    "many_bf16": C("g_many_bf16", T=1100, H=128, E=40, k=6, F=64, dtype="bf16"),
    "ragged_f32": C("g_ragged_f32", T=70, H=72, E=6, k=3, F=40, dtype="f32"),
}
REPLAYS = 3


def token_sets(cfg, L):
    """The layer's own tokens, then tokens of other seeds (same recipe)."""
    xs = [L["x"].clone()]
    for i in range(1, REPLAYS):
        other = dataclasses.replace(cfg, seed=cfg.seed + 1000 * i)
        xs.append(mi.make_x(other, "cuda"))
    return xs


def capture(fn):
    """fn captured in a graph after one eager warm-up run on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def scramble(*ts):
    for t in ts:
        if t.dtype in (torch.int32, torch.uint8):
            t.fill_(-3 if t.dtype == torch.int32 else 0x5A)
        else:
            t.fill_(7.0)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("entry", ["moe_forward", "moe_forward_noalloc"])
def test_forward_graph_replays(name, entry):
    cfg = CASES[name]
    L = gpu_layer(cfg)
    T, H, k = cfg.T, cfg.H, cfg.k
    x = L["x"].clone()
    y = torch.empty((T, H), dtype=x.dtype, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    args = (L["w_r"], L["router_bias"], L["w1"], L["w2"], k)
    if entry == "moe_forward":
        ws = torch.empty(moe.moe_workspace_bytes(T, H, cfg.E, k, cfg.F, x.dtype),
                         dtype=torch.uint8, device="cuda")

        def fwd():
            moe.moe_forward(x, *args, y=y, topk_ids_out=ids, topk_w_out=w, ws=ws)
    else:
        def fwd():
            moe.moe_forward_noalloc(x, *args, y, topk_ids_out=ids, topk_w_out=w)
    g = capture(fwd)
    eager = getattr(moe, entry)
    for i, xi in enumerate(token_sets(cfg, L)):
        print(f"[graph] {entry} {name} replay {i}", flush=True)
        x.copy_(xi)
        scramble(y, ids, w)
        g.replay()
        torch.cuda.synchronize()
        y_ref = torch.empty_like(y)
        ids_ref = torch.empty_like(ids)
        w_ref = torch.empty_like(w)
        eager(xi, *args, y_ref, topk_ids_out=ids_ref, topk_w_out=w_ref) \
            if entry == "moe_forward_noalloc" else \
            eager(xi, *args, y=y_ref, topk_ids_out=ids_ref, topk_w_out=w_ref)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_ref), f"replay {i}: ids"
        assert torch.equal(w, w_ref), f"replay {i}: gate weights"
        assert torch.equal(y, y_ref), f"replay {i}: y"


@pytest.mark.parametrize("name", ["ragged_bf16", "decode_bf16", "ksplit_bf16", "many_bf16",
                                  "ragged_f32"])
def test_training_step_graph_replays(name):
    cfg = CASES[name]
    L = gpu_layer(cfg)
    T, H, E, k, F = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F
    x = L["x"].clone()
    dt = x.dtype
    dy = mi.make_dy(cfg, "cuda")
    y = torch.empty((T, H), dtype=dt, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    saved = torch.empty(moe.moe_saved_bytes(T, H, E, k, F, dt), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(moe.moe_workspace_bytes(T, H, E, k, F, dt), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(moe.moe_backward_workspace_bytes(T, H, E, k, F, dt), dtype=torch.uint8,
                       device="cuda")
    shapes = {"dx": ((T, H), dt), "dw_r": ((H, E), L["w_r"].dtype), "db_r": ((E,), torch.float32),
              "dw1": ((E, H, F), dt), "dw2": ((E, F, H), dt), "dw": ((T, k), torch.float32)}
    out = {n: torch.empty(s, dtype=d, device="cuda") for n, (s, d) in shapes.items()}
    wargs = (L["w_r"], L["router_bias"], L["w1"], L["w2"], k)

    def step():
        moe.moe_forward_train(x, *wargs, y=y, topk_ids=ids, topk_w=w, saved=saved, ws=ws_f)
        moe.moe_backward(dy, x, L["w_r"], L["w1"], L["w2"], k, ids, w, saved,
                         with_bias_grad=True, out=out, ws=ws_b)
    g = capture(step)
    for i, xi in enumerate(token_sets(cfg, L)):
        print(f"[graph] training step {name} replay {i}", flush=True)
        x.copy_(xi)
        scramble(y, ids, w, saved, *out.values())
        g.replay()
        torch.cuda.synchronize()
        y_ref, ids_ref, w_ref, saved_ref = moe.moe_forward_train(xi, *wargs)
        ref = moe.moe_backward(dy, xi, L["w_r"], L["w1"], L["w2"], k, ids_ref, w_ref, saved_ref,
                               with_bias_grad=True)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_ref), f"replay {i}: ids"
        assert torch.equal(w, w_ref), f"replay {i}: gate weights"
        assert torch.equal(y, y_ref), f"replay {i}: y"
        for n in shapes:
            assert torch.equal(out[n], ref[n]), f"replay {i}: {n}"
