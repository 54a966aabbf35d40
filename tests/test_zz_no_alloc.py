"""moe_forward_noalloc (the forward for callers that cannot allocate; its
workspace is the library's fixed scratch array) against moe_forward on the
same inputs, through the C ABI: two calls in a row on the same GPU, the
second with a smaller layer, then the first layer again (the scratch keeps
the previous call's contents).  Expert ids and gate weights must be
identical; y within the forward's tolerance of moe_forward's y (the no-alloc
GEMMs do not split tiles along K, so rounding may differ), 2e-2 (bf16) or
1e-4 (fp32) of its largest magnitude.  Layers too large for the scratch are
refused with MOE_ERR_UNSUPPORTED before anything is enqueued."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from moe_check import TOL, assert_close_rel, f64

pytestmark = pytest.mark.gpu

import mixture_experts_layer_21_amd as moe  # fails loudly if the library is missing

C = mi.MoEConfig
# decode-sized layers: 64 tokens with every expert touched, so that the usual
# forward splits leftover tiles along K in both GEMMs (320 and 640 tiles: 64
# tiles split 4 ways, 128 split 2 ways) where the no-alloc one runs them
# whole; then a smaller layer
SEQS = {
    "bf16": [C("na_big_bf16", T=64, H=4096, E=40, k=8, F=2048, dtype="bf16"),
             C("na_small_bf16", T=24, H=1024, E=16, k=4, F=512, dtype="bf16", bias0=1.0)],
    "f32": [mi.CONFIGS["tiny_fp32"],
            C("na_small_f32", T=20, H=64, E=4, k=2, F=96, dtype="f32")],
}


def compare(cfg, L):
    T, k = cfg.T, cfg.k
    ids0 = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w0 = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y0 = moe.moe_forward(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], k,
                         topk_ids_out=ids0, topk_w_out=w0)
    ids1 = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w1 = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    y1 = torch.full((T, cfg.H), 7.0, dtype=cfg.torch_dtype, device="cuda")
    moe.moe_forward_noalloc(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], k, y1,
                            topk_ids_out=ids1, topk_w_out=w1)
    torch.cuda.synchronize()
    assert torch.equal(ids1, ids0)
    assert torch.equal(w1, w0)
    rel = assert_close_rel(f64(y1), f64(y0), TOL[cfg.dtype], f"{cfg.name} y")
    print(f"[{cfg.name}] no-alloc vs moe_forward: ids, w equal; y max|err|/max|y| {rel:.2e}",
          flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_forward_on_consecutive_calls(dtype):
    big, small = SEQS[dtype]
    Lb = mi.make_inputs(big, "cuda")
    Ls = mi.make_inputs(small, "cuda")
    print(f"\n[case] no-alloc {big.name} -> {small.name} -> {big.name}", flush=True)
    compare(big, Lb)
    compare(small, Ls)
    compare(big, Lb)


def test_noalloc_refuses_layers_beyond_its_scratch():
    cfg = mi.CONFIGS["mixtral_bf16"]
    x = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    w_r = torch.empty((cfg.H, cfg.E), dtype=torch.bfloat16, device="cuda")
    one = torch.empty((cfg.E, 8, 8), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    lib = moe.lib()
    st = lib.moe_forward_noalloc(x.data_ptr(), w_r.data_ptr(), None, one.data_ptr(),
                                 one.data_ptr(), cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, moe.MOE_BF16,
                                 y.data_ptr(), None, None, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
