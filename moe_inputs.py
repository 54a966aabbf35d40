"""Seeded synthetic inputs for the MoE layer forward, shared by the tests, the
bench and the oracle's callers.

This module holds none of the MoE arithmetic.  It only draws the layer's
inputs (x, W_r, router bias, W1, W2, and an output gradient dy for the
backward) for the five workloads, and it draws them
so that the bits are identical whether the tensors are made on the CPU or on a
GPU:

* uniform 32-bit words come from a counter-based hash evaluated with exact
  int64 tensor arithmetic (no float math, so CPU and GPU agree bit for bit);
* a standard normal is the Irwin-Hall approximation, the sum of 12 uniforms
  minus 6 (mean 0, variance 1, support +-6), with each uniform quantised to
  odd multiples of 2**-17 so that the sum is an integer below 2**21 and is
  exact in fp32;
* the fan-in scale 1/sqrt(fan_in) is applied as one fp32 multiply (correctly
  rounded on both devices) and bf16 inputs are rounded once, to nearest even.

The hash is Chris Wellons' "lowbias32" integer mixer (Hash Prospector, 2018),
applied twice per word with per-stream keys.  Every (tensor, expert) slab is
an independent stream, so any one expert's weights can be regenerated on its
own without materialising the others.

The workloads are the forward pass of one MoE layer as the pages state it
(fused MoE operator article, section "MoE computation flow"): tokens x[T,H],
router W_r[H,E], experts W1[E,H,F] and W2[E,F,H], top_k experts per token.
"""
from __future__ import annotations

import dataclasses
import math

import torch

MASK32 = 0xFFFFFFFF
_M1 = 0x7FEB352D
_M2 = 0x846CA68B
_STREAM_X, _STREAM_WR, _STREAM_W1, _STREAM_W2, _STREAM_DY = 1, 2, 3, 4, 5
_DRAWS = 6            # 6 hashed words -> 12 uniform 16-bit halves per value
_CHUNK_CPU = 1 << 22  # values per generation chunk (bounds temporaries)
_CHUNK_GPU = 1 << 25


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    H: int          # model (hidden) width
    E: int          # experts
    k: int          # experts per token
    F: int          # expert FFN width
    dtype: str      # "f32" or "bf16": dtype of x, W_r, W1, W2 and y
    bias0: float = 0.0   # router bias on expert 0 (skewed-routing workload)
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  "skewed_bf16" biases expert 0's logit by +3.0 through
# the router bias term, which sends roughly 80-90% of tokens to expert 0 as a
# top choice (the imbalance the routing article describes).
CONFIGS = {
    "tiny_fp32": MoEConfig("tiny_fp32", T=64, H=128, E=8, k=2, F=256, dtype="f32"),
    "mixtral_bf16": MoEConfig("mixtral_bf16", T=2048, H=4096, E=8, k=2, F=14336, dtype="bf16"),
    "skewed_bf16": MoEConfig("skewed_bf16", T=2048, H=4096, E=8, k=2, F=14336, dtype="bf16", bias0=3.0),
    "many_experts_bf16": MoEConfig("many_experts_bf16", T=4096, H=2048, E=128, k=8, F=768, dtype="bf16"),
    "weight_bound_bf16": MoEConfig("weight_bound_bf16", T=64, H=7168, E=256, k=8, F=2048, dtype="bf16"),
}
CONFIG_ORDER = ["tiny_fp32", "mixtral_bf16", "skewed_bf16", "many_experts_bf16", "weight_bound_bf16"]


def _lowbias32_int(v: int) -> int:
    v &= MASK32
    v ^= v >> 16
    v = (v * _M1) & MASK32
    v ^= v >> 15
    v = (v * _M2) & MASK32
    v ^= v >> 16
    return v


def _mul32(a: torch.Tensor, c: int) -> torch.Tensor:
    """(a * c) mod 2**32 for int64 a in [0, 2**32), without int64 overflow."""
    ch, cl = c >> 16, c & 0xFFFF
    return ((((a * ch) & 0xFFFF) << 16) + a * cl) & MASK32


def _lowbias32(v: torch.Tensor) -> torch.Tensor:
    v = v ^ (v >> 16)
    v = _mul32(v, _M1)
    v = v ^ (v >> 15)
    v = _mul32(v, _M2)
    return v ^ (v >> 16)


def stream_keys(seed: int, stream: int, expert: int) -> tuple[int, int]:
    k1 = _lowbias32_int(_lowbias32_int(seed * 0x9E3779B9 + 0x1234567) ^ (stream * 0x85EBCA6B))
    k1 = _lowbias32_int(k1 ^ ((expert + 1) * 0xC2B2AE35))
    k2 = _lowbias32_int(k1 ^ 0x5BD1E995)
    return k1, k2


def uniform_words(n: int, keys: tuple[int, int], start: int = 0, device="cpu") -> torch.Tensor:
    """int64 tensor [_DRAWS, n] of hashed 32-bit words for values start..start+n-1."""
    k1, k2 = keys
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    ctr = idx.unsqueeze(0) * _DRAWS + torch.arange(_DRAWS, dtype=torch.int64, device=device).unsqueeze(1)
    ctr = ctr & MASK32
    h = _lowbias32(ctr ^ k1)
    return _lowbias32(h ^ k2)


def normal_fp32(n: int, keys: tuple[int, int], scale: float, device="cpu") -> torch.Tensor:
    """n approximately-N(0, scale**2) fp32 values; bit-identical on CPU and GPU."""
    out = torch.empty(n, dtype=torch.float32, device=device)
    s32 = torch.tensor(scale, dtype=torch.float32, device=device)
    chunk = _CHUNK_CPU if torch.device(device).type == "cpu" else _CHUNK_GPU
    for start in range(0, n, chunk):
        m = min(chunk, n - start)
        w = uniform_words(m, keys, start, device)
        lo = w & 0xFFFF
        hi = w >> 16
        # sum over 12 uniforms of (2u+1); mean 12*65536
        s = (2 * lo + 1).sum(0) + (2 * hi + 1).sum(0) - 12 * 65536
        v = s.to(torch.float32) * (2.0 ** -17)     # exact: |s| < 2**21
        out[start:start + m] = v if scale == 1.0 else v * s32
    return out


def _fill(shape, stream: int, expert: int, scale: float, cfg: MoEConfig, device) -> torch.Tensor:
    n = math.prod(shape)
    v = normal_fp32(n, stream_keys(cfg.seed, stream, expert), scale, device).view(*shape)
    return v.to(cfg.torch_dtype)


def make_x(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    return _fill((cfg.T, cfg.H), _STREAM_X, 0, 1.0, cfg, device)


def make_w_r(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    return _fill((cfg.H, cfg.E), _STREAM_WR, 0, 1.0 / math.sqrt(cfg.H), cfg, device)


def make_w_r_f32(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """W_r from the same stream as make_w_r, kept in fp32 (an fp32 router for
    a layer whose other tensors are bf16)."""
    n = cfg.H * cfg.E
    return normal_fp32(n, stream_keys(cfg.seed, _STREAM_WR, 0), 1.0 / math.sqrt(cfg.H),
                       device).view(cfg.H, cfg.E)


def make_dy(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """An output gradient dy[T,H] ~ N(0, 1) in the layer's dtype (for the backward)."""
    return _fill((cfg.T, cfg.H), _STREAM_DY, 0, 1.0, cfg, device)


def make_router_bias(cfg: MoEConfig, device="cpu"):
    """fp32 [E] router bias, or None when the workload has no bias."""
    if cfg.bias0 == 0.0:
        return None
    b = torch.zeros(cfg.E, dtype=torch.float32, device=device)
    b[0] = cfg.bias0
    return b


def make_w1_expert(cfg: MoEConfig, e: int, device="cpu") -> torch.Tensor:
    return _fill((cfg.H, cfg.F), _STREAM_W1, e, 1.0 / math.sqrt(cfg.H), cfg, device)


def make_w2_expert(cfg: MoEConfig, e: int, device="cpu") -> torch.Tensor:
    return _fill((cfg.F, cfg.H), _STREAM_W2, e, 1.0 / math.sqrt(cfg.F), cfg, device)


def make_w1(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    w = torch.empty((cfg.E, cfg.H, cfg.F), dtype=cfg.torch_dtype, device=device)
    for e in range(cfg.E):
        w[e] = make_w1_expert(cfg, e, device)
    return w


def make_w2(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    w = torch.empty((cfg.E, cfg.F, cfg.H), dtype=cfg.torch_dtype, device=device)
    for e in range(cfg.E):
        w[e] = make_w2_expert(cfg, e, device)
    return w


def make_inputs(cfg: MoEConfig, device="cpu") -> dict:
    return {
        "x": make_x(cfg, device),
        "w_r": make_w_r(cfg, device),
        "router_bias": make_router_bias(cfg, device),
        "w1": make_w1(cfg, device),
        "w2": make_w2(cfg, device),
    }


def integer_inputs(T: int, H: int, E: int, F: int, lo: int, hi: int, seed: int,
                   dtype=torch.float32, device="cpu") -> dict:
    """Small-integer-valued inputs in [lo, hi]: every product and partial sum is
    exact in bf16 x bf16 -> fp32 and in fp64, so logits (and their ties) are
    reproduced exactly on every device."""
    g = torch.Generator().manual_seed(seed)

    def ri(*shape):
        return torch.randint(lo, hi + 1, shape, generator=g).to(dtype).to(device)

    return {"x": ri(T, H), "w_r": ri(H, E), "router_bias": None,
            "w1": ri(E, H, F), "w2": ri(E, F, H)}


def to_f64_numpy(t):
    """Exact upcast of a (CPU or GPU) fp32/bf16 tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
