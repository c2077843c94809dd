"""Seeded synthetic inputs for the fused MoE layer.

This module only draws random tensors; it holds none of the layer's
arithmetic, and both the HIP path and the CPU oracle receive the very bytes
it produces.  Recipe (one ``torch.Generator`` per workload, seeded with
``seed``, on the device the tensors are made on):

  draw order: x, router weights, router bias (if any), then W1 of experts
  0..E-1, then W2 of experts 0..E-1;
  x      [M,K]    ~ N(0, 1)          fp32 draw, cast to bf16 (RNE)
  W_r    [E,K]    ~ N(0, 1/K)        bf16
  bias   [E]      ~ N(0, bias_var)   fp32, only where the workload skews routing
  W1[e]  [2N,K]   ~ N(0, 1/K)        bf16, or e4m3 (see below)
  W2[e]  [K,N]    ~ N(0, 1/N)        bf16, or e4m3

The variances are fan-in variances (N(0, 1/fan_in) gives unit-variance
logits and pre-activations).  For e4m3 workloads each expert tensor is
stored per-tensor quantised, the way an FP8 per-tensor checkpoint arrives:
scale = amax/448 in fp32, codes = torch's float8_e4m3fn cast of W/scale
clamped to +-448 (with fp8_rowwise: the same per output row).  That offline weight preparation is input
generation, not a step of the layer; the activations are quantised by the
layer itself at run time.

The same seed gives different bytes on the CPU and on a GPU (different
generators), so a workload is named by (sizes, seed, device kind).  Large
workloads are drawn on the GPU, expert by expert, to keep host memory small.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    E: int
    topk: int
    fp8: bool = False
    fp8_rowwise: bool = False   # e4m3 scales per output row instead of per tensor
    mxfp4: bool = False         # MXFP4 weights (implies e4m3 activations)
    bias_var: Optional[float] = None
    seed: int = 0

    def resized(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def slots(self) -> int:
        return self.M * self.topk


# The five workloads of the layer's statement: a tiny correctness case,
# Mixtral-shaped decode, single-token decode, Mixtral-shaped prefill with a
# skewed router, and DeepSeek-V3-shaped routed experts in FP8.
WORKLOADS = {
    "tiny": Workload("tiny", M=64, K=256, N=512, E=8, topk=2),
    "mixtral_decode": Workload("mixtral_decode", M=8, K=4096, N=14336, E=8, topk=2),
    "single_token_decode": Workload("single_token_decode", M=1, K=4096, N=8192, E=16,
                                    topk=2),
    "mixtral_prefill": Workload("mixtral_prefill", M=4096, K=4096, N=14336, E=8, topk=2,
                                bias_var=0.5),
    "dsv3_fp8": Workload("dsv3_fp8", M=128, K=7168, N=2048, E=256, topk=8, fp8=True),
}


def _quant_tensor(w32: torch.Tensor, rowwise: bool = False):
    """e4m3 codes and fp32 scale(s) amax/448: one for the tensor, or one per
    row (output channel) with ``rowwise``."""
    if rowwise:
        amax = w32.abs().amax(dim=1).to(torch.float32)
        scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (w32 / scale[:, None]).clamp(-448.0, 448.0)
    else:
        amax = w32.abs().max().to(torch.float32)
        scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (w32 / scale).clamp(-448.0, 448.0)
    return q.to(torch.float8_e4m3fn).view(torch.uint8), scale


_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _quant_mxfp4(w32: torch.Tensor):
    """OCP MXFP4 of a [rows, cols] matrix: per 32-element block of a row the
    E8M0 scale 2^(floor(log2 amax) - 2) (6 = 1.5 * 2^2 is e2m1's largest
    value), elements rounded to the nearest e2m1 value (saturating at 6),
    packed two per byte with the even element in the low nibble.  Returns
    (packed uint8 [rows, cols/2], scales uint8 [rows, cols/32])."""
    rows, cols = w32.shape
    blk = w32.reshape(rows, cols // 32, 32)
    amax = blk.abs().amax(dim=2)
    ex = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.full_like(amax, -127))
    ex = ex.clamp(-127, 127)
    scales = (ex + 127).to(torch.uint8)
    v = blk / torch.exp2(ex)[..., None]
    table = torch.tensor(_E2M1, device=w32.device)
    mag = (v.abs()[..., None] - table).abs().argmin(dim=-1).to(torch.uint8)  # nearest value
    code = mag | ((v < 0).to(torch.uint8) << 3)
    code = code.reshape(rows, cols)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), scales.contiguous()


def generate(wl: Workload, device="cpu") -> dict:
    """Draw all tensors of ``wl`` on ``device``.

    Returns a dict with x [M,K] bf16, w_router [E,K] bf16, bias [E] fp32 or
    None, w1 [E,2N,K] and w2 [E,K,N] (bf16, or uint8 e4m3 codes), and
    w1_scale / w2_scale fp32: [E] per tensor, or [E,2N] / [E,K] per output
    row with ``fp8_rowwise`` (None for bf16).  With ``mxfp4``: w1 [E,2N,K/2]
    and w2 [E,K,N/2] packed e2m1, scales uint8 E8M0 [E,2N,K/32] / [E,K,N/32]."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed)
    M, K, N, E = wl.M, wl.K, wl.N, wl.E

    def normal(shape, var):
        return torch.randn(shape, generator=g, device=device,
                           dtype=torch.float32) * math.sqrt(var)

    x = normal((M, K), 1.0).to(torch.bfloat16)
    w_router = normal((E, K), 1.0 / K).to(torch.bfloat16)
    bias = normal((E,), wl.bias_var) if wl.bias_var is not None else None
    if wl.mxfp4:
        w1 = torch.empty((E, 2 * N, K // 2), dtype=torch.uint8, device=device)
        w2 = torch.empty((E, K, N // 2), dtype=torch.uint8, device=device)
        w1_scale = torch.empty((E, 2 * N, K // 32), dtype=torch.uint8, device=device)
        w2_scale = torch.empty((E, K, N // 32), dtype=torch.uint8, device=device)
        for e in range(E):
            w1[e], w1_scale[e] = _quant_mxfp4(normal((2 * N, K), 1.0 / K))
        for e in range(E):
            w2[e], w2_scale[e] = _quant_mxfp4(normal((K, N), 1.0 / N))
        return {"x": x, "w_router": w_router, "bias": bias, "w1": w1, "w2": w2,
                "w1_scale": w1_scale, "w2_scale": w2_scale}
    wdt = torch.uint8 if wl.fp8 else torch.bfloat16
    w1 = torch.empty((E, 2 * N, K), dtype=wdt, device=device)
    w2 = torch.empty((E, K, N), dtype=wdt, device=device)
    s1_shape = (E, 2 * N) if wl.fp8_rowwise else (E,)
    s2_shape = (E, K) if wl.fp8_rowwise else (E,)
    w1_scale = torch.empty(s1_shape, dtype=torch.float32, device=device) if wl.fp8 else None
    w2_scale = torch.empty(s2_shape, dtype=torch.float32, device=device) if wl.fp8 else None
    for e in range(E):
        w = normal((2 * N, K), 1.0 / K)
        if wl.fp8:
            w1[e], w1_scale[e] = _quant_tensor(w, wl.fp8_rowwise)
        else:
            w1[e] = w.to(torch.bfloat16)
        del w
    for e in range(E):
        w = normal((K, N), 1.0 / N)
        if wl.fp8:
            w2[e], w2_scale[e] = _quant_tensor(w, wl.fp8_rowwise)
        else:
            w2[e] = w.to(torch.bfloat16)
        del w
    return {"x": x, "w_router": w_router, "bias": bias, "w1": w1, "w2": w2,
            "w1_scale": w1_scale, "w2_scale": w2_scale}


def to_numpy_bits(t: Optional[torch.Tensor]):
    """Host numpy view of a tensor: bf16 -> uint16 bits, uint8 stays, fp32 stays."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
