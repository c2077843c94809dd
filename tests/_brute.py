"""Independent numpy brute force for tiny MoE layers (test-only).

Evaluates EVERY expert densely for every token and weights the experts a
token did not pick by zero, so it shares neither the oracle's loops nor its
gating code: selection is numpy's stable argsort, the routing weights are
the full softmax renormalised over the picked experts, the expert MLP is
numpy matmuls, and FP8 codes come from torch's float8_e4m3fn casts.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_codes_to_f64(codes) -> np.ndarray:
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def f32_to_e4m3_codes(v32) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quant_rows(v32: np.ndarray):
    """Per-row dynamic e4m3 codes and scales of fp32 rows."""
    v32 = np.asarray(v32, dtype=np.float32)
    amax = np.abs(v32).max(axis=-1).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    r = (v32 / s[..., None]).astype(np.float32)
    return f32_to_e4m3_codes(r), s


def silu(z):
    return z / (1.0 + np.exp(-z))


def dense_layer(x_bits, wr_bits, bias, w1, w2, k, *, fp8=False, w1_scale=None,
                w2_scale=None):
    """fp64 output [M,K], picked ids [M,k] and full weight matrix [M,E]."""
    x = bf16_bits_to_f64(x_bits)
    wr = bf16_bits_to_f64(wr_bits)
    M, K = x.shape
    E = wr.shape[0]
    lg = x @ wr.T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float64)[None, :]
    l32 = lg.astype(np.float32)
    order = np.argsort(-l32, axis=1, kind="stable")[:, :k]
    l64 = l32.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    wfull = np.zeros((M, E))
    for t in range(M):
        sel = order[t]
        wfull[t, sel] = p[t, sel] / p[t, sel].sum()
    out = np.zeros((M, K))
    if fp8:
        xq, sx = quant_rows(x.astype(np.float32))
        xd = e4m3_codes_to_f64(xq)
    for e in range(E):
        if fp8:
            W1 = e4m3_codes_to_f64(w1[e])
            W2 = e4m3_codes_to_f64(w2[e])
            s1 = np.asarray(w1_scale[e], dtype=np.float64).reshape(-1)  # [1] or [2N]
            h = (xd @ W1.T) * sx.astype(np.float64)[:, None] * s1[None, :]
        else:
            W1 = bf16_bits_to_f64(w1[e])
            W2 = bf16_bits_to_f64(w2[e])
            h = x @ W1.T
        N = W1.shape[0] // 2
        act = silu(h[:, :N]) * h[:, N:]
        if fp8:
            aq, sa = quant_rows(act.astype(np.float32))
            s2 = np.asarray(w2_scale[e], dtype=np.float64).reshape(-1)  # [1] or [K]
            y = (e4m3_codes_to_f64(aq) @ W2.T) * sa.astype(np.float64)[:, None] * s2[None, :]
        else:
            y = act @ W2.T
        out += wfull[:, e:e + 1] * y
    return out, order.astype(np.int32), wfull


def row_rel_err(got, ref) -> float:
    """max over rows of max|got-ref| / max|ref| (the layer's error metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(got - ref).max(axis=1) / den).max())
