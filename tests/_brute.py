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


def e2m1_as_e4m3_code(c):
    """The e4m3 code holding the same value as e2m1 code c (every e2m1 value is
    an e4m3 value): sign bit 3 -> 7; exponent e > 0 -> e4m3 exponent e + 6 and
    the mantissa bit to the top of e4m3's three; e = 0 (0 or 0.5) -> 0 / 0x30."""
    c = np.asarray(c, dtype=np.uint8)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    normal = (s << 7) | ((e + 6) << 3) | (m << 2)
    sub = (s << 7) | np.where(m == 1, 0x30, 0)
    return np.where(e > 0, normal, sub).astype(np.uint8)


def e8m0_to_f64(codes) -> np.ndarray:
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e8m0fnu).to(torch.float32).numpy().astype(np.float64)


def mx_dequant(packed, scales) -> np.ndarray:
    """MXFP4 [rows, cols/2] packed (even element in the low nibble) with E8M0
    scales [rows, cols/32] -> float64 [rows, cols], decoded through torch."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, 2 * half), np.uint8)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    vals = e4m3_codes_to_f64(e2m1_as_e4m3_code(codes))
    sc = np.repeat(e8m0_to_f64(scales), 32, axis=1)
    return vals * sc


def silu(z):
    return z / (1.0 + np.exp(-z))


def dense_layer(x_bits, wr_bits, bias, w1, w2, k, *, fp8=False, w1_scale=None,
                w2_scale=None, w_f64=None):
    """fp64 output [M,K], picked ids [M,k] and full weight matrix [M,E].

    ``w_f64`` = (W1 [E,2N,K], W2 [E,K,N]) already-dequantised float64 weights
    for the FP8 activation path (then w1/w2 and their scales are unused)."""
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
        if fp8 and w_f64 is not None:
            W1, W2 = w_f64[0][e], w_f64[1][e]
            h = (xd @ W1.T) * sx.astype(np.float64)[:, None]
        elif fp8:
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
            s2 = (np.ones(1) if w_f64 is not None
                  else np.asarray(w2_scale[e], dtype=np.float64).reshape(-1))  # [1] or [K]
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
