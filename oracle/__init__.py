"""fp64 CPU oracle of the fused MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never imports, links or loads it, and it imports nothing from the product
package.  The arithmetic lives in ``moe_oracle.c`` (plain C, fp64); this
module builds it with gcc and marshals numpy arrays through ctypes.

What each function computes, and the page passage it follows, is stated in
``moe_oracle.c``.  bf16 tensors travel as ``numpy.uint16`` bit patterns and
e4m3 tensors as ``numpy.uint8`` codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ORC_OK = 0
ORC_ERR_ARG = 1
ORC_ERR_MISSING_EXPERT = 2
ORC_ERR_NOMEM = 3

BF16 = 0
FP8_E4M3 = 1            # per-tensor weight scales [E]
FP8_E4M3_ROWWISE = 2    # per-channel weight scales [E,2N] / [E,K]
MXFP4 = 3               # e2m1 weights, E8M0 scale per 32 elements of a row


def build() -> str:
    """Compile ``moe_oracle.c`` into ``liboracle.so`` (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = ctypes.c_double
        lib.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_to_f64.restype = ctypes.c_double
        lib.orc_e2m1_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_e2m1_to_f64.restype = ctypes.c_double
        lib.orc_e8m0_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_e8m0_to_f64.restype = ctypes.c_double
        lib.orc_f32_to_e4m3.argtypes = [ctypes.c_float]
        lib.orc_f32_to_e4m3.restype = ctypes.c_uint8
        lib.orc_logits.argtypes = [P, P, P, I64, I64, I64, P]
        lib.orc_topk.argtypes = [P, I64, I64, I64, P, P]
        lib.orc_align.argtypes = [P, I64, I64, I64, I64, P, P, P, P]
        lib.orc_quant_rows_bf16.argtypes = [P, I64, I64, P, P]
        lib.orc_quant_rows_f32.argtypes = [P, I64, I64, P, P]
        lib.orc_moe_forward.argtypes = [ctypes.c_int, P, P, P, P, P, P, P,
                                        I64, I64, I64, I64, I64, P, I64, P, P, P]
        lib.orc_num_threads.restype = ctypes.c_int
        for name in ("orc_logits", "orc_topk", "orc_align", "orc_quant_rows_bf16",
                     "orc_quant_rows_f32", "orc_moe_forward"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != ORC_OK:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().orc_num_threads())


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Elementwise bf16 bit pattern -> float64."""
    lib = _load()
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    flat = out.reshape(-1)
    for i, v in enumerate(b.reshape(-1).tolist()):
        flat[i] = lib.orc_bf16_to_f64(v)
    return out


def e4m3_to_f64(codes) -> np.ndarray:
    """Elementwise OCP E4M3FN code -> float64 (NaN for 0x7F/0xFF)."""
    lib = _load()
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    flat = out.reshape(-1)
    for i, v in enumerate(c.reshape(-1).tolist()):
        flat[i] = lib.orc_e4m3_to_f64(v)
    return out


def f32_to_e4m3(values) -> np.ndarray:
    """Elementwise fp32 -> OCP E4M3FN code (RNE, saturating to +-448)."""
    lib = _load()
    v = _c(values, np.float32)
    out = np.empty(v.shape, np.uint8)
    flat = out.reshape(-1)
    for i, x in enumerate(v.reshape(-1).tolist()):
        flat[i] = lib.orc_f32_to_e4m3(x)
    return out


# --------------------------------------------------------------------------
# the layer's steps
# --------------------------------------------------------------------------

def logits(x, w_router, bias=None) -> np.ndarray:
    """fp32 router logits [M,E] (fp64 dot product, one rounding)."""
    lib = _load()
    x = _c(x, np.uint16)
    wr = _c(w_router, np.uint16)
    M, K = x.shape
    E = wr.shape[0]
    assert wr.shape[1] == K
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((M, E), np.float32)
    _check(lib.orc_logits(_ptr(x), _ptr(wr), _ptr(b), M, K, E, _ptr(out)), "logits")
    return out


def topk(lg, k):
    """(ids int32 [M,k], weights float64 [M,k]) from fp32 logits [M,E]."""
    lib = _load()
    lg = _c(lg, np.float32)
    M, E = lg.shape
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float64)
    _check(lib.orc_topk(_ptr(lg), M, E, k, _ptr(ids), _ptr(w)), "topk")
    return ids, w


def align(ids, E, block):
    """Expert-sorted, block-padded permutation of the flattened ids.

    Returns (sorted_ids [M*k + E*(B-1)], block_expert [that // B],
    expert_offsets [E+1], num_padded)."""
    lib = _load()
    ids = _c(ids, np.int32)
    M, k = ids.shape
    cap = M * k + E * (block - 1)
    sorted_ids = np.empty(cap, np.int32)
    block_expert = np.empty(cap // block, np.int32)
    offsets = np.empty(E + 1, np.int32)
    npad = np.empty(1, np.int32)
    _check(lib.orc_align(_ptr(ids), M, k, E, block, _ptr(sorted_ids),
                         _ptr(block_expert), _ptr(offsets), _ptr(npad)), "align")
    return sorted_ids, block_expert, offsets, int(npad[0])


def quant_rows_bf16(x):
    """Per-row dynamic e4m3 quantisation of bf16 rows: (codes, scales)."""
    lib = _load()
    x = _c(x, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty(M, np.float32)
    _check(lib.orc_quant_rows_bf16(_ptr(x), M, K, _ptr(q), _ptr(s)), "quant")
    return q, s


def quant_rows_f32(v):
    """Per-row dynamic e4m3 quantisation of fp32 rows: (codes, scales)."""
    lib = _load()
    v = _c(v, np.float32)
    M, K = v.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty(M, np.float32)
    _check(lib.orc_quant_rows_f32(_ptr(v), M, K, _ptr(q), _ptr(s)), "quant")
    return q, s


def e2m1_to_f64(codes) -> np.ndarray:
    """The oracle's e2m1 decoding of 4-bit codes (R9)."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_e2m1_to_f64(int(v)) for v in c.reshape(-1)]).reshape(c.shape)


def e8m0_to_f64(codes) -> np.ndarray:
    """The oracle's E8M0 scale decoding (R9)."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_e8m0_to_f64(int(v)) for v in c.reshape(-1)]).reshape(c.shape)


def moe_forward(x, w_router, bias, w1, w2, k, *, w1_scale=None, w2_scale=None,
                tokens=None, fp8=False, mxfp4=False):
    """The whole layer in fp64 for the given tokens (default: all).

    ``w1`` / ``w2`` are either full arrays [E,2N,K] / [E,K,N] or sequences of
    per-expert arrays (None where an expert's weights are not provided; the
    oracle fails if a routed expert is missing).  With ``fp8`` the scales are
    per expert tensor ([E]) or per output channel ([E,2N] and [E,K]).  With
    ``mxfp4`` the weights are packed e2m1 (w1[e] [2N,K/2], w2[e] [K,N/2]) and
    the scales E8M0 bytes (w1_scale [E,2N,K/32], w2_scale [E,K,N/32]).
    Returns (out float64 [n_tok,K], ids int32 [n_tok,k], weights float64
    [n_tok,k]).
    """
    lib = _load()
    x = _c(x, np.uint16)
    wr = _c(w_router, np.uint16)
    M, K = x.shape
    E = wr.shape[0]
    wdt = np.uint8 if (fp8 or mxfp4) else np.uint16
    w1_list = [None if w is None else _c(w, wdt) for w in w1]
    w2_list = [None if w is None else _c(w, wdt) for w in w2]
    assert len(w1_list) == E and len(w2_list) == E
    N = None
    for a, b in zip(w1_list, w2_list):
        if a is not None:
            N = a.shape[0] // 2
            if mxfp4:
                assert a.shape == (2 * N, K // 2) and b.shape == (K, N // 2)
            else:
                assert a.shape == (2 * N, K) and b.shape == (K, N)
    if N is None:
        raise ValueError("no expert weights given")
    arr1 = (ctypes.c_void_p * E)(*[None if a is None else a.ctypes.data for a in w1_list])
    arr2 = (ctypes.c_void_p * E)(*[None if a is None else a.ctypes.data for a in w2_list])
    b = None if bias is None else _c(bias, np.float32)
    sdt = np.uint8 if mxfp4 else np.float32
    s1 = None if w1_scale is None else _c(w1_scale, sdt)
    s2 = None if w2_scale is None else _c(w2_scale, sdt)
    toks = np.arange(M, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    n_tok = toks.shape[0]
    out = np.empty((n_tok, K), np.float64)
    ids = np.empty((n_tok, k), np.int32)
    wts = np.empty((n_tok, k), np.float64)
    dtype = BF16
    if mxfp4:
        assert s1 is not None and s1.shape == (E, 2 * N, K // 32)
        assert s2 is not None and s2.shape == (E, K, N // 32)
        dtype = MXFP4
    elif fp8:
        dtype = FP8_E4M3
        if s1 is not None and s1.ndim == 2:
            assert s1.shape == (E, 2 * N) and s2 is not None and s2.shape == (E, K)
            dtype = FP8_E4M3_ROWWISE
        else:
            assert s1 is not None and s1.shape == (E,) and s2 is not None and s2.shape == (E,)
    rc = lib.orc_moe_forward(dtype, _ptr(x), _ptr(wr), _ptr(b),
                             ctypes.cast(arr1, ctypes.c_void_p),
                             ctypes.cast(arr2, ctypes.c_void_p), _ptr(s1), _ptr(s2),
                             M, K, N, E, k, _ptr(toks), n_tok, _ptr(out), _ptr(ids),
                             _ptr(wts))
    _check(rc, "moe_forward")
    return out, ids, wts
