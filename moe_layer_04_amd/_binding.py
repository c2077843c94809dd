"""Thin ctypes binding of libmoe.so (the C ABI in include/moe.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs and the workspace are allocated with torch (plumbing),
and every step of the layer runs in the library's HIP kernels on the
current torch stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

from . import build as _build

LIB_PATH = _build.LIB

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

MOE_BF16 = 0
MOE_FP8_E4M3 = 1
MOE_FP8_E4M3_ROWWISE = 2
MOE_MXFP4_E2M1 = 3

MOE_REGIME_AUTO = 0
MOE_REGIME_DECODE = 1
MOE_REGIME_PREFILL = 2

EXPORTS = ("moe_topk", "moe_align", "moe_align_ex", "moe_quant_rows_e4m3", "moe_fused_forward",
           "moe_fused_forward_ex", "moe_fused_forward_timed", "moe_fused_plan",
           "moe_fused_forward_noalloc", "moe_fused_graph_create", "moe_fused_graph_launch",
           "moe_fused_graph_destroy", "moe_status_string")

NOALLOC_SCRATCH_BYTES = 128 << 20   # MOE_NOALLOC_SCRATCH_BYTES


class Plan(ctypes.Structure):
    """moe_plan of include/moe.h: the launch plan of the fused forward for a
    shape, and where its routing outputs sit in the workspace."""
    _fields_ = [("regime", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("sorted_rows", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("gemm2_splits", ctypes.c_int32), ("logit_splits", ctypes.c_int32),
                ("fused_decode", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("logits_offset", ctypes.c_uint64),
                ("topk_ids_offset", ctypes.c_uint64), ("topk_weights_offset", ctypes.c_uint64),
                ("sorted_ids_offset", ctypes.c_uint64), ("block_expert_offset", ctypes.c_uint64),
                ("expert_offsets_offset", ctypes.c_uint64),
                ("num_padded_offset", ctypes.c_uint64)]

_lock = threading.Lock()
_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)} ({status})")


def load_library(build_if_missing: bool = False):
    """Load libmoe.so (torch first, so the process has one HIP runtime)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            if not build_if_missing:
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m moe_layer_04_amd.build`")
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        P, I, SZP = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)
        lib.moe_topk.argtypes = [P, P, P, I, I, I, I, P, P, P, P]
        lib.moe_align.argtypes = [P, I, I, I, I, P, P, P, P, P]
        lib.moe_align_ex.argtypes = [P, I, I, I, I, P, P, P, P, P, SZP, P]
        lib.moe_quant_rows_e4m3.argtypes = [P, I, I, P, P, P]
        lib.moe_fused_forward.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, SZP, P]
        lib.moe_fused_forward_ex.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, P,
                                             SZP, P]
        lib.moe_fused_forward_timed.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, P,
                                                SZP, P, P]
        lib.moe_fused_plan.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(Plan)]
        lib.moe_fused_forward_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P]
        lib.moe_fused_graph_create.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, P,
                                               ctypes.c_size_t, P, ctypes.POINTER(P)]
        lib.moe_fused_graph_launch.argtypes = [P, P]
        lib.moe_fused_graph_destroy.argtypes = [P]
        for name in ("moe_topk", "moe_align", "moe_align_ex", "moe_quant_rows_e4m3",
                     "moe_fused_forward", "moe_fused_forward_ex", "moe_fused_forward_timed",
                     "moe_fused_plan", "moe_fused_forward_noalloc", "moe_fused_graph_create",
                     "moe_fused_graph_launch", "moe_fused_graph_destroy"):
            getattr(lib, name).restype = ctypes.c_int
        lib.moe_status_string.argtypes = [I]
        lib.moe_status_string.restype = ctypes.c_char_p
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().moe_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoEError(rc, what)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------

def moe_topk(x: torch.Tensor, w_router: torch.Tensor, router_bias: Optional[torch.Tensor],
             topk: int):
    """Router: (topk_ids int32 [M,k], topk_weights fp32 [M,k], logits fp32 [M,E])."""
    lib = load_library()
    M, K = x.shape
    E = w_router.shape[0]
    _dev(x, "x", torch.bfloat16)
    _dev(w_router, "w_router", torch.bfloat16, (E, K))
    if router_bias is not None:
        _dev(router_bias, "router_bias", torch.float32, (E,))
    dev = x.device
    ids = torch.empty((M, topk), dtype=torch.int32, device=dev)
    w = torch.empty((M, topk), dtype=torch.float32, device=dev)
    logits = torch.empty((M, E), dtype=torch.float32, device=dev)
    _check(lib.moe_topk(_ptr(x), _ptr(w_router), _ptr(router_bias), M, K, E, topk, _ptr(ids),
                        _ptr(w), _ptr(logits), _stream(dev)), "moe_topk")
    return ids, w, logits


def moe_align(topk_ids: torch.Tensor, num_experts: int, block_m: int):
    """(sorted_ids [M*k + E*(B-1)], block_expert [that // B], expert_offsets [E+1],
    num_padded [1]), all int32 on the device."""
    lib = load_library()
    _dev(topk_ids, "topk_ids", torch.int32)
    M, k = topk_ids.shape
    cap = M * k + num_experts * (block_m - 1)
    dev = topk_ids.device
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.moe_align(_ptr(topk_ids), M, k, num_experts, block_m, _ptr(sorted_ids),
                         _ptr(block_expert), _ptr(offsets), _ptr(npad), _stream(dev)),
           "moe_align")
    return sorted_ids, block_expert[: cap // block_m], offsets, npad


def moe_align_ex(topk_ids: torch.Tensor, num_experts: int, block_m: int):
    """moe_align through moe_align_ex (many workgroups above 2048 slots, with
    a workspace allocated here); the same outputs."""
    lib = load_library()
    _dev(topk_ids, "topk_ids", torch.int32)
    M, k = topk_ids.shape
    cap = M * k + num_experts * (block_m - 1)
    dev = topk_ids.device
    nbytes = ctypes.c_size_t(0)
    _check(lib.moe_align_ex(None, M, k, num_experts, block_m, None, None, None, None, None,
                            ctypes.byref(nbytes), None), "moe_align_ex (size query)")
    ws = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=dev)
    nbytes = ctypes.c_size_t(ws.numel())
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.moe_align_ex(_ptr(topk_ids), M, k, num_experts, block_m, _ptr(sorted_ids),
                            _ptr(block_expert), _ptr(offsets), _ptr(npad), _ptr(ws),
                            ctypes.byref(nbytes), _stream(dev)), "moe_align_ex")
    return sorted_ids, block_expert[: cap // block_m], offsets, npad


def moe_quant_rows_e4m3(x: torch.Tensor):
    """Per-row dynamic e4m3: (codes uint8 [M,K], scales fp32 [M])."""
    lib = load_library()
    _dev(x, "x", torch.bfloat16)
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib.moe_quant_rows_e4m3(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(x.device)),
           "moe_quant_rows_e4m3")
    return q, s


def _weight_dtype(w1: torch.Tensor, w1_scale: Optional[torch.Tensor]) -> int:
    """bf16 weights, or e4m3 codes (uint8) with per-tensor scales [E] or
    per-channel scales [E,2N] (MOE_FP8_E4M3_ROWWISE)."""
    if w1.dtype != torch.uint8:
        return MOE_BF16
    if w1_scale is not None and w1_scale.dtype == torch.uint8:
        return MOE_MXFP4_E2M1
    if w1_scale is not None and w1_scale.dim() == 2:
        return MOE_FP8_E4M3_ROWWISE
    return MOE_FP8_E4M3


def fused_plan(dtype: int, M: int, K: int, N: int, E: int, topk: int,
               regime: int = MOE_REGIME_AUTO) -> Plan:
    """The library's launch plan for this shape (no GPU call is made)."""
    plan = Plan()
    _check(load_library().moe_fused_plan(dtype, M, K, N, E, topk, regime, ctypes.byref(plan)),
           "moe_fused_plan")
    return plan


def fused_routing(workspace: torch.Tensor, plan: Plan, M: int, E: int, topk: int) -> dict:
    """Views of the routing outputs a completed moe_fused_forward left in its
    workspace (offsets from ``plan``): logits, topk_ids, topk_weights,
    sorted_ids, block_expert, expert_offsets, num_padded."""
    _dev(workspace, "workspace", torch.uint8)

    def view(off, n, dt):
        nbytes = n * 4
        return workspace[off: off + nbytes].view(dt)

    return {
        "logits": view(plan.logits_offset, M * E, torch.float32).view(M, E),
        "topk_ids": view(plan.topk_ids_offset, M * topk, torch.int32).view(M, topk),
        "topk_weights": view(plan.topk_weights_offset, M * topk, torch.float32).view(M, topk),
        "sorted_ids": view(plan.sorted_ids_offset, plan.sorted_rows, torch.int32),
        "block_expert": view(plan.block_expert_offset, plan.max_blocks, torch.int32),
        "expert_offsets": view(plan.expert_offsets_offset, E + 1, torch.int32),
        "num_padded": view(plan.num_padded_offset, 1, torch.int32),
    }


def workspace_size(dtype: int, M: int, K: int, N: int, E: int, topk: int,
                   regime: int = MOE_REGIME_AUTO) -> int:
    """Bytes of workspace moe_fused_forward needs (no GPU call is made)."""
    lib = load_library()
    nbytes = ctypes.c_size_t(0)
    dummy = ctypes.c_void_p(0x100)
    s1 = dummy if dtype in (MOE_FP8_E4M3, MOE_FP8_E4M3_ROWWISE, MOE_MXFP4_E2M1) else None
    _check(lib.moe_fused_forward_ex(dummy, dummy, None, dummy, dummy, s1, s1, dtype, M, K, N, E,
                                    topk, regime, dummy, None, ctypes.byref(nbytes), None),
           "workspace query")
    return int(nbytes.value)


def moe_fused_forward(x: torch.Tensor, w_router: torch.Tensor,
                      router_bias: Optional[torch.Tensor], w1: torch.Tensor, w2: torch.Tensor,
                      topk: int, *, w1_scale: Optional[torch.Tensor] = None,
                      w2_scale: Optional[torch.Tensor] = None, regime: int = MOE_REGIME_AUTO,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer; returns out bf16 [M,K].

    w1 [E,2N,K] / w2 [E,K,N] are bf16, or uint8 e4m3 codes with fp32 scales:
    per expert (w1_scale, w2_scale [E]) or per output row (w1_scale [E,2N],
    w2_scale [E,K]), or MXFP4: packed e2m1 w1 [E,2N,K/2] / w2 [E,K,N/2] with
    uint8 E8M0 block scales w1_scale [E,2N,K/32] / w2_scale [E,K,N/32].
    ``workspace`` (uint8, at least workspace_size bytes) may be passed to
    avoid an allocation per call."""
    lib = load_library()
    dtype, M, K, N, E = _fused_args(x, w_router, router_bias, w1, w2, w1_scale, w2_scale)
    dev = x.device
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    _dev(out, "out", torch.bfloat16, (M, K))
    need = workspace_size(dtype, M, K, N, E, topk, regime)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8)
    nbytes = ctypes.c_size_t(workspace.numel())
    _check(lib.moe_fused_forward_ex(_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w1),
                                    _ptr(w2), _ptr(w1_scale), _ptr(w2_scale), dtype, M, K, N, E,
                                    topk, regime, _ptr(out), _ptr(workspace),
                                    ctypes.byref(nbytes), _stream(dev)),
           "moe_fused_forward")
    return out


def _fused_args(x, w_router, router_bias, w1, w2, w1_scale, w2_scale):
    """Checks the layer's tensors; returns (dtype, M, K, N, E)."""
    fp8 = w1.dtype == torch.uint8
    dtype = _weight_dtype(w1, w1_scale)
    M, K = x.shape
    E, twoN, _ = w1.shape
    N = twoN // 2
    _dev(x, "x", torch.bfloat16)
    _dev(w_router, "w_router", torch.bfloat16, (E, K))
    if router_bias is not None:
        _dev(router_bias, "router_bias", torch.float32, (E,))
    wdt = torch.uint8 if fp8 else torch.bfloat16
    if dtype == MOE_MXFP4_E2M1:
        _dev(w1, "w1", wdt, (E, 2 * N, K // 2))
        _dev(w2, "w2", wdt, (E, K, N // 2))
        _dev(w1_scale, "w1_scale", torch.uint8, (E, 2 * N, K // 32))
        _dev(w2_scale, "w2_scale", torch.uint8, (E, K, N // 32))
    else:
        _dev(w1, "w1", wdt, (E, 2 * N, K))
        _dev(w2, "w2", wdt, (E, K, N))
        if dtype == MOE_FP8_E4M3_ROWWISE:
            _dev(w1_scale, "w1_scale", torch.float32, (E, 2 * N))
            _dev(w2_scale, "w2_scale", torch.float32, (E, K))
        elif fp8:
            _dev(w1_scale, "w1_scale", torch.float32, (E,))
            _dev(w2_scale, "w2_scale", torch.float32, (E,))
        elif w1_scale is not None or w2_scale is not None:
            raise ValueError("scales are only for e4m3 / MXFP4 weights")
    return dtype, M, K, N, E


def moe_fused_forward_noalloc(x: torch.Tensor, w_router: torch.Tensor,
                              router_bias: Optional[torch.Tensor], w1: torch.Tensor,
                              w2: torch.Tensor, topk: int, *,
                              w1_scale: Optional[torch.Tensor] = None,
                              w2_scale: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer through moe_fused_forward_noalloc: the library's static
    per-device scratch instead of a workspace (shapes whose plan needs more
    than NOALLOC_SCRATCH_BYTES raise MoEError with MOE_ERR_WORKSPACE).
    Only ``out`` may be allocated here, when not given."""
    lib = load_library()
    dtype = _weight_dtype(w1, w1_scale)
    M, K = x.shape
    E, twoN, _ = w1.shape
    N = twoN // 2
    _dev(x, "x", torch.bfloat16)
    _dev(w_router, "w_router", torch.bfloat16, (E, K))
    _dev(w1, "w1")
    _dev(w2, "w2")
    for t, name in ((router_bias, "router_bias"), (w1_scale, "w1_scale"), (w2_scale, "w2_scale")):
        if t is not None:
            _dev(t, name)
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16, (M, K))
    _check(lib.moe_fused_forward_noalloc(_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w1),
                                         _ptr(w2), _ptr(w1_scale), _ptr(w2_scale), dtype, M, K,
                                         N, E, topk, _ptr(out), _stream(x.device)),
           "moe_fused_forward_noalloc")
    return out


class FusedForwardGraph:
    """One moe_fused_forward captured in a HIP graph by the library
    (moe_fused_graph_create), for serving loops that re-run the layer on
    fixed buffers: ``replay()`` is one moe_fused_graph_launch on the current
    stream.

    The graph is bound to the tensors given here (this object keeps them
    alive): a replay recomputes ``out`` from whatever ``x`` (and the weights)
    hold at that moment.  ``out`` and the workspace are owned by this
    object.  Creating it runs the layer once eagerly on the current stream."""

    def __init__(self, x: torch.Tensor, w_router: torch.Tensor,
                 router_bias: Optional[torch.Tensor], w1: torch.Tensor, w2: torch.Tensor,
                 topk: int, *, w1_scale: Optional[torch.Tensor] = None,
                 w2_scale: Optional[torch.Tensor] = None, regime: int = MOE_REGIME_AUTO):
        lib = load_library()
        self._handle = None
        dtype, M, K, N, E = _fused_args(x, w_router, router_bias, w1, w2, w1_scale, w2_scale)
        self.device = x.device
        need = workspace_size(dtype, M, K, N, E, topk, regime)
        self.out = torch.empty((M, K), dtype=torch.bfloat16, device=self.device)
        self.workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        self._inputs = (x, w_router, router_bias, w1, w2, w1_scale, w2_scale)
        handle = ctypes.c_void_p()
        _check(lib.moe_fused_graph_create(_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w1),
                                          _ptr(w2), _ptr(w1_scale), _ptr(w2_scale), dtype, M, K,
                                          N, E, topk, regime, _ptr(self.out),
                                          _ptr(self.workspace), self.workspace.numel(),
                                          _stream(self.device), ctypes.byref(handle)),
               "moe_fused_graph_create")
        self._handle = handle

    def replay(self) -> torch.Tensor:
        _check(load_library().moe_fused_graph_launch(self._handle, _stream(self.device)),
               "moe_fused_graph_launch")
        return self.out

    def close(self) -> None:
        """Releases the graph (after the work already enqueued has run)."""
        if self._handle is not None:
            torch.cuda.synchronize(self.device)
            _check(load_library().moe_fused_graph_destroy(self._handle),
                   "moe_fused_graph_destroy")
            self._handle = None

    def __del__(self):
        if getattr(self, "_handle", None) is not None and _lib is not None:
            try:
                self.close()
            except Exception:
                pass
