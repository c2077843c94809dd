"""The C ABI on a host without a GPU: the library loads, exports every entry
point include/moe.h declares, and rejects bad arguments with the documented
status before making any HIP call (so no device is touched here)."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library links against)

import moe_layer_04_amd as moe
from moe_layer_04_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced on error paths
MISALIGNED = ctypes.c_void_p(0x10004)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char \*)\s*(moe_\w+)\s*\(", text,
                                 re.M)))


@pytest.fixture(scope="module")
def lib():
    return moe.load_library(build_if_missing=True)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"moe_topk", "moe_align", "moe_fused_forward"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTS)


def test_status_strings(lib):
    assert moe.status_string(0) == "MOE_OK"
    assert moe.status_string(3) == "MOE_ERR_WORKSPACE"
    assert moe.status_string(99) == "MOE_ERR_UNKNOWN"


def topk_call(lib, x=FAKE, wr=FAKE, bias=None, M=4, K=64, E=8, k=2, ids=FAKE, w=FAKE, lg=FAKE):
    return lib.moe_topk(x, wr, bias, M, K, E, k, ids, w, lg, None)


def test_topk_validation(lib):
    assert topk_call(lib, M=-1) == B.MOE_ERR_INVALID_ARG
    assert topk_call(lib, K=0) == B.MOE_ERR_INVALID_ARG
    assert topk_call(lib, k=0) == B.MOE_ERR_INVALID_ARG
    assert topk_call(lib, k=9) == B.MOE_ERR_INVALID_ARG          # topk > E
    assert topk_call(lib, E=300, k=2) == B.MOE_ERR_UNSUPPORTED
    assert topk_call(lib, E=32, k=17) == B.MOE_ERR_UNSUPPORTED
    assert topk_call(lib, x=None) == B.MOE_ERR_INVALID_ARG
    assert topk_call(lib, lg=None) == B.MOE_ERR_INVALID_ARG
    assert topk_call(lib, wr=MISALIGNED) == B.MOE_ERR_INVALID_ARG
    assert topk_call(lib, M=0, x=None, ids=None, w=None, lg=None) == B.MOE_OK   # no-op


def test_align_ex_validation(lib):
    f = lib.moe_align_ex
    n = ctypes.c_size_t(0)
    # size queries make no HIP call: a minimal 256 bytes up to 2048 slots
    # (never 0, so a buffer sized from the query is not NULL), chunk counts above
    assert f(None, 1024, 2, 8, 16, None, None, None, None, None, ctypes.byref(n), None) == 0
    assert n.value == 256
    assert f(None, 4096, 2, 256, 16, None, None, None, None, None, ctypes.byref(n), None) == 0
    assert n.value >= (8 * 256 + 256) * 4
    need = n.value
    assert f(FAKE, 4096, 2, 256, 16, FAKE, FAKE, FAKE, FAKE, None, None, None) == \
        B.MOE_ERR_INVALID_ARG                                          # null size pointer
    small = ctypes.c_size_t(need - 1)
    assert f(FAKE, 4096, 2, 256, 16, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(small),
             None) == B.MOE_ERR_WORKSPACE
    big = ctypes.c_size_t(need)
    assert f(FAKE, 4096, 2, 256, 16, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10010),
             ctypes.byref(big), None) == B.MOE_ERR_INVALID_ARG       # workspace not aligned
    assert f(FAKE, 4, 2, 257, 16, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(big), None) == \
        B.MOE_ERR_UNSUPPORTED
    assert f(FAKE, -1, 2, 8, 16, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(big), None) == \
        B.MOE_ERR_INVALID_ARG


def test_align_validation(lib):
    f = lib.moe_align
    assert f(FAKE, -1, 2, 8, 16, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 0, 8, 16, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 2, 8, 0, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 2, 257, 16, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert f(FAKE, 4, 2, 8, 2048, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert f(None, 4, 2, 8, 16, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 2, 8, 16, None, FAKE, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 2, 8, 16, MISALIGNED, FAKE, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG


def fused(lib, *, x=FAKE, wr=FAKE, bias=None, w1=FAKE, w2=FAKE, s1=None, s2=None, dtype=0,
          M=8, K=256, N=512, E=8, k=2, regime=0, out=FAKE, ws=FAKE, nbytes=None):
    n = ctypes.c_size_t(1 << 40 if nbytes is None else nbytes)
    rc = lib.moe_fused_forward_ex(x, wr, bias, w1, w2, s1, s2, dtype, M, K, N, E, k, regime, out,
                                  ws, ctypes.byref(n), None)
    return rc, n.value


def test_fused_validation(lib):
    INV, UNS, WSP = B.MOE_ERR_INVALID_ARG, B.MOE_ERR_UNSUPPORTED, B.MOE_ERR_WORKSPACE
    assert fused(lib, dtype=4)[0] == INV
    assert fused(lib, dtype=3)[0] == INV                              # MXFP4 without scales
    # MXFP4 full tiles (size query only)
    assert fused(lib, dtype=3, s1=FAKE, s2=FAKE, regime=2, ws=None)[0] == B.MOE_OK
    assert fused(lib, dtype=3, s1=FAKE, s2=FAKE, N=384)[0] == UNS       # MXFP4: multiples of 256
    assert fused(lib, dtype=3, s1=FAKE, s2=FAKE, K=16640)[0] == UNS     # MXFP4: K <= 16384
    # MXFP4: GEMM2 splits must hold <= 8192 reduction elements; 8448 = 33*256
    # cannot be halved into multiples of 256
    assert fused(lib, dtype=3, s1=FAKE, s2=FAKE, N=8448)[0] == UNS
    assert fused(lib, dtype=3, s1=FAKE, s2=FAKE, N=8192, ws=None)[0] == 0  # size query succeeds
    # the full tiles copy their scales per step: no such limit there
    assert fused(lib, dtype=3, s1=FAKE, s2=FAKE, N=8448, regime=2, ws=None)[0] == 0
    assert fused(lib, dtype=2)[0] == INV                              # rowwise fp8 without scales
    assert fused(lib, dtype=2, s1=FAKE, s2=None)[0] == INV
    # e4m3 weights have full-tile kernels too (size query only: no launch here)
    assert fused(lib, dtype=2, s1=FAKE, s2=FAKE, regime=2, ws=None)[0] == B.MOE_OK
    assert fused(lib, regime=3)[0] == INV
    assert fused(lib, M=-1)[0] == INV
    assert fused(lib, N=0)[0] == INV
    assert fused(lib, k=9)[0] == INV
    assert fused(lib, s1=FAKE, s2=FAKE)[0] == INV                     # scales with bf16
    assert fused(lib, dtype=1)[0] == INV                              # fp8 without scales
    assert fused(lib, dtype=1, s1=FAKE, s2=None)[0] == INV
    assert fused(lib, E=257, k=2)[0] == UNS
    assert fused(lib, E=64, k=17)[0] == UNS
    assert fused(lib, K=200)[0] == UNS                               # not a multiple of 128
    assert fused(lib, N=192)[0] == UNS
    assert fused(lib, dtype=1, s1=FAKE, s2=FAKE, regime=2, ws=None)[0] == B.MOE_OK
    # 32-bit offsets of the sorted activation rows GEMM2 reads: 2 bytes each
    # for bf16, 1 for the e4m3 codes
    assert fused(lib, M=65536, K=4096, N=14336, E=8, k=2, ws=None)[0] == UNS
    assert fused(lib, dtype=1, s1=FAKE, s2=FAKE, M=65536, K=4096, N=14336, E=8, k=2,
                 ws=None)[0] == B.MOE_OK
    assert fused(lib, dtype=1, s1=FAKE, s2=FAKE, M=4096, K=7168, N=2048, E=256, k=8,
                 ws=None)[0] == B.MOE_OK
    assert fused(lib, x=None)[0] == INV
    assert fused(lib, out=None)[0] == INV
    assert fused(lib, w2=MISALIGNED)[0] == INV
    assert fused(lib, ws=ctypes.c_void_p(0x10010))[0] == INV          # workspace not 256-aligned
    rc, need = fused(lib, ws=None)
    assert rc == B.MOE_OK and need > 0
    assert fused(lib, nbytes=need - 1)[0] == WSP
    assert lib.moe_fused_forward_ex(FAKE, FAKE, None, FAKE, FAKE, None, None, 0, 8, 256, 512, 8,
                                    2, 0, FAKE, FAKE, None, None) == INV  # null size pointer
    rc, _ = fused(lib, M=0, x=None, out=None)
    assert rc == B.MOE_OK                                             # M == 0: no-op


def test_workspace_query_sizes(lib):
    # the query makes no HIP call; sizes grow with M and follow the dtype
    s_dec = moe.workspace_size(moe.MOE_BF16, 8, 4096, 14336, 8, 2)
    s_pre = moe.workspace_size(moe.MOE_BF16, 4096, 4096, 14336, 8, 2)
    s_fp8 = moe.workspace_size(moe.MOE_FP8_E4M3, 128, 7168, 2048, 256, 8)
    assert 0 < s_dec < s_pre
    # prefill: the bf16 SiLU*up activation [M*k + E*255, N] dominates
    assert s_pre >= (4096 * 2 + 8 * 255) * 14336 * 2
    # fp8: fp32 + e4m3 activations of [M*k + E*15, N]
    assert s_fp8 >= (128 * 8 + 256 * 15) * 2048 * 5
    assert moe.workspace_size(moe.MOE_BF16, 8, 4096, 14336, 8, 2, moe.MOE_REGIME_PREFILL) > s_dec
    # per-channel scales change no workspace region
    assert moe.workspace_size(moe.MOE_FP8_E4M3_ROWWISE, 128, 7168, 2048, 256, 8) == s_fp8
    assert moe.workspace_size(moe.MOE_MXFP4_E2M1, 128, 7168, 2048, 256, 8) == s_fp8
    # e4m3 full tiles: 256-row blocks at 1024 rows per expert, 128-row blocks
    # at 128 (the fp32 + e4m3 activations of [M*k + E*(B-1), N] dominate)
    s_pre8 = moe.workspace_size(moe.MOE_FP8_E4M3, 4096, 4096, 14336, 8, 2)
    assert s_pre8 >= (8192 + 8 * 255) * 14336 * 5
    # (plus the fp32 partial rows [M*k, K], unsplit there)
    ypart = 32768 * 7168 * 4
    s_ds = moe.workspace_size(moe.MOE_FP8_E4M3, 4096, 7168, 2048, 256, 8)
    assert (32768 + 256 * 127) * 2048 * 5 + ypart <= s_ds
    assert s_ds < (32768 + 256 * 255) * 2048 * 5 + ypart
    # forcing the decode kernels there sizes 64-row blocks
    s_dsd = moe.workspace_size(moe.MOE_FP8_E4M3, 4096, 7168, 2048, 256, 8,
                               moe.MOE_REGIME_DECODE)
    assert (32768 + 256 * 63) * 2048 * 5 + ypart <= s_dsd < s_ds


def test_fused_plan(lib):
    """The plan query (no HIP call): kernel family per workload, block sizes,
    and routing regions that lie inside the workspace without overlapping."""
    P = B.Plan
    assert lib.moe_fused_plan(0, 8, 256, 512, 8, 2, 0, None) == B.MOE_ERR_INVALID_ARG
    p = P()
    assert lib.moe_fused_plan(0, 8, 200, 512, 8, 2, 0, ctypes.byref(p)) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_fused_plan(5, 8, 256, 512, 8, 2, 0, ctypes.byref(p)) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_fused_plan(3, 8, 256, 384, 8, 2, 2, ctypes.byref(p)) == B.MOE_ERR_UNSUPPORTED
    cases = {  # (dtype, M, K, N, E, k): regime, block
        (0, 64, 256, 512, 8, 2): (2, 128),      # 16 rows per expert: full tiles
        (0, 8, 4096, 14336, 8, 2): (1, 16),
        (0, 1, 4096, 8192, 16, 2): (1, 16),
        (0, 4096, 4096, 14336, 8, 2): (2, 256),
        (1, 128, 7168, 2048, 256, 8): (1, 16),
        (1, 4096, 7168, 2048, 256, 8): (2, 128),
        # MXFP4: the decode kernels up to 24 rows per expert, then the full
        # tiles, always with 256-row blocks
        (3, 128, 7168, 2048, 256, 8): (1, 16),
        (3, 8, 4096, 14336, 8, 2): (1, 16),
        (3, 4096, 7168, 2048, 256, 8): (2, 256),
        (3, 96, 4096, 14336, 8, 2): (1, 64),       # 24 rows per expert
        (3, 100, 4096, 14336, 8, 2): (2, 256),
        (3, 4096, 4096, 14336, 8, 2): (2, 256),
    }
    for (dt, M, K, N, E, k), (regime, block) in cases.items():
        p = moe.fused_plan(dt, M, K, N, E, k)
        assert p.regime == regime, (dt, M)
        if block is not None:
            assert p.block_m == block, (dt, M, p.block_m)
        assert p.sorted_rows == M * k + E * (p.block_m - 1)
        assert p.max_blocks == p.sorted_rows // p.block_m
        assert p.workspace_bytes == moe.workspace_size(dt, M, K, N, E, k)
        regions = sorted([(p.logits_offset, M * E * 4), (p.topk_ids_offset, M * k * 4),
                          (p.topk_weights_offset, M * k * 4),
                          (p.sorted_ids_offset, p.sorted_rows * 4),
                          (p.block_expert_offset, p.max_blocks * 4),
                          (p.expert_offsets_offset, (E + 1) * 4),
                          (p.num_padded_offset, 4)])
        for (a, na), (b, _) in zip(regions, regions[1:]):
            assert a % 256 == 0 and a + na <= b
        assert regions[-1][0] + regions[-1][1] <= p.workspace_bytes
        assert p.reserved == 0
        assert p.fused_decode == (1 if (dt, M) == (0, 1) else 0)
        if p.fused_decode:
            assert p.gemm2_splits == 1
    # a forced family is reported as such
    assert moe.fused_plan(0, 4096, 4096, 14336, 8, 2, moe.MOE_REGIME_DECODE).regime == 1
    assert moe.fused_plan(0, 8, 4096, 14336, 8, 2, moe.MOE_REGIME_PREFILL).regime == 2


def test_noalloc_validation(lib):
    """moe_fused_forward_noalloc rejects bad arguments and shapes whose plan
    needs more than its static scratch before any HIP call."""
    f = lib.moe_fused_forward_noalloc

    def call(x=FAKE, wr=FAKE, w1=FAKE, w2=FAKE, s1=None, s2=None, dtype=0, M=8, K=256, N=512,
             E=8, k=2, out=FAKE):
        return f(x, wr, None, w1, w2, s1, s2, dtype, M, K, N, E, k, out, None)

    assert call(M=-1) == B.MOE_ERR_INVALID_ARG
    assert call(K=200) == B.MOE_ERR_UNSUPPORTED
    assert call(dtype=1) == B.MOE_ERR_INVALID_ARG                   # e4m3 without scales
    assert call(x=None) == B.MOE_ERR_INVALID_ARG
    assert call(out=MISALIGNED) == B.MOE_ERR_INVALID_ARG
    assert call(M=0, x=None, out=None) == B.MOE_OK                  # no-op
    # the Mixtral-shaped prefill batch needs ~536 MiB of scratch: rejected
    p = moe.fused_plan(0, 4096, 4096, 14336, 8, 2)
    assert p.workspace_bytes > B.NOALLOC_SCRATCH_BYTES
    assert call(M=4096, K=4096, N=14336, E=8, k=2) == B.MOE_ERR_WORKSPACE
    # the decode batches fit
    for dt, M, K, N, E, k in ((0, 8, 4096, 14336, 8, 2), (0, 1, 4096, 8192, 16, 2)):
        assert moe.fused_plan(dt, M, K, N, E, k).workspace_bytes <= B.NOALLOC_SCRATCH_BYTES


def test_graph_validation(lib):
    """moe_fused_graph_create rejects bad arguments before any HIP call;
    launching a NULL handle is an argument error and destroying it a no-op."""
    create = lib.moe_fused_graph_create
    INV, UNS, WSP = B.MOE_ERR_INVALID_ARG, B.MOE_ERR_UNSUPPORTED, B.MOE_ERR_WORKSPACE

    def call(x=FAKE, w1=FAKE, s1=None, s2=None, dtype=0, M=8, K=256, N=512, E=8, k=2,
             regime=0, out=FAKE, ws=FAKE, nbytes=1 << 40, handle=True):
        h = ctypes.c_void_p(0x1234)
        rc = create(x, FAKE, None, w1, FAKE, s1, s2, dtype, M, K, N, E, k, regime, out, ws,
                    nbytes, None, ctypes.byref(h) if handle else None)
        # on every error the handle comes back NULL (or was never written)
        assert rc == B.MOE_OK or not handle or h.value is None
        return rc

    assert call(handle=False) == INV
    assert call(M=-1) == INV
    assert call(K=200) == UNS
    assert call(dtype=1) == INV                       # e4m3 without scales
    assert call(regime=3) == INV
    assert call(M=0) == INV                           # nothing to capture
    assert call(ws=None) == INV
    need = moe.workspace_size(0, 8, 256, 512, 8, 2)
    assert call(nbytes=need - 1) == WSP
    assert call(x=None) == INV                        # the eager call's pointer checks
    assert call(out=MISALIGNED) == INV
    assert lib.moe_fused_graph_launch(None, None) == INV
    assert lib.moe_fused_graph_destroy(None) == B.MOE_OK
