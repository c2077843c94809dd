"""The fused layer captured in a HIP graph by the library
(moe_fused_graph_create, through FusedForwardGraph).

A captured launch sequence must give, on every replay, exactly what an eager
call on the same inputs gives (the kernels are deterministic), and stay
within tolerance of the oracle.  Each case replays several times with new
inputs copied into the captured tensors and with the program's own eager
work and synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

from moe_layer_04_amd import workloads as wlm
from tests._brute import row_rel_err
from tests.test_gpu_parity import (TOL_BF16, TOL_FP8, gen_small, note, oracle_layer,
                                   out_f64)

pytestmark = pytest.mark.gpu

CASES = [
    # name, M, K, N, E, k, weights ("bf16" / "fp8" / "mxfp4"), regime
    ("decode_bf16", 8, 512, 768, 8, 2, "bf16", 0),
    ("decode_fp8", 6, 512, 384, 16, 4, "fp8", 0),
    ("full_tiles_bf16", 96, 512, 512, 6, 2, "bf16", 2),
    ("decode_mxfp4", 8, 512, 512, 8, 2, "mxfp4", 0),
    ("fp8_32_row_blocks", 48, 512, 256, 8, 2, "fp8", 0),
    ("full_tiles_fp8", 96, 512, 512, 6, 2, "fp8", 2),
    ("full_tiles_mxfp4", 300, 512, 512, 8, 2, "mxfp4", 0),
    # more than 2048 token-slots: the multi-workgroup align in the graph
    ("multi_align_tiles", 1100, 256, 256, 8, 2, "bf16", 0),
    ("multi_align_tiles_fp8", 1100, 256, 256, 8, 2, "fp8", 0),
    # one token: routing inside GEMM1 (bf16) and the single-wave top-k +
    # align (e4m3)
    ("single_token", 1, 512, 512, 16, 2, "bf16", 0),
    # two tokens, bf16: routing inside GEMM1, GEMM2 + combine
    ("two_tokens_fused", 2, 1024, 512, 8, 2, "bf16", 0),
    ("single_token_fp8", 1, 512, 512, 8, 2, "fp8", 0),
]


@pytest.fixture(scope="module")
def moe():
    import moe_layer_04_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(moe, case):
    name, M, K, N, E, k, weights, regime = case
    note(f"graph {case}")
    fp8, mx = weights == "fp8", weights == "mxfp4"
    wl = wlm.Workload(name, M=M, K=K, N=N, E=E, topk=k, fp8=fp8, mxfp4=mx, seed=21)
    d, g = gen_small(wl)
    x = g["x"].clone()
    graph = moe.FusedForwardGraph(x, g["w_router"], g["bias"], g["w1"], g["w2"], k,
                                  w1_scale=g["w1_scale"], w2_scale=g["w2_scale"],
                                  regime=regime)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(5)
    for rep in range(4):
        # a new batch in the captured input tensor
        xb = torch.randn((M, K), generator=gen).to(torch.bfloat16)
        x.copy_(xb.cuda())
        got = graph.replay().clone()
        torch.cuda.synchronize()
        # eager work between replays: the same layer on the same inputs
        ref = moe.moe_fused_forward(x, g["w_router"], g["bias"], g["w1"], g["w2"], k,
                                    w1_scale=g["w1_scale"], w2_scale=g["w2_scale"],
                                    regime=regime)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        if rep in (0, 3):
            dd = dict(d)
            dd["x"] = xb
            want, _, _ = oracle_layer(dd, wl)
            err = row_rel_err(out_f64(got), want)
            note(f"  replay {rep} err={err:.3e}")
            assert np.isfinite(out_f64(got)).all()
            assert err <= (TOL_FP8 if (fp8 or mx) else TOL_BF16)
