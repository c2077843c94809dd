"""The allocation-free entry point (moe_fused_forward_noalloc, static
per-device scratch) against moe_fused_forward (caller workspace), through
the C ABI: two calls in a row on each shape, the second with fewer tokens,
must give bitwise the same outputs as the workspace entry point (the same
kernels and plan), and one case is also checked against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_layer_04_amd import workloads as wlm
from tests._brute import row_rel_err

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moe():
    import moe_layer_04_amd as m
    m.load_library()
    return m


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


CASES = [
    # workload, smaller token count of the second call, generate on
    (wlm.WORKLOADS["tiny"], 5, "cpu"),                 # full tiles, then Swap-AB decode
    (wlm.WORKLOADS["single_token_decode"], 1, "cuda"),
    (wlm.WORKLOADS["mixtral_decode"], 3, "cuda"),
    (wlm.WORKLOADS["dsv3_fp8"], 16, "cuda"),           # e4m3, 77 MiB of scratch
    (wlm.Workload("fp8_rowwise_small", M=40, K=512, N=256, E=16, topk=4, fp8=True,
                  fp8_rowwise=True, seed=6), 7, "cpu"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_noalloc_matches_workspace_entry(moe, case):
    wl, m2, where = case
    note(f"noalloc {wl.name}: M={wl.M} then M={m2}")
    g = wlm.generate(wl, where)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in g.items()}
    for M in (wl.M, m2):
        x = g["x"][:M].contiguous()
        args = (x, g["w_router"], g["bias"], g["w1"], g["w2"], wl.topk)
        kw = dict(w1_scale=g["w1_scale"], w2_scale=g["w2_scale"])
        got = moe.moe_fused_forward_noalloc(*args, **kw)
        ref = moe.moe_fused_forward(*args, **kw)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert same_bits(got, ref), (wl.name, M)
    del g
    torch.cuda.empty_cache()


def test_noalloc_vs_oracle(moe):
    wl = wlm.Workload("noalloc_oracle", M=24, K=512, N=384, E=8, topk=2, bias_var=0.5, seed=9)
    note("noalloc vs oracle")
    d = wlm.generate(wl, "cpu")
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    got = moe.moe_fused_forward_noalloc(g["x"], g["w_router"], g["bias"], g["w1"], g["w2"],
                                        wl.topk).float().cpu().numpy().astype(np.float64)
    bits = wlm.to_numpy_bits
    ref, _, _ = oracle.moe_forward(bits(d["x"]), bits(d["w_router"]), d["bias"].numpy(),
                                   bits(d["w1"]), bits(d["w2"]), wl.topk)
    err = row_rel_err(got, ref)
    note(f"  err={err:.3e}")
    assert err <= 2e-2
