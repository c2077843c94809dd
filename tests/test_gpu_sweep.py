"""A seeded sweep of random layer shapes through the fused layer.

Each case draws M, K, N, E, top-k, the weight format (bf16, e4m3 per tensor
or per channel, MXFP4), an optional router bias and a kernel family
(automatic, or one forced) from a fixed generator, so the list is the same
on every run; bf16 cases of one or two tokens take K and N from multiples
of 512, so the automatic ones with few router pairs run the two-launch
decode.  Every case checks the layer's own routing bit for bit
against the oracle (logits, top-k ids, sorted permutation, block owners,
offsets, padded count; weights within 1e-6) and every token's output within
the format's tolerance, on a workspace poisoned with 0xFF.
"""
import numpy as np
import pytest

from moe_layer_04_amd import workloads as wlm
from tests._brute import row_rel_err
from tests.test_gpu_parity import (TOL_BF16, TOL_FP8, bits, check_fused_routing, gen_small,
                                   note, oracle_layer, out_f64, run_layer)

pytestmark = pytest.mark.gpu

N_CASES = 96


@pytest.fixture(scope="module")
def moe():
    import moe_layer_04_amd as m
    m.load_library()
    return m


def _cases():
    rng = np.random.default_rng(20261203)
    kinds = ["bf16", "fp8", "rowwise", "mxfp4"]
    experts = [1, 2, 3, 4, 5, 8, 12, 16, 32, 64, 128, 256]
    cases = []
    while len(cases) < N_CASES:
        kind = kinds[len(cases) % 4]
        dims = [256, 512, 768, 1024] if kind == "mxfp4" else [128, 256, 384, 512, 640, 1024]
        K, N = (int(v) for v in rng.choice(dims, 2))
        E = int(rng.choice(experts))
        k = int(min(E, rng.choice([1, 2, 2, 2, 4, 6, 8, 16])))
        band = rng.integers(4)
        M = int([rng.integers(1, 5), rng.integers(5, 65), rng.integers(65, 401),
                 rng.integers(401, 1300)][band])
        if kind == "bf16" and M <= 2:
            # shapes the two-launch decode of one or two tokens takes
            K, N = (int(v) for v in rng.choice([512, 1024, 1536, 2048], 2))
        regime = int(rng.choice([0, 0, 0, 1, 2]))
        bias = 0.5 if rng.random() < 0.4 else None
        # CPU cost of drawing the weights and of the oracle on every token
        if E * 3 * K * N > 48e6 or M * k * 3 * K * N > 3e9:
            continue
        cases.append((f"{len(cases):02d}_{kind}_M{M}_K{K}_N{N}_E{E}_k{k}_r{regime}", M, K, N, E,
                      k, kind, bias, regime, int(rng.integers(1 << 30))))
    return cases


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sweep(moe, case):
    name, M, K, N, E, k, kind, bias, regime, seed = case
    note(f"sweep {case}")
    wl = wlm.Workload(name, M=M, K=K, N=N, E=E, topk=k, fp8=kind in ("fp8", "rowwise"),
                      fp8_rowwise=kind == "rowwise", mxfp4=kind == "mxfp4", bias_var=bias,
                      seed=seed)
    d, g = gen_small(wl)
    out, ws = run_layer(moe, g, wl, regime, keep_ws=True)
    check_fused_routing(moe, ws, wl, regime, bits(d["x"]), bits(d["w_router"]),
                        None if d["bias"] is None else d["bias"].numpy())
    got = out_f64(out)
    assert np.isfinite(got).all()
    ref, _, _ = oracle_layer(d, wl)
    err = row_rel_err(got, ref)
    note(f"  err={err:.3e}")
    assert err <= (TOL_BF16 if kind == "bf16" else TOL_FP8)
