"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer work -- top-k ids, the sorted permutation, block owners, offsets,
e4m3 codes of the token quantiser -- must match bit for bit.  Floating
outputs must match within the layer's stated tolerances, measured as the
max over tokens of max|gpu - ref| / max|ref| (row max of the fp64 oracle):
2e-2 for bf16 weights, 6e-2 for e4m3 weights.  Routing weights: 1e-6
absolute (fp32 softmax vs the oracle's fp64 on the same logits).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_layer_04_amd import workloads as wlm
from tests._brute import row_rel_err

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_FP8 = 6e-2
TOL_WEIGHTS = 1e-6


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moe():
    import moe_layer_04_amd as m
    m.load_library()
    return m


def bits(t):
    return wlm.to_numpy_bits(t)


def gen_small(wl, seed=None):
    """Small workloads are drawn on the CPU and copied to the GPU."""
    if seed is not None:
        wl = wl.resized(seed=seed)
    d = wlm.generate(wl, "cpu")
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    return d, g


def dtype_of(moe, wl):
    return (moe.MOE_MXFP4_E2M1 if wl.mxfp4 else
            moe.MOE_FP8_E4M3_ROWWISE if wl.fp8_rowwise else
            moe.MOE_FP8_E4M3 if wl.fp8 else moe.MOE_BF16)


def run_layer(moe, g, wl, regime=0, poison=True, keep_ws=False):
    need = moe.workspace_size(dtype_of(moe, wl), wl.M, wl.K, wl.N, wl.E, wl.topk, regime)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    if poison:
        ws.fill_(0xFF)   # any read of a never-written workspace byte turns into NaN
    out = torch.full((wl.M, wl.K), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_fused_forward(g["x"], g["w_router"], g["bias"], g["w1"], g["w2"], wl.topk,
                          w1_scale=g["w1_scale"], w2_scale=g["w2_scale"], regime=regime,
                          out=out, workspace=ws)
    torch.cuda.synchronize()
    return (out, ws) if keep_ws else out


def check_fused_routing(moe, ws, wl, regime, x_bits, wr_bits, bias):
    """The routing the fused layer itself computed (left in its workspace at
    the offsets moe_fused_plan reports) against the oracle: logits, top-k ids,
    the sorted permutation, block owners, offsets and padded count bit for
    bit, routing weights within 1e-6.  Returns (plan, oracle ids, oracle
    sorted ids)."""
    plan = moe.fused_plan(dtype_of(moe, wl), wl.M, wl.K, wl.N, wl.E, wl.topk, regime)
    r = {k: v.cpu().numpy() for k, v in moe.fused_routing(ws, plan, wl.M, wl.E, wl.topk).items()}
    rlg = oracle.logits(x_bits, wr_bits, bias)
    assert np.array_equal(r["logits"], rlg), "fused logits"
    rids, rw = oracle.topk(rlg, wl.topk)
    assert np.array_equal(r["topk_ids"], rids), "fused top-k ids"
    assert np.abs(r["topk_weights"] - rw).max() <= TOL_WEIGHTS, "fused routing weights"
    rs, rb, ro, rn = oracle.align(rids, wl.E, plan.block_m)
    assert int(r["num_padded"][0]) == rn, "fused num_padded"
    assert np.array_equal(r["expert_offsets"], ro), "fused expert_offsets"
    assert np.array_equal(r["block_expert"], rb), "fused block_expert"
    assert np.array_equal(r["sorted_ids"], rs), "fused sorted_ids"
    return plan, rids, rs


def oracle_layer(d, wl, tokens=None):
    s1 = None if d["w1_scale"] is None else d["w1_scale"].numpy()
    s2 = None if d["w2_scale"] is None else d["w2_scale"].numpy()
    return oracle.moe_forward(bits(d["x"]), bits(d["w_router"]),
                              None if d["bias"] is None else d["bias"].numpy(),
                              bits(d["w1"]), bits(d["w2"]), wl.topk, w1_scale=s1, w2_scale=s2,
                              tokens=tokens, fp8=wl.fp8, mxfp4=wl.mxfp4)


def out_f64(out):
    return out.float().cpu().numpy().astype(np.float64)


# --------------------------------------------------------------------------
# token quantiser: bit-exact codes and scales
# --------------------------------------------------------------------------

def test_quant_rows_bit_exact_all_bf16_values(moe):
    note("quant_rows: every finite bf16 value")
    pat = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((pat & 0x7F80) != 0x7F80)
    vals = pat[finite]
    K = 640
    M = (vals.size + K - 1) // K
    xb = np.zeros(M * K, np.uint16)
    xb[: vals.size] = vals
    xb = xb.reshape(M, K)
    rng = np.random.default_rng(0)
    rng.shuffle(xb, axis=1)
    xb = np.concatenate([xb, np.zeros((1, K), np.uint16)])   # an all-zero row -> scale 1
    # rows with very different ranges: scale one row's magnitudes down
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    q, s = moe.moe_quant_rows_e4m3(x)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_rows_bf16(xb)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("M,K", [(1, 1), (3, 7), (5, 4096), (2, 7168 + 3), (4, 7168),
                                 (3, 8192), (2, 8192 + 2048 + 8)])
def test_quant_rows_ragged(moe, M, K):
    note(f"quant_rows M={M} K={K}")
    g = torch.Generator().manual_seed(M * 31 + K)
    x = (torch.randn((M, K), generator=g) * 3).to(torch.bfloat16)
    q, s = moe.moe_quant_rows_e4m3(x.cuda())
    torch.cuda.synchronize()
    rq, rs = oracle.quant_rows_bf16(bits(x))
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(q.cpu().numpy(), rq)


# --------------------------------------------------------------------------
# router: bit-exact logits, ids; weights within 1e-6
# --------------------------------------------------------------------------

def check_router(moe, x, wr, bias, k):
    ids, w, lg = moe.moe_topk(x.cuda(), wr.cuda(), None if bias is None else bias.cuda(), k)
    torch.cuda.synchronize()
    ids, w, lg = ids.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()
    rlg = oracle.logits(bits(x), bits(wr), None if bias is None else bias.numpy())
    # selection on the GPU's own logits must be the oracle's selection
    sids, sw = oracle.topk(lg, k)
    assert np.array_equal(ids, sids)
    assert np.abs(w - sw).max() <= TOL_WEIGHTS
    # and the logits themselves are the oracle's (fp64 dot product, one rounding)
    assert np.array_equal(lg, rlg)
    rids, _ = oracle.topk(rlg, k)
    assert np.array_equal(ids, rids)
    return ids


@pytest.mark.parametrize("name", list(wlm.WORKLOADS))
def test_router_full_size(moe, name):
    wl = wlm.WORKLOADS[name]
    note(f"router {name} M={wl.M} K={wl.K} E={wl.E} k={wl.topk}")
    g = torch.Generator().manual_seed(0)
    x = torch.randn((wl.M, wl.K), generator=g).to(torch.bfloat16)
    wr = (torch.randn((wl.E, wl.K), generator=g) / math.sqrt(wl.K)).to(torch.bfloat16)
    bias = (torch.randn(wl.E, generator=g) * math.sqrt(wl.bias_var)) if wl.bias_var else None
    check_router(moe, x, wr, bias, wl.topk)


# the last three take the fp64 matrix-core logits (M*E > 8192, K % 512 == 0)
# with token and expert counts that are not multiples of its 16 x 16 tile
@pytest.mark.parametrize("M,K,E,k,with_bias", [(1, 1, 1, 1, False), (7, 100, 3, 2, False),
                                               (33, 264, 256, 16, False), (64, 96, 64, 8, False),
                                               (5, 8, 200, 200 // 13, False),
                                               (37, 1024, 250, 8, False),
                                               (45, 512, 200, 4, True),
                                               (1000, 1536, 9, 2, True)])
def test_router_ragged(moe, M, K, E, k, with_bias):
    note(f"router ragged M={M} K={K} E={E} k={k} bias={with_bias}")
    g = torch.Generator().manual_seed(M + K + E)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16)
    wr = (torch.randn((E, K), generator=g)).to(torch.bfloat16)
    bias = torch.randn(E, generator=g) if with_bias else None
    check_router(moe, x, wr, bias, k)


def test_router_ties_lower_id(moe):
    note("router ties")
    g = torch.Generator().manual_seed(5)
    M, K, E = 40, 128, 12
    x = torch.randn((M, K), generator=g).to(torch.bfloat16)
    wr = torch.randn((E, K), generator=g).to(torch.bfloat16)
    wr[7] = wr[2]
    wr[9] = wr[2]
    wr[11] = wr[4]
    ids = check_router(moe, x, wr, None, 4)
    x0 = torch.zeros((3, K), dtype=torch.bfloat16)   # all logits equal -> experts 0..3
    ids0 = check_router(moe, x0, wr, None, 4)
    assert ids0.tolist() == [[0, 1, 2, 3]] * 3


# --------------------------------------------------------------------------
# align: bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,k,E,B", [(64, 2, 8, 16), (8, 2, 8, 16), (1, 2, 16, 16),
                                     (4096, 2, 8, 128), (128, 8, 256, 16), (0, 2, 8, 16),
                                     (37, 3, 17, 64), (20000, 4, 64, 128), (300, 1, 256, 1),
                                     (9, 5, 5, 1024), (1024, 2, 8, 256), (683, 3, 16, 256),
                                     (4096, 8, 256, 128), (2500, 1, 3, 1)])
def test_align_bit_exact(moe, M, k, E, B):
    note(f"align M={M} k={k} E={E} B={B}")
    rng = np.random.default_rng(M * 7 + E)
    if M:
        # skewed expert popularity, distinct experts per token
        pop = rng.dirichlet(np.full(E, 0.3))
        ids = np.stack([rng.choice(E, size=k, replace=False, p=pop) for _ in range(M)])
    else:
        ids = np.zeros((0, k))
    ids = ids.astype(np.int32)
    rs, rb, ro, rn = oracle.align(ids, E, B)
    # one workgroup (moe_align) and, above 2048 slots, many (moe_align_ex)
    for fn in (moe.moe_align, moe.moe_align_ex):
        s, b, o, npad = fn(torch.from_numpy(ids).cuda(), E, B)
        torch.cuda.synchronize()
        assert int(npad.item()) == rn
        assert np.array_equal(o.cpu().numpy(), ro)
        assert np.array_equal(b.cpu().numpy(), rb)
        assert np.array_equal(s.cpu().numpy(), rs)


# --------------------------------------------------------------------------
# the fused layer at small sizes (the oracle evaluates every token)
# --------------------------------------------------------------------------

SMALL = [
    # name, M, K, N, E, k, fp8, bias_var, regime
    ("tiny", 64, 256, 512, 8, 2, False, None, 0),
    ("tiny_prefill_tiles", 64, 256, 512, 8, 2, False, None, 2),
    ("decode_ragged", 5, 384, 640, 6, 2, False, None, 0),
    ("k1", 9, 256, 256, 4, 1, False, None, 0),
    ("k_eq_e", 6, 256, 384, 4, 4, False, None, 0),
    ("e1_dense", 3, 128, 256, 1, 1, False, None, 0),
    ("many_empty_experts", 3, 256, 256, 256, 8, False, None, 0),
    ("prefill_skewed", 700, 256, 384, 8, 2, False, 0.5, 0),
    ("prefill_ragged", 333, 384, 640, 5, 3, False, None, 2),
    ("fp8_tiny", 16, 512, 256, 16, 4, True, None, 0),
    ("fp8_ragged", 7, 384, 640, 32, 8, True, None, 0),
    ("fp8_many_rows", 300, 256, 384, 8, 2, True, None, 0),
    # bf16 Swap-AB kernels forced on 32-row (2 token tiles) and 64-row (4) blocks
    ("decode_two_tiles", 48, 512, 512, 8, 2, False, None, 1),
    ("decode_four_tiles", 160, 256, 384, 8, 2, False, 0.5, 1),
    # FP8 with fp64-MFMA logits (split over K) and the token rows quantised
    # by their own kernel
    ("fp8_router_mfma", 78, 1024, 256, 128, 4, True, None, 0),
    # more rows per expert: 32-row (2 token tiles) and 64-row (4) blocks (the
    # latter forced: the automatic choice takes the full tiles there)
    ("fp8_two_tiles", 48, 512, 256, 8, 2, True, None, 0),
    ("fp8_four_tiles", 160, 512, 384, 8, 2, True, 0.5, 1),
    ("fp8_rowwise_four_tiles", 200, 256, 256, 4, 2, "rowwise", None, 1),
    # e4m3 weights with per-channel scales (one per output row)
    ("fp8_rowwise_tiny", 16, 512, 256, 16, 4, "rowwise", None, 0),
    ("fp8_rowwise_ragged", 7, 384, 640, 32, 8, "rowwise", None, 0),
    ("fp8_rowwise_many_rows", 300, 256, 384, 8, 2, "rowwise", None, 0),
    # MXFP4 weights (e2m1, E8M0 per 32 elements) with e4m3 activations
    ("mxfp4_tiny", 16, 512, 256, 16, 4, "mxfp4", None, 0),
    ("mxfp4_ragged", 7, 768, 512, 32, 8, "mxfp4", None, 0),
    ("mxfp4_many_rows", 300, 256, 512, 8, 2, "mxfp4", None, 1),
    # tiny batches through the single-workgroup routing, with router bias;
    # FP8 with K > 1024 quantises the token rows in their own kernel
    ("tiny_route_bias", 8, 768, 512, 8, 2, False, 0.5, 0),
    ("tiny_route_fp8", 4, 1536, 256, 8, 2, True, 0.5, 0),
    # router logits on the fp64 matrix cores with K split over 4 workgroups
    # per 16x16 tile (finished by the top-k kernel)
    ("router_split_k", 80, 2048, 256, 128, 4, False, 0.5, 0),
    # MXFP4 with 32- and 64-row blocks
    ("mxfp4_two_tiles", 48, 512, 512, 8, 2, "mxfp4", None, 0),
    ("mxfp4_four_tiles", 160, 256, 512, 8, 2, "mxfp4", 0.5, 1),
    # many experts and a wider intermediate dimension
    ("mxfp4_wide_grid", 32, 512, 1024, 64, 4, "mxfp4", None, 0),
    ("single_token", 1, 512, 1024, 16, 2, False, None, 0),
    # e4m3 weights on the full tiles: forced, ragged (GEMM2 with 128 output
    # rows per tile as K % 256 != 0), reduction split in 2 and 4, per-channel
    # scales, and the automatic choice at many rows per expert
    ("fp8_prefill_tiles", 300, 256, 384, 8, 2, True, None, 2),
    ("fp8_prefill_ragged", 333, 384, 640, 5, 3, True, None, 2),
    ("fp8_prefill_split2", 150, 256, 256, 4, 2, True, None, 2),
    ("fp8_prefill_split4", 260, 512, 512, 4, 2, True, None, 2),
    ("fp8_rowwise_prefill", 200, 256, 256, 4, 2, "rowwise", None, 2),
    ("fp8_rowwise_prefill_ragged", 97, 384, 384, 3, 2, "rowwise", 0.5, 2),
    # per-channel scales on the 256-row (ping-pong) tiles: 160-250 rows per
    # expert, so every expert's last block is part padding
    ("fp8_rowwise_prefill_256", 333, 256, 512, 3, 2, "rowwise", 0.5, 2),
    ("fp8_prefill_auto_skewed", 700, 256, 384, 8, 2, True, 0.5, 0),
    # MXFP4 weights on the full tiles (256-row blocks): forced, ragged token
    # count and expert count, reduction split in 2 and 4, 256 experts with
    # a few rows each, top-16, and the automatic choice at many rows
    ("mxfp4_prefill_tiles", 300, 256, 512, 8, 2, "mxfp4", None, 2),
    ("mxfp4_prefill_ragged", 333, 512, 768, 5, 3, "mxfp4", None, 2),
    ("mxfp4_prefill_split2", 150, 256, 256, 4, 2, "mxfp4", None, 2),
    ("mxfp4_prefill_split4", 260, 512, 512, 4, 2, "mxfp4", 0.5, 2),
    ("mxfp4_prefill_many_experts", 300, 256, 256, 256, 8, "mxfp4", None, 2),
    ("mxfp4_topk16_tiles", 40, 256, 256, 32, 16, "mxfp4", None, 2),
    ("mxfp4_prefill_auto_skewed", 700, 256, 512, 8, 2, "mxfp4", 0.5, 0),
    # full tiles over 256 experts with a few rows each (one mostly-padding
    # block per expert, block owners and sentinels over a long sorted list)
    ("fp8_prefill_many_experts", 300, 256, 256, 256, 8, True, None, 2),
    ("prefill_many_experts", 100, 256, 256, 256, 8, False, None, 2),
    # more than 2048 token-slots: the multi-workgroup align (per-chunk counts,
    # one scan, per-chunk scatter), with decode blocks, FP8 (its amax rows
    # cleared and inverse permutation written by all workgroups) and a last
    # chunk of one slot
    ("decode_many_slots", 300, 256, 256, 256, 8, False, None, 1),
    ("fp8_decode_many_slots", 300, 256, 256, 128, 8, True, None, 1),
    ("align_multi_ragged", 683, 256, 256, 16, 3, False, None, 0),
    # the largest top-k (16), on the decode kernels and on the e4m3 full tiles
    ("topk16", 20, 256, 256, 64, 16, False, None, 0),
    ("fp8_topk16_tiles", 40, 256, 256, 32, 16, True, None, 2),
    # one or two tokens: the single-wave top-k + align, with bias, e4m3
    # (per-tensor and per-channel) and MXFP4 weights
    ("two_tokens_wave_route_bias", 2, 768, 512, 8, 2, False, 0.5, 0),
    ("one_token_wave_route_fp8", 1, 1536, 256, 8, 2, True, 0.5, 0),
    ("two_tokens_wave_route_fp8_rowwise", 2, 512, 256, 4, 3, "rowwise", None, 0),
    ("one_token_wave_route_mxfp4", 1, 512, 512, 12, 4, "mxfp4", None, 0),
    # bf16, one or two tokens, K and N multiples of 512, at most 32 router
    # pairs and 4 routed experts: the router, top-k and align inside the
    # GEMM1 launch and GEMM2 with the combine in one more; two tokens sharing
    # experts, top-1, top-k = E (every expert serves both tokens), router bias
    ("fused_decode_two_tokens_bias", 2, 1024, 512, 8, 2, False, 0.5, 0),
    ("fused_decode_top1", 1, 512, 512, 4, 1, False, None, 0),
    ("fused_decode_two_tokens_top1", 2, 512, 1024, 4, 1, False, None, 0),
    ("fused_decode_top4", 1, 512, 512, 8, 4, False, 0.5, 0),
    ("fused_decode_k_eq_e", 2, 512, 512, 4, 4, False, None, 0),
    ("fused_decode_e16", 2, 1536, 1024, 16, 2, False, None, 0),
    ("fused_decode_wide_k", 1, 4096, 512, 16, 2, False, 0.5, 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fused_small(moe, case):
    name, M, K, N, E, k, fp8, bias_var, regime = case
    note(f"fused small {case}")
    rowwise = fp8 == "rowwise"
    mx = fp8 == "mxfp4"
    fp8 = bool(fp8) and not mx
    wl = wlm.Workload(name, M=M, K=K, N=N, E=E, topk=k, fp8=fp8, fp8_rowwise=rowwise,
                      mxfp4=mx, bias_var=bias_var, seed=3)
    d, g = gen_small(wl)
    out, ws = run_layer(moe, g, wl, regime, keep_ws=True)
    plan, _, _ = check_fused_routing(moe, ws, wl, regime, bits(d["x"]), bits(d["w_router"]),
                                     None if d["bias"] is None else d["bias"].numpy())
    ref, _, _ = oracle_layer(d, wl)
    got = out_f64(out)
    assert np.isfinite(got).all()
    err = row_rel_err(got, ref)
    note(f"  routing bit-exact (family {plan.regime}, block {plan.block_m}, "
         f"logit splits {plan.logit_splits}); err={err:.3e}")
    assert err <= (TOL_FP8 if (fp8 or mx) else TOL_BF16)


@pytest.mark.parametrize("M,E,fp8", [(1, 16, False), (2, 8, False), (1, 8, True)])
def test_fused_tiny_routing_ties(moe, M, E, fp8):
    """The routing of one or two tokens (the single-wave top-k + align)
    breaks ties to the lower expert id inside the fused layer: with every
    router row equal all logits of a token tie and experts 0 and 1 must serve
    it; with some rows duplicated the oracle's tie rule decides.  A wrong
    pick routes through other experts' weights, which the output comparison
    sees."""
    note(f"fused tiny routing ties M={M} E={E} fp8={fp8}")
    # bf16 with K = N = 512: the routing GEMM1 of one or two tokens
    wl = wlm.Workload("tiny_ties", M=M, K=512, N=512, E=E, topk=2, fp8=fp8, seed=8)
    for dup in ("all", "pairs"):
        d, g = gen_small(wl)
        wr = d["w_router"].clone()
        if dup == "all":
            wr[:] = wr[0]
        else:
            wr[E - 1] = wr[1]
            wr[E - 2] = wr[0]
        d["w_router"] = wr
        g["w_router"] = wr.cuda()
        out, ws = run_layer(moe, g, wl, keep_ws=True)
        got = out_f64(out)
        check_fused_routing(moe, ws, wl, 0, bits(d["x"]), bits(wr), None)
        ref, ids, _ = oracle_layer(d, wl)
        if dup == "all":
            assert np.array_equal(np.asarray(ids).reshape(M, 2), np.tile([0, 1], (M, 1)))
        err = row_rel_err(got, ref)
        note(f"  {dup}: err={err:.3e}")
        assert err <= (TOL_FP8 if fp8 else TOL_BF16)


def test_fused_m0_is_noop(moe):
    note("fused M=0")
    wl = wlm.Workload("m0", M=0, K=256, N=256, E=4, topk=2)
    d, g = gen_small(wl)
    out = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    moe.moe_fused_forward(g["x"], g["w_router"], None, g["w1"], g["w2"], 2, out=out)
    torch.cuda.synchronize()


def test_swap_ab_identity_decode_vs_prefill(moe):
    """C^T = B^T.A^T: the Swap-AB decode kernels and the full-tile kernels give
    the same layer output on identical inputs (up to fp32 summation order and
    the bf16 rounding of the intermediate)."""
    note("swap-ab cross-check")
    wl = wlm.Workload("xcheck", M=96, K=512, N=768, E=6, topk=2, seed=11)
    d, g = gen_small(wl)
    a = out_f64(run_layer(moe, g, wl, 1))
    b = out_f64(run_layer(moe, g, wl, 2))
    ref, _, _ = oracle_layer(d, wl)
    assert row_rel_err(a, ref) <= TOL_BF16 and row_rel_err(b, ref) <= TOL_BF16
    assert row_rel_err(a, b) <= 1e-2


def test_fp8_decode_vs_tiles(moe):
    """The e4m3 Swap-AB decode kernels and the e4m3 full-tile kernels on
    identical inputs: both within tolerance of the oracle, and close to each
    other (they differ by fp32 summation order, which can move an activation
    code across an e4m3 rounding boundary)."""
    note("fp8 decode vs full tiles")
    wl = wlm.Workload("xcheck8", M=96, K=512, N=768, E=6, topk=2, fp8=True, seed=12)
    d, g = gen_small(wl)
    a = out_f64(run_layer(moe, g, wl, 1))
    b = out_f64(run_layer(moe, g, wl, 2))
    ref, _, _ = oracle_layer(d, wl)
    ea, eb, eab = row_rel_err(a, ref), row_rel_err(b, ref), row_rel_err(a, b)
    note(f"  decode {ea:.3e} tiles {eb:.3e} between {eab:.3e}")
    assert ea <= TOL_FP8 and eb <= TOL_FP8
    assert eab <= 2e-2


def test_mxfp4_decode_vs_tiles(moe):
    """MXFP4 weights on the decode kernels and on the full tiles, identical
    inputs: both within tolerance of the oracle and close to each other (the
    block scales act inside the MFMA on both; they differ by fp32 summation
    order and the e4m3 activation codes that order can move)."""
    note("mxfp4 decode vs full tiles")
    wl = wlm.Workload("xcheck_mx", M=96, K=512, N=768, E=6, topk=2, mxfp4=True, seed=13)
    d, g = gen_small(wl)
    a = out_f64(run_layer(moe, g, wl, 1))
    b = out_f64(run_layer(moe, g, wl, 2))
    ref, _, _ = oracle_layer(d, wl)
    ea, eb, eab = row_rel_err(a, ref), row_rel_err(b, ref), row_rel_err(a, b)
    note(f"  decode {ea:.3e} tiles {eb:.3e} between {eab:.3e}")
    assert ea <= TOL_FP8 and eb <= TOL_FP8
    assert eab <= 2e-2


def test_fused_deterministic(moe):
    """Ten calls on the same inputs are bitwise identical on every path: the
    decode and full-tile kernels, bf16, e4m3 and MXFP4, the multi-workgroup align
    and the routing GEMM1 with GEMM2 + combine of two tokens (no result
    depends on the order of atomics or on timing)."""
    note("determinism")
    wl = wlm.Workload("det", M=40, K=512, N=512, E=8, topk=2, seed=4)
    big = wlm.Workload("det_big", M=1100, K=256, N=256, E=8, topk=2, seed=5)
    two = wlm.Workload("det_two_tokens", M=2, K=512, N=512, E=8, topk=2, seed=6)
    for w, regimes in ((wl, (1, 2)), (wl.resized(fp8=True), (1, 2)),
                       (wl.resized(mxfp4=True), (1, 2)), (big, (0,)),
                       (big.resized(fp8=True), (0,)), (big.resized(mxfp4=True), (0,)),
                       (two, (0,))):
        d, g = gen_small(w)
        for regime in regimes:
            outs = [run_layer(moe, g, w, regime).clone() for _ in range(10)]
            for o in outs[1:]:
                assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16)), \
                    (w.name, w.fp8, regime)


# --------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the benchmark
# times; the oracle evaluates sampled tokens one by one
# --------------------------------------------------------------------------

def stratified_tokens(rids, E, B, M, k, n_min=64, max_experts=16):
    """Tokens whose slots sit at telling rows of the token blocks: in the
    segment of every expert (of at most max_experts, evenly spaced among
    those routed to) the first row, the rows either side of the block middle
    (the two halves of a 256-row block are different token waves) and the
    last row of the first, a middle and the last (padded) block, then random
    tokens up to n_min, plus the first and last token."""
    rs, _, ro, _ = oracle.align(rids, E, B)
    counts = np.bincount(rids.reshape(-1), minlength=E)
    rng = np.random.default_rng(M)
    toks = {0, M - 1}
    used = [e for e in range(E) if counts[e] > 0]
    n_pick = min(max_experts, len(used))
    pick = [used[i * len(used) // n_pick] for i in range(n_pick)]
    for e in pick:
        c = int(counts[e])
        nblk = (c + B - 1) // B
        for b in sorted({0, nblk // 2, nblk - 1}):
            for off in (0, B // 2 - 1, B // 2, B - 1):
                r = b * B + off
                if r < c:
                    toks.add(int(rs[ro[e] + r]) // k)
        toks.add(int(rs[ro[e] + c - 1]) // k)
    while len(toks) < n_min:
        toks.add(int(rng.integers(M)))
    return sorted(toks)


# the DeepSeek-shaped batch also with per-channel e4m3 weight scales and with
# MXFP4 weights and at 4096 tokens; the prefill batch also with e4m3 and with
# MXFP4 weights; the Mixtral decode batch with e4m3 and MXFP4 weights and the
# single token with MXFP4 weights
@pytest.mark.parametrize("name", list(wlm.WORKLOADS) + [
    "dsv3_fp8_rowwise", "dsv3_mxfp4", "mixtral_prefill_fp8", "mixtral_prefill_mxfp4",
    "dsv3_fp8_4096", "dsv3_mxfp4_4096", "mixtral_decode_fp8", "mixtral_decode_mxfp4",
    "single_token_decode_mxfp4"])
def test_fused_full_size_sampled(moe, name):
    if name in ("mixtral_decode_fp8", "mixtral_decode_mxfp4", "single_token_decode_mxfp4"):
        # the decode shapes with e4m3 and MXFP4 weights (every token checked)
        base, fmt = name.rsplit("_", 1)
        wl = wlm.WORKLOADS[base].resized(name=name, fp8=fmt == "fp8", mxfp4=fmt == "mxfp4")
    elif name == "dsv3_mxfp4_4096":
        # MXFP4 full tiles over 256 experts (about 128 rows each, 256-row blocks)
        wl = wlm.WORKLOADS["dsv3_fp8"].resized(name=name, M=4096, fp8=False, mxfp4=True)
    elif name == "mixtral_prefill_mxfp4":
        wl = wlm.WORKLOADS["mixtral_prefill"].resized(name=name, mxfp4=True)
    elif name == "dsv3_fp8_4096":
        # 4096 tokens on the DeepSeek shape: 32 768 token-slots over 256
        # experts (about 128 each): e4m3 full tiles with 128-row blocks and
        # the multi-workgroup align
        wl = wlm.WORKLOADS["dsv3_fp8"].resized(name=name, M=4096)
    elif name == "mixtral_prefill_fp8":
        # the prefill batch with e4m3 weights: the e4m3 full-tile kernels
        wl = wlm.WORKLOADS["mixtral_prefill"].resized(name=name, fp8=True)
    elif name == "dsv3_fp8_rowwise":
        wl = wlm.WORKLOADS["dsv3_fp8"].resized(name=name, fp8_rowwise=True)
    elif name == "dsv3_mxfp4":
        wl = wlm.WORKLOADS["dsv3_fp8"].resized(name=name, fp8=False, mxfp4=True)
    else:
        wl = wlm.WORKLOADS[name]
    note(f"full size {name}: generate on GPU")
    g = wlm.generate(wl, "cuda")
    out, ws = run_layer(moe, g, wl, keep_ws=True)
    got = out_f64(out)
    # the workspace was poisoned: a partial row never written would be NaN here
    assert np.isfinite(got).all()
    x_h, wr_h = bits(g["x"]), bits(g["w_router"])
    bias_h = None if g["bias"] is None else g["bias"].cpu().numpy()
    # the layer's own routing of every token is bit-exact with the oracle
    plan, rids, _ = check_fused_routing(moe, ws, wl, 0, x_h, wr_h, bias_h)
    del ws
    # and so is the standalone router on the same batch
    ids, _, lg = moe.moe_topk(g["x"], g["w_router"], g["bias"], wl.topk)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), rids)
    # every token for the decode batches (at most 128 tokens), else tokens at
    # the telling rows of every expert's blocks through the oracle
    if wl.M <= 128:
        toks = list(range(wl.M))
    else:
        toks = stratified_tokens(rids, wl.E, plan.block_m, wl.M, wl.topk)
    need = sorted(set(rids[toks].reshape(-1).tolist()))
    note(f"  oracle on {len(toks)} tokens, {len(need)} experts (block {plan.block_m})")
    w1 = [bits(g["w1"][e]) if e in need else None for e in range(wl.E)]
    w2 = [bits(g["w2"][e]) if e in need else None for e in range(wl.E)]
    s1 = None if g["w1_scale"] is None else g["w1_scale"].cpu().numpy()
    s2 = None if g["w2_scale"] is None else g["w2_scale"].cpu().numpy()
    ref, _, _ = oracle.moe_forward(x_h, wr_h, bias_h, w1, w2, wl.topk, w1_scale=s1,
                                   w2_scale=s2, tokens=toks, fp8=wl.fp8, mxfp4=wl.mxfp4)
    err = row_rel_err(got[toks], ref)
    note(f"  err={err:.3e}")
    assert err <= (TOL_FP8 if (wl.fp8 or wl.mxfp4) else TOL_BF16)
    del g, w1, w2
    torch.cuda.empty_cache()
