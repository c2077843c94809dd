"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against an independent source: a
library routine (numpy matmul / stable argsort, torch's bf16 and
float8_e4m3fn casts), a closed form, an invariant, brute-force dense
evaluation, or a value the pages print (tests/golden/pages_values.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests._brute import (bf16_bits_to_f64, dense_layer, e4m3_codes_to_f64,
                          f32_to_e4m3_codes, row_rel_err,
                          e2m1_as_e4m3_code, mx_dequant)
from tests._brute import e8m0_to_f64 as mx_e8m0_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")


def rand_bf16(rng, shape, std=1.0):
    v = torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
    return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_of(values):
    v = torch.tensor(values, dtype=torch.float32)
    return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f64(codes)
    ref = e4m3_codes_to_f64(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_exhaustive_bf16_values():
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) < 464.0)   # torch turns >=464 into NaN
    v = vals[keep]
    got = oracle.f32_to_e4m3(v)
    ref = f32_to_e4m3_codes(v)
    assert np.array_equal(got, ref)


def test_e4m3_encode_midpoints_ties_to_even():
    pos = e4m3_codes_to_f64(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal((mids.astype(np.float64)), (pos[:-1] + pos[1:]) / 2)  # exact in fp32
    got = oracle.f32_to_e4m3(np.concatenate([mids, -mids]))
    ref = f32_to_e4m3_codes(np.concatenate([mids, -mids]))
    assert np.array_equal(got, ref)
    # ties go to the even code
    assert np.all(got[: len(mids)] % 2 == 0)


def test_e4m3_encode_saturates_and_nan():
    got = oracle.f32_to_e4m3(np.array([448.0, 463.9, 464.0, 1e6, -1e6, np.inf, -np.inf,
                                       np.nan], np.float32))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F]


def test_quant_rows_amax_maps_to_448_and_half_ulp():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((6, 300)) * rng.uniform(0.01, 100, (6, 1))).astype(np.float32)
    q, s = oracle.quant_rows_f32(v)
    dq = e4m3_codes_to_f64(q)
    for r in range(v.shape[0]):
        i = int(np.argmax(np.abs(v[r])))
        assert abs(dq[r, i]) == 448.0
        assert s[r] == np.float32(np.abs(v[r]).max()) / np.float32(448.0)
        # |v/s - dequant| <= half the spacing of e4m3 at that magnitude
        y = v[r].astype(np.float64) / s[r]
        ay = np.maximum(np.abs(y), 2.0 ** -6)
        half_ulp = 2.0 ** (np.floor(np.log2(ay)) - 3) / 2
        assert np.all(np.abs(y - dq[r]) <= half_ulp * (1 + 1e-6))
    z, sz = oracle.quant_rows_f32(np.zeros((1, 8), np.float32))
    assert sz[0] == 1.0 and not z.any()


def test_quant_rows_bf16_matches_torch_codec():
    rng = np.random.default_rng(2)
    x = rand_bf16(rng, (5, 96))
    q, s = oracle.quant_rows_bf16(x)
    x32 = (x.astype(np.uint32) << 16).view(np.float32)
    s_ref = (np.abs(x32).max(axis=1) / np.float32(448)).astype(np.float32)
    assert np.array_equal(s, s_ref)
    ref = f32_to_e4m3_codes((x32 / s_ref[:, None]).astype(np.float32))
    assert np.array_equal(q, ref)


# --------------------------------------------------------------------------
# gating
# --------------------------------------------------------------------------

@pytest.mark.parametrize("with_bias", [False, True])
def test_logits_vs_numpy_matmul(with_bias):
    rng = np.random.default_rng(3)
    M, K, E = 9, 200, 13
    x = rand_bf16(rng, (M, K))
    wr = rand_bf16(rng, (E, K), 1 / math.sqrt(K))
    bias = (rng.standard_normal(E) * 0.7).astype(np.float32) if with_bias else None
    got = oracle.logits(x, wr, bias)
    ref64 = bf16_bits_to_f64(x) @ bf16_bits_to_f64(wr).T
    if with_bias:
        ref64 = ref64 + bias.astype(np.float64)
    assert np.array_equal(got, ref64.astype(np.float32))


def test_topk_vs_stable_argsort_and_softmax():
    rng = np.random.default_rng(4)
    M, E, k = 40, 11, 3
    lg = rng.standard_normal((M, E)).astype(np.float32)
    lg[:, 5] = lg[:, 2]          # exact ties: the lower id must come first
    lg[3, :] = 0.25              # a row of all-equal logits
    ids, w = oracle.topk(lg, k)
    ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, ref)
    assert ids[3].tolist() == [0, 1, 2]
    l64 = lg.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ref, axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=0, atol=1e-14)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)   # slots in descending weight


def test_topk_k2_closed_form_sigmoid():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((50, 6)).astype(np.float32) * 3
    ids, w = oracle.topk(lg, 2)
    l0 = np.take_along_axis(lg, ids[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(lg, ids[:, 1:], 1)[:, 0].astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-(l0 - l1)))
    assert np.allclose(w[:, 0], sig, rtol=0, atol=1e-14)
    assert np.allclose(w[:, 1], 1 - sig, rtol=0, atol=1e-14)


def test_topk_k_equals_e_returns_all_in_order():
    lg = np.array([[0.1, 2.0, -1.0, 2.0]], np.float32)
    ids, w = oracle.topk(lg, 4)
    assert ids.tolist() == [[1, 3, 0, 2]]
    assert abs(w[0].sum() - 1) < 1e-15 and w[0, 0] == w[0, 1]


def test_ties_from_duplicate_router_rows():
    rng = np.random.default_rng(6)
    M, K, E = 16, 64, 6
    x = rand_bf16(rng, (M, K))
    wr = rand_bf16(rng, (E, K), 0.2)
    wr[4] = wr[1]
    wr[5] = wr[1]
    lg = oracle.logits(x, wr)
    assert np.array_equal(lg[:, 1], lg[:, 4]) and np.array_equal(lg[:, 1], lg[:, 5])
    ids, _ = oracle.topk(lg, 3)
    for t in range(M):
        row = ids[t].tolist()
        # whenever duplicates are picked together, they appear in ascending id order
        dup = [e for e in row if e in (1, 4, 5)]
        assert dup == sorted(dup)
        if 4 in row or 5 in row:
            assert 1 in row


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------

def brute_align(ids, E, B):
    flat = ids.reshape(-1)
    n = flat.size
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    padded = -(-counts // B) * B
    offs = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    cap = n + E * (B - 1)
    sorted_ids = np.full(cap, n, np.int32)
    pos = 0
    for e in range(E):
        seg = order[pos:pos + counts[e]]
        sorted_ids[offs[e]:offs[e] + counts[e]] = seg
        pos += counts[e]
    blocks = np.full(cap // B, -1, np.int32)
    for e in range(E):
        blocks[offs[e] // B: offs[e + 1] // B] = e
    return sorted_ids, blocks, offs, int(offs[-1])


@pytest.mark.parametrize("M,k,E,B", [(64, 2, 8, 16), (37, 3, 17, 4), (5, 1, 40, 16),
                                     (128, 8, 256, 16), (300, 2, 8, 128), (1, 2, 16, 16),
                                     (0, 2, 8, 16), (20, 2, 5, 1)])
def test_align_vs_brute_and_invariants(M, k, E, B):
    rng = np.random.default_rng(M * 1000 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32) \
        if M else np.zeros((0, k), np.int32)
    s, b, o, npad = oracle.align(ids, E, B)
    rs, rb, ro, rn = brute_align(ids, E, B)
    assert np.array_equal(s, rs) and np.array_equal(b, rb)
    assert np.array_equal(o, ro) and npad == rn
    n = M * k
    real = s[s < n]
    assert np.array_equal(np.sort(real), np.arange(n))          # bijection
    counts = np.bincount(ids.reshape(-1), minlength=E)
    assert counts.sum() == n                                    # counts sum to M*k
    assert np.all(np.diff(o) % B == 0)                          # padded to B
    for e in range(E):
        seg = s[o[e]:o[e + 1]]
        segr = seg[seg < n]
        assert np.all(np.diff(segr) > 0)                        # stable / ascending
        assert np.all(ids.reshape(-1)[segr] == e)
        assert np.all(seg[len(segr):] == n)                     # sentinel padding


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

def make_layer(rng, M, K, N, E, fp8=False, bias=False):
    x = rand_bf16(rng, (M, K))
    wr = rand_bf16(rng, (E, K), 1 / math.sqrt(K))
    b = (rng.standard_normal(E) * math.sqrt(0.5)).astype(np.float32) if bias else None
    if fp8:
        w1 = rng.integers(0, 256, (E, 2 * N, K)).astype(np.uint8)
        w2 = rng.integers(0, 256, (E, K, N)).astype(np.uint8)
        w1[(w1 & 0x7F) == 0x7F] = 0x3C
        w2[(w2 & 0x7F) == 0x7F] = 0x3C
        s1 = (rng.uniform(0.5, 2, E) / 448 / math.sqrt(K)).astype(np.float32)
        s2 = (rng.uniform(0.5, 2, E) / 448 / math.sqrt(N)).astype(np.float32)
        return x, wr, b, w1, w2, s1, s2
    w1 = rand_bf16(rng, (E, 2 * N, K), 1 / math.sqrt(K))
    w2 = rand_bf16(rng, (E, K, N), 1 / math.sqrt(N))
    return x, wr, b, w1, w2, None, None


@pytest.mark.parametrize("M,K,N,E,k,bias", [(8, 32, 16, 4, 2, False), (5, 64, 32, 8, 1, True),
                                            (6, 48, 24, 3, 3, False), (4, 16, 8, 1, 1, False),
                                            (7, 40, 20, 6, 2, True)])
def test_layer_bf16_vs_dense_bruteforce(M, K, N, E, k, bias):
    rng = np.random.default_rng(M + 10 * K + 100 * E + k)
    x, wr, b, w1, w2, _, _ = make_layer(rng, M, K, N, E, bias=bias)
    out, ids, wts = oracle.moe_forward(x, wr, b, w1, w2, k)
    ref, rids, wfull = dense_layer(x, wr, b, w1, w2, k)
    assert np.array_equal(ids, rids)
    assert np.allclose(wts, np.take_along_axis(wfull, rids, 1), rtol=0, atol=1e-14)
    assert row_rel_err(out, ref) <= 1e-12


@pytest.mark.parametrize("M,K,N,E,k", [(6, 64, 32, 8, 2), (4, 128, 16, 5, 3), (3, 32, 64, 2, 2)])
def test_layer_fp8_vs_dense_bruteforce(M, K, N, E, k):
    rng = np.random.default_rng(7 + M + K + N)
    x, wr, b, w1, w2, s1, s2 = make_layer(rng, M, K, N, E, fp8=True)
    out, ids, _ = oracle.moe_forward(x, wr, b, w1, w2, k, w1_scale=s1, w2_scale=s2, fp8=True)
    ref, rids, _ = dense_layer(x, wr, b, w1, w2, k, fp8=True, w1_scale=s1, w2_scale=s2)
    assert np.array_equal(ids, rids)
    assert row_rel_err(out, ref) <= 1e-12


def rowwise_scales(rng, E, N, K):
    s1 = (rng.uniform(0.25, 4, (E, 2 * N)) / 448 / math.sqrt(K)).astype(np.float32)
    s2 = (rng.uniform(0.25, 4, (E, K)) / 448 / math.sqrt(N)).astype(np.float32)
    return s1, s2


@pytest.mark.parametrize("M,K,N,E,k", [(6, 64, 32, 8, 2), (4, 128, 16, 5, 3), (3, 32, 64, 2, 2)])
def test_layer_fp8_rowwise_vs_dense_bruteforce(M, K, N, E, k):
    """Per-channel weight scales (one per output row of W1 and of W2)."""
    rng = np.random.default_rng(17 + M + K + N)
    x, wr, b, w1, w2, _, _ = make_layer(rng, M, K, N, E, fp8=True)
    s1, s2 = rowwise_scales(rng, E, N, K)
    out, ids, _ = oracle.moe_forward(x, wr, b, w1, w2, k, w1_scale=s1, w2_scale=s2, fp8=True)
    ref, rids, _ = dense_layer(x, wr, b, w1, w2, k, fp8=True, w1_scale=s1, w2_scale=s2)
    assert np.array_equal(ids, rids)
    assert row_rel_err(out, ref) <= 1e-12


def test_layer_fp8_rowwise_equal_rows_is_per_tensor():
    """Row scales all equal to the expert's tensor scale give the per-tensor
    result bit for bit."""
    rng = np.random.default_rng(23)
    M, K, N, E, k = 7, 64, 48, 6, 2
    x, wr, b, w1, w2, s1, s2 = make_layer(rng, M, K, N, E, fp8=True)
    r1 = np.repeat(s1[:, None], 2 * N, axis=1)
    r2 = np.repeat(s2[:, None], K, axis=1)
    a, _, _ = oracle.moe_forward(x, wr, b, w1, w2, k, w1_scale=s1, w2_scale=s2, fp8=True)
    c, _, _ = oracle.moe_forward(x, wr, b, w1, w2, k, w1_scale=r1, w2_scale=r2, fp8=True)
    assert np.array_equal(a, c)


def test_layer_fp8_rowwise_w2_row_scale_hits_its_column():
    """Doubling the scale of W2 row c (of every expert) doubles output column
    c exactly and leaves every other column unchanged."""
    rng = np.random.default_rng(29)
    M, K, N, E, k = 5, 32, 16, 4, 2
    x, wr, b, w1, w2, _, _ = make_layer(rng, M, K, N, E, fp8=True)
    s1, s2 = rowwise_scales(rng, E, N, K)
    a, _, _ = oracle.moe_forward(x, wr, b, w1, w2, k, w1_scale=s1, w2_scale=s2, fp8=True)
    c = 11
    t2 = s2.copy()
    t2[:, c] *= 2
    d, _, _ = oracle.moe_forward(x, wr, b, w1, w2, k, w1_scale=s1, w2_scale=t2, fp8=True)
    assert np.array_equal(d[:, c], 2 * a[:, c])
    keep = np.arange(K) != c
    assert np.array_equal(d[:, keep], a[:, keep])


# --------------------------------------------------------------------------
# MXFP4 weights (e2m1 elements, E8M0 scale per 32 elements of a row)
# --------------------------------------------------------------------------

def test_e2m1_decode_matches_e4m3_codec():
    """Each of the 16 e2m1 codes decodes to the value of the e4m3 code with
    the same sign, exponent and mantissa (torch's e4m3 codec); the magnitudes
    are 8 distinct values up to 6, negatives mirror them."""
    c = np.arange(16, dtype=np.uint8)
    got = oracle.e2m1_to_f64(c)
    ref = e4m3_codes_to_f64(e2m1_as_e4m3_code(c))
    assert np.array_equal(got, ref)
    assert len(set(np.abs(got[:8]).tolist())) == 8 and np.abs(got).max() == 6.0
    assert np.array_equal(got[8:], -got[:8])


def test_e8m0_decode_matches_torch():
    c = np.arange(255, dtype=np.uint8)
    assert np.array_equal(oracle.e8m0_to_f64(c), mx_e8m0_to_f64(c))
    assert np.isnan(oracle.e8m0_to_f64([255])[0])


def make_mx_layer(rng, M, K, N, E, scale_lo=117, scale_hi=124):
    x = rand_bf16(rng, (M, K))
    wr = rand_bf16(rng, (E, K), 1 / math.sqrt(K))
    w1 = rng.integers(0, 256, (E, 2 * N, K // 2)).astype(np.uint8)
    w2 = rng.integers(0, 256, (E, K, N // 2)).astype(np.uint8)
    s1 = rng.integers(scale_lo, scale_hi, (E, 2 * N, K // 32)).astype(np.uint8)
    s2 = rng.integers(scale_lo, scale_hi, (E, K, N // 32)).astype(np.uint8)
    return x, wr, w1, w2, s1, s2


@pytest.mark.parametrize("M,K,N,E,k", [(6, 64, 32, 8, 2), (4, 128, 64, 5, 3), (3, 32, 96, 2, 2)])
def test_layer_mxfp4_vs_dense_bruteforce(M, K, N, E, k):
    rng = np.random.default_rng(31 + M + K + N)
    x, wr, w1, w2, s1, s2 = make_mx_layer(rng, M, K, N, E)
    out, ids, _ = oracle.moe_forward(x, wr, None, w1, w2, k, w1_scale=s1, w2_scale=s2,
                                     mxfp4=True)
    W1 = np.stack([mx_dequant(w1[e], s1[e]) for e in range(E)])
    W2 = np.stack([mx_dequant(w2[e], s2[e]) for e in range(E)])
    ref, rids, _ = dense_layer(x, wr, None, None, None, k, fp8=True, w_f64=(W1, W2))
    assert np.array_equal(ids, rids)
    assert row_rel_err(out, ref) <= 1e-12


def test_layer_mxfp4_unit_scales_equals_fp8_per_tensor():
    """With every block scale 1 (E8M0 127) the MXFP4 layer is the e4m3 layer
    with per-tensor scale 1 on the same weight values, bit for bit."""
    rng = np.random.default_rng(37)
    M, K, N, E, k = 7, 64, 64, 6, 2
    x, wr, w1, w2, s1, s2 = make_mx_layer(rng, M, K, N, E, 127, 128)
    a, _, _ = oracle.moe_forward(x, wr, None, w1, w2, k, w1_scale=s1, w2_scale=s2, mxfp4=True)

    def unpack_as_e4m3(p):
        c = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
        c[..., 0::2] = p & 15
        c[..., 1::2] = p >> 4
        return e2m1_as_e4m3_code(c)

    ones = np.ones(E, np.float32)
    b, _, _ = oracle.moe_forward(x, wr, None, unpack_as_e4m3(w1), unpack_as_e4m3(w2), k,
                                 w1_scale=ones, w2_scale=ones, fp8=True)
    assert np.array_equal(a, b)


def test_layer_mxfp4_w2_row_scales_hit_their_column():
    """One more E8M0 step on every block of W2 row c doubles output column c
    exactly and leaves every other column unchanged."""
    rng = np.random.default_rng(41)
    M, K, N, E, k = 5, 64, 64, 4, 2
    x, wr, w1, w2, s1, s2 = make_mx_layer(rng, M, K, N, E)
    a, _, _ = oracle.moe_forward(x, wr, None, w1, w2, k, w1_scale=s1, w2_scale=s2, mxfp4=True)
    c = 13
    t2 = s2.copy()
    t2[:, c, :] += 1
    d, _, _ = oracle.moe_forward(x, wr, None, w1, w2, k, w1_scale=s1, w2_scale=t2, mxfp4=True)
    assert np.array_equal(d[:, c], 2 * a[:, c])
    keep = np.arange(K) != c
    assert np.array_equal(d[:, keep], a[:, keep])


def test_dense_swiglu_special_case_page_decode_shape():
    """E=1, k=1: the layer is one dense SwiGLU MLP; shapes of the pages' decode
    example (A 1 x 4096, expert block 4096 x 8192)."""
    g = json.load(open(GOLDEN))["decode_gemv_example"]
    M, K = g["A"]
    N = g["B"][1]
    rng = np.random.default_rng(8)
    x = rand_bf16(rng, (M, K))
    wr = rand_bf16(rng, (1, K), 1 / math.sqrt(K))
    w1 = rand_bf16(rng, (1, 2 * N, K), 1 / math.sqrt(K))
    w2 = rand_bf16(rng, (1, K, N), 1 / math.sqrt(N))
    out, ids, wts = oracle.moe_forward(x, wr, None, w1, w2, 1)
    assert ids.tolist() == [[0]] and wts.tolist() == [[1.0]]
    xf = bf16_bits_to_f64(x)
    h = xf @ bf16_bits_to_f64(w1[0]).T
    ref = (h[:, :N] / (1 + np.exp(-h[:, :N])) * h[:, N:]) @ bf16_bits_to_f64(w2[0]).T
    assert row_rel_err(out, ref) <= 1e-12


def test_closed_form_hand_example():
    """M=1, K=2, N=1, E=3, k=2 worked by hand: logits (0.5, 0, -1) pick experts
    0 and 1 with weights sigmoid(0.5) and 1 - sigmoid(0.5)."""
    x = bf16_of([[1.0, 0.0]])
    wr = bf16_of([[0.5, 0.0], [0.0, 1.0], [-1.0, 0.0]])
    w1 = bf16_of([[[2.0, 0.0], [0.5, 0.0]],        # expert 0: gate 2, up 0.5
                  [[-1.0, 0.0], [4.0, 0.0]],       # expert 1: gate -1, up 4
                  [[9.0, 9.0], [9.0, 9.0]]])       # expert 2: not picked
    w2 = bf16_of([[[1.0], [-3.0]], [[0.25], [2.0]], [[7.0], [7.0]]])
    out, ids, wts = oracle.moe_forward(x, wr, None, w1, w2, 2)
    w0 = 1.0 / (1.0 + math.exp(-0.5))
    a0 = (2.0 / (1.0 + math.exp(-2.0))) * 0.5
    a1 = (-1.0 / (1.0 + math.exp(1.0))) * 4.0
    ref = [w0 * a0 * 1.0 + (1 - w0) * a1 * 0.25, w0 * a0 * -3.0 + (1 - w0) * a1 * 2.0]
    assert ids.tolist() == [[0, 1]]
    assert abs(wts[0, 0] - w0) < 1e-15
    assert np.allclose(out[0], ref, rtol=1e-14, atol=0)


def test_linearity_in_w2():
    rng = np.random.default_rng(9)
    x, wr, b, w1, w2, _, _ = make_layer(rng, 6, 32, 16, 4)
    out, _, _ = oracle.moe_forward(x, wr, b, w1, w2, 2)
    w2x2 = (torch.from_numpy(w2.view(np.int16)).view(torch.bfloat16) * 2).view(torch.int16)
    out2, _, _ = oracle.moe_forward(x, wr, b, w1, w2x2.numpy().view(np.uint16), 2)
    assert np.array_equal(out2, 2 * out)     # scaling by 2 is exact throughout


def test_token_subset_and_missing_expert():
    rng = np.random.default_rng(10)
    x, wr, b, w1, w2, _, _ = make_layer(rng, 12, 32, 16, 6)
    full, ids, _ = oracle.moe_forward(x, wr, b, w1, w2, 2)
    toks = [11, 0, 5]
    sub, sids, _ = oracle.moe_forward(x, wr, b, w1, w2, 2, tokens=toks)
    assert np.array_equal(sub, full[toks]) and np.array_equal(sids, ids[toks])
    needed = set(ids[toks].reshape(-1).tolist())
    w1l = [w1[e] if e in needed else None for e in range(6)]
    w2l = [w2[e] if e in needed else None for e in range(6)]
    sub2, _, _ = oracle.moe_forward(x, wr, b, w1l, w2l, 2, tokens=toks)
    assert np.array_equal(sub2, sub)
    missing = sorted(set(range(6)) - needed)
    if missing:
        w1l[ids[toks[0], 0]] = None
        with pytest.raises(RuntimeError):
            oracle.moe_forward(x, wr, b, w1l, w2l, 2, tokens=toks)


def test_poisson_load_value_from_pages():
    g = json.load(open(GOLDEN))["poisson_load"]
    M, k, E = g["tokens"], g["topk"], g["experts"]
    lam = M * k / E
    assert lam == g["lambda"]
    p2 = 1 - math.exp(-lam) * (1 + lam)
    assert p2 >= g["p_at_least_two"]        # the page prints the value as ~0.9999
    # routing random tokens through the oracle gives mean load lambda exactly and,
    # as the Poisson model says, practically every expert gets >= 2 rows
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((M, E)).astype(np.float32)
    ids, _ = oracle.topk(lg, k)
    s, _, o, _ = oracle.align(ids, E, 1)
    counts = np.diff(o)
    assert counts.sum() == M * k and counts.mean() == lam
    assert (counts >= 2).mean() >= 0.99
