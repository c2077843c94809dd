// router.hip -- the MoE router on gfx950: logits, top-k, routing weights and
// (FP8 path) per-token dynamic e4m3 quantisation of the tokens.
//
// "Mixture-of-Experts kernel engineering on Amazon SageMaker AI" (summary
// text) puts token routing inside the fused MoE operation instead of host
// loops; "AI混合专家模型性能优化全链路解析" (chapter 1) picks experts by top-k
// over the router logits.  Readings used here: a logit is the fp32 rounding
// of the fp64-accumulated dot product x_t.W_r[e] (+ bias[e]); the k largest
// logits are taken in descending order with ties to the lower expert id;
// the weights are the softmax over the picked logits (equal to the full
// softmax renormalised over them).
#include "routing.hpp"
#include "tuning.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Logits.  A workgroup (4 waves) computes a TT-token x TE-expert tile; its
// waves split K into four contiguous quarters, each lane accumulates
// bf16*bf16 products (exact in fp64) in fp64 over 8-element slices, the
// wave sums its lanes with DPP/ds_swizzle, and the four wave partials are
// added in wave order through LDS (a fixed order: deterministic).  Small
// problems use 1x1 tiles so every (token, expert) pair gets a workgroup.
// ---------------------------------------------------------------------------
template <int TT, int TE, bool VEC>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int M, int K, int E, float* __restrict__ logits) {
    __shared__ double part[4][TT * TE];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int tiles_e = (E + TE - 1) / TE;
    const int t0 = ((int)blockIdx.x / tiles_e) * TT;
    const int e0 = ((int)blockIdx.x % tiles_e) * TE;

    double acc[TT][TE];
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
        for (int b = 0; b < TE; ++b) acc[a][b] = 0.0;

    // Rows past M / E are clamped to a valid row; their sums are discarded.
    const uint16_t* xr[TT];
    const uint16_t* wrr[TE];
#pragma unroll
    for (int a = 0; a < TT; ++a) xr[a] = x + (size_t)min(t0 + a, M - 1) * K;
#pragma unroll
    for (int b = 0; b < TE; ++b) wrr[b] = wr + (size_t)min(e0 + b, E - 1) * K;

    if constexpr (VEC) {
        // K % 8 == 0: wave w covers [kb, ke) in 16-byte slices, lane-strided
        const int kq = ((K / 8 + 3) / 4) * 8;
        const int kb = wave * kq, ke = min(K, kb + kq);
        for (int k = kb + lane * 8; k < ke; k += kWave * 8) {
            double xv[TT][8], wv[TE][8];
#pragma unroll
            for (int a = 0; a < TT; ++a) {
                const i32x4_t v = *reinterpret_cast<const i32x4_t*>(xr[a] + k);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xv[a][2 * q] = (double)bf16_bits_to_f32((uint32_t)v[q] & 0xffffu);
                    xv[a][2 * q + 1] = (double)bf16_bits_to_f32((uint32_t)v[q] >> 16);
                }
            }
#pragma unroll
            for (int b = 0; b < TE; ++b) {
                const i32x4_t v = *reinterpret_cast<const i32x4_t*>(wrr[b] + k);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    wv[b][2 * q] = (double)bf16_bits_to_f32((uint32_t)v[q] & 0xffffu);
                    wv[b][2 * q + 1] = (double)bf16_bits_to_f32((uint32_t)v[q] >> 16);
                }
            }
#pragma unroll
            for (int a = 0; a < TT; ++a)
#pragma unroll
                for (int b = 0; b < TE; ++b)
#pragma unroll
                    for (int q = 0; q < 8; ++q) acc[a][b] = __fma_rn(xv[a][q], wv[b][q], acc[a][b]);
        }
    } else {
        const int kq = (K + 3) / 4;
        const int kb = wave * kq, ke = min(K, kb + kq);
        for (int k = kb + lane; k < ke; k += kWave) {
            double xv[TT], wv[TE];
#pragma unroll
            for (int a = 0; a < TT; ++a) xv[a] = (double)bf16_bits_to_f32(xr[a][k]);
#pragma unroll
            for (int b = 0; b < TE; ++b) wv[b] = (double)bf16_bits_to_f32(wrr[b][k]);
#pragma unroll
            for (int a = 0; a < TT; ++a)
#pragma unroll
                for (int b = 0; b < TE; ++b) acc[a][b] = __fma_rn(xv[a], wv[b], acc[a][b]);
        }
    }

#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
        for (int b = 0; b < TE; ++b) {
            const double s = wave_sum_f64(acc[a][b]);
            if (lane == 0) part[wave][a * TE + b] = s;
        }
    __syncthreads();
    const int tid = (int)threadIdx.x;
    if (tid < TT * TE) {
        const int t = t0 + tid / TE, e = e0 + tid % TE;
        if (t < M && e < E) {
            double s = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
            if (bias) s += (double)bias[e];
            logits[(size_t)t * E + e] = (float)s;
        }
    }

}

// ---------------------------------------------------------------------------
// Logits of large batches on the fp64 matrix cores: a workgroup computes a
// 16-token x 16-expert tile with v_mfma_f64_16x16x4_f64; its 16 waves split
// K into contiguous ranges (K % 512 == 0) and the per-wave fp64 sums are
// added in wave order through LDS (deterministic), then the bias and one
// fp32 rounding.  The kernel is bound by the fp64 matrix rate of the CU a
// tile runs on, so with fewer tiles than CUs the reduction is also split
// over nks workgroups per tile (ks-th contiguous range of K each), which
// store fp64 partial sums; the top-k kernel then adds them in ks order,
// adds the bias and rounds once.  Operand layout: lane l supplies token / expert row l % 16
// at k-slot l / 16, and each 16-byte load of a row gives the elements of 8
// successive MFMAs (MFMA m takes element m of every lane's 8-element run,
// the same k for both operands).  Accumulator element q of lane l is tile
// entry (token 4q + l/16, expert l % 16).
// ---------------------------------------------------------------------------
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kLogitWaves = 16;

__global__ __launch_bounds__(kLogitWaves * 64) void router_logits_f64mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int M, int K, int E, float* __restrict__ logits, int nks,
    double* __restrict__ lpart) {
    __shared__ double part[kLogitWaves][256];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int tiles_e = (E + 15) / 16;
    const int tile = (int)blockIdx.x / nks, ks = (int)blockIdx.x % nks;
    const int t0 = (tile / tiles_e) * 16;
    const int e0 = (tile % tiles_e) * 16;
    const int r = lane & 15, kq = lane >> 4;
    // rows past M / E are clamped to a valid row; their sums are discarded
    const uint16_t* xr = x + (size_t)min(t0 + r, M - 1) * K + kq * 8;
    const uint16_t* wrr = wr + (size_t)min(e0 + r, E - 1) * K + kq * 8;
    const int kw = K / nks / kLogitWaves;
    const int kb = ks * (K / nks) + wave * kw;
    const int nblk = kw / 32;

    f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
    auto mma8 = [&](i32x4_t va, i32x4_t vb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(
                (double)bf16_bits_to_f32((uint32_t)va[q] & 0xffffu),
                (double)bf16_bits_to_f32((uint32_t)vb[q] & 0xffffu), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(
                (double)bf16_bits_to_f32((uint32_t)va[q] >> 16),
                (double)bf16_bits_to_f32((uint32_t)vb[q] >> 16), acc, 0, 0, 0);
        }
    };
    // two 32-deep blocks in flight ahead of the one being multiplied
    i32x4_t a0 = *reinterpret_cast<const i32x4_t*>(xr + kb);
    i32x4_t b0 = *reinterpret_cast<const i32x4_t*>(wrr + kb);
    i32x4_t a1 = a0, b1 = b0;
    if (nblk > 1) {
        a1 = *reinterpret_cast<const i32x4_t*>(xr + kb + 32);
        b1 = *reinterpret_cast<const i32x4_t*>(wrr + kb + 32);
    }
    for (int i = 0; i < nblk; ++i) {
        i32x4_t a2 = a1, b2 = b1;
        if (i + 2 < nblk) {
            a2 = *reinterpret_cast<const i32x4_t*>(xr + kb + (i + 2) * 32);
            b2 = *reinterpret_cast<const i32x4_t*>(wrr + kb + (i + 2) * 32);
        }
        mma8(a0, b0);
        a0 = a1; b0 = b1;
        a1 = a2; b1 = b2;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) part[wave][(4 * q + kq) * 16 + r] = acc[q];
    __syncthreads();
    const int tid = (int)threadIdx.x;
    if (tid < 256) {
        const int t = t0 + tid / 16, e = e0 + tid % 16;
        if (t < M && e < E) {
            double s = part[0][tid];
#pragma unroll
            for (int w = 1; w < kLogitWaves; ++w) s += part[w][tid];
            if (nks > 1) {
                lpart[((size_t)ks * M + t) * E + e] = s;
            } else {
                if (bias) s += (double)bias[e];
                logits[(size_t)t * E + e] = (float)s;
            }
        }
    }
}

// Per-token dynamic e4m3 quantisation for the fused FP8 path: one workgroup
// per token row, 16-byte loads (K % 8 == 0), s = amax/448 (1 if amax == 0),
// code = E4M3(x/s) with one correctly rounded fp32 division.
__global__ __launch_bounds__(256) void quant_rows_vec_kernel(const uint16_t* __restrict__ x,
                                                             int M, int K,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ scale) {
    __shared__ uint32_t wmax[4];
    const int t = (int)blockIdx.x;
    const int tid = (int)threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint16_t* row = x + (size_t)t * K;
    uint32_t amax = 0;
    for (int k = tid * 8; k < K; k += 256 * 8) {
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(row + k);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            amax = max(amax, max((uint32_t)v[u] & 0x7fffu, ((uint32_t)v[u] >> 16) & 0x7fffu));
    }
    amax = wave_max_bits(amax << 16);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const float am = __uint_as_float(amax);
    const float sc = (am == 0.0f) ? 1.0f : am / 448.0f;
    uint8_t* dst = q + (size_t)t * K;
    for (int k = tid * 8; k < K; k += 256 * 8) {
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(row + k);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            lo |= f32_to_e4m3(bf16_bits_to_f32((uint32_t)v[u] & 0xffffu) / sc) << (16 * u);
            lo |= f32_to_e4m3(bf16_bits_to_f32((uint32_t)v[u] >> 16) / sc) << (16 * u + 8);
            hi |= f32_to_e4m3(bf16_bits_to_f32((uint32_t)v[u + 2] & 0xffffu) / sc) << (16 * u);
            hi |= f32_to_e4m3(bf16_bits_to_f32((uint32_t)v[u + 2] >> 16) / sc) << (16 * u + 8);
        }
        *reinterpret_cast<uint2*>(dst + k) = make_uint2(lo, hi);
    }
    if (tid == 0) scale[t] = sc;
}

// ---------------------------------------------------------------------------
// Top-k + weights: one wave per token (topk_wave in routing.hpp).
// ---------------------------------------------------------------------------
// With nks > 1 the wave first forms its token's logits from the fp64
// partial sums (ascending ks, then the bias, one fp32 rounding) and stores
// them; lane l handles experts l, l+64, ..., the same lanes that read them
// back in topk_wave.
__global__ __launch_bounds__(256) void router_topk_kernel(
    float* __restrict__ logits, int M, int E, int topk,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    const double* __restrict__ lpart, int nks, const float* __restrict__ bias) {
    const int t = (int)(blockIdx.x * 4 + threadIdx.x / kWave);
    if (t >= M) return;  // wave-uniform
    if (nks > 1) {
        for (int e = lane_id(); e < E; e += kWave) {
            double s = lpart[(size_t)t * E + e];
            for (int ks = 1; ks < nks; ++ks) s += lpart[((size_t)ks * M + t) * E + e];
            if (bias) s += (double)bias[e];
            logits[(size_t)t * E + e] = (float)s;
        }
    }
    topk_wave(logits + (size_t)t * E, E, topk, topk_ids + (size_t)t * topk,
              topk_weights + (size_t)t * topk, nullptr);
}

// ---------------------------------------------------------------------------
// Per-row e4m3 quantisation of bf16 rows, exported on its own.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int M,
                                                         int K, uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
    const int lane = lane_id();
    const int t = (int)(blockIdx.x * 4 + threadIdx.x / kWave);
    if (t >= M) return;
    const uint16_t* xr = x + (size_t)t * K;
    uint32_t amax = 0;
    for (int k = lane; k < K; k += kWave) amax = max(amax, (uint32_t)xr[k] & 0x7fffu);
    amax = wave_max_bits(amax << 16);
    const float a = __uint_as_float(amax);
    const float s = (a == 0.0f) ? 1.0f : a / 448.0f;
    for (int k = lane; k < K; k += kWave)
        q[(size_t)t * K + k] = (uint8_t)f32_to_e4m3(bf16_bits_to_f32(xr[k]) / s);
    if (lane == 0) scale[t] = s;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int router_logit_splits(int M, int K, int E) {
    if ((long)M * E <= 8192 || K % (kLogitWaves * 32)) return 1;
    // fp64 matrix work is the bound: split K until every CU holds a tile
    const long tiles = (long)((M + 15) / 16) * ((E + 15) / 16);
    int nks = 1;
    while (tiles * nks < tune::kRouterSplitTargetTiles && nks < 4 &&
           K % (kLogitWaves * 32 * nks * 2) == 0)
        nks *= 2;
    return nks;
}

void launch_router_logits(const void* x, const void* wr, const float* bias, int M, int K, int E,
                          float* logits, uint8_t* xq, float* xscale, int nks, double* lpart,
                          hipStream_t s) {
    const uint16_t* xp = (const uint16_t*)x;
    const uint16_t* wp = (const uint16_t*)wr;
    if ((long)M * E <= 8192) {
        const int grid = M * E;
        if (K % 8 == 0)
            router_logits_kernel<1, 1, true><<<grid, 256, 0, s>>>(xp, wp, bias, M, K, E, logits);
        else
            router_logits_kernel<1, 1, false><<<grid, 256, 0, s>>>(xp, wp, bias, M, K, E, logits);
    } else if (K % (kLogitWaves * 32) == 0) {
        const int grid = ((M + 15) / 16) * ((E + 15) / 16) * nks;
        router_logits_f64mfma_kernel<<<grid, kLogitWaves * 64, 0, s>>>(xp, wp, bias, M, K, E,
                                                                      logits, nks, lpart);
    } else {
        const int grid = ((M + 3) / 4) * ((E + 3) / 4);
        if (K % 8 == 0)
            router_logits_kernel<4, 4, true><<<grid, 256, 0, s>>>(xp, wp, bias, M, K, E, logits);
        else
            router_logits_kernel<4, 4, false><<<grid, 256, 0, s>>>(xp, wp, bias, M, K, E, logits);
    }
    if (xq) quant_rows_vec_kernel<<<M, 256, 0, s>>>(xp, M, K, xq, xscale);
}

void launch_router_topk(float* logits, int M, int E, int topk, int32_t* ids, float* w,
                        const double* lpart, int nks, const float* bias, hipStream_t s) {
    const int grid = (M + 3) / 4;
    router_topk_kernel<<<grid, 256, 0, s>>>(logits, M, E, topk, ids, w, lpart, nks, bias);
}

void launch_quant_rows(const void* x, int M, int K, uint8_t* q, float* scale, hipStream_t s) {
    if (K % 8 == 0) {
        quant_rows_vec_kernel<<<M, 256, 0, s>>>((const uint16_t*)x, M, K, q, scale);
    } else {
        const int grid = (M + 3) / 4;
        quant_rows_kernel<<<grid, 256, 0, s>>>((const uint16_t*)x, M, K, q, scale);
    }
}

}  // namespace moe
