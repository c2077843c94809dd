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
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Logits.  One wave computes a TT-token x TE-expert tile: its 64 lanes split
// K into 8-element slices, each lane accumulates bf16*bf16 products (exact in
// fp64) in fp64, and the tile is summed across lanes with DPP/ds_swizzle.
// ---------------------------------------------------------------------------
constexpr int kTT = 4;
constexpr int kTE = 4;

template <bool VEC>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int M, int K, int E, float* __restrict__ logits) {
    const int lane = lane_id();
    const int wave = (int)(blockIdx.x * 4 + threadIdx.x / kWave);
    const int tiles_e = (E + kTE - 1) / kTE;
    const int t0 = (wave / tiles_e) * kTT;
    const int e0 = (wave % tiles_e) * kTE;
    if (t0 >= M) return;  // wave-uniform

    double acc[kTT][kTE];
#pragma unroll
    for (int a = 0; a < kTT; ++a)
#pragma unroll
        for (int b = 0; b < kTE; ++b) acc[a][b] = 0.0;

    // Rows past M / E are clamped to a valid row; their sums are discarded.
    const uint16_t* xr[kTT];
    const uint16_t* wrr[kTE];
#pragma unroll
    for (int a = 0; a < kTT; ++a) xr[a] = x + (size_t)min(t0 + a, M - 1) * K;
#pragma unroll
    for (int b = 0; b < kTE; ++b) wrr[b] = wr + (size_t)min(e0 + b, E - 1) * K;

    if constexpr (VEC) {
        // K % 8 == 0: 16-byte loads, lane owns elements [k, k+8) of each row.
        for (int k = lane * 8; k < K; k += kWave * 8) {
            double xv[kTT][8], wv[kTE][8];
#pragma unroll
            for (int a = 0; a < kTT; ++a) {
                i32x4_t v = *reinterpret_cast<const i32x4_t*>(xr[a] + k);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xv[a][2 * q] = (double)bf16_bits_to_f32((uint32_t)v[q] & 0xffffu);
                    xv[a][2 * q + 1] = (double)bf16_bits_to_f32((uint32_t)v[q] >> 16);
                }
            }
#pragma unroll
            for (int b = 0; b < kTE; ++b) {
                i32x4_t v = *reinterpret_cast<const i32x4_t*>(wrr[b] + k);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    wv[b][2 * q] = (double)bf16_bits_to_f32((uint32_t)v[q] & 0xffffu);
                    wv[b][2 * q + 1] = (double)bf16_bits_to_f32((uint32_t)v[q] >> 16);
                }
            }
#pragma unroll
            for (int a = 0; a < kTT; ++a)
#pragma unroll
                for (int b = 0; b < kTE; ++b)
#pragma unroll
                    for (int q = 0; q < 8; ++q) acc[a][b] = __fma_rn(xv[a][q], wv[b][q], acc[a][b]);
        }
    } else {
        for (int k = lane; k < K; k += kWave) {
            double xv[kTT], wv[kTE];
#pragma unroll
            for (int a = 0; a < kTT; ++a) xv[a] = (double)bf16_bits_to_f32(xr[a][k]);
#pragma unroll
            for (int b = 0; b < kTE; ++b) wv[b] = (double)bf16_bits_to_f32(wrr[b][k]);
#pragma unroll
            for (int a = 0; a < kTT; ++a)
#pragma unroll
                for (int b = 0; b < kTE; ++b) acc[a][b] = __fma_rn(xv[a], wv[b], acc[a][b]);
        }
    }

#pragma unroll
    for (int a = 0; a < kTT; ++a)
#pragma unroll
        for (int b = 0; b < kTE; ++b) {
            double s = wave_sum_f64(acc[a][b]);
            const int t = t0 + a, e = e0 + b;
            if (lane == 0 && t < M && e < E) {
                if (bias) s += (double)bias[e];
                logits[(size_t)t * E + e] = (float)s;
            }
        }
}

// ---------------------------------------------------------------------------
// Top-k + weights (+ optional per-token e4m3 quantisation of x).  One wave per
// token.  Lane l holds logits of experts l, l+64, l+128, l+192.  A 64-bit key
// orders (logit, -expert): the high word maps the float to an unsigned with
// the same order, the low word is ~expert, so the wave max (DPP/ds_swizzle)
// is the largest logit with ties to the lower id.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ logits, int M, int E, int topk,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    const uint16_t* __restrict__ x, int K, uint8_t* __restrict__ xq,
    float* __restrict__ xscale) {
    const int lane = lane_id();
    const int t = (int)(blockIdx.x * 4 + threadIdx.x / kWave);
    if (t >= M) return;  // wave-uniform

    uint64_t key[4];
    float lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            lv[i] = logits[(size_t)t * E + e];
            key[i] = ((uint64_t)ordered_bits(lv[i]) << 32) | (uint32_t)(~(uint32_t)e);
        } else {
            lv[i] = 0.0f;
            key[i] = 0;
        }
    }

    float sel_l[MOE_KERNEL_MAX_TOPK];
    int sel_e[MOE_KERNEL_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_KERNEL_MAX_TOPK; ++j) {
        if (j >= topk) break;
        uint64_t best = max_u64(max_u64(key[0], key[1]), max_u64(key[2], key[3]));
        best = wave_max_u64(best);
        const int e = (int)(~(uint32_t)best);
        sel_e[j] = e;
        // the owning lane removes it and broadcasts its logit
        float l = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == e) { key[i] = 0; l = lv[i]; }
        sel_l[j] = __shfl(l, e & 63);
    }
    if (lane < topk) {
        // every lane holds the same sel_l[]; lane j writes slot j
        const float l0 = sel_l[0];
        float den = 0.0f, mine = 0.0f;
        int mye = 0;
#pragma unroll
        for (int j = 0; j < MOE_KERNEL_MAX_TOPK; ++j) {
            if (j >= topk) break;
            const float w = expf(sel_l[j] - l0);
            den += w;
            if (j == lane) { mine = w; mye = sel_e[j]; }
        }
        topk_ids[(size_t)t * topk + lane] = mye;
        topk_weights[(size_t)t * topk + lane] = mine / den;
    }

    if (xq) {
        // per-token dynamic e4m3: s = amax/448 (1 if amax == 0), code = E4M3(x/s)
        const uint16_t* xr = x + (size_t)t * K;
        uint32_t amax = 0;
        for (int k = lane; k < K; k += kWave) amax = max(amax, (uint32_t)xr[k] & 0x7fffu);
        amax = wave_max_bits(amax << 16);
        const float a = __uint_as_float(amax);
        const float s = (a == 0.0f) ? 1.0f : a / 448.0f;
        for (int k = lane; k < K; k += kWave)
            xq[(size_t)t * K + k] = (uint8_t)f32_to_e4m3(bf16_bits_to_f32(xr[k]) / s);
        if (lane == 0) xscale[t] = s;
    }
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
void launch_router_logits(const void* x, const void* wr, const float* bias, int M, int K, int E,
                          float* logits, hipStream_t s) {
    const long tiles = (long)((M + kTT - 1) / kTT) * ((E + kTE - 1) / kTE);
    const int grid = (int)((tiles + 3) / 4);
    if (K % 8 == 0)
        router_logits_kernel<true><<<grid, 256, 0, s>>>((const uint16_t*)x, (const uint16_t*)wr,
                                                         bias, M, K, E, logits);
    else
        router_logits_kernel<false><<<grid, 256, 0, s>>>((const uint16_t*)x, (const uint16_t*)wr,
                                                          bias, M, K, E, logits);
}

void launch_router_topk(const float* logits, int M, int E, int topk, int32_t* ids, float* w,
                        const void* x, int K, uint8_t* xq, float* xscale, hipStream_t s) {
    const int grid = (M + 3) / 4;
    router_topk_kernel<<<grid, 256, 0, s>>>(logits, M, E, topk, ids, w, (const uint16_t*)x, K,
                                            xq, xscale);
}

void launch_quant_rows(const void* x, int M, int K, uint8_t* q, float* scale, hipStream_t s) {
    const int grid = (M + 3) / 4;
    quant_rows_kernel<<<grid, 256, 0, s>>>((const uint16_t*)x, M, K, q, scale);
}

}  // namespace moe
