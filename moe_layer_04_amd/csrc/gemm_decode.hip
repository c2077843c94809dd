// gemm_decode.hip -- grouped expert GEMMs for few rows per expert, with the
// operands swapped (Swap-AB) so that expert weight rows, not tokens, sit on
// the MFMA row dimension.
//
// "Mixture-of-Experts kernel engineering on Amazon SageMaker AI" (summary
// text, decode-phase passage and Figure 1): in decode the token matrix is a
// thin 1..64-row block while the expert weights are a large dense block, so
// the product is computed as C^T[N,M] = B^T[N,K].A^T[K,M], with the large
// weight dimension in the fixed-height operand slot; the weights, held as
// B^T (output-major, reduction dimension contiguous), then stream as large
// contiguous blocks.  On gfx950 the MFMA row dimension is 16 (not Hopper's
// 64), so the swap wastes at most 15 of 16 token columns while every byte of
// weights read from HBM feeds a full MFMA row.  The weights are loaded from
// HBM straight into registers, 16 contiguous bytes per lane, two K-steps in
// flight per wave; decode is bound by that HBM stream.
//
// Work split: one workgroup (4 waves) per (16-row block of one expert,
// tile of weight rows).  GEMM1 waves own 16 gate rows and the matching 16
// up rows, so SiLU(gate)*up is formed in registers (the fused epilogue);
// GEMM2 waves own 32 output rows and may split the reduction (N) across
// workgroups, writing fp32 partial rows scattered back to slot order and
// already multiplied by the routing weight.
//
// MFMA operand layout used (16x16 family): lane l supplies row (l % 16) of
// the A tile and column (l % 16) of the B tile, each with a K-slice chosen
// by l / 16; A and B use the same K-slice assignment, so the sum over K is
// the full dot product whatever order the hardware adds the slices in.  The
// accumulator lane l holds D[4*(l/16) + v][l % 16], v = 0..3.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kDecRows = 16;  // token rows per block (the align block size)

__device__ __forceinline__ bf16x8_t ld16(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8_t*>(p);
}
__device__ __forceinline__ i32x8_t ld32(const uint8_t* p) {
    return *reinterpret_cast<const i32x8_t*>(p);
}

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// e4m3 x e4m3, block scales fixed at 2^0 (E8M0 code 127).
__device__ __forceinline__ f32x4_t mfma_fp8(i32x8_t a, i32x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------------------
// GEMM1 + SiLU*up, bf16.  grid = (N/64, blocks); wave w of workgroup x owns
// gate rows n0..n0+15 with n0 = (4x + w)*16 and up rows N+n0..N+n0+15.
// ---------------------------------------------------------------------------
struct FragBf16G1 {
    bf16x8_t g[4], u[4], b[4];
};

__global__ __launch_bounds__(256) void gemm1_decode_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int topk, int nslots, int K, int N,
    uint16_t* __restrict__ act) {
    const int blk = (int)blockIdx.y;
    if (blk * kDecRows >= *num_padded) return;
    const int e = block_expert[blk];
    const int lane = lane_id();
    const int wave = (int)threadIdx.x / kWave;
    const int n0 = ((int)blockIdx.x * 4 + wave) * 16;
    const int i = lane & 15, kq = lane >> 4;
    const int p = sorted_ids[blk * kDecRows + i];
    const bool valid = p < nslots;
    const uint16_t* xr = x + (size_t)(valid ? p / topk : 0) * K + kq * 8;
    const uint16_t* gr = w1 + ((size_t)e * 2 * N + n0 + i) * K + kq * 8;
    const uint16_t* ur = gr + (size_t)N * K;

    auto load = [&](FragBf16G1& f, int k) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f.g[s] = ld16(gr + k + s * 32);
            f.u[s] = ld16(ur + k + s * 32);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) f.b[s] = valid ? ld16(xr + k + s * 32) : bf16x8_t{};
    };

    f32x4_t accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
    FragBf16G1 cur, nxt;
    load(cur, 0);
    for (int k = 0; k < K; k += 128) {
        const bool more = k + 128 < K;
        if (more) load(nxt, k + 128);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            accg = mfma_bf16(cur.g[s], cur.b[s], accg);
            accu = mfma_bf16(cur.u[s], cur.b[s], accu);
        }
        if (more) cur = nxt;
    }

    if (valid) {
        u16x4_t o;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = f32_to_bf16_bits(silu(accg[v]) * accu[v]);
        *reinterpret_cast<u16x4_t*>(act + (size_t)(blk * kDecRows + i) * N + n0 + 4 * kq) = o;
    }
}

// ---------------------------------------------------------------------------
// GEMM2 (down projection), bf16.  grid = (K/128, blocks, nsplit); wave w of
// workgroup x owns output rows c0..c0+31, c0 = (4x + w)*32, over the
// reduction range [z*N/nsplit, (z+1)*N/nsplit).
// ---------------------------------------------------------------------------
struct FragBf16G2 {
    bf16x8_t a0[4], a1[4], b[4];
};

__global__ __launch_bounds__(256) void gemm2_decode_bf16_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    int nslots, int K, int N, int nsplit, float* __restrict__ ypart) {
    const int blk = (int)blockIdx.y;
    if (blk * kDecRows >= *num_padded) return;
    const int e = block_expert[blk];
    const int lane = lane_id();
    const int wave = (int)threadIdx.x / kWave;
    const int c0 = ((int)blockIdx.x * 4 + wave) * 32;
    const int i = lane & 15, kq = lane >> 4;
    const int z = (int)blockIdx.z;
    const int nlen = N / nsplit;
    const int nbeg = z * nlen;
    const int p = sorted_ids[blk * kDecRows + i];
    const bool valid = p < nslots;
    const uint16_t* ar = act + (size_t)(blk * kDecRows + i) * N + nbeg + kq * 8;
    const uint16_t* w0 = w2 + ((size_t)e * K + c0 + i) * N + nbeg + kq * 8;
    const uint16_t* w1r = w0 + (size_t)16 * N;

    auto load = [&](FragBf16G2& f, int n) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f.a0[s] = ld16(w0 + n + s * 32);
            f.a1[s] = ld16(w1r + n + s * 32);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) f.b[s] = valid ? ld16(ar + n + s * 32) : bf16x8_t{};
    };

    f32x4_t acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    FragBf16G2 cur, nxt;
    load(cur, 0);
    for (int n = 0; n < nlen; n += 128) {
        const bool more = n + 128 < nlen;
        if (more) load(nxt, n + 128);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            acc0 = mfma_bf16(cur.a0[s], cur.b[s], acc0);
            acc1 = mfma_bf16(cur.a1[s], cur.b[s], acc1);
        }
        if (more) cur = nxt;
    }

    if (valid) {
        const float w = topk_w[p];
        float* yr = ypart + ((size_t)z * nslots + p) * K + c0 + 4 * kq;
        *reinterpret_cast<f32x4_t*>(yr) = acc0 * w;
        *reinterpret_cast<f32x4_t*>(yr + 16) = acc1 * w;
    }
}

// ---------------------------------------------------------------------------
// FP8 (OCP e4m3) versions.  One 16x16x128 MFMA consumes 32 codes per lane.
// GEMM1 applies s_x[t] * w1_scale[e] to the fp32 accumulators, forms
// SiLU*up in fp32, stores it and folds each row's |act| max into amax[r]
// (float bits, atomicMax: exact and order-free for non-negative floats).
// ---------------------------------------------------------------------------
struct FragFp8G1 {
    i32x8_t g[2], u[2], b[2];
};

__global__ __launch_bounds__(256) void gemm1_decode_fp8_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xscale,
    const uint8_t* __restrict__ w1, const float* __restrict__ w1_scale,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int topk, int nslots, int K, int N,
    float* __restrict__ act, uint32_t* __restrict__ amax) {
    const int blk = (int)blockIdx.y;
    if (blk * kDecRows >= *num_padded) return;
    const int e = block_expert[blk];
    const int lane = lane_id();
    const int wave = (int)threadIdx.x / kWave;
    const int n0 = ((int)blockIdx.x * 4 + wave) * 16;
    const int i = lane & 15, kq = lane >> 4;
    const int p = sorted_ids[blk * kDecRows + i];
    const bool valid = p < nslots;
    const int t = valid ? p / topk : 0;
    const uint8_t* xr = xq + (size_t)t * K + kq * 32;
    const uint8_t* gr = w1 + ((size_t)e * 2 * N + n0 + i) * K + kq * 32;
    const uint8_t* ur = gr + (size_t)N * K;

    // K is a multiple of 128; a step covers two 128-code chunks, and the
    // second chunk is neither loaded nor used past the end of the row.
    const int ksteps = K / 128;
    auto load = [&](FragFp8G1& f, int c) {
        const int k = c * 128;
        const bool two = c + 1 < ksteps;
        f.g[0] = ld32(gr + k);
        f.u[0] = ld32(ur + k);
        f.g[1] = two ? ld32(gr + k + 128) : i32x8_t{};
        f.u[1] = two ? ld32(ur + k + 128) : i32x8_t{};
        f.b[0] = valid ? ld32(xr + k) : i32x8_t{};
        f.b[1] = (valid && two) ? ld32(xr + k + 128) : i32x8_t{};
    };

    f32x4_t accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
    FragFp8G1 cur, nxt;
    load(cur, 0);
    for (int c = 0; c < ksteps; c += 2) {
        const bool more = c + 2 < ksteps;
        if (more) load(nxt, c + 2);
        accg = mfma_fp8(cur.g[0], cur.b[0], accg);
        accu = mfma_fp8(cur.u[0], cur.b[0], accu);
        if (c + 1 < ksteps) {
            accg = mfma_fp8(cur.g[1], cur.b[1], accg);
            accu = mfma_fp8(cur.u[1], cur.b[1], accu);
        }
        if (more) cur = nxt;
    }

    float m = 0.0f;
    f32x4_t o;
    if (valid) {
        const float sc = xscale[t] * w1_scale[e];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            o[v] = silu(accg[v] * sc) * (accu[v] * sc);
            m = fmaxf(m, fabsf(o[v]));
        }
        *reinterpret_cast<f32x4_t*>(act + (size_t)(blk * kDecRows + i) * N + n0 + 4 * kq) = o;
    }
    const uint32_t mb = col_max_bits(__float_as_uint(m));
    if (valid && kq == 0) atomicMax(amax + blk * kDecRows + i, mb);
}

// act32 [cap,N] + amax [cap] -> act_q [cap,N] e4m3 and s_a [cap]; one wave per row.
__global__ __launch_bounds__(256) void act_quant_kernel(
    const float* __restrict__ act, const uint32_t* __restrict__ amax,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ num_padded, int nslots,
    int N, uint8_t* __restrict__ act_q, float* __restrict__ ascale) {
    const int r = (int)(blockIdx.x * 4 + threadIdx.x / kWave);
    if (r >= *num_padded) return;
    if (sorted_ids[r] >= nslots) return;
    const int lane = lane_id();
    const float a = __uint_as_float(amax[r]);
    const float s = (a == 0.0f) ? 1.0f : a / 448.0f;
    const float* src = act + (size_t)r * N;
    uint8_t* dst = act_q + (size_t)r * N;
    for (int n = lane * 4; n < N; n += kWave * 4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + n);
        const uint32_t q = f32_to_e4m3(v[0] / s) | (f32_to_e4m3(v[1] / s) << 8) |
                           (f32_to_e4m3(v[2] / s) << 16) | (f32_to_e4m3(v[3] / s) << 24);
        *reinterpret_cast<uint32_t*>(dst + n) = q;
    }
    if (lane == 0) ascale[r] = s;
}

struct FragFp8G2 {
    i32x8_t a0[2], a1[2], b[2];
};

__global__ __launch_bounds__(256) void gemm2_decode_fp8_kernel(
    const uint8_t* __restrict__ act_q, const float* __restrict__ ascale,
    const uint8_t* __restrict__ w2, const float* __restrict__ w2_scale,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    int nslots, int K, int N, int nsplit, float* __restrict__ ypart) {
    const int blk = (int)blockIdx.y;
    if (blk * kDecRows >= *num_padded) return;
    const int e = block_expert[blk];
    const int lane = lane_id();
    const int wave = (int)threadIdx.x / kWave;
    const int c0 = ((int)blockIdx.x * 4 + wave) * 32;
    const int i = lane & 15, kq = lane >> 4;
    const int z = (int)blockIdx.z;
    const int nlen = N / nsplit;
    const int nbeg = z * nlen;
    const int r = blk * kDecRows + i;
    const int p = sorted_ids[r];
    const bool valid = p < nslots;
    const uint8_t* ar = act_q + (size_t)r * N + nbeg + kq * 32;
    const uint8_t* w0 = w2 + ((size_t)e * K + c0 + i) * N + nbeg + kq * 32;
    const uint8_t* w1r = w0 + (size_t)16 * N;

    const int nsteps = nlen / 128;
    auto load = [&](FragFp8G2& f, int c) {
        const int n = c * 128;
        const bool two = c + 1 < nsteps;
        f.a0[0] = ld32(w0 + n);
        f.a1[0] = ld32(w1r + n);
        f.a0[1] = two ? ld32(w0 + n + 128) : i32x8_t{};
        f.a1[1] = two ? ld32(w1r + n + 128) : i32x8_t{};
        f.b[0] = valid ? ld32(ar + n) : i32x8_t{};
        f.b[1] = (valid && two) ? ld32(ar + n + 128) : i32x8_t{};
    };

    f32x4_t acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    FragFp8G2 cur, nxt;
    load(cur, 0);
    for (int c = 0; c < nsteps; c += 2) {
        const bool more = c + 2 < nsteps;
        if (more) load(nxt, c + 2);
        acc0 = mfma_fp8(cur.a0[0], cur.b[0], acc0);
        acc1 = mfma_fp8(cur.a1[0], cur.b[0], acc1);
        if (c + 1 < nsteps) {
            acc0 = mfma_fp8(cur.a0[1], cur.b[1], acc0);
            acc1 = mfma_fp8(cur.a1[1], cur.b[1], acc1);
        }
        if (more) cur = nxt;
    }

    if (valid) {
        const float w = topk_w[p] * ascale[r] * w2_scale[e];
        float* yr = ypart + ((size_t)z * nslots + p) * K + c0 + 4 * kq;
        *reinterpret_cast<f32x4_t*>(yr) = acc0 * w;
        *reinterpret_cast<f32x4_t*>(yr + 16) = acc1 * w;
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
void launch_gemm1_decode_bf16(const void* x, const void* w1, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded, int topk,
                              int nslots, int K, int N, int max_blocks, void* act,
                              hipStream_t s) {
    dim3 grid(N / 64, max_blocks);
    gemm1_decode_bf16_kernel<<<grid, 256, 0, s>>>((const uint16_t*)x, (const uint16_t*)w1,
                                                  sorted_ids, block_expert, num_padded, topk,
                                                  nslots, K, N, (uint16_t*)act);
}

void launch_gemm2_decode_bf16(const void* act, const void* w2, const float* topk_w,
                              const int32_t* sorted_ids, const int32_t* block_expert,
                              const int32_t* num_padded, int nslots, int K, int N, int nsplit,
                              int max_blocks, float* ypart, hipStream_t s) {
    dim3 grid(K / 128, max_blocks, nsplit);
    gemm2_decode_bf16_kernel<<<grid, 256, 0, s>>>((const uint16_t*)act, (const uint16_t*)w2,
                                                  topk_w, sorted_ids, block_expert, num_padded,
                                                  nslots, K, N, nsplit, ypart);
}

void launch_gemm1_decode_fp8(const uint8_t* xq, const float* xscale, const void* w1,
                             const float* w1_scale, const int32_t* sorted_ids,
                             const int32_t* block_expert, const int32_t* num_padded, int topk,
                             int nslots, int K, int N, int max_blocks, float* act,
                             uint32_t* amax, hipStream_t s) {
    dim3 grid(N / 64, max_blocks);
    gemm1_decode_fp8_kernel<<<grid, 256, 0, s>>>(xq, xscale, (const uint8_t*)w1, w1_scale,
                                                 sorted_ids, block_expert, num_padded, topk,
                                                 nslots, K, N, act, amax);
}

void launch_act_quant(const float* act, const uint32_t* amax, const int32_t* sorted_ids,
                      const int32_t* num_padded, int nslots, int N, int cap, uint8_t* act_q,
                      float* ascale, hipStream_t s) {
    act_quant_kernel<<<(cap + 3) / 4, 256, 0, s>>>(act, amax, sorted_ids, num_padded, nslots, N,
                                                   act_q, ascale);
}

void launch_gemm2_decode_fp8(const uint8_t* act_q, const float* ascale, const void* w2,
                             const float* w2_scale, const float* topk_w,
                             const int32_t* sorted_ids, const int32_t* block_expert,
                             const int32_t* num_padded, int nslots, int K, int N, int nsplit,
                             int max_blocks, float* ypart, hipStream_t s) {
    dim3 grid(K / 128, max_blocks, nsplit);
    gemm2_decode_fp8_kernel<<<grid, 256, 0, s>>>(act_q, ascale, (const uint8_t*)w2, w2_scale,
                                                 topk_w, sorted_ids, block_expert, num_padded,
                                                 nslots, K, N, nsplit, ypart);
}

}  // namespace moe
