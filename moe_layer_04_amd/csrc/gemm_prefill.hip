// gemm_prefill.hip -- grouped expert GEMMs with full MFMA tiles, for many
// rows per expert.
//
// The fused MoE of "Mixture-of-Experts kernel engineering on Amazon
// SageMaker AI" (summary text) groups all active experts into one launch;
// with hundreds of token rows per expert the GEMMs are MFMA-bound, so each
// workgroup computes a full 128 (weight rows) x 128 (token rows) tile from
// LDS with 32x32x16 bf16 MFMAs.  Weights stay as the pages' B^T layout
// (output-major, reduction dimension contiguous) and sit on the MFMA row
// dimension as in the decode kernels; tokens are the columns, gathered
// through the expert-sorted row list for GEMM1 and contiguous for GEMM2.
//
// Per workgroup (4 waves, 2x2): each wave owns 64 weight rows x 64 token
// columns = 2x2 MFMA tiles of 32x32.  In GEMM1 the workgroup's 128 weight
// rows are 64 gate rows and the matching 64 up rows, and each wave takes 32
// of each, so SiLU(gate)*up is formed from its own accumulators.
//
// Staging: K advances 64 at a time; the next stage's global loads are issued
// into registers before the current stage's MFMAs and written to LDS after
// them.  LDS rows are padded by 16 bytes to spread banks.
//
// Tile order: the linear workgroup id is dealt to the 8 XCDs round-robin by
// the hardware; each XCD is given a contiguous range of tiles, and tiles are
// numbered so that a run of consecutive ids covers kGroup weight tiles for
// successive token blocks, so workgroups resident on one XCD share both
// operands in its L2.
//
// 32x32x16 layouts (gfx950): lane l supplies row/column (l % 32) with the
// K-slice 8*(l/32)..+8 for both operands; the accumulator lane l holds
// D[8*(v/4) + 4*(l/32) + v%4][l % 32], v = 0..15.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kPreRows = 128;     // token rows per block (the align block size)
constexpr int kBK = 64;           // K per LDS stage
constexpr int kLdsStride = kBK + 8;  // bf16 elements per LDS row
constexpr int kGroup = 8;

__device__ __forceinline__ f32x16_t mfma32_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Map the linear workgroup id to (weight tile, token block); false if idle.
__device__ __forceinline__ bool tile_of(int g, int n_wtiles, int n_blocks, int& wt, int& blk) {
    const int total = n_wtiles * n_blocks;
    const int per_xcd = (total + 7) / 8;
    const int t = (g % 8) * per_xcd + g / 8;
    if (t >= total) return false;
    const int span = kGroup * n_blocks;
    const int grp = t / span;
    const int in = t % span;
    const int gsize = min(kGroup, n_wtiles - grp * kGroup);
    wt = grp * kGroup + in % gsize;
    blk = in / gsize;
    return true;
}

// ---------------------------------------------------------------------------
// GEMM1 + SiLU*up (bf16).  Weight tile wt covers gate rows wt*64..+64 and up
// rows N+wt*64..+64.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm1_prefill_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int topk, int nslots, int K, int N, int max_blocks,
    uint16_t* __restrict__ act) {
    __shared__ __attribute__((aligned(16))) uint16_t sW[kPreRows * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t sX[kPreRows * kLdsStride];

    int wt, blk;
    if (!tile_of((int)blockIdx.x, N / 64, max_blocks, wt, blk)) return;
    if (blk * kPreRows >= *num_padded) return;
    const int e = block_expert[blk];
    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int wa = wave & 1, wb = wave >> 1;

    // global -> LDS assignment: 4 chunks of 16 B per operand per thread
    const uint16_t* wsrc[4];
    const uint16_t* xsrc[4];
    bool xval[4];
    int lds_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = tid + 256 * q;
        const int row = c >> 3, col = (c & 7) * 8;
        lds_off[q] = row * kLdsStride + col;
        const int wrow = (row < 64) ? (wt * 64 + row) : (N + wt * 64 + row - 64);
        wsrc[q] = w1 + ((size_t)e * 2 * N + wrow) * K + col;
        const int p = sorted_ids[blk * kPreRows + row];
        xval[q] = p < nslots;
        xsrc[q] = x + (size_t)(xval[q] ? p / topk : 0) * K + col;
    }

    bf16x8_t rw[4], rx[4];
    auto gload = [&](int k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            rw[q] = *reinterpret_cast<const bf16x8_t*>(wsrc[q] + k);
            rx[q] = xval[q] ? *reinterpret_cast<const bf16x8_t*>(xsrc[q] + k) : bf16x8_t{};
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<bf16x8_t*>(sW + lds_off[q]) = rw[q];
            *reinterpret_cast<bf16x8_t*>(sX + lds_off[q]) = rx[q];
        }
    };

    f32x16_t accg[2], accu[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) { accg[b][v] = 0.0f; accu[b][v] = 0.0f; }

    const int li = lane & 31, lk = (lane >> 5) * 8;
    const int ga = (wa * 32 + li) * kLdsStride + lk;        // gate rows of this wave
    const int ua = (64 + wa * 32 + li) * kLdsStride + lk;   // matching up rows
    const int xb0 = (wb * 64 + li) * kLdsStride + lk;
    const int xb1 = (wb * 64 + 32 + li) * kLdsStride + lk;

    gload(0);
    lstore();
    __syncthreads();
    for (int k = 0; k < K; k += kBK) {
        const bool more = k + kBK < K;
        if (more) gload(k + kBK);
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 16) {
            const bf16x8_t ag = *reinterpret_cast<const bf16x8_t*>(sW + ga + ks);
            const bf16x8_t au = *reinterpret_cast<const bf16x8_t*>(sW + ua + ks);
            const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(sX + xb0 + ks);
            const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(sX + xb1 + ks);
            accg[0] = mfma32_bf16(ag, b0, accg[0]);
            accu[0] = mfma32_bf16(au, b0, accu[0]);
            accg[1] = mfma32_bf16(ag, b1, accg[1]);
            accu[1] = mfma32_bf16(au, b1, accu[1]);
        }
        __syncthreads();
        if (more) {
            lstore();
            __syncthreads();
        }
    }

    // epilogue: lane holds token column li of each 32-col sub-tile and, for
    // each v-group, 4 consecutive n
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int r = blk * kPreRows + wb * 64 + b * 32 + li;
        if (sorted_ids[r] >= nslots) continue;
        uint16_t* dst = act + (size_t)r * N + wt * 64 + wa * 32 + 4 * (lane >> 5);
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
            u16x4_t o;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                o[v] = f32_to_bf16_bits(silu(accg[b][vg * 4 + v]) * accu[b][vg * 4 + v]);
            *reinterpret_cast<u16x4_t*>(dst + 8 * vg) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// GEMM2 (bf16): weight tile wt covers output rows wt*128..+128; epilogue
// multiplies by the routing weight and scatters token row r to slot p.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm2_prefill_bf16_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    int nslots, int K, int N, int max_blocks, float* __restrict__ ypart) {
    __shared__ __attribute__((aligned(16))) uint16_t sW[kPreRows * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t sX[kPreRows * kLdsStride];

    int wt, blk;
    if (!tile_of((int)blockIdx.x, K / 128, max_blocks, wt, blk)) return;
    if (blk * kPreRows >= *num_padded) return;
    const int e = block_expert[blk];
    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int wa = wave & 1, wb = wave >> 1;

    const uint16_t* wsrc[4];
    const uint16_t* asrc[4];
    bool aval[4];
    int lds_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = tid + 256 * q;
        const int row = c >> 3, col = (c & 7) * 8;
        lds_off[q] = row * kLdsStride + col;
        wsrc[q] = w2 + ((size_t)e * K + wt * 128 + row) * N + col;
        const int r = blk * kPreRows + row;
        aval[q] = sorted_ids[r] < nslots;
        asrc[q] = act + (size_t)r * N + col;
    }

    bf16x8_t rw[4], ra[4];
    auto gload = [&](int n) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            rw[q] = *reinterpret_cast<const bf16x8_t*>(wsrc[q] + n);
            ra[q] = aval[q] ? *reinterpret_cast<const bf16x8_t*>(asrc[q] + n) : bf16x8_t{};
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<bf16x8_t*>(sW + lds_off[q]) = rw[q];
            *reinterpret_cast<bf16x8_t*>(sX + lds_off[q]) = ra[q];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

    const int li = lane & 31, lk = (lane >> 5) * 8;
    const int wa0 = (wa * 64 + li) * kLdsStride + lk;
    const int wa1 = (wa * 64 + 32 + li) * kLdsStride + lk;
    const int xb0 = (wb * 64 + li) * kLdsStride + lk;
    const int xb1 = (wb * 64 + 32 + li) * kLdsStride + lk;

    gload(0);
    lstore();
    __syncthreads();
    for (int n = 0; n < N; n += kBK) {
        const bool more = n + kBK < N;
        if (more) gload(n + kBK);
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 16) {
            const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(sW + wa0 + ks);
            const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(sW + wa1 + ks);
            const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(sX + xb0 + ks);
            const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(sX + xb1 + ks);
            acc[0][0] = mfma32_bf16(a0, b0, acc[0][0]);
            acc[1][0] = mfma32_bf16(a1, b0, acc[1][0]);
            acc[0][1] = mfma32_bf16(a0, b1, acc[0][1]);
            acc[1][1] = mfma32_bf16(a1, b1, acc[1][1]);
        }
        __syncthreads();
        if (more) {
            lstore();
            __syncthreads();
        }
    }

#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int r = blk * kPreRows + wb * 64 + b * 32 + li;
        const int p = sorted_ids[r];
        if (p >= nslots) continue;
        const float w = topk_w[p];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            float* dst = ypart + (size_t)p * K + wt * 128 + wa * 64 + a * 32 + 4 * (lane >> 5);
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                f32x4_t o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = acc[a][b][vg * 4 + v] * w;
                *reinterpret_cast<f32x4_t*>(dst + 8 * vg) = o;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
static int grid_for(int tiles) { return (tiles + 7) / 8 * 8; }

void launch_gemm1_prefill_bf16(const void* x, const void* w1, const int32_t* sorted_ids,
                               const int32_t* block_expert, const int32_t* num_padded, int topk,
                               int nslots, int K, int N, int max_blocks, void* act,
                               hipStream_t s) {
    const int grid = grid_for((N / 64) * max_blocks);
    gemm1_prefill_bf16_kernel<<<grid, 256, 0, s>>>((const uint16_t*)x, (const uint16_t*)w1,
                                                   sorted_ids, block_expert, num_padded, topk,
                                                   nslots, K, N, max_blocks, (uint16_t*)act);
}

void launch_gemm2_prefill_bf16(const void* act, const void* w2, const float* topk_w,
                               const int32_t* sorted_ids, const int32_t* block_expert,
                               const int32_t* num_padded, int nslots, int K, int N,
                               int max_blocks, float* ypart, hipStream_t s) {
    const int grid = grid_for((K / 128) * max_blocks);
    gemm2_prefill_bf16_kernel<<<grid, 256, 0, s>>>((const uint16_t*)act, (const uint16_t*)w2,
                                                   topk_w, sorted_ids, block_expert, num_padded,
                                                   nslots, K, N, max_blocks, ypart);
}

}  // namespace moe
