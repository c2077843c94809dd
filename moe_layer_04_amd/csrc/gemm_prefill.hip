// gemm_prefill.hip -- grouped expert GEMMs with full MFMA tiles, for many
// rows per expert.
//
// The fused MoE of "Mixture-of-Experts kernel engineering on Amazon
// SageMaker AI" (summary text) groups all active experts into one launch;
// with hundreds of token rows per expert the GEMMs are MFMA-bound, so each
// workgroup computes a full TW (weight rows) x 128 (token rows) tile from
// LDS with 32x32x16 bf16 MFMAs.  Weights stay in the pages' B^T layout
// (output-major, reduction dimension contiguous) on the MFMA row dimension,
// as in the decode kernels; tokens are the columns, gathered through the
// expert-sorted row list for GEMM1 and contiguous for GEMM2.
//
// Per workgroup (4 waves, 2x2): each wave owns TW/2 weight rows x 64 token
// columns, i.e. (TW/64) x 2 MFMA tiles of 32x32.  In GEMM1 the workgroup's
// weight rows are TW/2 gate rows followed by the matching TW/2 up rows and
// each wave takes the same n-range from both halves, so SiLU(gate)*up is
// formed from its own accumulators.
//
// Staging: K advances BK at a time through two LDS buffers.  Each step
// issues the next step's global loads (buffer loads into registers), runs
// the MFMAs of the current buffer, writes the registers into the other
// buffer and meets the workgroup at one barrier.  LDS rows are padded by
// 16 bytes so the 32 rows one MFMA operand read touches fall in distinct
// banks.  Padding token rows (sentinels) load token row 0 for GEMM1 / their
// own in-bounds act row for GEMM2: an MFMA output column depends only on its
// own B column, and those columns are never stored.
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

constexpr int kPreRows = 128;  // token rows per block (the align block size)
constexpr int kGroup = 8;

typedef __amdgpu_buffer_rsrc_t prsrc_t;

__device__ __forceinline__ prsrc_t pmake_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8_t pload(prsrc_t r, uint32_t off) {
    return (bf16x8_t)__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
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

// The shared main loop.  wrow_off(q) / xrow_off(q): byte offsets (at k = 0)
// of the rows this thread stages; FW = A tiles per wave (TW/64).
template <int TW, int BK>
struct PrefillCore {
    static constexpr int kStride = BK + 8;                 // bf16 per LDS row
    static constexpr int kWChunks = TW * BK / 8 / 256;     // 16-B chunks per thread (weights)
    static constexpr int kXChunks = kPreRows * BK / 8 / 256;
    static constexpr int kCPR = BK / 8;                    // chunks per row
    static constexpr int FW = TW / 64;
    static constexpr int kLdsW = TW * kStride;
    static constexpr int kLdsX = kPreRows * kStride;
    static constexpr int kLdsBytes = 2 * (kLdsW + kLdsX) * 2;

    f32x16_t acc[FW][2];

    __device__ __forceinline__ void run(uint16_t* lds, prsrc_t rw, const uint32_t* woff,
                                        prsrc_t rx, const uint32_t* xoff, int K, int wa, int wb,
                                        const int* arow) {
        const int tid = (int)threadIdx.x;
        const int lane = lane_id();
#pragma unroll
        for (int a = 0; a < FW; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

        int wl[kWChunks], xl[kXChunks];
#pragma unroll
        for (int q = 0; q < kWChunks; ++q) {
            const int c = tid + 256 * q;
            wl[q] = (c / kCPR) * kStride + (c % kCPR) * 8;
        }
#pragma unroll
        for (int q = 0; q < kXChunks; ++q) {
            const int c = tid + 256 * q;
            xl[q] = (c / kCPR) * kStride + (c % kCPR) * 8;
        }
        bf16x8_t rw_[kWChunks], rx_[kXChunks];
        auto gload = [&](int k) {
            const uint32_t kb = (uint32_t)k * 2;
#pragma unroll
            for (int q = 0; q < kWChunks; ++q) rw_[q] = pload(rw, woff[q] + kb);
#pragma unroll
            for (int q = 0; q < kXChunks; ++q) rx_[q] = pload(rx, xoff[q] + kb);
        };
        auto lstore = [&](int buf) {
            uint16_t* sw = lds + buf * (kLdsW + kLdsX);
            uint16_t* sx = sw + kLdsW;
#pragma unroll
            for (int q = 0; q < kWChunks; ++q) *reinterpret_cast<bf16x8_t*>(sw + wl[q]) = rw_[q];
#pragma unroll
            for (int q = 0; q < kXChunks; ++q) *reinterpret_cast<bf16x8_t*>(sx + xl[q]) = rx_[q];
        };
        const int li = lane & 31, lk = (lane >> 5) * 8;
        int ar[FW];
#pragma unroll
        for (int a = 0; a < FW; ++a) ar[a] = (arow[a] + li) * kStride + lk;
        const int xb0 = (wb * 64 + li) * kStride + lk;
        const int xb1 = xb0 + 32 * kStride;
        auto compute = [&](int buf) {
            const uint16_t* sw = lds + buf * (kLdsW + kLdsX);
            const uint16_t* sx = sw + kLdsW;
#pragma unroll
            for (int ks = 0; ks < BK; ks += 16) {
                bf16x8_t av[FW];
#pragma unroll
                for (int a = 0; a < FW; ++a)
                    av[a] = *reinterpret_cast<const bf16x8_t*>(sw + ar[a] + ks);
                const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(sx + xb0 + ks);
                const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(sx + xb1 + ks);
#pragma unroll
                for (int a = 0; a < FW; ++a) {
                    acc[a][0] = mfma32_bf16(av[a], b0, acc[a][0]);
                    acc[a][1] = mfma32_bf16(av[a], b1, acc[a][1]);
                }
            }
        };

        const int steps = K / BK;
        gload(0);
        lstore(0);
        __syncthreads();
        for (int s = 0; s + 1 < steps; ++s) {
            gload((s + 1) * BK);
            // keep the next step's loads ahead of this step's MFMAs (the
            // scheduler would otherwise sink them to just before their use)
            __builtin_amdgcn_sched_barrier(0);
            compute(s & 1);
            lstore((s + 1) & 1);
            __syncthreads();
        }
        compute((steps - 1) & 1);
#pragma unroll
        for (int a = 0; a < FW; ++a) {
            pin(acc[a][0]);
            pin(acc[a][1]);
        }
    }
};

// ---------------------------------------------------------------------------
// GEMM1 + SiLU*up (bf16).  Weight tile wt covers n in [wt*TW/2, (wt+1)*TW/2):
// LDS weight rows [0,TW/2) are those gate rows, [TW/2,TW) the up rows.
// ---------------------------------------------------------------------------
template <int TW, int BK>
__global__ __launch_bounds__(256, 2) void gemm1_prefill_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int M, int topk, int nslots, int K, int N,
    int max_blocks, uint16_t* __restrict__ act) {
    using Core = PrefillCore<TW, BK>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[Core::kLdsBytes / 2];
    constexpr int HW = TW / 2;  // n-values per tile

    int wt, blk;
    if (!tile_of((int)blockIdx.x, N / HW, max_blocks, wt, blk)) return;
    if (blk * kPreRows >= *num_padded) return;
    const int e = block_expert[blk];
    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wa = wave & 1, wb = wave >> 1;

    const size_t row_bytes = (size_t)K * 2;
    const prsrc_t rw = pmake_rsrc(w1 + (size_t)e * 2 * N * K, (uint32_t)(2 * (size_t)N * row_bytes));
    const prsrc_t rx = pmake_rsrc(x, (uint32_t)((size_t)M * row_bytes));
    uint32_t woff[Core::kWChunks], xoff[Core::kXChunks];
#pragma unroll
    for (int q = 0; q < Core::kWChunks; ++q) {
        const int c = tid + 256 * q;
        const int row = c / Core::kCPR, col = (c % Core::kCPR) * 8;
        const int wrow = (row < HW) ? (wt * HW + row) : (N + wt * HW + row - HW);
        woff[q] = (uint32_t)(wrow * row_bytes) + col * 2;
    }
#pragma unroll
    for (int q = 0; q < Core::kXChunks; ++q) {
        const int c = tid + 256 * q;
        const int row = c / Core::kCPR, col = (c % Core::kCPR) * 8;
        const int p = sorted_ids[blk * kPreRows + row];
        const int t = p < nslots ? p / topk : 0;
        xoff[q] = (uint32_t)(t * row_bytes) + col * 2;
    }
    // A tiles of this wave: gate frags then the matching up frags
    int arow[Core::FW];
#pragma unroll
    for (int a = 0; a < Core::FW / 2; ++a) {
        arow[a] = wa * (HW / 2) + a * 32;
        arow[a + Core::FW / 2] = HW + wa * (HW / 2) + a * 32;
    }
    Core core;
    core.run(lds, rw, woff, rx, xoff, K, wa, wb, arow);

    const int li = lane & 31;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int r = blk * kPreRows + wb * 64 + b * 32 + li;
        if (sorted_ids[r] >= nslots) continue;
#pragma unroll
        for (int a = 0; a < Core::FW / 2; ++a) {
            uint16_t* dst = act + (size_t)r * N + wt * HW + wa * (HW / 2) + a * 32 + 4 * (lane >> 5);
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                u16x4_t o;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    o[v] = f32_to_bf16_bits(silu(core.acc[a][b][vg * 4 + v]) *
                                            core.acc[a + Core::FW / 2][b][vg * 4 + v]);
                *reinterpret_cast<u16x4_t*>(dst + 8 * vg) = o;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// GEMM2 (bf16): weight tile wt covers output rows wt*TW..+TW; the epilogue
// multiplies by the routing weight and scatters token row r to slot p.
// ---------------------------------------------------------------------------
template <int TW, int BK>
__global__ __launch_bounds__(256, 2) void gemm2_prefill_bf16_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int cap,
    int nslots, int K, int N, int max_blocks, float* __restrict__ ypart) {
    using Core = PrefillCore<TW, BK>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[Core::kLdsBytes / 2];

    int wt, blk;
    if (!tile_of((int)blockIdx.x, K / TW, max_blocks, wt, blk)) return;
    if (blk * kPreRows >= *num_padded) return;
    const int e = block_expert[blk];
    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wa = wave & 1, wb = wave >> 1;

    const size_t row_bytes = (size_t)N * 2;
    const prsrc_t rw = pmake_rsrc(w2 + ((size_t)e * K + (size_t)wt * TW) * N,
                                  (uint32_t)(TW * row_bytes));
    const prsrc_t ra = pmake_rsrc(act, (uint32_t)((size_t)cap * row_bytes));
    uint32_t woff[Core::kWChunks], aoff[Core::kXChunks];
#pragma unroll
    for (int q = 0; q < Core::kWChunks; ++q) {
        const int c = tid + 256 * q;
        woff[q] = (uint32_t)((c / Core::kCPR) * row_bytes) + (c % Core::kCPR) * 16;
    }
#pragma unroll
    for (int q = 0; q < Core::kXChunks; ++q) {
        const int c = tid + 256 * q;
        const int r = blk * kPreRows + c / Core::kCPR;
        aoff[q] = (uint32_t)(r * row_bytes) + (c % Core::kCPR) * 16;
    }
    int arow[Core::FW];
#pragma unroll
    for (int a = 0; a < Core::FW; ++a) arow[a] = wa * (TW / 2) + a * 32;
    Core core;
    core.run(lds, rw, woff, ra, aoff, N, wa, wb, arow);

    const int li = lane & 31;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int r = blk * kPreRows + wb * 64 + b * 32 + li;
        const int p = sorted_ids[r];
        if (p >= nslots) continue;
        const float w = topk_w[p];
#pragma unroll
        for (int a = 0; a < Core::FW; ++a) {
            float* dst = ypart + (size_t)p * K + wt * TW + wa * (TW / 2) + a * 32 + 4 * (lane >> 5);
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                f32x4_t o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = core.acc[a][b][vg * 4 + v] * w;
                *reinterpret_cast<f32x4_t*>(dst + 8 * vg) = o;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
static int grid_for(int tiles) { return (tiles + 7) / 8 * 8; }

constexpr int kG1TW = 256, kG1BK = 32;
constexpr int kG2BK = 32;

void launch_gemm1_prefill_bf16(const void* x, const void* w1, const int32_t* sorted_ids,
                               const int32_t* block_expert, const int32_t* num_padded, int M,
                               int topk, int nslots, int K, int N, int max_blocks, void* act,
                               hipStream_t s) {
    const int grid = grid_for((N / (kG1TW / 2)) * max_blocks);
    gemm1_prefill_bf16_kernel<kG1TW, kG1BK><<<grid, 256, 0, s>>>(
        (const uint16_t*)x, (const uint16_t*)w1, sorted_ids, block_expert, num_padded, M, topk,
        nslots, K, N, max_blocks, (uint16_t*)act);
}

void launch_gemm2_prefill_bf16(const void* act, const void* w2, const float* topk_w,
                               const int32_t* sorted_ids, const int32_t* block_expert,
                               const int32_t* num_padded, int cap, int nslots, int K, int N,
                               int max_blocks, float* ypart, hipStream_t s) {
    if (K % 256 == 0) {
        const int grid = grid_for((K / 256) * max_blocks);
        gemm2_prefill_bf16_kernel<256, kG2BK><<<grid, 256, 0, s>>>(
            (const uint16_t*)act, (const uint16_t*)w2, topk_w, sorted_ids, block_expert,
            num_padded, cap, nslots, K, N, max_blocks, ypart);
    } else {
        const int grid = grid_for((K / 128) * max_blocks);
        gemm2_prefill_bf16_kernel<128, kG2BK><<<grid, 256, 0, s>>>(
            (const uint16_t*)act, (const uint16_t*)w2, topk_w, sorted_ids, block_expert,
            num_padded, cap, nslots, K, N, max_blocks, ypart);
    }
}

}  // namespace moe
