// decode_fused.hip -- router, top-k, align and GEMM1 + SiLU*up of one or two
// tokens (bf16 weights) in one launch.
//
// "Amazon SageMaker AI上的混合专家模型内核工程优化" (H200 bottleneck section)
// names kernel-launch overhead among the costs of MoE decode, and
// "AI混合专家模型性能优化全链路解析" (§3.1) fuses work at expert granularity to
// cut launches.  With one or two tokens the layer is a pure weight stream
// (the 1x4096 . 4096x8192 expert GEMM of "Mixture-of-Experts kernel
// engineering on Amazon SageMaker AI", decode-phase passage): the router's
// own launches (logits, then top-k + align) leave HBM idle for their whole
// duration.  Here every workgroup computes the router itself -- the logits
// of every (token, expert) pair as fp64 dot products rounded once to fp32,
// then the top-k in one wave -- so no workgroup waits for another, and
// workgroup (c, a) streams the gate and up rows of n-chunk c of the a-th
// routed expert (ascending id) exactly as gemm1_decode_bf16_kernel does
// (Swap-AB: weight rows on the 16-row MFMA dimension, the expert's token
// slots on the columns), writing SiLU*up as bf16 to the sorted activation
// rows.  Workgroup 0 also stores the logits, top-k ids and weights and the
// expert-sorted permutation (align_wave, 16-row blocks: with at most 16
// slots per expert the a-th routed expert owns block a), which the decode
// GEMM2 and the combine then read as in the five-launch sequence.
#include "routing.hpp"
#include "tuning.hpp"

namespace moe {

constexpr int kFusedChunk = 64;       // intermediate (n) columns per workgroup
constexpr int kFusedMaxTokens = 2;
constexpr int kFusedMaxPairs = tune::kFusedDecodeMaxPairs;
constexpr uint32_t kFusedOob = 0x80000000u;  // past every buffer: loads return 0
constexpr int kFusedRot = 7;                 // GEMM1 K-step rotation per wave
constexpr int kFusedSliceGroup = 8;         // router: row slices loaded together
constexpr int kFusedExpertGroup = 4;        // router: expert rows of a wave in flight
constexpr int kFusedMaxBlocks = 4;          // routed experts (16-row blocks) of the layer
// GEMM2 + combine: waves splitting N (8 when N % 1024 == 0: single-token
// decode, 1 x 4096 and 4096 x 8192 experts, 78.3-78.6 against 79.9 us per
// layer call with 4).  Both kernels stream with two fragments (the next
// step's loads issued before the current step's MFMAs); rotations of 3 or 4
// fragments with the loads of 2 or 3 steps in flight measured slower on
// that shape: routing GEMM1 57.4 (3) and 57.5 (4) against 54.5 us, GEMM2
// 35.3 (3) and 48.9 (4, spilling) against 28.3 us.

typedef __amdgpu_buffer_rsrc_t frsrc_t;

__device__ __forceinline__ frsrc_t fmake_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ i32x4_t fload(frsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ f32x4_t fmfma(i32x4_t a, i32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8_t)a, (bf16x8_t)b, c, 0, 0, 0);
}

// MT tokens (1 or 2); grid = (N / kFusedChunk) * min(E, MT*topk) workgroups
// of 4 waves; K % 512 == 0, N % kFusedChunk == 0.  act [cap, N] bf16 in sorted-row order
// (block size 16); the align outputs as align_wave writes them.
template <int MT>
__global__ __launch_bounds__(256) void decode_route_gemm1_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, const uint16_t* __restrict__ w1, int K, int N,
    int E, int topk, int cap, float* __restrict__ logits_out, int32_t* __restrict__ ids_out,
    float* __restrict__ wts_out, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ num_padded, uint16_t* __restrict__ act) {
    __shared__ double part[MT][MOE_KERNEL_MAX_EXPERTS];
    __shared__ float lg[kFusedMaxPairs];
    __shared__ int32_t sid[kWave];
    __shared__ float swt[kWave];
    __shared__ int blk_e, blk_cnt;
    __shared__ int blk_slot[16];
    __shared__ int acnt[MOE_KERNEL_MAX_EXPERTS];
    __shared__ int aoff[MOE_KERNEL_MAX_EXPERTS + 1];

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int nchunks = N / kFusedChunk;
    constexpr int M = MT;
    const int a = (int)blockIdx.x / nchunks;  // routed expert, by ascending id (its block)
    const int c = (int)blockIdx.x % nchunks;  // chunk of the intermediate dimension
    const int nslots = M * topk;

    // ---- router logits: wave w takes experts w, w+4, ..., kFusedExpertGroup
    // at a time; each lane accumulates the bf16*bf16 products (exact in
    // fp64) of its 8-element slices k = 8*lane + 512*j in fp64 with all the
    // group's row loads in flight together, and a DPP wave sum finishes each
    // dot product; part[t][e] then gets the bias and one fp32 rounding.
    {
        const int nsl = K / (kWave * 8);  // 8-element slices per lane (K % 512 == 0)
        for (int e0 = wave; e0 < E; e0 += 4 * kFusedExpertGroup) {
            double acc[kFusedExpertGroup][MT];
#pragma unroll
            for (int u = 0; u < kFusedExpertGroup; ++u)
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[u][t] = 0.0;
            for (int j0 = 0; j0 < nsl; j0 += kFusedSliceGroup) {
                i32x4_t wv[kFusedExpertGroup][kFusedSliceGroup];
                i32x4_t xv[MT][kFusedSliceGroup];
#pragma unroll
                for (int jj = 0; jj < kFusedSliceGroup; ++jj) {
                    const int k = (j0 + jj) * 512 + lane * 8;
                    const bool in = j0 + jj < nsl;
#pragma unroll
                    for (int u = 0; u < kFusedExpertGroup; ++u) {
                        const int e = e0 + 4 * u;
                        wv[u][jj] = (in && e < E)
                                        ? *reinterpret_cast<const i32x4_t*>(wr + (size_t)e * K + k)
                                        : i32x4_t{0, 0, 0, 0};
                    }
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        xv[t][jj] = in ? *reinterpret_cast<const i32x4_t*>(x + (size_t)t * K + k)
                                       : i32x4_t{0, 0, 0, 0};
                }
#pragma unroll
                for (int jj = 0; jj < kFusedSliceGroup; ++jj)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int t = 0; t < MT; ++t) {
                            const uint32_t xa = (uint32_t)xv[t][jj][q];
                            const double x_lo = (double)bf16_bits_to_f32(xa & 0xffffu);
                            const double x_hi = (double)bf16_bits_to_f32(xa >> 16);
#pragma unroll
                            for (int u = 0; u < kFusedExpertGroup; ++u) {
                                const uint32_t wa = (uint32_t)wv[u][jj][q];
                                acc[u][t] = __fma_rn(x_lo, (double)bf16_bits_to_f32(wa & 0xffffu),
                                                     acc[u][t]);
                                acc[u][t] = __fma_rn(x_hi, (double)bf16_bits_to_f32(wa >> 16),
                                                     acc[u][t]);
                            }
                        }
            }
#pragma unroll
            for (int u = 0; u < kFusedExpertGroup; ++u)
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const double sum = wave_sum_f64(acc[u][t]);
                    const int e = e0 + 4 * u;
                    if (lane == 0 && e < E) part[t][e] = sum;
                }
        }
    }
    __syncthreads();
    for (int i = (int)threadIdx.x; i < M * E; i += 256) {
        double s = part[i / E][i % E];
        if (bias) s += (double)bias[i % E];
        lg[i] = (float)s;
        if (blockIdx.x == 0) logits_out[i] = (float)s;
    }
    __syncthreads();

    // ---- top-k per token, then this workgroup's expert and its slots
    if (wave == 0) {
        for (int t = 0; t < M; ++t)
            topk_wave(lg + t * E, E, topk, sid + t * topk, swt + t * topk, nullptr);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
        __builtin_amdgcn_wave_barrier();
        const bool valid = lane < nslots;
        const int my = valid ? sid[lane] : 0x7fffffff;
        if (blockIdx.x == 0 && valid) {
            ids_out[lane] = my;
            wts_out[lane] = swt[lane];
        }
        // first occurrence of its expert, and the column = earlier slots of it
        bool first = valid;
        int col = 0;
        for (int q = 0; q < nslots; ++q) {
            const int o = __shfl(my, q);
            if (q < lane && o == my) { first = false; ++col; }
        }
        // rank of the expert among the distinct routed experts
        int rk = 0;
        for (int q = 0; q < nslots; ++q) {
            const int o = __shfl(my, q);
            const int fq = __shfl((int)first, q);
            if (fq && o < my) ++rk;
        }
        const uint64_t hit = __ballot(valid && first && rk == a);
        const int ea = hit ? __shfl(my, __builtin_ctzll(hit)) : -1;
        const bool mine = valid && my == ea;
        if (mine && col < 16) blk_slot[col] = lane;
        const int cnt = __popcll(__ballot(mine));
        if (lane == 0) {
            blk_e = ea;
            blk_cnt = cnt;
        }
        if (blockIdx.x == 0)
            align_wave(sid, nslots, E, 16, cap, acnt, aoff, sorted_ids, block_expert,
                       expert_offsets, num_padded, nullptr, 0, nullptr);
    }
    __syncthreads();
    const int e = blk_e;
    if (e < 0) return;  // fewer routed experts than expert slots of the grid
    const int cnt = blk_cnt;

    const int i = lane & 15, kq = lane >> 4;

    // ---- GEMM1 + SiLU*up: wave w owns gate rows n0..n0+15 and up rows N+n0..
    const int n0 = c * kFusedChunk + wave * 16;
    const size_t row1 = (size_t)K * 2;
    const frsrc_t rg = fmake_rsrc(w1 + ((size_t)e * 2 * N + n0) * K, (uint32_t)(16 * row1));
    const frsrc_t ru = fmake_rsrc(w1 + ((size_t)e * 2 * N + N + n0) * K, (uint32_t)(16 * row1));
    const frsrc_t rx = fmake_rsrc(x, (uint32_t)((size_t)M * row1));
    const uint32_t wo = (uint32_t)(i * row1) + kq * 16;
    const int slot_i = i < cnt ? blk_slot[i] : -1;
    const uint32_t xo = slot_i >= 0 ? (uint32_t)((size_t)slot_token(slot_i, topk) * row1) + kq * 16
                                    : kFusedOob;

    struct Frag { i32x4_t g[4], u[4], b[4]; };
    auto load1 = [&](Frag& f, int k) {
        const uint32_t kb = (uint32_t)k * 2;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f.g[s] = fload(rg, wo + kb + s * 64);
            f.u[s] = fload(ru, wo + kb + s * 64);
            f.b[s] = fload(rx, xo + kb + s * 64);
        }
    };
    f32x4_t accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
    auto compute1 = [&](const Frag& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            accg = fmfma(f.g[s], f.b[s], accg);
            accu = fmfma(f.u[s], f.b[s], accu);
        }
    };
    const int nst = K / 128;
    const int gw = (int)blockIdx.x * 4 + wave;
    const int rot = (gw * kFusedRot) % nst;
    {
        Frag cur;
        int q = rot;
        load1(cur, q * 128);
        for (int j = 1; j < nst; ++j) {
            Frag nxt;
            q = q + 1 == nst ? 0 : q + 1;
            load1(nxt, q * 128);
            compute1(cur);
            cur = nxt;
        }
        compute1(cur);
    }
    pin(accg);
    pin(accu);

    // ---- SiLU*up of the valid columns to the sorted activation rows
    if (i < cnt) {
        u16x4_t o;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = f32_to_bf16_bits(silu(accg[v]) * accu[v]);
        *reinterpret_cast<u16x4_t*>(act + (size_t)(a * 16 + i) * N + n0 + 4 * kq) = o;
    }
}

// ---------------------------------------------------------------------------
// GEMM2 and the combine of one or two tokens in one launch: workgroup g owns
// output rows r0 = 16*g .. r0+15 of every routed expert (NB 16-row blocks of
// the sorted rows, block b owned by block_expert[b], -1 if unused); its
// kG2Waves waves split the reduction (N) into equal ranges and stream those
// rows of W2[e] against the block's activation rows (Swap-AB, as
// gemm2_decode_bf16_kernel).
// The wave partials meet in LDS, and out[t][r] = bf16( sum over the token's
// slots j in ascending order of w[t,j] * (sum over the waves in order of the
// partial of its block and column) ): a fixed order, and no partial rows
// leave the workgroup.
// ---------------------------------------------------------------------------
template <int MT, int NB, int kG2Waves>
__global__ __launch_bounds__(kG2Waves * 64) void decode_gemm2_combine_bf16_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, int K, int N, int topk, int cap,
    uint16_t* __restrict__ out) {
    __shared__ float red[kG2Waves][NB][16][17];  // [wave][block][row][column], padded
    __shared__ int spos[kWave];            // sorted row of each slot
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int nslots = MT * topk;
    const int r0 = (int)blockIdx.x * 16;
    const int i = lane & 15, kq = lane >> 4;
    const int nq = N / kG2Waves, nbeg = wave * nq;

    int eb[NB];
    bool vb[NB];
    uint32_t ao[NB];
    const size_t row_bytes = (size_t)N * 2;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        eb[b] = block_expert[b];
        const int p = sorted_ids[b * 16 + i];
        vb[b] = p < nslots;
        ao[b] = vb[b] ? (uint32_t)((size_t)(b * 16 + i) * row_bytes) + nbeg * 2 + kq * 16
                      : kFusedOob;
    }
    const frsrc_t ra = fmake_rsrc(act, (uint32_t)((size_t)cap * row_bytes));
    const uint32_t wo = (uint32_t)(i * row_bytes) + nbeg * 2 + kq * 16;
    frsrc_t rw[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
        rw[b] = fmake_rsrc(w2 + ((size_t)max(eb[b], 0) * K + r0) * N,
                           eb[b] >= 0 ? (uint32_t)(16 * row_bytes) : 0u);

    struct Frag { i32x4_t a[NB][4], b[NB][4]; };
    auto load = [&](Frag& f, int n) {
        const uint32_t nb = (uint32_t)n * 2;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                f.a[b][s] = fload(rw[b], wo + nb + s * 64);
                f.b[b][s] = fload(ra, ao[b] + nb + s * 64);
            }
    };
    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0, 0, 0, 0};
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = fmfma(f.a[b][s], f.b[b][s], acc[b]);
    };
    const int nst = nq / 128;
    const int rot = ((int)blockIdx.x * kFusedRot + wave * 3) % nst;
    {
        Frag cur;
        int q = rot;
        load(cur, q * 128);
        for (int j = 1; j < nst; ++j) {
            Frag nxt;
            q = q + 1 == nst ? 0 : q + 1;
            load(nxt, q * 128);
            compute(cur);
            cur = nxt;
        }
        compute(cur);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        pin(acc[b]);
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][b][4 * kq + v][i] = acc[b][v];
    }
    if (wave == 0) {
        // sorted row of every slot (the routed rows of the NB blocks)
        for (int r = lane; r < NB * 16; r += kWave) {
            const int p = sorted_ids[r];
            if (p < nslots) spos[p] = r;
        }
    }
    __syncthreads();
    const int tid = (int)threadIdx.x;
    if (tid < MT * 16) {
        const int t = tid / 16, row = tid % 16;
        float y = 0.0f;
        for (int j = 0; j < topk; ++j) {
            const int p = t * topk + j;
            const int r = spos[p];
            const int b = r / 16, col = r % 16;
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kG2Waves; ++w) s += red[w][b][row][col];
            y += topk_w[p] * s;
        }
        out[(size_t)t * K + r0 + row] = f32_to_bf16_bits(y);
    }
}

bool decode_fused_fits(int M, int K, int N, int E, int topk) {
    // the router takes K in 512-element slices; every workgroup computes all
    // M*E router logits; each routed expert owns one 16-row block, and the
    // GEMM2 + combine keeps at most kFusedMaxBlocks of them in flight; its
    // waves take N in 128-element steps of quarters
    return M >= 1 && M <= kFusedMaxTokens && K % 512 == 0 && N % 512 == 0 &&
           M * E <= tune::kFusedDecodeMaxPairs && min(E, M * topk) <= kFusedMaxBlocks;
}

void launch_decode_route_gemm1_bf16(const void* x, const void* wr, const float* bias,
                                    const void* w1, int M, int K, int N, int E, int topk, int cap,
                                    float* logits, int32_t* ids, float* wts, int32_t* sorted_ids,
                                    int32_t* block_expert, int32_t* expert_offsets,
                                    int32_t* num_padded, void* act, hipStream_t s) {
    const int blocks = min(E, M * topk) * (N / kFusedChunk);
#define MOE_RG1(MT)                                                                        \
    decode_route_gemm1_bf16_kernel<MT><<<blocks, 256, 0, s>>>(                             \
        (const uint16_t*)x, (const uint16_t*)wr, bias, (const uint16_t*)w1, K, N, E, topk, \
        cap, logits, ids, wts, sorted_ids, block_expert, expert_offsets, num_padded,       \
        (uint16_t*)act)
    if (M == 2) MOE_RG1(2);
    else MOE_RG1(1);
#undef MOE_RG1
}

void launch_decode_gemm2_combine_bf16(const void* act, const void* w2, const float* topk_w,
                                      const int32_t* sorted_ids, const int32_t* block_expert,
                                      int M, int K, int N, int E, int topk, int cap, void* out,
                                      hipStream_t s) {
    const int nb = min(E, M * topk);
#define MOE_G2C(MT, NB)                                                                      \
    do {                                                                                     \
        if (N % 1024 == 0)                                                                   \
            decode_gemm2_combine_bf16_kernel<MT, NB, 8><<<K / 16, 512, 0, s>>>(              \
                (const uint16_t*)act, (const uint16_t*)w2, topk_w, sorted_ids, block_expert, \
                K, N, topk, cap, (uint16_t*)out);                                            \
        else                                                                                 \
            decode_gemm2_combine_bf16_kernel<MT, NB, 4><<<K / 16, 256, 0, s>>>(              \
                (const uint16_t*)act, (const uint16_t*)w2, topk_w, sorted_ids, block_expert, \
                K, N, topk, cap, (uint16_t*)out);                                            \
    } while (0)
    if (M == 2) {
        if (nb <= 2) MOE_G2C(2, 2);
        else MOE_G2C(2, 4);
    } else {
        if (nb <= 1) MOE_G2C(1, 1);
        else if (nb <= 2) MOE_G2C(1, 2);
        else MOE_G2C(1, 4);
    }
#undef MOE_G2C
}

}  // namespace moe
