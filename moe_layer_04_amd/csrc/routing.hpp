// routing.hpp -- device pieces of the MoE routing shared by the separate
// router / align kernels and the single-workgroup routing kernel for small
// batches: the top-k selection of one token by one wave, the per-token e4m3
// quantisation of one row by one wave, and the body of the expert-sorted
// permutation (moe_align) run by a 1024-thread workgroup.
//
// Readings (see the kernels' headers for the citations): a logit is the fp32
// rounding of the fp64-accumulated dot product (+ bias); the k largest logits
// are picked in descending order with ties to the lower expert id; the
// weights are the softmax over the picked logits; slot p = t*topk + j is
// sorted stably by expert, each expert's segment padded to a multiple of the
// block size with the sentinel n = M*topk.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;

// ---------------------------------------------------------------------------
// top-k of one token
// ---------------------------------------------------------------------------

// float -> unsigned with the same order (-0 and +0 equal)
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave selects the topk largest of the E <= 256 logits in `row` (lane l
// holds experts l, l+64, l+128, l+192).  A 64-bit key orders (logit,
// -expert): the high word is the ordered float, the low word ~expert, so the
// wave max (DPP/ds_swizzle) is the largest logit with ties to the lower id.
// Lane j < topk writes slot j: ids_out[j], w_out[j] and, when ids_copy is
// not null, ids_copy[j].  Wave-uniform call.
__device__ __forceinline__ void topk_wave(const float* row, int E, int topk,
                                          int32_t* __restrict__ ids_out,
                                          float* __restrict__ w_out, int32_t* ids_copy) {
    const int lane = lane_id();
    uint64_t key[4];
    float lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            lv[i] = row[e];
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
        ids_out[lane] = mye;
        w_out[lane] = mine / den;
        if (ids_copy) ids_copy[lane] = mye;
    }
}

// The same selection and weights for E <= 16 experts with one token per
// 16-lane row of the wave (four tokens at once): lane r of a row holds
// expert r of its token, and the row max takes only the four in-row
// exchange steps of the wave max.  Rows whose `valid` is false take no part
// in any write.  ids, weights and arithmetic are those of topk_wave.
// Wave-uniform call.
__device__ __forceinline__ void topk_row16(const float* row, bool valid, int E, int topk,
                                           int32_t* __restrict__ ids_out,
                                           float* __restrict__ w_out) {
    const int lane = lane_id();
    const int r = lane & 15;
    float lv = 0.0f;
    uint64_t key = 0;
    if (valid && r < E) {
        lv = row[r];
        key = ((uint64_t)ordered_bits(lv) << 32) | (uint32_t)(~(uint32_t)r);
    }
    float sel_l[MOE_KERNEL_MAX_TOPK];
    int sel_e[MOE_KERNEL_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_KERNEL_MAX_TOPK; ++j) {
        if (j >= topk) break;
        uint64_t best = key;
        best = max_u64(best, xchg_u64<0>(best));
        best = max_u64(best, xchg_u64<1>(best));
        best = max_u64(best, xchg_u64<2>(best));
        best = max_u64(best, xchg_u64<3>(best));
        const int e = (int)(~(uint32_t)best) & 15;
        sel_e[j] = e;
        float l = 0.0f;
        if (r == e) { key = 0; l = lv; }
        sel_l[j] = __shfl(l, (lane & ~15) | e);
    }
    if (valid && r < topk) {
        const float l0 = sel_l[0];
        float den = 0.0f, mine = 0.0f;
        int mye = 0;
#pragma unroll
        for (int j = 0; j < MOE_KERNEL_MAX_TOPK; ++j) {
            if (j >= topk) break;
            const float w = expf(sel_l[j] - l0);
            den += w;
            if (j == r) { mine = w; mye = sel_e[j]; }
        }
        ids_out[r] = mye;
        w_out[r] = mine / den;
    }
}

// ---------------------------------------------------------------------------
// one router logit, one e4m3 row
// ---------------------------------------------------------------------------

// Per-token dynamic e4m3 quantisation of one bf16 row (K % 8 == 0) by one
// wave: s = amax/448 (1 if amax == 0), code = E4M3(x/s) with one correctly
// rounded fp32 division.  Lane 0 writes the scale.
__device__ __forceinline__ void quant_row_wave(const uint16_t* row, int K, uint8_t* dst,
                                               float* scale_out) {
    const int lane = lane_id();
    uint32_t amax = 0;
    for (int k = lane * 8; k < K; k += kWave * 8) {
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(row + k);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            amax = max(amax, max((uint32_t)v[u] & 0x7fffu, ((uint32_t)v[u] >> 16) & 0x7fffu));
    }
    amax = wave_max_bits(amax << 16);
    const float am = __uint_as_float(amax);
    const float sc = (am == 0.0f) ? 1.0f : am / 448.0f;
    for (int k = lane * 8; k < K; k += kWave * 8) {
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
    if (lane == 0) *scale_out = sc;
}

// ---------------------------------------------------------------------------
// moe_align body
// ---------------------------------------------------------------------------

struct AlignShared {
    int cnt[MOE_KERNEL_MAX_EXPERTS];
    int off[MOE_KERNEL_MAX_EXPERTS + 1];
    int run[MOE_KERNEL_MAX_EXPERTS];
    int wc[kAlignWaves][MOE_KERNEL_MAX_EXPERTS];
};

// Run by all kAlignThreads threads of a workgroup.  ids may point to global
// or shared memory.  An LDS histogram, a wave prefix scan of the padded
// counts, then the slots in chunks of 1024 in ascending p.  Inside a chunk,
// each lane's rank among earlier lanes of the same expert comes from 8
// ballots over the bits of the expert id (a wave-level match) plus the
// per-wave counts of earlier waves, so the order never depends on atomics.
// zero_buf[0 .. zero_words) is cleared on the way (a caller buffer); with
// inv not null, inv[p] receives the sorted position of slot p.
__device__ __forceinline__ void align_body(AlignShared& sh, const int32_t* ids, int n, int E,
                                           int B, int cap, int32_t* __restrict__ sorted_ids,
                                           int32_t* __restrict__ block_expert,
                                           int32_t* __restrict__ expert_offsets,
                                           int32_t* __restrict__ num_padded,
                                           uint32_t* __restrict__ zero_buf, int zero_words,
                                           int32_t* __restrict__ inv) {
    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;

    for (int i = tid; i < zero_words; i += kAlignThreads) zero_buf[i] = 0u;

    for (int e = tid; e < E; e += kAlignThreads) { sh.cnt[e] = 0; sh.run[e] = 0; }
    __syncthreads();
    for (int p = tid; p < n; p += kAlignThreads) {
        const int e = min(max(ids[p], 0), E - 1);
        atomicAdd(&sh.cnt[e], 1);  // counts are order-free
    }
    __syncthreads();

    // exclusive scan of padded counts over E <= 256 experts: wave 0, 4 per lane
    if (wave == 0) {
        int v[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            v[i] = (e < E) ? (sh.cnt[e] + B - 1) / B * B : 0;
            sum += v[i];
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        int base = incl - sum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            if (e < E) sh.off[e] = base;
            base += v[i];
        }
        if (lane == kWave - 1) sh.off[E] = incl;
    }
    __syncthreads();

    for (int e = tid; e <= E; e += kAlignThreads) expert_offsets[e] = sh.off[e];
    if (tid == 0) *num_padded = sh.off[E];
    const int npad = sh.off[E];

    // sentinels: padding inside a segment and everything past npad
    for (int i = tid; i < cap; i += kAlignThreads) {
        bool pad = (i >= npad);
        if (!pad) {
            int lo = 0, hi = E - 1;  // last e with off[e] <= i
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sh.off[mid] <= i) lo = mid; else hi = mid - 1;
            }
            pad = (i - sh.off[lo]) >= sh.cnt[lo];
        }
        if (pad) sorted_ids[i] = n;
    }
    // block owners
    const int nblk = cap / B;
    for (int b = tid; b < nblk; b += kAlignThreads) {
        const int i = b * B;
        int owner = -1;
        if (i < npad) {
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sh.off[mid] <= i) lo = mid; else hi = mid - 1;
            }
            owner = lo;
        }
        block_expert[b] = owner;
    }

    // stable scatter in chunks of 1024 slots
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < n; base += kAlignThreads) {
        for (int i = tid; i < kAlignWaves * MOE_KERNEL_MAX_EXPERTS; i += kAlignThreads)
            (&sh.wc[0][0])[i] = 0;
        __syncthreads();
        const int p = base + tid;
        const bool valid = p < n;
        const int e = valid ? min(max(ids[p], 0), E - 1) : 0;
        uint64_t match = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bb = __ballot(valid && bit);
            match &= bit ? bb : ~bb;
        }
        const int rank = __popcll(match & lt_mask);
        if (valid && (match >> lane) == 1ull) sh.wc[wave][e] = __popcll(match);  // last lane of its group
        __syncthreads();
        if (valid) {
            int before = 0;
            for (int w = 0; w < wave; ++w) before += sh.wc[w][e];
            const int pos = sh.off[e] + sh.run[e] + before + rank;
            sorted_ids[pos] = p;
            if (inv) inv[p] = pos;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kAlignThreads) {
            int s = 0;
            for (int w = 0; w < kAlignWaves; ++w) s += sh.wc[w][x];
            sh.run[x] += s;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// The align of at most 64 slots by one wave (no workgroup barriers): lane p
// holds slot p of sid (LDS); an LDS histogram in cnt, the padded exclusive
// scan over the experts (four per lane) in off, then each slot's rank among
// earlier slots of its expert from 8 ballots over the expert-id bits.  The
// order is the stable one of align_body, so the results are identical.
// cnt [E] and off [E+1] are LDS arrays of the caller.  Wave-uniform call.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void align_wave(const int32_t* sid, int n, int E, int B, int cap,
                                           int* cnt, int* off, int32_t* __restrict__ sorted_ids,
                                           int32_t* __restrict__ block_expert,
                                           int32_t* __restrict__ expert_offsets,
                                           int32_t* __restrict__ num_padded,
                                           uint32_t* __restrict__ zero_buf, int zero_words,
                                           int32_t* __restrict__ inv) {
    const int lane = lane_id();
    for (int i = lane; i < zero_words; i += kWave) zero_buf[i] = 0u;
    for (int e = lane; e < E; e += kWave) cnt[e] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    const bool valid = lane < n;
    const int e = valid ? min(max(sid[lane], 0), E - 1) : 0;
    if (valid) atomicAdd(&cnt[e], 1);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
    {
        int v[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ex = lane * 4 + q;
            v[q] = (ex < E) ? (cnt[ex] + B - 1) / B * B : 0;
            sum += v[q];
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        int base = incl - sum;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ex = lane * 4 + q;
            if (ex < E) off[ex] = base;
            base += v[q];
        }
        if (lane == kWave - 1) off[E] = incl;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
    for (int ex = lane; ex <= E; ex += kWave) expert_offsets[ex] = off[ex];
    const int npad = off[E];
    if (lane == 0) *num_padded = npad;
    // sentinels: padding inside a segment and everything past npad
    for (int i = lane; i < cap; i += kWave) {
        bool pad = (i >= npad);
        if (!pad) {
            int lo = 0, hi = E - 1;  // last expert with off <= i
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= i) lo = mid; else hi = mid - 1;
            }
            pad = (i - off[lo]) >= cnt[lo];
        }
        if (pad) sorted_ids[i] = n;
    }
    for (int b = lane; b < cap / B; b += kWave) {
        const int i = b * B;
        int owner = -1;
        if (i < npad) {
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= i) lo = mid; else hi = mid - 1;
            }
            owner = lo;
        }
        block_expert[b] = owner;
    }
    // stable scatter: rank among the earlier slots of the same expert
    uint64_t match = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(valid && bit);
        match &= bit ? bb : ~bb;
    }
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (valid) {
        const int pos = off[e] + __popcll(match & lt_mask);
        sorted_ids[pos] = lane;
        if (inv) inv[lane] = pos;
    }
}

}  // namespace moe
