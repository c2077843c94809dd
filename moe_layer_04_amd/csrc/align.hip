// align.hip -- moe_align on gfx950: the expert-sorted, block-padded
// permutation of token slots ("data shuffling" of the fused MoE in
// "Mixture-of-Experts kernel engineering on Amazon SageMaker AI", summary
// text; per-expert batch sizes that change from call to call, "Amazon
// SageMaker AI上的混合专家模型内核工程优化", H200 bottleneck section).
//
// Slot p = t*topk + j is sorted stably by expert; each expert's segment is
// padded to a multiple of the block size with the sentinel n = M*topk.
// One 1024-thread workgroup: an LDS histogram, a wave prefix scan of the
// padded counts, then the slots in chunks of 1024 in ascending p.  Inside a
// chunk, each lane's rank among earlier lanes of the same expert comes from
// 8 ballots over the bits of the expert id (a wave-level match) plus the
// per-wave counts of earlier waves, so the order never depends on atomics.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int n, int E, int B, int cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ num_padded,
    uint32_t* __restrict__ zero_buf, int zero_words) {
    __shared__ int cnt[MOE_KERNEL_MAX_EXPERTS];
    __shared__ int off[MOE_KERNEL_MAX_EXPERTS + 1];
    __shared__ int run[MOE_KERNEL_MAX_EXPERTS];
    __shared__ int wc[kAlignWaves][MOE_KERNEL_MAX_EXPERTS];

    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;

    // optional: clear a caller buffer (the fused path's per-row amax)
    for (int i = tid; i < zero_words; i += kAlignThreads) zero_buf[i] = 0u;

    for (int e = tid; e < E; e += kAlignThreads) { cnt[e] = 0; run[e] = 0; }
    __syncthreads();
    for (int p = tid; p < n; p += kAlignThreads) {
        const int e = min(max(ids[p], 0), E - 1);
        atomicAdd(&cnt[e], 1);  // counts are order-free
    }
    __syncthreads();

    // exclusive scan of padded counts over E <= 256 experts: wave 0, 4 per lane
    if (wave == 0) {
        int v[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            v[i] = (e < E) ? (cnt[e] + B - 1) / B * B : 0;
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
            if (e < E) off[e] = base;
            base += v[i];
        }
        if (lane == kWave - 1) off[E] = incl;
    }
    __syncthreads();

    for (int e = tid; e <= E; e += kAlignThreads) expert_offsets[e] = off[e];
    if (tid == 0) *num_padded = off[E];
    const int npad = off[E];

    // sentinels: padding inside a segment and everything past npad
    for (int i = tid; i < cap; i += kAlignThreads) {
        bool pad = (i >= npad);
        if (!pad) {
            int lo = 0, hi = E - 1;  // last e with off[e] <= i
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= i) lo = mid; else hi = mid - 1;
            }
            pad = (i - off[lo]) >= cnt[lo];
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
                if (off[mid] <= i) lo = mid; else hi = mid - 1;
            }
            owner = lo;
        }
        block_expert[b] = owner;
    }

    // stable scatter in chunks of 1024 slots
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < n; base += kAlignThreads) {
        for (int i = tid; i < kAlignWaves * MOE_KERNEL_MAX_EXPERTS; i += kAlignThreads)
            (&wc[0][0])[i] = 0;
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
        if (valid && (match >> lane) == 1ull) wc[wave][e] = __popcll(match);  // last lane of its group
        __syncthreads();
        if (valid) {
            int before = 0;
            for (int w = 0; w < wave; ++w) before += wc[w][e];
            sorted_ids[off[e] + run[e] + before + rank] = p;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kAlignThreads) {
            int s = 0;
            for (int w = 0; w < kAlignWaves; ++w) s += wc[w][x];
            run[x] += s;
        }
        __syncthreads();
    }
}

void launch_align(const int32_t* ids, int n, int E, int B, int cap, int32_t* sorted_ids,
                  int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded,
                  uint32_t* zero_buf, int zero_words, hipStream_t s) {
    align_kernel<<<1, kAlignThreads, 0, s>>>(ids, n, E, B, cap, sorted_ids, block_expert,
                                             expert_offsets, num_padded, zero_buf, zero_words);
}

}  // namespace moe
