// launch.hpp -- host-side launchers of the layer's kernels (internal to the
// library; the public interface is include/moe.h).  Every launcher only
// enqueues on the given stream; shapes are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_KERNEL_MAX_EXPERTS 256
#define MOE_KERNEL_MAX_TOPK 16

namespace moe {
// token rows per block of the sorted list (the align block size) for the
// Swap-AB decode kernels and for the full-tile kernels
constexpr int kDecodeRows = 16;
constexpr int kPrefillRows = 256;
constexpr int kPrefillSmallRows = 128;  // full-tile blocks for few rows per expert
}

namespace moe {

// logits [M,E]; with xq/xscale non-null also the per-token e4m3 codes and
// scales (a second kernel; K % 8 == 0).  With nks > 1 (a value from
// router_logit_splits) the logits are left as nks fp64 partial sums in
// lpart [nks,M,E], which launch_router_topk (same nks, lpart and bias)
// turns into the logits before selecting.
int router_logit_splits(int M, int K, int E);
void launch_router_logits(const void* x, const void* wr, const float* bias, int M, int K, int E,
                          float* logits, uint8_t* xq, float* xscale, int nks, double* lpart,
                          hipStream_t s);
void launch_router_topk(float* logits, int M, int E, int topk, int32_t* ids, float* w,
                        const double* lpart, int nks, const float* bias, hipStream_t s);
void launch_quant_rows(const void* x, int M, int K, uint8_t* q, float* scale, hipStream_t s);

// inv (optional): inv[p] = sorted position of slot p
void launch_align(const int32_t* ids, int n, int E, int B, int cap, int32_t* sorted_ids,
                  int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded,
                  uint32_t* zero_buf, int zero_words, int32_t* inv, hipStream_t s);

// The align of launch_align over many workgroups (three launches, identical
// result) for batches of more than kAlignMultiMinSlots slots; scratch:
// chunk_cnt [align_chunks(n) * E] and cnt_total [E] int32.
constexpr int kAlignMultiMinSlots = 2048;
inline int align_chunks(int n) { return (n + 1023) / 1024; }
bool align_multi_fits(int n);
void launch_align_multi(const int32_t* ids, int n, int E, int B, int cap, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded,
                        uint32_t* zero_buf, int zero_words, int32_t* inv, int32_t* chunk_cnt,
                        int32_t* cnt_total, hipStream_t s);

// Top-k + align (and, with xq not null, the FP8 token codes; meant for a
// few tokens) in one single-workgroup launch, for at most kRouteSmallMaxTokens
// tokens and kRouteSmallMaxSlots token-slots.
constexpr int kRouteSmallMaxTokens = 64;
constexpr int kRouteSmallMaxSlots = 1024;
bool topk_align_fits(int M, int topk);
void launch_topk_align(const float* logits, const void* x, int M, int K, int E, int topk,
                       int32_t* ids, float* w, uint8_t* xq, float* xscale, int B, int cap,
                       int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                       int32_t* num_padded, uint32_t* zero_buf, int zero_words, int32_t* inv,
                       hipStream_t s);

void launch_gemm1_decode_bf16(const void* x, const void* w1, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded, int M,
                              int topk, int nslots, int K, int N, int max_blocks, int nt, void* act,
                              hipStream_t s);
void launch_gemm2_decode_bf16(const void* act, const void* w2, const float* topk_w,
                              const int32_t* sorted_ids, const int32_t* block_expert,
                              const int32_t* num_padded, int cap, int nslots, int K, int N,
                              int nsplit, int max_blocks, int nt, float* ypart, hipStream_t s);
// rowwise: w1_scale [E,2N] / w2_scale [E,K] (one per output row) instead of [E]
// nt: 16-row token tiles per block (1, 2 or 4; the align block size is 16*nt)
void launch_gemm1_decode_fp8(const uint8_t* xq, const float* xscale, const void* w1,
                             const float* w1_scale, int rowwise, const int32_t* sorted_ids,
                             const int32_t* block_expert, const int32_t* num_padded, int M,
                             int topk, int nslots, int K, int N, int max_blocks, int nt,
                             float* act, uint32_t* amax, hipStream_t s);
// rows of the nslots slots only: slot p is sorted row inv[p]
void launch_act_quant(const float* act, const uint32_t* amax, const int32_t* inv, int nslots,
                      int N, uint8_t* act_q, float* ascale, hipStream_t s);
void launch_gemm2_decode_fp8(const uint8_t* act_q, const float* ascale, const void* w2,
                             const float* w2_scale, int rowwise, const float* topk_w,
                             const int32_t* sorted_ids, const int32_t* block_expert,
                             const int32_t* num_padded, int cap, int nslots, int K, int N,
                             int nsplit, int max_blocks, int nt, float* ypart, hipStream_t s);

// MXFP4 weights: w1 [E,2N,K/2] / w2 [E,K,N/2] packed e2m1 with E8M0 scales
// w1e8 [E,2N,K/32] / w2e8 [E,K,N/32]; activations as the e4m3 path
void launch_gemm1_decode_mxfp4(const uint8_t* xq, const float* xscale, const void* w1,
                               const uint8_t* w1e8, const int32_t* sorted_ids,
                               const int32_t* block_expert, const int32_t* num_padded, int M,
                               int topk, int nslots, int K, int N, int max_blocks, int nt, float* act,
                               uint32_t* amax, hipStream_t s);
void launch_gemm2_decode_mxfp4(const uint8_t* act_q, const float* ascale, const void* w2,
                               const uint8_t* w2e8, const float* topk_w,
                               const int32_t* sorted_ids, const int32_t* block_expert,
                               const int32_t* num_padded, int cap, int nslots, int K, int N,
                               int nsplit, int max_blocks, int nt, float* ypart, hipStream_t s);

// Full tiles: tt = token rows per block, kPrefillRows or kPrefillSmallRows
// (the latter only with K % 256 == 0).
void launch_gemm1_prefill_bf16(const void* x, const void* w1, const int32_t* sorted_ids,
                               const int32_t* block_expert, const int32_t* num_padded, int M,
                               int topk, int nslots, int K, int N, int max_blocks, int tt,
                               void* act, hipStream_t s);
// reduction splits the full-tile GEMM2 uses for (K, N) over `blocks` token
// blocks, each split a multiple of `gran` reduction elements (the kernel's
// K-step: 64 bf16, 128 e4m3); its partial rows go to ypart[split] like the
// decode kernel's
int prefill_gemm2_splits(int K, int N, int blocks, int gran);
void launch_gemm2_prefill_bf16(const void* act, const void* w2, const float* topk_w,
                               const int32_t* sorted_ids, const int32_t* block_expert,
                               const int32_t* num_padded, int cap, int nslots, int K, int N,
                               int nsplit, int max_blocks, int tt, float* ypart, hipStream_t s);

// e4m3 weights on the full tiles (K % 128 == 0, N % 128 == 0; with nsplit
// > 1, (N / nsplit) % 128 == 0): GEMM1 writes the fp32 activation rows and
// their |act| maxima (amax cleared by the align step), GEMM2 reads act_q /
// ascale from launch_act_quant; scales as the decode FP8 kernels
void launch_gemm1_prefill_fp8(const uint8_t* xq, const float* xscale, const void* w1,
                              const float* w1_scale, int rowwise, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded, int M,
                              int topk, int nslots, int K, int N, int max_blocks, int tt,
                              float* act, uint32_t* amax, hipStream_t s);
void launch_gemm2_prefill_fp8(const uint8_t* act_q, const float* ascale, const void* w2,
                              const float* w2_scale, int rowwise, const float* topk_w,
                              const int32_t* sorted_ids, const int32_t* block_expert,
                              const int32_t* num_padded, int cap, int nslots, int K, int N,
                              int nsplit, int max_blocks, int tt, float* ypart, hipStream_t s);

// MXFP4 weights on the full tiles (256-row blocks only; K, N multiples of
// 256; with nsplit > 1, (N / nsplit) % 128 == 0): the activations as the
// e4m3 full tiles
void launch_gemm1_prefill_mx(const uint8_t* xq, const float* xscale, const void* w1,
                             const uint8_t* w1e8, const int32_t* sorted_ids,
                             const int32_t* block_expert, const int32_t* num_padded, int M,
                             int topk, int nslots, int K, int N, int max_blocks, float* act,
                             uint32_t* amax, hipStream_t s);
void launch_gemm2_prefill_mx(const uint8_t* act_q, const float* ascale, const void* w2,
                             const uint8_t* w2e8, const float* topk_w, const int32_t* sorted_ids,
                             const int32_t* block_expert, const int32_t* num_padded, int cap,
                             int nslots, int K, int N, int nsplit, int max_blocks, float* ypart,
                             hipStream_t s);

void launch_combine(const float* ypart, int M, int K, int topk, int nsplit, void* out,
                    hipStream_t s);

// Router (logits, top-k), align (16-row blocks) and GEMM1 + SiLU*up of one
// or two tokens with bf16 weights in one launch (decode_fused.hip): logits
// [M,E], ids / weights [M*topk], the align outputs and act [cap,N] bf16 as
// the separate launches write them.
bool decode_fused_fits(int M, int K, int N, int E, int topk);
void launch_decode_route_gemm1_bf16(const void* x, const void* wr, const float* bias,
                                    const void* w1, int M, int K, int N, int E, int topk, int cap,
                                    float* logits, int32_t* ids, float* wts, int32_t* sorted_ids,
                                    int32_t* block_expert, int32_t* expert_offsets,
                                    int32_t* num_padded, void* act, hipStream_t s);
// GEMM2 and the combine of those tokens in one launch (no partial rows):
// out [M,K] bf16 from act, the block owners and the routing weights.
void launch_decode_gemm2_combine_bf16(const void* act, const void* w2, const float* topk_w,
                                      const int32_t* sorted_ids, const int32_t* block_expert,
                                      int M, int K, int N, int E, int topk, int cap, void* out,
                                      hipStream_t s);

}  // namespace moe
