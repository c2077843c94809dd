// combine.hip -- the weighted un-permute combine ("expert aggregation", one
// of the steps the FP8 passage of "Mixture-of-Experts kernel engineering on
// Amazon SageMaker AI" names as fused into a single pass).  The GEMM2
// epilogues already multiplied each slot's rows by its routing weight and
// wrote them at slot position p = t*topk + j (split partials z apart), so
// out[t,c] = bf16_rne( sum_j sum_z ypart[z][t*topk + j][c] ), summed in fp32
// in ascending j, then z: a fixed order, so the result is deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ypart, int M,
                                                      int K, int topk, int nsplit,
                                                      uint16_t* __restrict__ out) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;  // one thread per 4 columns
    const int kq = K / 4;
    if (idx >= (long)M * kq) return;
    const int t = (int)(idx / kq);
    const int c = (int)(idx % kq) * 4;
    const size_t nslots = (size_t)M * topk;
    f32x4_t acc = {0, 0, 0, 0};
    for (int j = 0; j < topk; ++j)
        for (int z = 0; z < nsplit; ++z)
            acc += *reinterpret_cast<const f32x4_t*>(
                ypart + ((size_t)z * nslots + (size_t)t * topk + j) * K + c);
    u16x4_t o;
#pragma unroll
    for (int v = 0; v < 4; ++v) o[v] = f32_to_bf16_bits(acc[v]);
    *reinterpret_cast<u16x4_t*>(out + (size_t)t * K + c) = o;
}

void launch_combine(const float* ypart, int M, int K, int topk, int nsplit, void* out,
                    hipStream_t s) {
    const long n = (long)M * (K / 4);
    const int grid = (int)((n + 255) / 256);
    combine_kernel<<<grid, 256, 0, s>>>(ypart, M, K, topk, nsplit, (uint16_t*)out);
}

}  // namespace moe
