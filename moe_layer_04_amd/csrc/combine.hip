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

// One thread per 4 columns when there are many tokens; per column when few
// (then the partial rows of one token are read by more threads at once).
template <int V>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ypart, int M,
                                                      int K, int topk, int nsplit,
                                                      uint16_t* __restrict__ out) {
    typedef float fv_t __attribute__((ext_vector_type(V)));
    typedef unsigned short uv_t __attribute__((ext_vector_type(V)));
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const int kq = K / V;
    if (idx >= (long)M * kq) return;
    const int t = (int)(idx / kq);
    const int c = (int)(idx % kq) * V;
    const size_t nslots = (size_t)M * topk;
    // partial i = j*nsplit + z lives at ypart[z][t*topk + j]; loads are issued
    // eight at a time and added in ascending i (a fixed order)
    const int n = topk * nsplit;
    auto at = [&](int i) {
        const int j = i / nsplit, z = i - j * nsplit;
        return *reinterpret_cast<const fv_t*>(ypart +
                                              ((size_t)z * nslots + (size_t)t * topk + j) * K + c);
    };
    fv_t acc = {};
    int i = 0;
    for (; i + 8 <= n; i += 8) {
        fv_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = at(i + u);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; i < n; ++i) acc += at(i);
    uv_t o;
#pragma unroll
    for (int v = 0; v < V; ++v) o[v] = f32_to_bf16_bits(acc[v]);
    *reinterpret_cast<uv_t*>(out + (size_t)t * K + c) = o;
}

void launch_combine(const float* ypart, int M, int K, int topk, int nsplit, void* out,
                    hipStream_t s) {
    if ((long)M * K >= 256L * 256) {
        const long n = (long)M * (K / 4);
        combine_kernel<4><<<(int)((n + 255) / 256), 256, 0, s>>>(ypart, M, K, topk, nsplit,
                                                                 (uint16_t*)out);
    } else {
        const long n = (long)M * K;
        combine_kernel<1><<<(int)((n + 255) / 256), 256, 0, s>>>(ypart, M, K, topk, nsplit,
                                                                 (uint16_t*)out);
    }
}

}  // namespace moe
