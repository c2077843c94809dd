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
// weights read from HBM feeds a full MFMA row.  Decode is bound by that HBM
// stream; the kernels load weights straight into registers.
//
// Work split: one workgroup (4 waves) per (block of one expert's sorted
// rows, tile of weight rows).  A block holds 16, 32 or 64 rows (NT = 1, 2 or
// 4 token tiles of 16): every weight fragment is multiplied by all NT token
// fragments, so an expert with up to 16*NT rows streams its weights once.
// GEMM1 waves own 16 gate rows and the matching 16 up rows, so
// SiLU(gate)*up is formed in registers (the fused epilogue); GEMM2 waves own
// 32 output rows and may split the reduction (N) across workgroups, writing
// fp32 partial rows scattered back to slot order and already multiplied by
// the routing weight.
//
// Memory access: all operands go through buffer loads.  A buffer resource is
// bounds-checked by the hardware, so padding lanes of a block (sentinel rows)
// get zeros by passing an offset past the end -- no branch, no traffic.
// Each wave starts its reduction at a different, rotated K-step: waves that
// all began at k = 0 would hit the same column slab of rows that are K*2
// bytes apart, concentrating the stream on few HBM channels.
//
// MFMA operand layout used (16x16 family): lane l supplies row (l % 16) of
// the A tile and column (l % 16) of the B tile, each with a K-slice chosen
// by l / 16; A and B use the same K-slice assignment, so the sum over K is
// the full dot product whatever order the hardware adds the slices in.  The
// accumulator lane l holds D[4*(l/16) + v][l % 16], v = 0..3.
#include "common.hpp"
#include "launch.hpp"
#include "tuning.hpp"

namespace moe {

constexpr int kDecRows = kDecodeRows;   // token rows per block (the align block size)
constexpr uint32_t kOob = 0x80000000u;  // offset past every resource: loads return 0
constexpr int kRot = 7;                 // K-step rotation per wave

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // dword3 = 0x00020000: raw (untyped) 32-bit buffer access on CDNA
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ i32x4_t bload(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ i32x8_t bload32(rsrc_t r, uint32_t off) {
    const i32x4_t a = bload(r, off), b = bload(r, off + 16);
    return i32x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ f32x4_t mfma_bf16(i32x4_t a, i32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8_t)a, (bf16x8_t)b, c, 0, 0, 0);
}
// e4m3 x e4m3, block scales fixed at 2^0 (E8M0 code 127).
__device__ __forceinline__ f32x4_t mfma_fp8(i32x8_t a, i32x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// A = 32 e2m1 codes per lane (4 dwords; cbsz 4) with the lane's E8M0 block
// scale, B = 32 e4m3 codes per lane with scale 1 (E8M0 127).
__device__ __forceinline__ f32x4_t mfma_fp4_fp8(i32x4_t a, int scale_a, i32x8_t b, f32x4_t c) {
    const i32x8_t a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, 4, 0, 0, scale_a, 0, 127);
}
__device__ __forceinline__ uint32_t bload_u32(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// K-step j of a wave whose sequence is rotated by `rot` (steps in [0, n)).
__device__ __forceinline__ int rotated(int j, int rot, int n) {
    const int q = j + rot;
    return q >= n ? q - n : q;
}

// ---------------------------------------------------------------------------
// GEMM1 + SiLU*up, bf16.  grid = (N/64, blocks); wave w of workgroup x owns
// gate rows n0..n0+15 with n0 = (4x + w)*16 and up rows N+n0..N+n0+15.
// A K-step is 128 elements: 4 MFMAs per row tile.
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void gemm1_decode_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int M, int topk, int nslots, int K, int N,
    uint16_t* __restrict__ act) {
    constexpr int BR = kDecRows * NT;  // sorted rows per block (NT token tiles)
    const int blk = (int)blockIdx.y;
    // a block past the padded end has no owner (-1 from the align step): the
    // owner alone decides, one dependent load fewer than reading num_padded
    const int e = block_expert[blk];
    if (e < 0) return;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);  // wave-uniform
    const int gw = (int)blockIdx.x * 4 + wave;
    const int n0 = gw * 16;
    const int i = lane & 15, kq = lane >> 4;

    const size_t row_bytes = (size_t)K * 2;
    const rsrc_t rg = make_rsrc(w1 + ((size_t)e * 2 * N + n0) * K, (uint32_t)(16 * row_bytes));
    const rsrc_t ru = make_rsrc(w1 + ((size_t)e * 2 * N + N + n0) * K, (uint32_t)(16 * row_bytes));
    const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)M * row_bytes));
    const uint32_t wo = (uint32_t)(i * row_bytes) + kq * 16;
    bool vj[NT];
    uint32_t xo[NT];
    int pj[NT];  // the rows' slots, loaded together
#pragma unroll
    for (int j = 0; j < NT; ++j) pj[j] = sorted_ids[blk * BR + 16 * j + i];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        vj[j] = pj[j] < nslots;
        xo[j] = vj[j] ? (uint32_t)((size_t)slot_token(pj[j], topk) * row_bytes) + kq * 16 : kOob;
    }

    struct Frag { i32x4_t g[4], u[4], b[NT][4]; };
    auto load = [&](Frag& f, int k) {
        const uint32_t kb = (uint32_t)k * 2;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f.g[s] = bload(rg, wo + kb + s * 64);
            f.u[s] = bload(ru, wo + kb + s * 64);
#pragma unroll
            for (int j = 0; j < NT; ++j) f.b[j][s] = bload(rx, xo[j] + kb + s * 64);
        }
    };
    f32x4_t accg[NT], accu[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) accg[j] = accu[j] = f32x4_t{0, 0, 0, 0};
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                accg[j] = mfma_bf16(f.g[s], f.b[j][s], accg[j]);
                accu[j] = mfma_bf16(f.u[s], f.b[j][s], accu[j]);
            }
    };
    const int nst = K / 128;
    const int rot = (gw * kRot + blk * 5) % nst;
    Frag cur;
    load(cur, rotated(0, rot, nst) * 128);
    for (int j = 1; j < nst; ++j) {
        Frag nxt;
        load(nxt, rotated(j, rot, nst) * 128);
        compute(cur);
        cur = nxt;
    }
    compute(cur);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        pin(accg[j]);
        pin(accu[j]);
    }

#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if (vj[j]) {
            u16x4_t o;
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = f32_to_bf16_bits(silu(accg[j][v]) * accu[j][v]);
            *reinterpret_cast<u16x4_t*>(act + (size_t)(blk * BR + 16 * j + i) * N + n0 +
                                        4 * kq) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// GEMM2 (down projection), bf16.  grid = (K/128, blocks, nsplit); wave w of
// workgroup x owns output rows c0..c0+31, c0 = (4x + w)*32, over the
// reduction range [z*N/nsplit, (z+1)*N/nsplit).
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void gemm2_decode_bf16_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int cap,
    int nslots, int K, int N, int nsplit, float* __restrict__ ypart) {
    constexpr int BR = kDecRows * NT;  // sorted rows per block (NT token tiles)
    const int blk = (int)blockIdx.y;
    // a block past the padded end has no owner (-1 from the align step): the
    // owner alone decides, one dependent load fewer than reading num_padded
    const int e = block_expert[blk];
    if (e < 0) return;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);  // wave-uniform
    const int gw = (int)blockIdx.x * 4 + wave;
    const int c0 = gw * 32;
    const int i = lane & 15, kq = lane >> 4;
    const int z = (int)blockIdx.z;
    const int nlen = N / nsplit;
    const int nbeg = z * nlen;

    const size_t row_bytes = (size_t)N * 2;
    const rsrc_t rw = make_rsrc(w2 + ((size_t)e * K + c0) * N, (uint32_t)(32 * row_bytes));
    const rsrc_t ra = make_rsrc(act, (uint32_t)((size_t)cap * row_bytes));
    const uint32_t wo = (uint32_t)(i * row_bytes) + nbeg * 2 + kq * 16;
    const uint32_t wo1 = wo + (uint32_t)(16 * row_bytes);
    int pj[NT];
    uint32_t ao[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int r = blk * BR + 16 * j + i;
        pj[j] = sorted_ids[r];
        ao[j] = pj[j] < nslots ? (uint32_t)((size_t)r * row_bytes) + nbeg * 2 + kq * 16 : kOob;
    }

    struct Frag { i32x4_t a0[4], a1[4], b[NT][4]; };
    auto load = [&](Frag& f, int n) {
        const uint32_t nb = (uint32_t)n * 2;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f.a0[s] = bload(rw, wo + nb + s * 64);
            f.a1[s] = bload(rw, wo1 + nb + s * 64);
#pragma unroll
            for (int j = 0; j < NT; ++j) f.b[j][s] = bload(ra, ao[j] + nb + s * 64);
        }
    };
    f32x4_t acc0[NT], acc1[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc0[j] = acc1[j] = f32x4_t{0, 0, 0, 0};
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                acc0[j] = mfma_bf16(f.a0[s], f.b[j][s], acc0[j]);
                acc1[j] = mfma_bf16(f.a1[s], f.b[j][s], acc1[j]);
            }
    };
    const int nst = nlen / 128;
    const int rot = (gw * kRot + blk * 5 + z * 3) % nst;
    Frag cur;
    load(cur, rotated(0, rot, nst) * 128);
    for (int j = 1; j < nst; ++j) {
        Frag nxt;
        load(nxt, rotated(j, rot, nst) * 128);
        compute(cur);
        cur = nxt;
    }
    compute(cur);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        pin(acc0[j]);
        pin(acc1[j]);
    }

#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if (pj[j] < nslots) {
            const float w = topk_w[pj[j]];
            float* yr = ypart + ((size_t)z * nslots + pj[j]) * K + c0 + 4 * kq;
            *reinterpret_cast<f32x4_t*>(yr) = acc0[j] * w;
            *reinterpret_cast<f32x4_t*>(yr + 16) = acc1[j] * w;
        }
    }
}

// ---------------------------------------------------------------------------
// FP8 (OCP e4m3) versions.  One 16x16x128 MFMA consumes 32 codes per lane; a
// K-step is one 128-code chunk.  GEMM1 applies s_x[t] * w1_scale[e] to the
// fp32 accumulators, forms SiLU*up in fp32, stores it and folds each row's
// |act| max into amax[r] (float bits, atomicMax: exact and order-free for
// non-negative floats).
// ---------------------------------------------------------------------------
// NT token tiles of 16 rows per block (block = 16*NT sorted rows): every
// wave multiplies its weight fragment by all NT token fragments, so an
// expert with up to 16*NT rows streams its weights once.
template <int NT>
__global__ __launch_bounds__(256) void gemm1_decode_fp8_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xscale,
    const uint8_t* __restrict__ w1, const float* __restrict__ w1_scale, int rowwise,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int M, int topk, int nslots, int K, int N,
    float* __restrict__ act, uint32_t* __restrict__ amax) {
    constexpr int BR = kDecRows * NT;  // sorted rows per block
    const int blk = (int)blockIdx.y;
    // a block past the padded end has no owner (-1 from the align step): the
    // owner alone decides, one dependent load fewer than reading num_padded
    const int e = block_expert[blk];
    if (e < 0) return;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);  // wave-uniform
    const int gw = (int)blockIdx.x * 4 + wave;
    const int n0 = gw * 16;
    const int i = lane & 15, kq = lane >> 4;

    const size_t row_bytes = (size_t)K;
    const rsrc_t rg = make_rsrc(w1 + ((size_t)e * 2 * N + n0) * K, (uint32_t)(16 * row_bytes));
    const rsrc_t ru = make_rsrc(w1 + ((size_t)e * 2 * N + N + n0) * K, (uint32_t)(16 * row_bytes));
    const rsrc_t rx = make_rsrc(xq, (uint32_t)((size_t)M * row_bytes));
    const uint32_t wo = (uint32_t)(i * row_bytes) + kq * 32;
    // token tile j: sorted row blk*BR + 16j + i
    int tj[NT];
    bool vj[NT];
    uint32_t xo[NT];
    int pj[NT];  // the rows' slots, loaded together
#pragma unroll
    for (int j = 0; j < NT; ++j) pj[j] = sorted_ids[blk * BR + 16 * j + i];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        vj[j] = pj[j] < nslots;
        tj[j] = vj[j] ? slot_token(pj[j], topk) : 0;
        xo[j] = vj[j] ? (uint32_t)((size_t)tj[j] * row_bytes) + kq * 32 : kOob;
    }

    struct Frag { i32x8_t g, u, b[NT]; };
    auto load = [&](Frag& f, int k) {
        f.g = bload32(rg, wo + k);
        f.u = bload32(ru, wo + k);
#pragma unroll
        for (int j = 0; j < NT; ++j) f.b[j] = bload32(rx, xo[j] + k);
    };
    f32x4_t accg[NT], accu[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) accg[j] = accu[j] = f32x4_t{0, 0, 0, 0};
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            accg[j] = mfma_fp8(f.g, f.b[j], accg[j]);
            accu[j] = mfma_fp8(f.u, f.b[j], accu[j]);
        }
    };
    const int nst = K / 128;
    const int rot = (gw * kRot + blk * 5) % nst;
    if constexpr (NT == 1) {
        // one token tile: three fragments in turn, loads two steps ahead
        // (DeepSeek shape 1265 -> 1252 us; the bf16 kernel measured slower
        // with it); loads past the end repeat the last step (never multiplied)
        auto kstep = [&](int j) { return rotated(j < nst ? j : nst - 1, rot, nst) * 128; };
        Frag fa, fb, fc;
        load(fa, kstep(0));
        load(fb, kstep(1));
        for (int j = 0; j < nst; j += 3) {
            load(fc, kstep(j + 2));
            compute(fa);
            load(fa, kstep(j + 3));
            if (j + 1 < nst) compute(fb);
            load(fb, kstep(j + 4));
            if (j + 2 < nst) compute(fc);
        }
    } else {
        Frag cur;
        load(cur, rotated(0, rot, nst) * 128);
        for (int j = 1; j < nst; ++j) {
            Frag nxt;
            load(nxt, rotated(j, rot, nst) * 128);
            compute(cur);
            cur = nxt;
        }
        compute(cur);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        pin(accg[j]);
        pin(accu[j]);
    }

    // accumulator element v is gate row n0 + 4*kq + v (and that up row)
    float sg[4], su[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        if (rowwise) {
            const float* sr = w1_scale + (size_t)e * 2 * N + n0 + 4 * kq + v;
            sg[v] = sr[0];
            su[v] = sr[N];
        } else {
            sg[v] = su[v] = w1_scale[e];
        }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int row = blk * BR + 16 * j + i;
        float m = 0.0f;
        if (vj[j]) {
            const float sx = xscale[tj[j]];
            f32x4_t o;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                o[v] = silu(accg[j][v] * (sx * sg[v])) * (accu[j][v] * (sx * su[v]));
                m = fmaxf(m, fabsf(o[v]));
            }
            *reinterpret_cast<f32x4_t*>(act + (size_t)row * N + n0 + 4 * kq) = o;
        }
        const uint32_t mb = col_max_bits(__float_as_uint(m));
        if (vj[j] && kq == 0) atomicMax(amax + row, mb);
    }
}

// act32 [cap,N] + amax [cap] -> act_q [cap,N] e4m3 and s_a [cap]; one wave per row.
// A wave per (row, chunk of kActChunk elements): the row's scale comes from
// the amax GEMM1 folded, so the chunks of a row are independent.
constexpr int kActChunk = 8 * kWave * 4;

__global__ __launch_bounds__(256) void act_quant_kernel(
    const float* __restrict__ act, const uint32_t* __restrict__ amax,
    const int32_t* __restrict__ inv, int nslots, int N, int nchunk,
    uint8_t* __restrict__ act_q, float* __restrict__ ascale) {
    // waves cover the slots (padding rows are never read): slot p's row is
    // its sorted position inv[p], written by the align step
    const int w = (int)(blockIdx.x * 4 + threadIdx.x / kWave);
    const int p = w / nchunk, ch = w % nchunk;
    if (p >= nslots) return;
    const int r = inv[p];
    const int lane = lane_id();
    const float a = __uint_as_float(amax[r]);
    const float s = (a == 0.0f) ? 1.0f : a / 448.0f;
    const float* src = act + (size_t)r * N;
    uint8_t* dst = act_q + (size_t)r * N;
    // the chunk's loads are issued (8 per lane) before any is used
    constexpr int G = 8;
    const int n0 = ch * kActChunk + lane * 4;
    f32x4_t v[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int n = n0 + g * kWave * 4;
        if (n < N) v[g] = *reinterpret_cast<const f32x4_t*>(src + n);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int n = n0 + g * kWave * 4;
        if (n < N) {
            const uint32_t q = f32_to_e4m3(v[g][0] / s) | (f32_to_e4m3(v[g][1] / s) << 8) |
                               (f32_to_e4m3(v[g][2] / s) << 16) |
                               (f32_to_e4m3(v[g][3] / s) << 24);
            *reinterpret_cast<uint32_t*>(dst + n) = q;
        }
    }
    if (ch == 0 && lane == 0) ascale[r] = s;
}

template <int NT>
__global__ __launch_bounds__(256) void gemm2_decode_fp8_kernel(
    const uint8_t* __restrict__ act_q, const float* __restrict__ ascale,
    const uint8_t* __restrict__ w2, const float* __restrict__ w2_scale, int rowwise,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int cap,
    int nslots, int K, int N, int nsplit, float* __restrict__ ypart) {
    constexpr int BR = kDecRows * NT;
    const int blk = (int)blockIdx.y;
    // a block past the padded end has no owner (-1 from the align step): the
    // owner alone decides, one dependent load fewer than reading num_padded
    const int e = block_expert[blk];
    if (e < 0) return;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);  // wave-uniform
    const int gw = (int)blockIdx.x * 4 + wave;
    const int c0 = gw * 32;
    const int i = lane & 15, kq = lane >> 4;
    const int z = (int)blockIdx.z;
    const int nlen = N / nsplit;
    const int nbeg = z * nlen;

    const size_t row_bytes = (size_t)N;
    const rsrc_t rw = make_rsrc(w2 + ((size_t)e * K + c0) * N, (uint32_t)(32 * row_bytes));
    const rsrc_t ra = make_rsrc(act_q, (uint32_t)((size_t)cap * row_bytes));
    const uint32_t wo = (uint32_t)(i * row_bytes) + nbeg + kq * 32;
    const uint32_t wo1 = wo + (uint32_t)(16 * row_bytes);
    int rj[NT], pj[NT];
    uint32_t ao[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        rj[j] = blk * BR + 16 * j + i;
        pj[j] = sorted_ids[rj[j]];
        ao[j] = pj[j] < nslots ? (uint32_t)((size_t)rj[j] * row_bytes) + nbeg + kq * 32 : kOob;
    }

    struct Frag { i32x8_t a0, a1, b[NT]; };
    auto load = [&](Frag& f, int n) {
        f.a0 = bload32(rw, wo + n);
        f.a1 = bload32(rw, wo1 + n);
#pragma unroll
        for (int j = 0; j < NT; ++j) f.b[j] = bload32(ra, ao[j] + n);
    };
    f32x4_t acc0[NT], acc1[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc0[j] = acc1[j] = f32x4_t{0, 0, 0, 0};
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            acc0[j] = mfma_fp8(f.a0, f.b[j], acc0[j]);
            acc1[j] = mfma_fp8(f.a1, f.b[j], acc1[j]);
        }
    };
    const int nst = nlen / 128;
    const int rot = (gw * kRot + blk * 5 + z * 3) % nst;
    Frag cur;
    load(cur, rotated(0, rot, nst) * 128);
    for (int j = 1; j < nst; ++j) {
        Frag nxt;
        load(nxt, rotated(j, rot, nst) * 128);
        compute(cur);
        cur = nxt;
    }
    compute(cur);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        pin(acc0[j]);
        pin(acc1[j]);
    }

    // accumulator element v of acc0 / acc1 is output column
    // c0 + 4*kq + v / c0 + 16 + 4*kq + v
    f32x4_t s0, s1;
    if (rowwise) {
        const float* sr = w2_scale + (size_t)e * K + c0 + 4 * kq;
        s0 = *reinterpret_cast<const f32x4_t*>(sr);
        s1 = *reinterpret_cast<const f32x4_t*>(sr + 16);
    } else {
        const float ws = w2_scale[e];
        s0 = s1 = f32x4_t{ws, ws, ws, ws};
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if (pj[j] < nslots) {
            const float w = topk_w[pj[j]] * ascale[rj[j]];
            float* yr = ypart + ((size_t)z * nslots + pj[j]) * K + c0 + 4 * kq;
            *reinterpret_cast<f32x4_t*>(yr) = acc0[j] * (s0 * w);
            *reinterpret_cast<f32x4_t*>(yr + 16) = acc1[j] * (s1 * w);
        }
    }
}

// ---------------------------------------------------------------------------
// MXFP4 weights (OCP microscaling: e2m1 codes two per byte, even element in
// the low nibble, one E8M0 scale per 32 elements of a row) against the
// layer's per-token e4m3 activations.  In the scaled 16x16x128 MFMA an FP4
// lane holds 32 consecutive K (lane group q: K 32q .. 32q+31 of the step),
// exactly one MX block, so the block scale is the lane's scale operand; the
// e4m3 operand's lane group q holds K 16q .. 16q+15 and 64+16q .. 64+16q+15
// (its two 16-byte halves).  Both layouts were measured on gfx950.
// ---------------------------------------------------------------------------
// Each wave covers RT 16-row tiles of gate rows and the matching up rows
// (GEMM1) or RT 16-row tiles of output rows (GEMM2) with one token fragment;
// a step is two 128-deep chunks, the scale bytes of a step are one 8-byte
// read per row tile from the wave's LDS copy of its rows' scales, and the
// steps rotate through two fragments (four in GEMM1 with one token tile).
constexpr int kMxTiles1 = tune::kMxTiles1;  // GEMM1: 16 gate + 16 up rows per wave
constexpr int kMxTiles2 = tune::kMxTiles2;  // GEMM2: 64 output rows per wave

// per-wave E8M0 scale copies of the MXFP4 kernels (dynamic LDS, sized by
// the launchers)
extern __shared__ __attribute__((aligned(16))) char mx_scale_lds[];

__device__ __forceinline__ uint64_t bload_u64(rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return ((uint64_t)(uint32_t)v[1] << 32) | (uint32_t)v[0];
}

template <int NT>
__global__ __launch_bounds__(256) void gemm1_decode_mxfp4_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xscale,
    const uint8_t* __restrict__ w1, const uint8_t* __restrict__ w1e8,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int M, int topk, int nslots, int K, int N,
    float* __restrict__ act, uint32_t* __restrict__ amax) {
    constexpr int RT = kMxTiles1;
    constexpr int BR = kDecRows * NT;  // sorted rows per block (NT token tiles)
    const int blk = (int)blockIdx.y;
    // a block past the padded end has no owner (-1 from the align step): the
    // owner alone decides, one dependent load fewer than reading num_padded
    const int e = block_expert[blk];
    if (e < 0) return;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);  // wave-uniform
    const int gw = (int)blockIdx.x * 4 + wave;
    const int n0 = gw * 16 * RT;
    const int i = lane & 15, kq = lane >> 4;
    int tj[NT];
    bool vj[NT];
    int pj[NT];  // the rows' slots, loaded together
#pragma unroll
    for (int j = 0; j < NT; ++j) pj[j] = sorted_ids[blk * BR + 16 * j + i];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        vj[j] = pj[j] < nslots;
        tj[j] = vj[j] ? slot_token(pj[j], topk) : 0;
    }

    const size_t row_bytes = (size_t)K / 2;   // packed e2m1
    const size_t srow = (size_t)K / 32;       // E8M0 scales per row
    const size_t g0 = (size_t)e * 2 * N + n0, u0 = g0 + N;
    const rsrc_t rg = make_rsrc(w1 + g0 * row_bytes, (uint32_t)(16 * RT * row_bytes));
    const rsrc_t ru = make_rsrc(w1 + u0 * row_bytes, (uint32_t)(16 * RT * row_bytes));
    const rsrc_t rsg = make_rsrc(w1e8 + g0 * srow, (uint32_t)(16 * RT * srow));
    const rsrc_t rsu = make_rsrc(w1e8 + u0 * srow, (uint32_t)(16 * RT * srow));
    const rsrc_t rx = make_rsrc(xq, (uint32_t)((size_t)M * K));
    const uint32_t wo = (uint32_t)(i * row_bytes) + kq * 16;
    const uint32_t so = (uint32_t)(i * srow);
    uint32_t xo[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) xo[j] = vj[j] ? (uint32_t)((size_t)tj[j] * K) + kq * 16 : kOob;
    const int sh = 8 * kq;

    // The E8M0 scales of this wave's gate rows and of its up rows (each
    // 16*RT rows of K/32 bytes, contiguous in memory) are copied once into
    // the wave's LDS region with 16-byte loads; every step then reads its 8
    // bytes per row from LDS.  (Per-step 8-byte global loads of 16 scattered
    // rows measured 25 % slower on the whole kernel.)
    const int sbytes = 16 * RT * (int)srow;  // a multiple of 128 (K % 256 == 0)
    char* sl = mx_scale_lds + (size_t)wave * 2 * sbytes;
    for (int off = lane * 16; off < sbytes; off += kWave * 16) {
        *reinterpret_cast<i32x4_t*>(sl + off) = bload(rsg, (uint32_t)off);
        *reinterpret_cast<i32x4_t*>(sl + sbytes + off) = bload(rsu, (uint32_t)off);
    }
    __syncthreads();

    // one step = chunks k and k+128 of every row tile
    struct Frag {
        i32x4_t g[2][RT], u[2][RT], b[2][NT][2];
        uint64_t sg[RT], su[RT];
    };
    auto load = [&](Frag& f, int k) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int kc = k + 128 * c;
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                f.g[c][r] = bload(rg, wo + (uint32_t)(16 * r * row_bytes) + kc / 2);
                f.u[c][r] = bload(ru, wo + (uint32_t)(16 * r * row_bytes) + kc / 2);
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                f.b[c][j][0] = bload(rx, xo[j] + kc);
                f.b[c][j][1] = bload(rx, xo[j] + kc + 64);
            }
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const char* q = sl + so + 16 * r * srow + k / 32;  // 8-byte aligned
            f.sg[r] = *reinterpret_cast<const uint64_t*>(q);
            f.su[r] = *reinterpret_cast<const uint64_t*>(q + sbytes);
        }
    };
    f32x4_t accg[NT][RT], accu[NT][RT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < RT; ++r) accg[j][r] = accu[j][r] = f32x4_t{0, 0, 0, 0};
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const i32x4_t b0 = f.b[c][j][0], b1 = f.b[c][j][1];
                const i32x8_t b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    accg[j][r] = mfma_fp4_fp8(f.g[c][r], (int)((f.sg[r] >> (32 * c + sh)) & 0xffu),
                                              b, accg[j][r]);
                    accu[j][r] = mfma_fp4_fp8(f.u[c][r], (int)((f.su[r] >> (32 * c + sh)) & 0xffu),
                                              b, accu[j][r]);
                }
            }
    };
    const int nst = K / 256;  // K is a multiple of 256 here (checked by the launcher)
    const int rot = (gw * kRot + blk * 5) % nst;
    auto kstep = [&](int j) { return rotated(j < nst ? j : nst - 1, rot, nst) * 256; };
    // fragments in turn, no copies; loads past the end repeat the last step
    // (never multiplied), so every wait count is exact.  One token tile:
    // four fragments (loads three steps ahead; against three: single-token
    // 23.7 -> 22.6 us, Mixtral shape 109 -> 105 us, DeepSeek shape 718 ->
    // 708 us); more tiles: two, as more would cost occupancy.
    if constexpr (NT == 1) {
        Frag fa, fb, fc, fd;
        load(fa, kstep(0));
        load(fb, kstep(1));
        load(fc, kstep(2));
        for (int j = 0; j < nst; j += 4) {
            load(fd, kstep(j + 3));
            compute(fa);
            load(fa, kstep(j + 4));
            if (j + 1 < nst) compute(fb);
            load(fb, kstep(j + 5));
            if (j + 2 < nst) compute(fc);
            load(fc, kstep(j + 6));
            if (j + 3 < nst) compute(fd);
        }
    } else {
        Frag fa, fb;
        load(fa, kstep(0));
        for (int j = 0; j < nst; j += 2) {
            load(fb, kstep(j + 1));
            compute(fa);
            load(fa, kstep(j + 2));
            if (j + 1 < nst) compute(fb);
        }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            pin(accg[j][r]);
            pin(accu[j][r]);
        }

#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int row = blk * BR + 16 * j + i;
        float m = 0.0f;
        if (vj[j]) {
            const float sx = xscale[tj[j]];
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                f32x4_t o;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    o[v] = silu(accg[j][r][v] * sx) * (accu[j][r][v] * sx);
                    m = fmaxf(m, fabsf(o[v]));
                }
                *reinterpret_cast<f32x4_t*>(act + (size_t)row * N + n0 + 16 * r + 4 * kq) = o;
            }
        }
        const uint32_t mb = col_max_bits(__float_as_uint(m));
        if (vj[j] && kq == 0) atomicMax(amax + row, mb);
    }
}

template <int NT>
__global__ __launch_bounds__(256) void gemm2_decode_mxfp4_kernel(
    const uint8_t* __restrict__ act_q, const float* __restrict__ ascale,
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2e8,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int cap,
    int nslots, int K, int N, int nsplit, float* __restrict__ ypart) {
    constexpr int RT = kMxTiles2;
    constexpr int BR = kDecRows * NT;  // sorted rows per block (NT token tiles)
    const int blk = (int)blockIdx.y;
    // a block past the padded end has no owner (-1 from the align step): the
    // owner alone decides, one dependent load fewer than reading num_padded
    const int e = block_expert[blk];
    if (e < 0) return;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);  // wave-uniform
    const int gw = (int)blockIdx.x * 4 + wave;
    const int c0 = gw * 16 * RT;
    const int i = lane & 15, kq = lane >> 4;
    const int z = (int)blockIdx.z;
    const int nlen = N / nsplit;
    const int nbeg = z * nlen;
    int rj[NT], pj[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        rj[j] = blk * BR + 16 * j + i;
        pj[j] = sorted_ids[rj[j]];
    }

    const size_t row_bytes = (size_t)N / 2;
    const size_t srow = (size_t)N / 32;
    const size_t r0 = (size_t)e * K + c0;
    const rsrc_t rw = make_rsrc(w2 + r0 * row_bytes, (uint32_t)(16 * RT * row_bytes));
    const rsrc_t rs = make_rsrc(w2e8 + r0 * srow, (uint32_t)(16 * RT * srow));
    const rsrc_t ra = make_rsrc(act_q, (uint32_t)((size_t)cap * N));
    const uint32_t wo = (uint32_t)(i * row_bytes) + nbeg / 2 + kq * 16;
    uint32_t ao[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
        ao[j] = pj[j] < nslots ? (uint32_t)((size_t)rj[j] * N) + nbeg + kq * 16 : kOob;
    const int sh = 8 * kq;

    // the split's E8M0 bytes of the wave's 16*RT rows (nlen/32 per row),
    // copied once into the wave's LDS region in 8-byte pieces, row-major
    const int sspan = nlen / 32;  // a multiple of 8 (nlen % 256 == 0)
    char* sl = mx_scale_lds + (size_t)wave * 16 * RT * sspan;
    {
        const int upr = sspan / 8;
        for (int u = lane; u < 16 * RT * upr; u += kWave) {
            const int row = u / upr, col = u - row * upr;
            *reinterpret_cast<uint64_t*>(sl + row * sspan + col * 8) =
                bload_u64(rs, (uint32_t)(row * srow) + nbeg / 32 + col * 8);
        }
    }
    __syncthreads();

    struct Frag {
        i32x4_t a[2][RT], b[2][NT][2];
        uint64_t s[RT];
    };
    auto load = [&](Frag& f, int n) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int nc = n + 128 * c;
#pragma unroll
            for (int q = 0; q < RT; ++q)
                f.a[c][q] = bload(rw, wo + (uint32_t)(16 * q * row_bytes) + nc / 2);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                f.b[c][j][0] = bload(ra, ao[j] + nc);
                f.b[c][j][1] = bload(ra, ao[j] + nc + 64);
            }
        }
#pragma unroll
        for (int q = 0; q < RT; ++q)
            f.s[q] = *reinterpret_cast<const uint64_t*>(sl + (i + 16 * q) * sspan + n / 32);
    };
    f32x4_t acc[NT][RT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < RT; ++q) acc[j][q] = f32x4_t{0, 0, 0, 0};
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const i32x4_t b0 = f.b[c][j][0], b1 = f.b[c][j][1];
                const i32x8_t b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
                for (int q = 0; q < RT; ++q)
                    acc[j][q] = mfma_fp4_fp8(f.a[c][q], (int)((f.s[q] >> (32 * c + sh)) & 0xffu),
                                             b, acc[j][q]);
            }
    };
    const int nst = nlen / 256;  // nlen is a multiple of 256 here (checked by the launcher)
    const int rot = (gw * kRot + blk * 5 + z * 3) % nst;
    auto kstep = [&](int j) { return rotated(j < nst ? j : nst - 1, rot, nst) * 256; };
    Frag fa, fb;
    load(fa, kstep(0));
    for (int j = 0; j < nst; j += 2) {
        load(fb, kstep(j + 1));
        compute(fa);
        load(fa, kstep(j + 2));
        if (j + 1 < nst) compute(fb);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < RT; ++q) pin(acc[j][q]);

#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if (pj[j] < nslots) {
            const float w = topk_w[pj[j]] * ascale[rj[j]];
            float* yr = ypart + ((size_t)z * nslots + pj[j]) * K + c0 + 4 * kq;
#pragma unroll
            for (int q = 0; q < RT; ++q)
                *reinterpret_cast<f32x4_t*>(yr + 16 * q) = acc[j][q] * w;
        }
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
void launch_gemm1_decode_bf16(const void* x, const void* w1, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded, int M,
                              int topk, int nslots, int K, int N, int max_blocks, int nt,
                              void* act, hipStream_t s) {
    dim3 grid(N / 64, max_blocks);
#define MOE_G1BF(NT)                                                                          \
    gemm1_decode_bf16_kernel<NT><<<grid, 256, 0, s>>>((const uint16_t*)x, (const uint16_t*)w1, \
                                                      sorted_ids, block_expert, num_padded, M, \
                                                      topk, nslots, K, N, (uint16_t*)act)
    if (nt == 4) MOE_G1BF(4);
    else if (nt == 2) MOE_G1BF(2);
    else MOE_G1BF(1);
#undef MOE_G1BF
}

void launch_gemm2_decode_bf16(const void* act, const void* w2, const float* topk_w,
                              const int32_t* sorted_ids, const int32_t* block_expert,
                              const int32_t* num_padded, int cap, int nslots, int K, int N,
                              int nsplit, int max_blocks, int nt, float* ypart, hipStream_t s) {
    dim3 grid(K / 128, max_blocks, nsplit);
#define MOE_G2BF(NT)                                                                          \
    gemm2_decode_bf16_kernel<NT><<<grid, 256, 0, s>>>((const uint16_t*)act, (const uint16_t*)w2,\
                                                      topk_w, sorted_ids, block_expert,        \
                                                      num_padded, cap, nslots, K, N, nsplit,   \
                                                      ypart)
    if (nt == 4) MOE_G2BF(4);
    else if (nt == 2) MOE_G2BF(2);
    else MOE_G2BF(1);
#undef MOE_G2BF
}

void launch_gemm1_decode_fp8(const uint8_t* xq, const float* xscale, const void* w1,
                             const float* w1_scale, int rowwise, const int32_t* sorted_ids,
                             const int32_t* block_expert, const int32_t* num_padded, int M,
                             int topk, int nslots, int K, int N, int max_blocks, int nt,
                             float* act, uint32_t* amax, hipStream_t s) {
    dim3 grid(N / 64, max_blocks);
#define MOE_G1F8(NT)                                                                         \
    gemm1_decode_fp8_kernel<NT><<<grid, 256, 0, s>>>(xq, xscale, (const uint8_t*)w1, w1_scale, \
                                                     rowwise, sorted_ids, block_expert,        \
                                                     num_padded, M, topk, nslots, K, N, act, amax)
    if (nt == 4) MOE_G1F8(4);
    else if (nt == 2) MOE_G1F8(2);
    else MOE_G1F8(1);
#undef MOE_G1F8
}

void launch_act_quant(const float* act, const uint32_t* amax, const int32_t* inv, int nslots,
                      int N, uint8_t* act_q, float* ascale, hipStream_t s) {
    const int nchunk = (N + kActChunk - 1) / kActChunk;
    const long waves = (long)nslots * nchunk;
    act_quant_kernel<<<(int)((waves + 3) / 4), 256, 0, s>>>(act, amax, inv, nslots, N, nchunk,
                                                             act_q, ascale);
}

void launch_gemm2_decode_fp8(const uint8_t* act_q, const float* ascale, const void* w2,
                             const float* w2_scale, int rowwise, const float* topk_w,
                             const int32_t* sorted_ids, const int32_t* block_expert,
                             const int32_t* num_padded, int cap, int nslots, int K, int N,
                             int nsplit, int max_blocks, int nt, float* ypart, hipStream_t s) {
    dim3 grid(K / 128, max_blocks, nsplit);
#define MOE_G2F8(NT)                                                                          \
    gemm2_decode_fp8_kernel<NT><<<grid, 256, 0, s>>>(act_q, ascale, (const uint8_t*)w2,         \
                                                     w2_scale, rowwise, topk_w, sorted_ids,    \
                                                     block_expert, num_padded, cap, nslots, K, \
                                                     N, nsplit, ypart)
    if (nt == 4) MOE_G2F8(4);
    else if (nt == 2) MOE_G2F8(2);
    else MOE_G2F8(1);
#undef MOE_G2F8
}

void launch_gemm1_decode_mxfp4(const uint8_t* xq, const float* xscale, const void* w1,
                               const uint8_t* w1e8, const int32_t* sorted_ids,
                               const int32_t* block_expert, const int32_t* num_padded, int M,
                               int topk, int nslots, int K, int N, int max_blocks, int nt,
                               float* act, uint32_t* amax, hipStream_t s) {
    dim3 grid(N / (64 * kMxTiles1), max_blocks);
    // 4 waves x (gate + up) x 16*RT rows x K/32 scale bytes; K <= 16384 keeps
    // it within the default 64 KB (checked by the caller)
    const size_t lds = (size_t)4 * 2 * 16 * kMxTiles1 * (K / 32);
#define MOE_G1MX(NT)                                                                          \
    gemm1_decode_mxfp4_kernel<NT><<<grid, 256, lds, s>>>(xq, xscale, (const uint8_t*)w1, w1e8, \
                                                         sorted_ids, block_expert, num_padded, \
                                                         M, topk, nslots, K, N, act, amax)
    if (nt == 4) MOE_G1MX(4);
    else if (nt == 2) MOE_G1MX(2);
    else MOE_G1MX(1);
#undef MOE_G1MX
}

void launch_gemm2_decode_mxfp4(const uint8_t* act_q, const float* ascale, const void* w2,
                               const uint8_t* w2e8, const float* topk_w,
                               const int32_t* sorted_ids, const int32_t* block_expert,
                               const int32_t* num_padded, int cap, int nslots, int K, int N,
                               int nsplit, int max_blocks, int nt, float* ypart, hipStream_t s) {
    dim3 grid(K / (64 * kMxTiles2), max_blocks, nsplit);
    // 4 waves x 16*RT rows x (N/nsplit)/32 scale bytes; N/nsplit <= 8192
    // keeps it within 64 KB (ensured by the caller's split choice)
    const size_t lds = (size_t)4 * 16 * kMxTiles2 * (N / nsplit / 32);
#define MOE_G2MX(NT)                                                                          \
    gemm2_decode_mxfp4_kernel<NT><<<grid, 256, lds, s>>>(act_q, ascale, (const uint8_t*)w2,     \
                                                         w2e8, topk_w, sorted_ids, block_expert,\
                                                         num_padded, cap, nslots, K, N, nsplit, \
                                                         ypart)
    if (nt == 4) MOE_G2MX(4);
    else if (nt == 2) MOE_G2MX(2);
    else MOE_G2MX(1);
#undef MOE_G2MX
}

}  // namespace moe
