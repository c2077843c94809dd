// gemm_prefill.hip -- grouped expert GEMMs with full MFMA tiles, for many
// rows per expert.
//
// The fused MoE of "Mixture-of-Experts kernel engineering on Amazon
// SageMaker AI" (summary text) groups all active experts into one launch;
// with hundreds of token rows per expert the GEMMs are MFMA-bound, so each
// workgroup computes a full TW (weight rows) x TT (token rows) tile from
// LDS with 32x32x16 bf16 (or 32x32x64 e4m3) MFMAs; the launchers use
// 256 x 256 tiles, or 256 weight rows x 128 tokens when the experts receive
// few rows (each token block re-reads its expert's weights, so the token
// tile sets the weight traffic).  Weights stay in the pages' B^T layout
// (output-major, reduction dimension contiguous) on the MFMA row dimension,
// as in the decode kernels; tokens are the columns, gathered through the
// expert-sorted row list for GEMM1 and contiguous for GEMM2.
//
// Waves: NW per workgroup, WW along the weight rows and NW/WW along the
// token columns.  In GEMM1 the workgroup's weight rows are TW/2 gate rows followed
// by the matching TW/2 up rows and each wave takes the same n-range from
// both halves, so SiLU(gate)*up is formed from its own accumulators.
//
// Staging: both operand tiles are copied global -> LDS by the gfx950 buffer
// loads with an LDS destination (no register round trip) into rings of
// slots (one for the weights, one for the tokens; their lengths may differ
// by one).  The bf16 256 x 256 tiles run the ping-pong core (PingPongCore:
// two groups of four waves a phase apart, so one group's LDS reads, copies
// and barrier waits overlap the other group's MFMAs); the other tiles run
// PrefillCore, whose waves all read, copy and compute in step.
// Each K-step waits (vmcnt) for its own slots, meets the workgroup at one raw
// s_barrier (the __syncthreads fence would wait for every in-flight copy),
// issues each operand's copy as many steps ahead as its ring allows and runs
// its MFMAs.  Padding token rows (sentinels) copy token row 0 for GEMM1 / the
// block's first act row for GEMM2: an MFMA output column depends only on its
// own B column, and those columns are never stored.
//
// GEMM2 may split its reduction (N) across workgroups into fp32 partial
// rows (combined later in a fixed order), because K/TW weight tiles per
// token block are too few to fill the chip in whole waves of workgroups.
//
// Tile order: the linear workgroup id is dealt to the 8 XCDs round-robin by
// the hardware; each XCD is given a contiguous range of tiles, and tiles are
// numbered so that a run of consecutive ids covers G weight tiles for
// successive token blocks, so workgroups resident on one XCD share both
// operands in its L2 (G = 4 for both GEMMs: the measured minimum of time).
//
// 32x32x16 layouts (gfx950): lane l supplies row/column (l % 32) with the
// K-slice 8*(l/32)..+8 for both operands; the accumulator lane l holds
// D[8*(v/4) + 4*(l/32) + v%4][l % 32], v = 0..15.
#include "common.hpp"
#include "launch.hpp"
#include "tuning.hpp"

#include <type_traits>

namespace moe {

typedef __amdgpu_buffer_rsrc_t prsrc_t;

__device__ __forceinline__ prsrc_t pmake_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x16_t mfma32_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// e4m3 x e4m3, 64-deep; block scales fixed at 2^0 (E8M0 code 127)
__device__ __forceinline__ f32x16_t mfma32_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Tile schedule.  The hardware deals workgroup g to XCD g % 8; each XCD is
// given a contiguous range of tiles, numbered with G weight tiles varying
// fastest, then token blocks, so the workgroups resident on one XCD at a
// time cover a G x (resident/G) block of tiles whose weight
// and token panels they share in that XCD's L2.  The walk below also
// supports a persistent grid (fewer workgroups than tiles, each taking
// every nslot-th tile of its XCD's range); the launchers size the grid to
// one tile per workgroup, which measured less memory traffic.
template <int G>
struct TileWalk {
    int xcd, slot, nslot, per_xcd, total, n_wtiles, n_blocks, r;
    __device__ TileWalk(int n_wt, int n_blk) {
        const int g = (int)blockIdx.x;
        xcd = g % 8;
        slot = g / 8;
        nslot = (int)gridDim.x / 8;
        n_wtiles = n_wt;
        n_blocks = n_blk;
        total = n_wt * n_blk;
        per_xcd = (total + 7) / 8;
        r = 0;
    }
    // next tile of this workgroup; false when its share is done
    __device__ bool next(int& wt, int& blk) {
        const int local = r * nslot + slot;
        ++r;
        if (local >= per_xcd) return false;
        const int t = xcd * per_xcd + local;
        if (t >= total) return false;
        const int span = G * n_blocks;
        const int grp = t / span;
        const int in = t % span;
        const int gsize = min(G, n_wtiles - grp * G);
        wt = grp * G + in % gsize;
        blk = in / gsize;
        return true;
    }
};

// LDS rows: each operand row of a K-step is its BK elements (64 or 128
// bytes) without padding, its 16-byte chunks permuted by an XOR of the row
// index (swz, keyed by the chunks per row) so
// that the 16 consecutive rows an MFMA operand read touches in one LDS cycle
// land in distinct banks.  The DMA writes 1 KB per wave instruction in lane
// order, so lane l of an instruction covering rows r0.. stores physical
// chunk (l % CPR) of row r0 + l / CPR and therefore fetches logical chunk
// (l % CPR) ^ swz(row) from global memory.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    static_assert(CPR == 4 || CPR == 8, "64- or 128-byte LDS rows");
    if constexpr (CPR == 4) return ((r >> 1) & 3) ^ ((r >> 3) & 1);
    else return (r & 7) ^ ((r >> 3) & 1);
}

// s_waitcnt vmcnt(N) leaving the LDS/export counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The wave's LDS accesses issued so far are complete (lgkmcnt(0)), and the
// compiler moves no memory access across this point.  A wave's LDS
// instructions execute in order, so after it the wave's lanes read what its
// other lanes wrote before it.
__device__ __forceinline__ void lds_wave_fence() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// v, computed where it is used: an epilogue address derived from it is not
// hoisted to the kernel's start, where it would hold a register through the
// main loop (the ping-pong loops use all 256)
__device__ __forceinline__ int late_uniform(int v) {
    __asm__ volatile("" : "+s"(v));
    return v;
}

// Epilogue staging of fp32 results through a ping-pong wave's own LDS area
// (kStagedRowsBytes: 64 token rows x 64 columns plus the rows' 64 slots).
// Stored straight from the 32x32 accumulator layout, a store instruction
// writes 16 or 32 bytes to each of 32 rows; staged, it writes four rows'
// whole 256-byte segments.  stage_put places the values of output columns
// 32a + 8vg + 4*(lane/32) + 0..3 (a = 0, 1: a 64-column pass) of token row
// 32b + lane%32; stage_slots records the rows' slots; stage_flush sends the
// 64 staged rows to their destination rows, row j to dst + j*ld (contiguous
// rows) or with SCATTER to dst + slot[j]*ld, skipping padding rows (slot[j]
// >= nslots).
constexpr int kStagedRowBytes = 64 * 4 + 16;  // the pad spreads a column's rows over the banks
constexpr int kStagedRowsBytes = 64 * kStagedRowBytes + 64 * 4;

// the lane's index, computed where it is used: per-lane epilogue addresses
// are not hoisted to the kernel's start, where they would hold registers
// through the main loop
__device__ __forceinline__ int late_lane() {
    int v;
    __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
    return v;
}

// lane: late_lane() of the epilogue
__device__ __forceinline__ void stage_put(char* st, int lane, int b, int a, int vg, f32x4_t v) {
    *reinterpret_cast<f32x4_t*>(st + (b * 32 + (lane & 31)) * kStagedRowBytes +
                                (a * 32 + 8 * vg + 4 * (lane >> 5)) * 4) = v;
}

// slot of token row 32b + lane%32: row_p[b] (both lane halves write the same value)
template <int FT>
__device__ __forceinline__ void stage_slots(char* st, int lane, const int (&row_p)[FT]) {
    int* slot = reinterpret_cast<int*>(st + 64 * kStagedRowBytes);
#pragma unroll
    for (int b = 0; b < FT; ++b) slot[b * 32 + (lane & 31)] = row_p[b];
}

template <bool SCATTER>
__device__ __forceinline__ void stage_flush(const char* st, int lane, float* dst, size_t ld,
                                            int nslots) {
    const int rr = lane >> 4, c = lane & 15;
    const int* slot = reinterpret_cast<const int*>(st + 64 * kStagedRowBytes);
    lds_wave_fence();  // the wave's stage_put writes are done
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = 4 * i + rr;
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(st + row * kStagedRowBytes + c * 16);
        const int p = slot[row];
        if (p < nslots)
            *reinterpret_cast<f32x4_t*>(dst + (size_t)(SCATTER ? p : row) * ld + c * 4) = v;
    }
    lds_wave_fence();  // its reads are done before the area is written again
}

// A wave's 64 token rows x WR results scattered to the rows of their slots
// (row_p[j / 32] of lane j % 32 for token row j) in 64-column passes;
// val(a, b, vg) gives accumulator (a, b)'s values 4vg..4vg+3.
template <int WR, int FT, typename Val>
__device__ __forceinline__ void store_rows_staged(char* st, const Val& val, const int (&row_p)[FT],
                                                  int nslots, float* dst, int ld) {
    static_assert(FT == 2 && WR % 64 == 0, "64 token rows, 64-column passes");
    const int lane = late_lane();
    lds_wave_fence();
    stage_slots(st, lane, row_p);
#pragma unroll
    for (int pass = 0; pass < WR / 64; ++pass) {
#pragma unroll
        for (int b = 0; b < FT; ++b)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) stage_put(st, lane, b, a, vg, val(2 * pass + a, b, vg));
        stage_flush<true>(st, lane, dst + pass * 64, (size_t)ld, nslots);
    }
}

// The shared main loop.  The weight rows and the token rows of each K-step
// stream through two LDS rings, of WST and XST slots: the weight copy of a
// step is issued WST-1 steps ahead, the token copy XST-1 steps ahead (when
// LDS runs out one operand gets the shorter lead).  At step s every wave
// issues the token copy of step s+XST-1 and the weight copy of step s+WST-1
// into the slots step s-1 used; before the last MFMAs of step s it waits
// (vmcnt) for its own copies of step s+1, meets the workgroup at one raw
// s_barrier (the __syncthreads fence would wait for every copy in flight),
// and reads the first fragments of step s+1, so those MFMAs cover the
// barrier and the LDS latency.  The barrier also proves that every wave is
// done reading step s, whose slots the copies issued at step s+1 overwrite.
template <int TW, int TT, int BK, int WST, int XST, int WW, int NW, bool F8 = false>
struct PrefillCore {
    static constexpr int kRowBytes = F8 ? BK : BK * 2;
    static constexpr int kCPR = kRowBytes / 16;             // 16-B chunks per row
    static constexpr int kRowsPerInstr = 64 / kCPR;         // rows one wave instruction covers
    static constexpr int kWInstr = TW / kRowsPerInstr / NW; // per wave per step
    static constexpr int kXInstr = TT / kRowsPerInstr / NW;
    static constexpr int kWSlot = TW * kRowBytes;
    static constexpr int kXSlot = TT * kRowBytes;
    static constexpr int kXBase = WST * kWSlot;
    static constexpr int kLdsBytes = WST * kWSlot + XST * kXSlot;
    static constexpr int WT = NW / WW;                      // waves along the token dimension
    static constexpr int FW = TW / WW / 32;                 // 32-row A tiles per wave
    static constexpr int FT = TT / WT / 32;                 // 32-column B tiles per wave
    // MFMA k-slices per step: 16 bf16 (32x32x16) or 64 e4m3 (32x32x64)
    static constexpr int KS = F8 ? BK / 64 : BK / 16;
    static_assert(kWInstr * kRowsPerInstr * NW == TW && kXInstr * kRowsPerInstr * NW == TT,
                  "tile rows must split evenly over the waves' DMA instructions");
    static_assert(WST >= 2 && XST >= 2 && WST - XST <= 1 && XST - WST <= 1,
                  "the two rings' leads differ by at most one step");
    static_assert(KS % 2 == 0, "fragment double buffer alternates per k-slice");
    // Per step the operand with the shorter lead is issued first.  Copies a
    // wave may leave in flight when step s must have landed, given that every
    // younger copy was issued:
    static constexpr bool kWFirst = XST > WST;
    static constexpr int kMinSt = WST < XST ? WST : XST;
    static constexpr int kMaxSt = WST < XST ? XST : WST;
    static constexpr int kLongInstr = WST > XST ? kWInstr : (XST > WST ? kXInstr : 0);
    static constexpr int kYounger = (kMinSt - 2) * (kWInstr + kXInstr) + kLongInstr;

    f32x16_t acc[FW][FT];

    // Row (within the weight / token rows of a step) that lane `lane` of DMA
    // instruction q of wave `wave` fills, and the logical chunk it fetches.
    __device__ static __forceinline__ int dma_row(int wave, int q, int lane) {
        return (q * NW + wave) * kRowsPerInstr + lane / kCPR;
    }
    // the wave's weight-row group (wa) and token-row group of TT/WT rows (wb)
    __device__ static __forceinline__ int wave_a(int wave) { return wave % WW; }
    __device__ static __forceinline__ int wave_b(int wave) { return wave / WW; }
    // after the tile's epilogue (the ping-pong core's last barrier)
    __device__ __forceinline__ void finish(int) {}
    __device__ static __forceinline__ int dma_chunk(int row, int lane) {
        return (lane % kCPR) ^ swz<kCPR>(row);
    }

    // Source offsets at k = kbeg of this lane's chunk: weight copy q reads
    // wvoff + wsoff[q] (wsoff wave-uniform, a scalar operand: the weight rows
    // of a wave's copies differ by whole-row amounts the same for every
    // lane), token copy q reads xoff[q] (gathered rows, per lane).  The A
    // fragments of the wave are LDS rows arow0 + (a % AH)*32 + (a / AH)*AJUMP
    // with AH = FW/2 when AJUMP is non-zero (GEMM1's gate and up halves),
    // else FW; those rows differ by multiples of 16, so they share one
    // swizzle and their LDS offsets differ by constants.  The loop covers
    // klen reduction elements.  With COMPUTE false the wave only takes its
    // share of the copies and barriers (its token columns are all padding):
    // no LDS reads, no MFMAs, accumulators stay zero.
    template <int AJUMP>
    __device__ static constexpr int arow_delta(int a) {
        return AJUMP ? (a % (FW / 2)) * 32 + (a / (FW / 2)) * AJUMP : a * 32;
    }
    template <bool COMPUTE, int AJUMP>
    __device__ __forceinline__ void run(char* lds, prsrc_t rw, uint32_t wvoff,
                                        const uint32_t* wsoff, prsrc_t rx, const uint32_t* xoff,
                                        int klen, int wave, int wb, int arow0) {
        static_assert(AJUMP % 16 == 0, "fragment rows must share one swizzle");
        const int lane = lane_id();
#pragma unroll
        for (int a = 0; a < FW; ++a)
#pragma unroll
            for (int b = 0; b < FT; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

        typedef __attribute__((address_space(3))) void* lds_ptr_t;
        auto dma_w = [&](int step, int slot) {
            const uint32_t kb = (uint32_t)step * kRowBytes;
            char* base = lds + slot * kWSlot;
#pragma unroll
            for (int q = 0; q < kWInstr; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (lds_ptr_t)(base + (q * NW + wave) * 1024), 16, wvoff + kb, wsoff[q], 0,
                    0);
        };
        auto dma_x = [&](int step, int slot) {
            const uint32_t kb = (uint32_t)step * kRowBytes;
            char* base = lds + kXBase + slot * kXSlot;
#pragma unroll
            for (int q = 0; q < kXInstr; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (lds_ptr_t)(base + (q * NW + wave) * 1024), 16, xoff[q] + kb, 0, 0, 0);
        };

        // per-lane LDS read offsets (bytes within a slot) of the first A and
        // B fragment for each k-slice; the other fragments are constant
        // offsets away.  bf16: lane half h reads chunk 2*ks + h (8 elements);
        // e4m3: chunks 4*ks + 2h and 4*ks + 2h + 1 (32 codes), two reads as
        // the swizzle may separate them.  A and B fragments come from the
        // same chunks of their rows, so whatever K order the MFMA assigns to
        // a lane's bytes, each product pairs matching reduction indices.
        const int li = lane & 31, half = lane >> 5;
        constexpr int NC = F8 ? 2 : 1;  // 16-byte reads per fragment
        int aoff[KS][NC], boff[KS][NC];
        {
            const int ra = arow0 + li, rb = wb * (TT / WT) + li;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int h = 0; h < NC; ++h) {
                    const int c = F8 ? 4 * ks + 2 * half + h : 2 * ks + half;
                    aoff[ks][h] = ra * kRowBytes + ((c ^ swz<kCPR>(ra)) << 4);
                    boff[ks][h] = rb * kRowBytes + ((c ^ swz<kCPR>(rb)) << 4);
                }
        }
        typedef typename std::conditional<F8, i32x8_t, bf16x8_t>::type frag_t;
        struct Frags { frag_t a[FW], b[FT]; };
        auto ld = [&](const char* base, const int (&off)[NC]) {
            if constexpr (F8) {
                const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(base + off[0]);
                const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(base + off[1]);
                return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                return *reinterpret_cast<const bf16x8_t*>(base + off[0]);
            }
        };
        auto read = [&](Frags& f, int wslot, int xslot, int ks) {
            if constexpr (!COMPUTE) return;
            const char* wbase = lds + wslot * kWSlot;
            const char* xbase = lds + kXBase + xslot * kXSlot;
#pragma unroll
            for (int a = 0; a < FW; ++a)
                f.a[a] = ld(wbase + arow_delta<AJUMP>(a) * kRowBytes, aoff[ks]);
#pragma unroll
            for (int b = 0; b < FT; ++b) f.b[b] = ld(xbase + b * 32 * kRowBytes, boff[ks]);
        };
        auto mfmas = [&](const Frags& f) {
            if constexpr (!COMPUTE) return;
#pragma unroll
            for (int a = 0; a < FW; ++a)
#pragma unroll
                for (int b = 0; b < FT; ++b) {
                    if constexpr (F8)
                        acc[a][b] = mfma32_fp8(f.a[a], f.b[b], acc[a][b]);
                    else
                        acc[a][b] = mfma32_bf16(f.a[a], f.b[b], acc[a][b]);
                }
        };

        const int steps = klen / BK;
        // the previous tile's last reads of the rings are done before refilling them
        __builtin_amdgcn_s_barrier();
        // prologue: the copies steps 1-kMaxSt .. -1 would have issued
#pragma unroll
        for (int v = 1 - kMaxSt; v < 0; ++v) {
            const int xs = v + XST - 1, ws = v + WST - 1;
            if constexpr (kWFirst) {
                if (ws >= 0 && ws < steps) dma_w(ws, ws);
                if (xs >= 0 && xs < steps) dma_x(xs, xs);
            } else {
                if (xs >= 0 && xs < steps) dma_x(xs, xs);
                if (ws >= 0 && ws < steps) dma_w(ws, ws);
            }
        }
        // wait for step s (issued through step s-1): vmcnt takes an
        // immediate, so the two counts that occur are branches
        auto arrive = [&](int s) {
            if (s + kMaxSt - 2 < steps) wait_vmcnt<kYounger>();
            else wait_vmcnt<0>();
            // this wave's LDS reads of older steps are complete: after the
            // barrier another wave may refill their slots
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
        };
        Frags f[2];
        // one K-step from slots (wsl, xsl); with MORE, step s+1 is published
        // and its first fragments read from (nwsl, nxsl) before the last MFMAs
        auto step = [&](auto more, int s, int wsl, int xsl, int nwsl, int nxsl) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 1 < KS) {
                    read(f[(ks + 1) & 1], wsl, xsl, ks + 1);
                } else if constexpr (decltype(more)::value) {
                    arrive(s + 1);
                    read(f[0], nwsl, nxsl, 0);
                }
                // keep the reads ahead of the MFMAs that hide their latency
                __builtin_amdgcn_sched_barrier(0);
                mfmas(f[ks & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        arrive(0);
        read(f[0], 0, 0, 0);
        int wsl = 0, xsl = 0;  // slots of step s
        int s = 0;
        for (; s + 1 < steps; ++s) {
            const int pw = wsl == 0 ? WST - 1 : wsl - 1;  // slots of step s-1
            const int px = xsl == 0 ? XST - 1 : xsl - 1;
            if constexpr (kWFirst) {
                if (s + WST - 1 < steps) dma_w(s + WST - 1, pw);
                if (s + XST - 1 < steps) dma_x(s + XST - 1, px);
            } else {
                if (s + XST - 1 < steps) dma_x(s + XST - 1, px);
                if (s + WST - 1 < steps) dma_w(s + WST - 1, pw);
            }
            const int nw = wsl + 1 == WST ? 0 : wsl + 1;
            const int nx = xsl + 1 == XST ? 0 : xsl + 1;
            step(std::true_type{}, s, wsl, xsl, nw, nx);
            wsl = nw;
            xsl = nx;
        }
        if (steps > 0) step(std::false_type{}, s, wsl, xsl, wsl, xsl);
#pragma unroll
        for (int a = 0; a < FW; ++a)
#pragma unroll
            for (int b = 0; b < FT; ++b) pin(acc[a][b]);
    }
};

// ---------------------------------------------------------------------------
// The ping-pong main loop for TW x 256 tiles with 8 waves.  The waves form
// two groups of four, A (waves 0-3) and B (waves 4-7), one wave of each per
// SIMD; group A computes token rows 0-127, group B rows 128-255, each wave a
// (TW/2) x 64 tile as in PrefillCore (2 x 2 waves per group).  A K-step is
// two phases per group: a memory phase (read all of the step's fragments
// from LDS into registers, issue DMA copies, wait for earlier copies) and a
// compute phase (the step's MFMAs from registers).  Group B runs one phase
// behind group A, and every phase ends at a workgroup barrier, so while one
// group waits on LDS reads, copies and the barrier the other keeps its
// SIMD's matrix core busy:
//
//   phase    1     2     3     4    ...   2s+1   2s+2  ...  2S+1
//   A       M0    C0    M1    C1          Ms     Cs         (idle)
//   B      (idle) M0    C0    M1          Cs-1   Ms          CS-1
//
// Group A copies the token rows (XST ring slots, issued one step ahead in
// its memory phase, waited for at the end of its compute phase), group B the
// weight rows (WST slots, issued two steps ahead in its memory phase and
// waited for one step later).  A slot of step s is overwritten only after
// the barrier that ends B's memory phase of step s, and a step's copies are
// complete before the barrier that starts A's memory phase of it.
// ---------------------------------------------------------------------------
template <int TW, int BK, int WST, int XST, bool F8 = false>
struct PingPongCore {
    static constexpr int TT = 256, NW = 8;
    static constexpr int kRowBytes = F8 ? BK : BK * 2;
    static constexpr int kCPR = kRowBytes / 16;
    static constexpr int kRowsPerInstr = 64 / kCPR;
    static constexpr int kWInstr = TW / kRowsPerInstr / 4;  // per wave of group B
    static constexpr int kXInstr = TT / kRowsPerInstr / 4;  // per wave of group A
    static constexpr int kWSlot = TW * kRowBytes;
    static constexpr int kXSlot = TT * kRowBytes;
    static constexpr int kXBase = WST * kWSlot;
    static constexpr int kLdsBytes = WST * kWSlot + XST * kXSlot;
    static constexpr int WW = 2;                // waves along the weight rows (per group)
    static constexpr int WT = 4;                // 64-row token quarters of the tile
    static constexpr int FW = TW / WW / 32;     // 32-row A tiles per wave
    static constexpr int FT = 2;                // 32-column B tiles per wave
    // MFMA k-slices per step: 32x32x16 bf16 or 32x32x64 e4m3
    static constexpr int KS = F8 ? BK / 64 : BK / 16;
    static_assert(WST == 3 && XST == 2, "the copy schedule below is written for 3 + 2 slots");
    static_assert(kWInstr * kRowsPerInstr * 4 == TW && kXInstr * kRowsPerInstr * 4 == TT,
                  "tile rows must split evenly over a group's DMA instructions");

    f32x16_t acc[FW][FT];

    // rows copied by instruction q of a wave (its group copies one operand)
    __device__ static __forceinline__ int dma_row(int wave, int q, int lane) {
        return (q * 4 + (wave & 3)) * kRowsPerInstr + lane / kCPR;
    }
    __device__ static __forceinline__ int dma_chunk(int row, int lane) {
        return (lane % kCPR) ^ swz<kCPR>(row);
    }
    __device__ static __forceinline__ int wave_a(int wave) { return (wave & 3) % WW; }
    __device__ static __forceinline__ int wave_b(int wave) { return 2 * (wave >> 2) + (wave & 3) / WW; }
    template <int AJUMP>
    __device__ static constexpr int arow_delta(int a) {
        return AJUMP ? (a % (FW / 2)) * 32 + (a / (FW / 2)) * AJUMP : a * 32;
    }
    // group A's last barrier, matching group B's last compute phase; taken
    // after the tile's epilogue so that A's stores overlap B's last MFMAs,
    // and B's epilogue, which may stage through the same LDS, follows A's
    // (dropping this pairing, so that the two epilogues overlap, measured
    // no faster for the bf16 tiles and 9-18 % slower for the e4m3 and MXFP4
    // GEMM1s)
    __device__ __forceinline__ void finish(int wave) {
        if (wave < 4) __builtin_amdgcn_s_barrier();
    }

    template <bool COMPUTE, int AJUMP>
    __device__ __forceinline__ void run(char* lds, prsrc_t rw, uint32_t wvoff,
                                        const uint32_t* wsoff, prsrc_t rx, const uint32_t* xoff,
                                        int klen, int wave, int wb, int arow0) {
        static_assert(AJUMP % 16 == 0, "fragment rows must share one swizzle");
        const int lane = lane_id();
        const bool grp_b = wave >= 4;  // wave-uniform
        const int gw = wave & 3;
#pragma unroll
        for (int a = 0; a < FW; ++a)
#pragma unroll
            for (int b = 0; b < FT; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

        typedef __attribute__((address_space(3))) void* lds_ptr_t;
        auto dma_w = [&](int step, int slot) {
            const uint32_t kb = (uint32_t)step * kRowBytes;
            char* base = lds + slot * kWSlot;
#pragma unroll
            for (int q = 0; q < kWInstr; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (lds_ptr_t)(base + (q * 4 + gw) * 1024), 16, wvoff + kb, wsoff[q], 0, 0);
        };
        auto dma_x = [&](int step, int slot) {
            const uint32_t kb = (uint32_t)step * kRowBytes;
            char* base = lds + kXBase + slot * kXSlot;
#pragma unroll
            for (int q = 0; q < kXInstr; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (lds_ptr_t)(base + (q * 4 + gw) * 1024), 16, xoff[q] + kb, 0, 0, 0);
        };
        // per-lane LDS offsets of the first A and B fragment of each k-slice
        // (as PrefillCore): bf16 lane half h reads chunk 2*ks + h; e4m3
        // chunks 4*ks + 2h and 4*ks + 2h + 1, the same chunks for both
        // operands, so each product pairs matching reduction indices
        const int li = lane & 31, half = lane >> 5;
        constexpr int NC = F8 ? 2 : 1;  // 16-byte reads per fragment
        int aoff[KS][NC], boff[KS][NC];
        {
            const int ra = arow0 + li, rb = wb * (TT / WT) + li;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int h = 0; h < NC; ++h) {
                    const int c = F8 ? 4 * ks + 2 * half + h : 2 * ks + half;
                    aoff[ks][h] = ra * kRowBytes + ((c ^ swz<kCPR>(ra)) << 4);
                    boff[ks][h] = rb * kRowBytes + ((c ^ swz<kCPR>(rb)) << 4);
                }
        }
        typedef typename std::conditional<F8, i32x8_t, bf16x8_t>::type frag_t;
        auto ld = [&](const char* base, const int (&off)[NC]) {
            if constexpr (F8) {
                const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(base + off[0]);
                const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(base + off[1]);
                return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                return *reinterpret_cast<const bf16x8_t*>(base + off[0]);
            }
        };
        frag_t fa[KS][FW], fb[KS][FT];
        auto read_all = [&](int wslot, int xslot) {
            const char* wbase = lds + wslot * kWSlot;
            const char* xbase = lds + kXBase + xslot * kXSlot;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int a = 0; a < FW; ++a)
                    fa[ks][a] = ld(wbase + arow_delta<AJUMP>(a) * kRowBytes, aoff[ks]);
#pragma unroll
                for (int b = 0; b < FT; ++b) fb[ks][b] = ld(xbase + b * 32 * kRowBytes, boff[ks]);
            }
        };
        auto mfma_all = [&]() {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int a = 0; a < FW; ++a)
#pragma unroll
                    for (int b = 0; b < FT; ++b) {
                        if constexpr (F8)
                            acc[a][b] = mfma32_fp8(fa[ks][a], fb[ks][b], acc[a][b]);
                        else
                            acc[a][b] = mfma32_bf16(fa[ks][a], fb[ks][b], acc[a][b]);
                    }
        };
        auto barrier = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        };

        const int steps = klen / BK;
        // the previous tile's last LDS reads are done before refilling
        barrier();
        // prologue: the token rows of step 0 (A), the weight rows of steps 0
        // and 1 (B); step 0 complete at the first barrier
        if (!grp_b) {
            if (steps > 0) dma_x(0, 0);
            wait_vmcnt<0>();
        } else {
            if (steps > 0) dma_w(0, 0);
            if (steps > 1) {
                dma_w(1, 1);
                wait_vmcnt<kWInstr>();
            } else {
                wait_vmcnt<0>();
            }
        }
        barrier();
        if (grp_b) barrier();  // B sits out phase 1
        int wsl = 0, xsl = 0;  // slots of step s
        for (int s = 0; s < steps; ++s) {
            // ---- memory phase of step s
            if constexpr (COMPUTE) read_all(wsl, xsl);
            if (!grp_b) {
                if (s + 1 < steps) dma_x(s + 1, xsl ^ 1);
            } else {
                if (s + 2 < steps) {
                    dma_w(s + 2, wsl == 0 ? 2 : wsl - 1);  // the slot of step s-1
                    wait_vmcnt<kWInstr>();                  // step s+1 has landed
                } else {
                    wait_vmcnt<0>();
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS reads of step s are done
            barrier();
            // ---- compute phase of step s
            if constexpr (COMPUTE) mfma_all();
            if (!grp_b) wait_vmcnt<0>();  // token rows of step s+1 have landed
            barrier();
            wsl = wsl + 1 == WST ? 0 : wsl + 1;
            xsl ^= 1;
        }
#pragma unroll
        for (int a = 0; a < FW; ++a)
#pragma unroll
            for (int b = 0; b < FT; ++b) pin(acc[a][b]);
    }
};

// ---------------------------------------------------------------------------
// The ping-pong loop for MXFP4 weights (OCP microscaling: e2m1 codes two per
// byte, even element in the low nibble, one E8M0 scale per 32 elements of a
// row) against e4m3 token rows, TW x 256 tiles, 8 waves in the two groups
// and phases of PingPongCore.  A K-step is 128 codes: a weight row is 64
// bytes (16 KB per slot), its 4 scale bytes go to a scale slot (1 KB), a
// token row is 128 bytes (32 KB per slot).  The MFMA is the scaled
// 16x16x128 one with A = e2m1: an FP4 lane of group q holds K 32q ..
// 32q+31 of the step, exactly one MX block, whose E8M0 byte is the lane's
// scale operand; the e4m3 operand's lane group q holds K 16q .. 16q+15 and
// 64+16q .. 64+16q+15 (the layouts the decode MXFP4 kernels use, measured
// on gfx950).  A wave covers (TW/2) x 64 of the tile as 8 x 4 16x16 tiles.
// Group B copies the weight rows and their scales (two steps ahead), group
// A the token rows (one step ahead).
// ---------------------------------------------------------------------------
template <int TW>
struct PingPongMxCore {
    static constexpr int TT = 256, NW = 8, BK = 128;
    static constexpr int WST = 3, XST = 2;
    static constexpr int kWRowBytes = BK / 2;                 // 64
    static constexpr int kXRowBytes = BK;                     // 128
    static constexpr int kWCPR = kWRowBytes / 16;             // 4 chunks per weight row
    static constexpr int kXCPR = kXRowBytes / 16;             // 8 chunks per token row
    static constexpr int kWRowsPerInstr = 64 / kWCPR;         // 16
    static constexpr int kXRowsPerInstr = 64 / kXCPR;         // 8
    static constexpr int kWInstr = TW / kWRowsPerInstr / 4;   // per wave of group B
    static constexpr int kXInstr = TT / kXRowsPerInstr / 4;   // per wave of group A
    static constexpr int kSInstr = 1;                         // TW/4 rows of 4 scale bytes
    static constexpr int kWSlot = TW * kWRowBytes;
    static constexpr int kSSlot = TW * 4;
    static constexpr int kXSlot = TT * kXRowBytes;
    static constexpr int kSBase = WST * kWSlot;
    static constexpr int kXBase = kSBase + WST * kSSlot;
    static constexpr int kLdsBytes = kXBase + XST * kXSlot;
    static constexpr int WW = 2, WT = 4;
    static constexpr int FW = TW / WW / 16;   // 16-row A tiles per wave (8)
    static constexpr int FT = 4;              // 16-column B tiles per wave
    static constexpr int kBInstr = kWInstr + kSInstr;  // a group-B wave's copies per step
    static_assert(TW == 256, "MXFP4 tiles are 256 weight rows");
    static_assert(kWInstr * kWRowsPerInstr * 4 == TW && kXInstr * kXRowsPerInstr * 4 == TT,
                  "tile rows must split evenly over a group's DMA instructions");

    f32x4_t acc[FW][FT];

    // weight row copied by lane `lane` of weight instruction q (group B)
    __device__ static __forceinline__ int w_dma_row(int wave, int q, int lane) {
        return (q * 4 + (wave & 3)) * kWRowsPerInstr + lane / kWCPR;
    }
    __device__ static __forceinline__ int w_dma_chunk(int row, int lane) {
        return (lane % kWCPR) ^ swz<kWCPR>(row);
    }
    // token row copied by lane `lane` of token instruction q (group A)
    __device__ static __forceinline__ int dma_row(int wave, int q, int lane) {
        return (q * 4 + (wave & 3)) * kXRowsPerInstr + lane / kXCPR;
    }
    __device__ static __forceinline__ int dma_chunk(int row, int lane) {
        return (lane % kXCPR) ^ swz<kXCPR>(row);
    }
    // weight row whose 4 scale bytes lane `lane` of a group-B wave copies
    __device__ static __forceinline__ int s_dma_row(int wave, int lane) {
        return (wave & 3) * 64 + lane;
    }
    __device__ static __forceinline__ int wave_a(int wave) { return (wave & 3) % WW; }
    __device__ static __forceinline__ int wave_b(int wave) { return 2 * (wave >> 2) + (wave & 3) / WW; }
    template <int AJUMP>
    __device__ static constexpr int arow_delta(int a) {
        return AJUMP ? (a % (FW / 2)) * 16 + (a / (FW / 2)) * AJUMP : a * 16;
    }
    __device__ __forceinline__ void finish(int wave) {
        if (wave < 4) __builtin_amdgcn_s_barrier();
    }

    // wvoff + wsoff[q]: weight instruction q's source (row offsets and the
    // lane's chunk, at k = 0); svoff: the lane's scale row (at k = 0);
    // xoff[q]: token instruction q's source.  klen in codes.
    template <bool COMPUTE, int AJUMP>
    __device__ __forceinline__ void run(char* lds, prsrc_t rw, uint32_t wvoff,
                                        const uint32_t* wsoff, prsrc_t rs, uint32_t svoff,
                                        prsrc_t rx, const uint32_t* xoff, int klen, int wave,
                                        int wb, int arow0) {
        static_assert(AJUMP % 16 == 0, "fragment rows must share one swizzle");
        const int lane = lane_id();
        const bool grp_b = wave >= 4;
        const int gw = wave & 3;
#pragma unroll
        for (int a = 0; a < FW; ++a)
#pragma unroll
            for (int b = 0; b < FT; ++b) acc[a][b] = f32x4_t{0, 0, 0, 0};

        typedef __attribute__((address_space(3))) void* lds_ptr_t;
        auto dma_w = [&](int step, int slot) {
            char* base = lds + slot * kWSlot;
#pragma unroll
            for (int q = 0; q < kWInstr; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (lds_ptr_t)(base + (q * 4 + gw) * 1024), 16,
                    wvoff + (uint32_t)step * kWRowBytes, wsoff[q], 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (lds_ptr_t)(lds + kSBase + slot * kSSlot + gw * 256), 4,
                svoff + (uint32_t)step * 4, 0, 0, 0);
        };
        auto dma_x = [&](int step, int slot) {
            char* base = lds + kXBase + slot * kXSlot;
#pragma unroll
            for (int q = 0; q < kXInstr; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (lds_ptr_t)(base + (q * 4 + gw) * 1024), 16,
                    xoff[q] + (uint32_t)step * kXRowBytes, 0, 0, 0);
        };
        const int li = lane & 15, q4 = lane >> 4;
        int aoff, boff[2], soff;
        {
            const int ra = arow0 + li, rb = wb * (TT / WT) + li;
            aoff = ra * kWRowBytes + ((q4 ^ swz<kWCPR>(ra)) << 4);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                boff[h] = rb * kXRowBytes + (((4 * h + q4) ^ swz<kXCPR>(rb)) << 4);
            soff = ra * 4;
        }
        i32x4_t fa[FW];
        i32x8_t fb[FT];
        int sc[FW];
        auto read_all = [&](int wslot, int xslot) {
            const char* wbase = lds + wslot * kWSlot;
            const char* sbase = lds + kSBase + wslot * kSSlot;
            const char* xbase = lds + kXBase + xslot * kXSlot;
#pragma unroll
            for (int a = 0; a < FW; ++a) {
                fa[a] = *reinterpret_cast<const i32x4_t*>(wbase + arow_delta<AJUMP>(a) * kWRowBytes +
                                                          aoff);
                sc[a] = *reinterpret_cast<const int*>(sbase + arow_delta<AJUMP>(a) * 4 + soff);
            }
#pragma unroll
            for (int b = 0; b < FT; ++b) {
                const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(xbase + b * 16 * kXRowBytes +
                                                                     boff[0]);
                const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(xbase + b * 16 * kXRowBytes +
                                                                     boff[1]);
                fb[b] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        };
        auto mfma_all = [&]() {
#pragma unroll
            for (int a = 0; a < FW; ++a) {
                const int sa = (sc[a] >> (8 * q4)) & 0xff;
                const i32x8_t a8 = {fa[a][0], fa[a][1], fa[a][2], fa[a][3], 0, 0, 0, 0};
#pragma unroll
                for (int b = 0; b < FT; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a8, fb[b], acc[a][b], 4, 0, 0, sa, 0, 127);
            }
        };
        auto barrier = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        };

        const int steps = klen / BK;
        barrier();
        if (!grp_b) {
            if (steps > 0) dma_x(0, 0);
            wait_vmcnt<0>();
        } else {
            if (steps > 0) dma_w(0, 0);
            if (steps > 1) {
                dma_w(1, 1);
                wait_vmcnt<kBInstr>();
            } else {
                wait_vmcnt<0>();
            }
        }
        barrier();
        if (grp_b) barrier();
        int wsl = 0, xsl = 0;
        for (int s = 0; s < steps; ++s) {
            if constexpr (COMPUTE) read_all(wsl, xsl);
            if (!grp_b) {
                if (s + 1 < steps) dma_x(s + 1, xsl ^ 1);
            } else {
                if (s + 2 < steps) {
                    dma_w(s + 2, wsl == 0 ? 2 : wsl - 1);
                    wait_vmcnt<kBInstr>();
                } else {
                    wait_vmcnt<0>();
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            barrier();
            if constexpr (COMPUTE) mfma_all();
            if (!grp_b) wait_vmcnt<0>();
            barrier();
            wsl = wsl + 1 == WST ? 0 : wsl + 1;
            xsl ^= 1;
        }
#pragma unroll
        for (int a = 0; a < FW; ++a)
#pragma unroll
            for (int b = 0; b < FT; ++b) pin(acc[a][b]);
    }
};

// ---------------------------------------------------------------------------
// GEMM1 + SiLU*up (bf16).  Weight tile wt covers n in [wt*TW/2, (wt+1)*TW/2):
// LDS weight rows [0,TW/2) are those gate rows, [TW/2,TW) the up rows.
// ---------------------------------------------------------------------------
template <int TW, int TT, int BK, int WST, int XST, int WW, int NW, int OCC, int GROUP,
          bool PP = false>
__global__ __launch_bounds__(NW * 64, OCC) void gemm1_prefill_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int M, int topk, int nslots, int K, int N,
    int max_blocks, uint16_t* __restrict__ act) {
    // PP: the ping-pong core (256 token rows, 8 waves)
    using Core = typename std::conditional<PP, PingPongCore<TW, BK, WST, XST>,
                                           PrefillCore<TW, TT, BK, WST, XST, WW, NW>>::type;
    static_assert(!PP || (TT == 256 && NW == 8), "the ping-pong core takes 256-row tiles");
    __shared__ __attribute__((aligned(1024))) char lds[Core::kLdsBytes];
    constexpr int HW = TW / 2;  // n-values per tile
    constexpr int WN = HW / WW; // n-values per wave

    const int npad = *num_padded;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int wa = Core::wave_a(wave), wb = Core::wave_b(wave);
    TileWalk<GROUP> walk(N / HW, max_blocks);
    int wt, blk;
    while (walk.next(wt, blk)) {
    if (blk * TT >= npad) continue;
    const int e = block_expert[blk];

    const size_t row_bytes = (size_t)K * 2;
    const prsrc_t rw = pmake_rsrc(w1 + (size_t)e * 2 * N * K, (uint32_t)(2 * (size_t)N * row_bytes));
    const prsrc_t rx = pmake_rsrc(x, (uint32_t)((size_t)M * row_bytes));
    // weight copy q covers LDS rows q*NW*R + wave*R .. +R (R rows per copy,
    // a multiple of 8 never straddling the gate/up boundary HW): its global
    // rows are those of copy 0 moved by a wave-uniform amount
    uint32_t wsoff[Core::kWInstr], xoff[Core::kXInstr];
    const int row0 = Core::dma_row(wave, 0, lane);
    const uint32_t wvoff = (uint32_t)((wt * HW + row0) * row_bytes) +
                           Core::dma_chunk(row0, lane) * 16;
#pragma unroll
    for (int q = 0; q < Core::kWInstr; ++q) {
        const int first = Core::dma_row(wave, q, 0);  // wave-uniform
        const int shift = first - Core::dma_row(wave, 0, 0) + (first >= HW ? N - HW : 0);
        wsoff[q] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(shift * row_bytes));
    }
    // all of the wave's row loads first, in flight together
    int pv[Core::kXInstr];
#pragma unroll
    for (int q = 0; q < Core::kXInstr; ++q) pv[q] = sorted_ids[blk * TT + Core::dma_row(wave, q, lane)];
#pragma unroll
    for (int q = 0; q < Core::kXInstr; ++q) {
        const int row = Core::dma_row(wave, q, lane);
        const int t = pv[q] < nslots ? slot_token(pv[q], topk) : 0;
        xoff[q] = (uint32_t)(t * row_bytes) + Core::dma_chunk(row, lane) * 16;
    }
    // A tiles of this wave: its gate frags (LDS rows wa*WN + 32a), then the
    // matching up frags HW rows further
    // the epilogue's rows, looked up before the main loop: their loads
    // overlap the first copies instead of trailing the last MFMAs
    bool row_ok[Core::FT];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b)
        row_ok[b] = sorted_ids[blk * TT + wb * (TT / Core::WT) + b * 32 + (lane & 31)] < nslots;
    Core core;
    // a wave whose token rows are all padding (the tail of an expert's last
    // block) skips its MFMAs
    const bool wave_valid = sorted_ids[blk * TT + wb * (TT / Core::WT)] < nslots;
    if (wave_valid)
        core.template run<true, HW>(lds, rw, wvoff, wsoff, rx, xoff, K, wave, wb, wa * WN);
    else
        core.template run<false, HW>(lds, rw, wvoff, wsoff, rx, xoff, K, wave, wb, wa * WN);

    const int li = lane & 31;
    if constexpr (PP) {
        // The wave's 64 token rows x WN values go out through its own LDS
        // area (the rings are idle once the group's last step is done), so
        // that each store instruction writes whole 128-byte row segments
        // (from the accumulator layout an instruction would write 16 bytes
        // of each of 32 rows); the rows' validity is staged beside them.
        if (wave_valid) {
            constexpr int kSt = WN * 2 + 16;  // staged row bytes; the pad spreads the banks
            constexpr int kArea = 64 * kSt + 64 * 4;
            static_assert(4 * kArea <= Core::kLdsBytes, "the staging fits the rings");
            char* st = lds + (wave & 3) * kArea;
            int* ok = reinterpret_cast<int*>(st + 64 * kSt);
            const int ln = late_lane(), lj = ln & 31;
            // the rows' slots, loaded here (through the main loop they would
            // hold registers) and needed only after the SiLU products
            int pe[Core::FT];
#pragma unroll
            for (int b = 0; b < Core::FT; ++b)
                pe[b] = sorted_ids[blk * TT + wb * (TT / Core::WT) + b * 32 + lj];
            lds_wave_fence();
#pragma unroll
            for (int b = 0; b < Core::FT; ++b) {
#pragma unroll
                for (int a = 0; a < Core::FW / 2; ++a)
#pragma unroll
                    for (int vg = 0; vg < 4; ++vg) {
                        float h[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            h[v] = silu(core.acc[a][b][vg * 4 + v]) *
                                   core.acc[a + Core::FW / 2][b][vg * 4 + v];
                        *reinterpret_cast<uint2*>(st + (b * 32 + lj) * kSt +
                                                  (a * 32 + 8 * vg + 4 * (ln >> 5)) * 2) =
                            make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                    }
            }
#pragma unroll
            for (int b = 0; b < Core::FT; ++b)
                ok[b * 32 + lj] = pe[b] < nslots;  // both lane halves write the same value
            lds_wave_fence();
            constexpr int kCpr = WN * 2 / 16;  // 16-byte chunks per row
            constexpr int kRpi = 64 / kCpr;    // rows per instruction
            const int rr = ln / kCpr, c = ln % kCpr;
            uint16_t* dst = act + (size_t)(blk * TT + wb * (TT / Core::WT) + rr) * N + wt * HW +
                            wa * WN + c * 8;
#pragma unroll
            for (int i = 0; i < 64 / kRpi; ++i) {
                const uint4 v = *reinterpret_cast<const uint4*>(st + (i * kRpi + rr) * kSt + c * 16);
                if (ok[i * kRpi + rr]) *reinterpret_cast<uint4*>(dst + (size_t)i * kRpi * N) = v;
            }
            lds_wave_fence();
        }
    } else {
#pragma unroll
    for (int b = 0; b < Core::FT; ++b) {
        const int r = blk * TT + wb * (TT / Core::WT) + b * 32 + li;
        if (!row_ok[b]) continue;
#pragma unroll
        for (int a = 0; a < Core::FW / 2; ++a) {
            uint16_t* dst = act + (size_t)r * N + wt * HW + wa * WN + a * 32 + 4 * (lane >> 5);
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                float h[4];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    h[v] = silu(core.acc[a][b][vg * 4 + v]) *
                           core.acc[a + Core::FW / 2][b][vg * 4 + v];
                *reinterpret_cast<uint2*>(dst + 8 * vg) =
                    make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
            }
        }
    }
    }
    core.finish(wave);
    }  // tiles
}

// ---------------------------------------------------------------------------
// GEMM2 (bf16): weight tile wt covers output rows wt*TW..+TW; the epilogue
// multiplies by the routing weight and scatters token row r to slot p.
// ---------------------------------------------------------------------------
template <int TW, int TT, int BK, int WST, int XST, int WW, int NW, int OCC, int GROUP,
          bool PP = false>
__global__ __launch_bounds__(NW * 64, OCC) void gemm2_prefill_bf16_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int cap,
    int nslots, int K, int N, int nsplit, int max_blocks, float* __restrict__ ypart) {
    using Core = typename std::conditional<PP, PingPongCore<TW, BK, WST, XST>,
                                           PrefillCore<TW, TT, BK, WST, XST, WW, NW>>::type;
    static_assert(!PP || (TT == 256 && NW == 8), "the ping-pong core takes 256-row tiles");
    __shared__ __attribute__((aligned(1024))) char lds[Core::kLdsBytes];
    constexpr int WR = TW / WW;  // output rows per wave

    // the split index is the slowest-varying part of the weight-tile index
    const int n_wt = K / TW;
    const int npad = *num_padded;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int wa = Core::wave_a(wave), wb = Core::wave_b(wave);
    TileWalk<GROUP> walk(n_wt * nsplit, max_blocks);
    int wtz, blk;
    while (walk.next(wtz, blk)) {
    if (blk * TT >= npad) continue;
    const int wt = wtz % n_wt, z = wtz / n_wt;
    const int nlen = N / nsplit, nbeg = z * nlen;
    const int e = block_expert[blk];

    const size_t row_bytes = (size_t)N * 2;
    const prsrc_t rw = pmake_rsrc(w2 + ((size_t)e * K + (size_t)wt * TW) * N,
                                  (uint32_t)(TW * row_bytes));
    const prsrc_t ra = pmake_rsrc(act, (uint32_t)((size_t)cap * row_bytes));
    uint32_t wsoff[Core::kWInstr], aoff[Core::kXInstr];
    const int row0 = Core::dma_row(wave, 0, lane);
    const uint32_t wvoff = (uint32_t)(row0 * row_bytes) + nbeg * 2 +
                           Core::dma_chunk(row0, lane) * 16;
#pragma unroll
    for (int q = 0; q < Core::kWInstr; ++q)
        wsoff[q] = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)((Core::dma_row(wave, q, 0) - Core::dma_row(wave, 0, 0)) * row_bytes));
#pragma unroll
    for (int q = 0; q < Core::kXInstr; ++q) {
        const int row = Core::dma_row(wave, q, lane);
        // padding rows (never written by GEMM1) copy the block's first row
        // instead, an L2 hit; their columns are never stored
        const int src = sorted_ids[blk * TT + row] < nslots ? blk * TT + row : blk * TT;
        aoff[q] = (uint32_t)(src * row_bytes) + nbeg * 2 + Core::dma_chunk(row, lane) * 16;
    }
    Core core;
    // A tiles of this wave: LDS rows wa*WR + 32a
    const bool wave_valid = sorted_ids[blk * TT + wb * (TT / Core::WT)] < nslots;
    if (wave_valid)
        core.template run<true, 0>(lds, rw, wvoff, wsoff, ra, aoff, nlen, wave, wb, wa * WR);
    else
        core.template run<false, 0>(lds, rw, wvoff, wsoff, ra, aoff, nlen, wave, wb, wa * WR);

    const int li = lane & 31;
    // the epilogue's rows: all slots, then all routing weights, loaded
    // together (kept out of the main loop, whose registers are full)
    int row_p[Core::FT];
    float row_w[Core::FT];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b)
        row_p[b] = sorted_ids[blk * TT + wb * (TT / Core::WT) + b * 32 + li];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b) row_w[b] = row_p[b] < nslots ? topk_w[row_p[b]] : 0.0f;
    if constexpr (PP) {
        // the wave's 64 token rows x WR partial sums go out through its own
        // LDS area (the rings are idle once the group's last step is done)
        static_assert(4 * kStagedRowsBytes <= Core::kLdsBytes, "the staging fits the rings");
        if (wave_valid)
            store_rows_staged<WR>(
                lds + late_uniform(wave & 3) * kStagedRowsBytes,
                [&](int a, int b, int vg) {
                    f32x4_t o;
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[v] = core.acc[a][b][vg * 4 + v] * row_w[b];
                    return o;
                },
                row_p, nslots, ypart + (size_t)z * nslots * K + wt * TW + wa * WR, K);
    } else {
#pragma unroll
    for (int b = 0; b < Core::FT; ++b) {
        const int p = row_p[b];
        if (p >= nslots) continue;
        const float w = row_w[b];
#pragma unroll
        for (int a = 0; a < Core::FW; ++a) {
            float* dst = ypart + ((size_t)z * nslots + p) * K + wt * TW + wa * WR + a * 32 +
                         4 * (lane >> 5);
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
    core.finish(wave);
    }  // tiles
}

// ---------------------------------------------------------------------------
// FP8 (OCP e4m3) weights and per-token e4m3 activations on the same tiles:
// 128-code K-steps (128-byte LDS rows, as the bf16 kernels' 64-element
// steps), two 32x32x64 MFMAs per step and fragment.  The epilogues apply the
// scales where the decode FP8 kernels do: GEMM1 multiplies the gate and up
// accumulators by s_x[t] times the row's (or the expert's) W1 scale, forms
// SiLU(gate)*up in fp32, stores it and folds each row's |act| max into
// amax[r] (float bits, atomicMax: exact and order-free for non-negative
// values); GEMM2 multiplies by the output row's (or expert's) W2 scale, the
// sorted row's activation scale s_a[r] and the routing weight.
// ---------------------------------------------------------------------------
template <int TW, int TT, int BK, int WST, int XST, int WW, int NW, int OCC, int GROUP,
          bool PP = false>
__global__ __launch_bounds__(NW * 64, OCC) void gemm1_prefill_fp8_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xscale,
    const uint8_t* __restrict__ w1, const float* __restrict__ w1_scale, int rowwise,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int M, int topk, int nslots, int K, int N,
    int max_blocks, float* __restrict__ act, uint32_t* __restrict__ amax) {
    using Core = typename std::conditional<PP, PingPongCore<TW, BK, WST, XST, true>,
                                           PrefillCore<TW, TT, BK, WST, XST, WW, NW, true>>::type;
    static_assert(!PP || (TT == 256 && NW == 8), "the ping-pong core takes 256-row tiles");
    __shared__ __attribute__((aligned(1024))) char lds[Core::kLdsBytes];
    constexpr int HW = TW / 2;  // n-values per tile
    constexpr int WN = HW / WW; // n-values per wave

    const int npad = *num_padded;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int wa = Core::wave_a(wave), wb = Core::wave_b(wave);
    TileWalk<GROUP> walk(N / HW, max_blocks);
    int wt, blk;
    while (walk.next(wt, blk)) {
    if (blk * TT >= npad) continue;
    const int e = block_expert[blk];

    const size_t row_bytes = (size_t)K;
    const prsrc_t rw = pmake_rsrc(w1 + (size_t)e * 2 * N * K, (uint32_t)(2 * (size_t)N * row_bytes));
    const prsrc_t rx = pmake_rsrc(xq, (uint32_t)((size_t)M * row_bytes));
    uint32_t wsoff[Core::kWInstr], xoff[Core::kXInstr];
    const int row0 = Core::dma_row(wave, 0, lane);
    const uint32_t wvoff = (uint32_t)((wt * HW + row0) * row_bytes) +
                           Core::dma_chunk(row0, lane) * 16;
#pragma unroll
    for (int q = 0; q < Core::kWInstr; ++q) {
        const int first = Core::dma_row(wave, q, 0);  // wave-uniform
        const int shift = first - Core::dma_row(wave, 0, 0) + (first >= HW ? N - HW : 0);
        wsoff[q] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(shift * row_bytes));
    }
    // all of the wave's row loads first, in flight together
    int pv[Core::kXInstr];
#pragma unroll
    for (int q = 0; q < Core::kXInstr; ++q) pv[q] = sorted_ids[blk * TT + Core::dma_row(wave, q, lane)];
#pragma unroll
    for (int q = 0; q < Core::kXInstr; ++q) {
        const int row = Core::dma_row(wave, q, lane);
        const int t = pv[q] < nslots ? slot_token(pv[q], topk) : 0;
        xoff[q] = (uint32_t)(t * row_bytes) + Core::dma_chunk(row, lane) * 16;
    }
    // the epilogue's rows, looked up before the main loop: their loads
    // overlap the first copies instead of trailing the last MFMAs
    int row_p[Core::FT];
    float row_sx[Core::FT];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b)
        row_p[b] = sorted_ids[blk * TT + wb * (TT / Core::WT) + b * 32 + (lane & 31)];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b)
        row_sx[b] = row_p[b] < nslots ? xscale[slot_token(row_p[b], topk)] : 0.0f;
    Core core;
    const bool wave_valid = sorted_ids[blk * TT + wb * (TT / Core::WT)] < nslots;
    if (wave_valid)
        core.template run<true, HW>(lds, rw, wvoff, wsoff, rx, xoff, K, wave, wb, wa * WN);
    else
        core.template run<false, HW>(lds, rw, wvoff, wsoff, rx, xoff, K, wave, wb, wa * WN);

    const int li = lane & 31;
    const float ws = rowwise ? 0.0f : w1_scale[e];
    if constexpr (PP) {
        // the wave's 64 token rows x WN activations go out through its own
        // LDS area, whole 256-byte row segments per store instruction
        static_assert(WN == 64 && 4 * kStagedRowsBytes <= Core::kLdsBytes, "one staged pass");
        if (wave_valid) {
            char* st = lds + late_uniform(wave & 3) * kStagedRowsBytes;
            const int ln = late_lane();
            // the rows' slots, loaded again here rather than held through the
            // main loop (only their activation scales are)
            int pe[Core::FT];
#pragma unroll
            for (int b = 0; b < Core::FT; ++b)
                pe[b] = sorted_ids[blk * TT + wb * (TT / Core::WT) + b * 32 + (ln & 31)];
            lds_wave_fence();
#pragma unroll
            for (int b = 0; b < Core::FT; ++b) {
                const int r = blk * TT + wb * (TT / Core::WT) + b * 32 + (ln & 31);
                const float sx = row_sx[b];
                float m = 0.0f;
#pragma unroll
                for (int a = 0; a < Core::FW / 2; ++a) {
                    const int n0 = wt * HW + wa * WN + a * 32 + 4 * (ln >> 5);
#pragma unroll
                    for (int vg = 0; vg < 4; ++vg) {
                        f32x4_t sg, su;
                        if (rowwise) {
                            const float* sr = w1_scale + (size_t)e * 2 * N + n0 + 8 * vg;
                            sg = *reinterpret_cast<const f32x4_t*>(sr);
                            su = *reinterpret_cast<const f32x4_t*>(sr + N);
                        } else {
                            sg = su = f32x4_t{ws, ws, ws, ws};
                        }
                        f32x4_t o;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            o[v] = silu(core.acc[a][b][vg * 4 + v] * (sx * sg[v])) *
                                   (core.acc[a + Core::FW / 2][b][vg * 4 + v] * (sx * su[v]));
                            m = fmaxf(m, fabsf(o[v]));
                        }
                        stage_put(st, ln, b, a, vg, o);
                    }
                }
                // lanes l and l ^ 32 hold the same token row
                const uint32_t mb =
                    max(__float_as_uint(m), (uint32_t)__shfl_xor((int)__float_as_uint(m), 32));
                if (pe[b] < nslots && ln < 32) atomicMax(amax + r, mb);
            }
            stage_slots(st, ln, pe);
            stage_flush<false>(st, ln,
                               act + (size_t)(blk * TT + wb * (TT / Core::WT)) * N + wt * HW + wa * WN,
                               (size_t)N, nslots);
        }
    } else {
#pragma unroll
    for (int b = 0; b < Core::FT; ++b) {
        const int r = blk * TT + wb * (TT / Core::WT) + b * 32 + li;
        const bool valid = row_p[b] < nslots;
        const float sx = row_sx[b];
        float m = 0.0f;
#pragma unroll
        for (int a = 0; a < Core::FW / 2; ++a) {
            // accumulator element 4*vg + v is gate row n0 + 8*vg + v (and that up row)
            const int n0 = wt * HW + wa * WN + a * 32 + 4 * (lane >> 5);
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                f32x4_t sg, su;
                if (rowwise) {
                    const float* sr = w1_scale + (size_t)e * 2 * N + n0 + 8 * vg;
                    sg = *reinterpret_cast<const f32x4_t*>(sr);
                    su = *reinterpret_cast<const f32x4_t*>(sr + N);
                } else {
                    sg = su = f32x4_t{ws, ws, ws, ws};
                }
                f32x4_t o;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    o[v] = silu(core.acc[a][b][vg * 4 + v] * (sx * sg[v])) *
                           (core.acc[a + Core::FW / 2][b][vg * 4 + v] * (sx * su[v]));
                    m = fmaxf(m, fabsf(o[v]));
                }
                if (valid)
                    *reinterpret_cast<f32x4_t*>(act + (size_t)r * N + n0 + 8 * vg) = o;
            }
        }
        // lanes l and l ^ 32 hold the same token row
        const uint32_t mb = max(__float_as_uint(m), (uint32_t)__shfl_xor((int)__float_as_uint(m), 32));
        if (valid && lane < 32) atomicMax(amax + r, mb);
    }
    }
    core.finish(wave);
    }  // tiles
}

template <int TW, int TT, int BK, int WST, int XST, int WW, int NW, int OCC, int GROUP,
          bool PP = false>
__global__ __launch_bounds__(NW * 64, OCC) void gemm2_prefill_fp8_kernel(
    const uint8_t* __restrict__ act_q, const float* __restrict__ ascale,
    const uint8_t* __restrict__ w2, const float* __restrict__ w2_scale, int rowwise,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int cap,
    int nslots, int K, int N, int nsplit, int max_blocks, float* __restrict__ ypart) {
    using Core = typename std::conditional<PP, PingPongCore<TW, BK, WST, XST, true>,
                                           PrefillCore<TW, TT, BK, WST, XST, WW, NW, true>>::type;
    static_assert(!PP || (TT == 256 && NW == 8), "the ping-pong core takes 256-row tiles");
    __shared__ __attribute__((aligned(1024))) char lds[Core::kLdsBytes];
    constexpr int WR = TW / WW;  // output rows per wave

    const int n_wt = K / TW;
    const int npad = *num_padded;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int wa = Core::wave_a(wave), wb = Core::wave_b(wave);
    TileWalk<GROUP> walk(n_wt * nsplit, max_blocks);
    int wtz, blk;
    while (walk.next(wtz, blk)) {
    if (blk * TT >= npad) continue;
    const int wt = wtz % n_wt, z = wtz / n_wt;
    const int nlen = N / nsplit, nbeg = z * nlen;
    const int e = block_expert[blk];

    const size_t row_bytes = (size_t)N;
    const prsrc_t rw = pmake_rsrc(w2 + ((size_t)e * K + (size_t)wt * TW) * N,
                                  (uint32_t)(TW * row_bytes));
    const prsrc_t ra = pmake_rsrc(act_q, (uint32_t)((size_t)cap * row_bytes));
    uint32_t wsoff[Core::kWInstr], aoff[Core::kXInstr];
    const int row0 = Core::dma_row(wave, 0, lane);
    const uint32_t wvoff = (uint32_t)(row0 * row_bytes) + nbeg +
                           Core::dma_chunk(row0, lane) * 16;
#pragma unroll
    for (int q = 0; q < Core::kWInstr; ++q)
        wsoff[q] = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)((Core::dma_row(wave, q, 0) - Core::dma_row(wave, 0, 0)) * row_bytes));
#pragma unroll
    for (int q = 0; q < Core::kXInstr; ++q) {
        const int row = Core::dma_row(wave, q, lane);
        // padding rows (never quantised) copy the block's first row instead
        const int src = sorted_ids[blk * TT + row] < nslots ? blk * TT + row : blk * TT;
        aoff[q] = (uint32_t)(src * row_bytes) + nbeg + Core::dma_chunk(row, lane) * 16;
    }
    Core core;
    const bool wave_valid = sorted_ids[blk * TT + wb * (TT / Core::WT)] < nslots;
    if (wave_valid)
        core.template run<true, 0>(lds, rw, wvoff, wsoff, ra, aoff, nlen, wave, wb, wa * WR);
    else
        core.template run<false, 0>(lds, rw, wvoff, wsoff, ra, aoff, nlen, wave, wb, wa * WR);

    const int li = lane & 31;
    // the epilogue's rows: all slots, then all routing weights and row
    // scales, loaded together (kept out of the main loop, whose registers
    // are full)
    int row_p[Core::FT];
    float row_w[Core::FT];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b)
        row_p[b] = sorted_ids[blk * TT + wb * (TT / Core::WT) + b * 32 + li];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b) {
        const int r = blk * TT + wb * (TT / Core::WT) + b * 32 + li;
        row_w[b] = row_p[b] < nslots ? topk_w[row_p[b]] * ascale[r] : 0.0f;
    }
    const float ws = rowwise ? 0.0f : w2_scale[e];
    if constexpr (PP) {
        // the wave's 64 token rows x WR partial sums go out through its own
        // LDS area (the rings are idle once the group's last step is done)
        static_assert(4 * kStagedRowsBytes <= Core::kLdsBytes, "the staging fits the rings");
        if (wave_valid)
            store_rows_staged<WR>(
                lds + late_uniform(wave & 3) * kStagedRowsBytes,
                [&](int a, int b, int vg) {
                    const int c0 = wt * TW + wa * WR + a * 32 + 4 * (lane >> 5);
                    f32x4_t sc;
                    if (rowwise)
                        sc = *reinterpret_cast<const f32x4_t*>(w2_scale + (size_t)e * K + c0 + 8 * vg);
                    else
                        sc = f32x4_t{ws, ws, ws, ws};
                    f32x4_t o;
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[v] = core.acc[a][b][vg * 4 + v] * (sc[v] * row_w[b]);
                    return o;
                },
                row_p, nslots, ypart + (size_t)z * nslots * K + wt * TW + wa * WR, K);
    } else {
#pragma unroll
    for (int b = 0; b < Core::FT; ++b) {
        const int p = row_p[b];
        if (p >= nslots) continue;
        const float w = row_w[b];
#pragma unroll
        for (int a = 0; a < Core::FW; ++a) {
            const int c0 = wt * TW + wa * WR + a * 32 + 4 * (lane >> 5);
            float* dst = ypart + ((size_t)z * nslots + p) * K + c0;
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                f32x4_t sc;
                if (rowwise)
                    sc = *reinterpret_cast<const f32x4_t*>(w2_scale + (size_t)e * K + c0 + 8 * vg);
                else
                    sc = f32x4_t{ws, ws, ws, ws};
                f32x4_t o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = core.acc[a][b][vg * 4 + v] * (sc[v] * w);
                *reinterpret_cast<f32x4_t*>(dst + 8 * vg) = o;
            }
        }
    }
    }
    core.finish(wave);
    }  // tiles
}

// ---------------------------------------------------------------------------
// MXFP4 weights on the full tiles (PingPongMxCore), against the per-token
// e4m3 activations of the e4m3 path: GEMM1 applies s_x[t] (the E8M0 block
// scales are inside the MFMA), forms SiLU(gate)*up in fp32, stores it and
// folds each row's |act| max into amax[r]; GEMM2 multiplies by the sorted
// row's activation scale s_a[r] and the routing weight.
// ---------------------------------------------------------------------------
template <int GROUP>
__global__ __launch_bounds__(512, 1) void gemm1_prefill_mx_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xscale,
    const uint8_t* __restrict__ w1, const uint8_t* __restrict__ w1e8,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, int M, int topk, int nslots, int K, int N,
    int max_blocks, float* __restrict__ act, uint32_t* __restrict__ amax) {
    using Core = PingPongMxCore<256>;
    __shared__ __attribute__((aligned(1024))) char lds[Core::kLdsBytes];
    constexpr int TT = Core::TT;
    constexpr int HW = 128;     // n-values per tile (128 gate + 128 up weight rows)
    constexpr int WN = HW / Core::WW;

    const int npad = *num_padded;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int wa = Core::wave_a(wave), wb = Core::wave_b(wave);
    TileWalk<GROUP> walk(N / HW, max_blocks);
    int wt, blk;
    while (walk.next(wt, blk)) {
    if (blk * TT >= npad) continue;
    const int e = block_expert[blk];

    const size_t wrow = (size_t)K / 2, srow = (size_t)K / 32, xrow = (size_t)K;
    const prsrc_t rw = pmake_rsrc(w1 + (size_t)e * 2 * N * wrow, (uint32_t)(2 * (size_t)N * wrow));
    const prsrc_t rs = pmake_rsrc(w1e8 + (size_t)e * 2 * N * srow, (uint32_t)(2 * (size_t)N * srow));
    const prsrc_t rx = pmake_rsrc(xq, (uint32_t)((size_t)M * xrow));
    // tile weight row lr is gate row wt*HW + lr (lr < HW) or up row
    // N + wt*HW + lr - HW; a weight copy's 16 rows never straddle the two
    uint32_t wsoff[Core::kWInstr], xoff[Core::kXInstr];
    const int row0 = Core::w_dma_row(wave, 0, lane);
    const uint32_t wvoff = (uint32_t)((wt * HW + row0) * wrow) + Core::w_dma_chunk(row0, lane) * 16;
#pragma unroll
    for (int q = 0; q < Core::kWInstr; ++q) {
        const int first = Core::w_dma_row(wave, q, 0);
        const int shift = first - Core::w_dma_row(wave, 0, 0) + (first >= HW ? N - HW : 0);
        wsoff[q] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(shift * wrow));
    }
    const int sr = Core::s_dma_row(wave, lane);
    const uint32_t svoff = (uint32_t)((sr < HW ? wt * HW + sr : N + wt * HW + sr - HW) * srow);
    // all of the wave's row loads first, in flight together
    int pv[Core::kXInstr];
#pragma unroll
    for (int q = 0; q < Core::kXInstr; ++q) pv[q] = sorted_ids[blk * TT + Core::dma_row(wave, q, lane)];
#pragma unroll
    for (int q = 0; q < Core::kXInstr; ++q) {
        const int row = Core::dma_row(wave, q, lane);
        const int t = pv[q] < nslots ? slot_token(pv[q], topk) : 0;
        xoff[q] = (uint32_t)(t * xrow) + Core::dma_chunk(row, lane) * 16;
    }
    // the epilogue's rows, looked up before the main loop: their loads
    // overlap the first copies instead of trailing the last MFMAs
    int row_p[Core::FT];
    float row_sx[Core::FT];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b)
        row_p[b] = sorted_ids[blk * TT + wb * (TT / Core::WT) + b * 16 + (lane & 15)];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b)
        row_sx[b] = row_p[b] < nslots ? xscale[slot_token(row_p[b], topk)] : 0.0f;
    Core core;
    if (sorted_ids[blk * TT + wb * (TT / Core::WT)] < nslots)
        core.template run<true, HW>(lds, rw, wvoff, wsoff, rs, svoff, rx, xoff, K, wave, wb, wa * WN);
    else
        core.template run<false, HW>(lds, rw, wvoff, wsoff, rs, svoff, rx, xoff, K, wave, wb, wa * WN);

    const int li = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int b = 0; b < Core::FT; ++b) {
        const int r = blk * TT + wb * (TT / Core::WT) + b * 16 + li;
        const bool valid = row_p[b] < nslots;
        const float sx = row_sx[b];
        float m = 0.0f;
#pragma unroll
        for (int a = 0; a < Core::FW / 2; ++a) {
            // accumulator element v: gate row n0 + v (and that up row)
            const int n0 = wt * HW + wa * WN + a * 16 + 4 * q4;
            f32x4_t o;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                o[v] = silu(core.acc[a][b][v] * sx) * (core.acc[a + Core::FW / 2][b][v] * sx);
                m = fmaxf(m, fabsf(o[v]));
            }
            if (valid) *reinterpret_cast<f32x4_t*>(act + (size_t)r * N + n0) = o;
        }
        // lanes l, l^16, l^32, l^48 hold the same token row
        const uint32_t mb = col_max_bits(__float_as_uint(m));
        if (valid && lane < 16) atomicMax(amax + r, mb);
    }
    core.finish(wave);
    }  // tiles
}

template <int GROUP>
__global__ __launch_bounds__(512, 1) void gemm2_prefill_mx_kernel(
    const uint8_t* __restrict__ act_q, const float* __restrict__ ascale,
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2e8,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded, int cap,
    int nslots, int K, int N, int nsplit, int max_blocks, float* __restrict__ ypart) {
    using Core = PingPongMxCore<256>;
    __shared__ __attribute__((aligned(1024))) char lds[Core::kLdsBytes];
    constexpr int TT = Core::TT, TW = 256;
    constexpr int WR = TW / Core::WW;  // output rows per wave

    const int n_wt = K / TW;
    const int npad = *num_padded;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int wa = Core::wave_a(wave), wb = Core::wave_b(wave);
    TileWalk<GROUP> walk(n_wt * nsplit, max_blocks);
    int wtz, blk;
    while (walk.next(wtz, blk)) {
    if (blk * TT >= npad) continue;
    const int wt = wtz % n_wt, z = wtz / n_wt;
    const int nlen = N / nsplit, nbeg = z * nlen;
    const int e = block_expert[blk];

    const size_t wrow = (size_t)N / 2, srow = (size_t)N / 32, xrow = (size_t)N;
    const prsrc_t rw = pmake_rsrc(w2 + ((size_t)e * K + (size_t)wt * TW) * wrow,
                                  (uint32_t)(TW * wrow));
    const prsrc_t rs = pmake_rsrc(w2e8 + ((size_t)e * K + (size_t)wt * TW) * srow,
                                  (uint32_t)(TW * srow));
    const prsrc_t ra = pmake_rsrc(act_q, (uint32_t)((size_t)cap * xrow));
    uint32_t wsoff[Core::kWInstr], aoff[Core::kXInstr];
    const int row0 = Core::w_dma_row(wave, 0, lane);
    const uint32_t wvoff = (uint32_t)(row0 * wrow) + nbeg / 2 + Core::w_dma_chunk(row0, lane) * 16;
#pragma unroll
    for (int q = 0; q < Core::kWInstr; ++q)
        wsoff[q] = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)((Core::w_dma_row(wave, q, 0) - Core::w_dma_row(wave, 0, 0)) * wrow));
    const uint32_t svoff = (uint32_t)(Core::s_dma_row(wave, lane) * srow) + nbeg / 32;
#pragma unroll
    for (int q = 0; q < Core::kXInstr; ++q) {
        const int row = Core::dma_row(wave, q, lane);
        // padding rows (never written) copy the block's first row; their
        // columns are never stored
        const int src = sorted_ids[blk * TT + row] < nslots ? blk * TT + row : blk * TT;
        aoff[q] = (uint32_t)(src * xrow) + nbeg + Core::dma_chunk(row, lane) * 16;
    }
    // the epilogue's rows, looked up before the main loop: their loads
    // overlap the first copies instead of trailing the last MFMAs
    int row_p[Core::FT];
    float row_w[Core::FT];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b)
        row_p[b] = sorted_ids[blk * TT + wb * (TT / Core::WT) + b * 16 + (lane & 15)];
#pragma unroll
    for (int b = 0; b < Core::FT; ++b) {
        const int r = blk * TT + wb * (TT / Core::WT) + b * 16 + (lane & 15);
        row_w[b] = row_p[b] < nslots ? topk_w[row_p[b]] * ascale[r] : 0.0f;
    }
    Core core;
    if (sorted_ids[blk * TT + wb * (TT / Core::WT)] < nslots)
        core.template run<true, 0>(lds, rw, wvoff, wsoff, rs, svoff, ra, aoff, nlen, wave, wb, wa * WR);
    else
        core.template run<false, 0>(lds, rw, wvoff, wsoff, rs, svoff, ra, aoff, nlen, wave, wb, wa * WR);

    const int li = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int b = 0; b < Core::FT; ++b) {
        const int r = blk * TT + wb * (TT / Core::WT) + b * 16 + li;
        const int p = row_p[b];
        if (p >= nslots) continue;
        const float w = row_w[b];
        float* dst = ypart + ((size_t)z * nslots + p) * K + wt * TW + wa * WR + 4 * q4;
#pragma unroll
        for (int a = 0; a < Core::FW; ++a)
            *reinterpret_cast<f32x4_t*>(dst + a * 16) = core.acc[a][b] * w;
    }
    core.finish(wave);
    }  // tiles
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
// One workgroup per tile, rounded up to whole XCD groups of 8.
static int tile_grid(int tiles) { return (tiles + 7) / 8 * 8; }

// Token blocks of tt = 256 rows, or 128 for batches with few rows per expert
// (the plan's choice, tuning.hpp): 128-row tiles put 4 waves along the weight
// rows and 2 along the tokens, with a 3-slot weight ring and a 4-slot token
// ring (160 KB of LDS).
void launch_gemm1_prefill_bf16(const void* x, const void* w1, const int32_t* sorted_ids,
                               const int32_t* block_expert, const int32_t* num_padded, int M,
                               int topk, int nslots, int K, int N, int max_blocks, int tt,
                               void* act, hipStream_t s) {
    const int grid = tile_grid((N / 128) * max_blocks);
    if (tt == kPrefillSmallRows)
        gemm1_prefill_bf16_kernel<256, kPrefillSmallRows, 64, 3, 4, 4, 8, 1,
                                  tune::kPrefillGemm1Group><<<grid, 512, 0, s>>>(
            (const uint16_t*)x, (const uint16_t*)w1, sorted_ids, block_expert, num_padded, M,
            topk, nslots, K, N, max_blocks, (uint16_t*)act);
    else
        gemm1_prefill_bf16_kernel<256, kPrefillRows, 64, 3, 2, 2, 8, 1, tune::kPrefillGemm1Group,
                                  true><<<grid, 512, 0, s>>>(
            (const uint16_t*)x, (const uint16_t*)w1, sorted_ids, block_expert, num_padded, M,
            topk, nslots, K, N, max_blocks, (uint16_t*)act);
}

int prefill_gemm2_splits(int K, int N, int blocks, int gran) {
    // split the reduction until the target tile count (tuning.hpp): fewer
    // tiles leave the last round of workgroups part-empty, every split adds
    // a partial row per slot for the combine to read
    const long tiles = (long)(K % 256 == 0 ? K / 256 : K / 128) * blocks;
    int ns = 1;
    while (tiles * ns < tune::kPrefillSplitTargetTiles && ns < 4 && (N / (2 * ns)) % gran == 0)
        ns *= 2;
    return ns;
}

void launch_gemm2_prefill_bf16(const void* act, const void* w2, const float* topk_w,
                               const int32_t* sorted_ids, const int32_t* block_expert,
                               const int32_t* num_padded, int cap, int nslots, int K, int N,
                               int nsplit, int max_blocks, int tt, float* ypart, hipStream_t s) {
    if (tt == kPrefillSmallRows) {
        // the plan picks 128-row blocks only with K % 256 == 0; its splits
        // keep N / nsplit a multiple of 64
        const int grid = tile_grid((K / 256) * nsplit * max_blocks);
        gemm2_prefill_bf16_kernel<256, kPrefillSmallRows, 64, 3, 4, 4, 8, 1,
                                  tune::kPrefillGemm2Group><<<grid, 512, 0, s>>>(
            (const uint16_t*)act, (const uint16_t*)w2, topk_w, sorted_ids, block_expert,
            num_padded, cap, nslots, K, N, nsplit, max_blocks, ypart);
    } else if (K % 256 == 0 && (N / nsplit) % 64 == 0) {
        // 64-deep K-steps: each row copy is a whole 128-byte line
        const int grid = tile_grid((K / 256) * nsplit * max_blocks);
        gemm2_prefill_bf16_kernel<256, kPrefillRows, 64, 3, 2, 2, 8, 1, tune::kPrefillGemm2Group,
                                  true><<<grid, 512, 0, s>>>(
            (const uint16_t*)act, (const uint16_t*)w2, topk_w, sorted_ids, block_expert,
            num_padded, cap, nslots, K, N, nsplit, max_blocks, ypart);
    } else if (K % 256 == 0) {
        const int grid = tile_grid((K / 256) * nsplit * max_blocks);
        gemm2_prefill_bf16_kernel<256, kPrefillRows, 32, 3, 3, 4, 8, 1, 8><<<grid, 512, 0, s>>>(
            (const uint16_t*)act, (const uint16_t*)w2, topk_w, sorted_ids, block_expert,
            num_padded, cap, nslots, K, N, nsplit, max_blocks, ypart);
    } else {
        const int grid = tile_grid((K / 128) * nsplit * max_blocks);
        gemm2_prefill_bf16_kernel<128, kPrefillRows, 32, 3, 3, 4, 8, 1, 8><<<grid, 512, 0, s>>>(
            (const uint16_t*)act, (const uint16_t*)w2, topk_w, sorted_ids, block_expert,
            num_padded, cap, nslots, K, N, nsplit, max_blocks, ypart);
    }
}


// e4m3: 128-code K-steps; GEMM2's reduction split keeps each split a
// multiple of 128 codes (the caller's split choice)
void launch_gemm1_prefill_fp8(const uint8_t* xq, const float* xscale, const void* w1,
                              const float* w1_scale, int rowwise, const int32_t* sorted_ids,
                              const int32_t* block_expert, const int32_t* num_padded, int M,
                              int topk, int nslots, int K, int N, int max_blocks, int tt,
                              float* act, uint32_t* amax, hipStream_t s) {
    const int grid = tile_grid((N / 128) * max_blocks);
    if (tt == kPrefillSmallRows)
        gemm1_prefill_fp8_kernel<256, kPrefillSmallRows, 128, 3, 4, 4, 8, 1,
                                 tune::kPrefillFp8Gemm1Group><<<grid, 512, 0, s>>>(
            xq, xscale, (const uint8_t*)w1, w1_scale, rowwise, sorted_ids, block_expert,
            num_padded, M, topk, nslots, K, N, max_blocks, act, amax);
    else
        gemm1_prefill_fp8_kernel<256, kPrefillRows, 128, 3, 2, 2, 8, 1,
                                 tune::kPrefillFp8Gemm1Group, true><<<grid, 512, 0, s>>>(
            xq, xscale, (const uint8_t*)w1, w1_scale, rowwise, sorted_ids, block_expert,
            num_padded, M, topk, nslots, K, N, max_blocks, act, amax);
}

void launch_gemm2_prefill_fp8(const uint8_t* act_q, const float* ascale, const void* w2,
                              const float* w2_scale, int rowwise, const float* topk_w,
                              const int32_t* sorted_ids, const int32_t* block_expert,
                              const int32_t* num_padded, int cap, int nslots, int K, int N,
                              int nsplit, int max_blocks, int tt, float* ypart, hipStream_t s) {
    if (tt == kPrefillSmallRows) {
        // 128-row blocks come with K % 256 == 0 (the plan's choice)
        const int grid = tile_grid((K / 256) * nsplit * max_blocks);
        gemm2_prefill_fp8_kernel<256, kPrefillSmallRows, 128, 3, 4, 4, 8, 1,
                                 tune::kPrefillFp8Gemm2Group><<<grid, 512, 0, s>>>(
            act_q, ascale, (const uint8_t*)w2, w2_scale, rowwise, topk_w, sorted_ids,
            block_expert, num_padded, cap, nslots, K, N, nsplit, max_blocks, ypart);
    } else if (K % 256 == 0) {
        const int grid = tile_grid((K / 256) * nsplit * max_blocks);
        gemm2_prefill_fp8_kernel<256, kPrefillRows, 128, 3, 2, 2, 8, 1,
                                 tune::kPrefillFp8Gemm2Group, true>
            <<<grid, 512, 0, s>>>(act_q, ascale, (const uint8_t*)w2, w2_scale, rowwise, topk_w,
                                  sorted_ids, block_expert, num_padded, cap, nslots, K, N, nsplit,
                                  max_blocks, ypart);
    } else {
        const int grid = tile_grid((K / 128) * nsplit * max_blocks);
        gemm2_prefill_fp8_kernel<128, kPrefillRows, 128, 3, 3, 4, 8, 1, 8><<<grid, 512, 0, s>>>(
            act_q, ascale, (const uint8_t*)w2, w2_scale, rowwise, topk_w, sorted_ids,
            block_expert, num_padded, cap, nslots, K, N, nsplit, max_blocks, ypart);
    }
}

// MXFP4 weights on the full tiles (256-row blocks; K, N multiples of 256;
// GEMM2 splits of multiples of 128 codes)
void launch_gemm1_prefill_mx(const uint8_t* xq, const float* xscale, const void* w1,
                             const uint8_t* w1e8, const int32_t* sorted_ids,
                             const int32_t* block_expert, const int32_t* num_padded, int M,
                             int topk, int nslots, int K, int N, int max_blocks, float* act,
                             uint32_t* amax, hipStream_t s) {
    const int grid = tile_grid((N / 128) * max_blocks);
    gemm1_prefill_mx_kernel<tune::kPrefillMxGemm1Group><<<grid, 512, 0, s>>>(
        xq, xscale, (const uint8_t*)w1, w1e8, sorted_ids, block_expert, num_padded, M, topk,
        nslots, K, N, max_blocks, act, amax);
}

void launch_gemm2_prefill_mx(const uint8_t* act_q, const float* ascale, const void* w2,
                             const uint8_t* w2e8, const float* topk_w, const int32_t* sorted_ids,
                             const int32_t* block_expert, const int32_t* num_padded, int cap,
                             int nslots, int K, int N, int nsplit, int max_blocks, float* ypart,
                             hipStream_t s) {
    const int grid = tile_grid((K / 256) * nsplit * max_blocks);
    gemm2_prefill_mx_kernel<tune::kPrefillMxGemm2Group><<<grid, 512, 0, s>>>(
        act_q, ascale, (const uint8_t*)w2, w2e8, topk_w, sorted_ids, block_expert, num_padded,
        cap, nslots, K, N, nsplit, max_blocks, ypart);
}

}  // namespace moe
