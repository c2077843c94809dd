// tuning.hpp -- the launch choices of the fused MoE layer, per token bucket
// and shape, frozen from measurements on one MI355X (the batch sweep is
// `bench.py --regime-sweep`; the other figures are quoted at each entry).
// Everything that picks a kernel family, a block size, a reduction split, a
// tile order or a ring shape reads it from here.
#pragma once

#include <cmath>

namespace moe {
namespace tune {

// ---- kernel family per token bucket -----------------------------------------
// bf16 weights: the Swap-AB decode kernels up to this many token-slots per
// expert, the full-tile kernels above.  Sweep of both families over
// M = 8 .. 1024 (K, N, E, k = 4096, 14336, 8, 2 / 4096, 8192, 16, 2 /
// 7168, 2048, 256, 8): decode faster up to 8 rows per expert on all three
// shapes, full tiles from 12 on; re-measured with the 32- and 64-row decode
// blocks (Mixtral shape, 16 rows: 0.586 ms decode against 0.548 tiles).
constexpr long kDecodeMaxRowsPerExpert = 8;
// e4m3 weights: the decode kernels up to this many token-slots per expert,
// the full tiles above.  Sweep
// of both families (bench.py --fp8 --regime-sweep), ms per layer call at
// 8 / 16 / 32 / 64 rows per expert, decode against tiles:
//   K, N, E, k = 4096, 14336, 8, 2: 0.300/0.330, 0.332/0.338, 0.422/0.353,
//                                   0.735/0.378 (128 rows: 1.198/0.441)
//   K, N, E, k = 7168, 2048, 256, 8: 2.14/2.42, 2.43/2.54, 3.09/2.82,
//                                   4.85/3.20 (128 rows: 8.73/4.16)
constexpr long kFp8DecodeMaxRowsPerExpert = 16;
// MXFP4 weights: the same rule.  Sweep (bench.py --mxfp4 --regime-sweep),
// ms per layer call at 8 / 16 / 24 / 32 / 48 / 64 rows per expert, decode
// against tiles:
//   K, N, E, k = 4096, 14336, 8, 2: 0.234/0.311, 0.252/0.311, 0.319/0.314,
//                                   0.338/0.319, 0.387/0.330, 0.575/0.344
//   K, N, E, k = 7168, 2048, 256, 8: 1.35/2.11, 1.68/2.18, 2.17/2.28,
//                                   2.38/2.39, 2.85/2.54, 3.89/2.75
constexpr long kMxDecodeMaxRowsPerExpert = 24;

// ---- decode block rows ------------------------------------------------------
// 16, 32 or 64 sorted rows per block (1, 2 or 4 token tiles multiplied by
// every weight fragment), sized for the mean rows per active expert plus two
// Poisson standard deviations, so most experts stream their weights once.
// DeepSeek shape, e4m3: 16 rows on average best in 32-row blocks (2.44 ms
// against 2.82 ms in 16-row ones), 32 rows in 64-row blocks (3.09 / 4.35).
inline int decode_block_rows(long slots, int E) {
    const double active = (double)(slots < E ? slots : E);
    const double rows = active > 0 ? (double)slots / active : 0.0;
    const double need = rows + 2.0 * std::sqrt(rows);
    return need > 32 ? 64 : (need > 16 ? 32 : 16);
}

// ---- decode GEMM2 reduction split ----------------------------------------
// tiles = (block, output-row tile) pairs of one split.  A grid already
// holding a workgroup per CU stays unsplit (8 experts x 4096 x 14336 bf16:
// 160 us unsplit, 166-171 us in 2-16 splits); a smaller one splits until
// about two workgroups per CU while each wave keeps at least 32 KB of
// weights (2 experts x 4096 x 8192: bf16 and MXFP4 best in 8 splits; 16
// splits, 16 KB per wave, measured 12 % slower for MXFP4).
constexpr long kDecodeSplitUnsplitTiles = 256;
constexpr long kDecodeSplitTargetTiles = 512;
constexpr long kDecodeSplitMinWaveBytes = 32 * 1024;
// MXFP4 GEMM2 keeps a split's E8M0 bytes in LDS: at most this many reduction
// elements per split (64 KB of dynamic LDS per workgroup)
constexpr int kMxMaxSplitLen = 8192;
// MXFP4 GEMM1 keeps K/32 scale bytes per row of its waves in LDS
constexpr int kMxMaxK = 16384;

// ---- MXFP4 row tiles per wave -------------------------------------------------
// GEMM1: one 16-row gate tile and its up tile (two: 12-30 % slower as the
// grid halves); GEMM2: four 16-row output tiles (two: 1-2 % slower).
constexpr int kMxTiles1 = 1;
constexpr int kMxTiles2 = 4;

// ---- prefill ------------------------------------------------------------------
// token rows per full-tile block: 128 while the mean rows per active expert
// stay at or below this, else 256.  Full-tile ms per layer call with 128- /
// 256-row blocks at 16, 32, 64, 128 rows per expert:
//   e4m3, K, N, E, k = 7168, 2048, 256, 8: 2.18/2.44, 2.35/2.63, 2.63/2.95, 3.58/3.57
//   e4m3, K, N, E, k = 4096, 14336, 8, 2: 0.301/0.351, 0.315/0.365, 0.348/0.384, 0.424/0.444
//   bf16, K, N, E, k = 4096, 14336, 8, 2: 0.513/0.551, 0.525/0.562, 0.562/0.604, 0.701/0.697
// and on the skewed Mixtral-shaped prefill (1024 rows per expert on
// average) 3.15 against 2.78 ms (GEMM1 1908/1720 us, GEMM2 unsplit
// 1167/945 us although the combine halves, 30/53 us).
constexpr long kPrefillSmallTileMaxRows = 128;
// e4m3 weights: the same bound.  128-row blocks at every size measured
// worse on the skewed Mixtral-shaped prefill (1.82 -> 1.87 ms per layer
// call, 1024 rows per expert on average) and better on the DeepSeek shape
// with 8192 tokens (256 rows per expert: 6.01 -> 5.82 ms; GEMM1 faster by
// 11 %, GEMM2 slower by 5 %).
constexpr long kPrefillFp8SmallTileMaxRows = 128;

// GEMM2 reduction split until about four workgroups per CU exist (Mixtral
// prefill, 39 blocks: 1118 us unsplit, 999 us in 2 splits, 1007 us in 4
// with a combine twice as long).
constexpr long kPrefillSplitTargetTiles = 1024;
// weight tiles varying fastest in a tile group of the XCD-aware order
// (GEMM1: 1705-1715 us with 4 against 1725-1740 with 2; GEMM2: 936 us with
// 4 against 990 with 8 and 1042 with 16)
constexpr int kPrefillGemm1Group = 4;
constexpr int kPrefillGemm2Group = 4;
// Measured and dropped for the bf16 256 x 256 tiles: a four-wave core (one
// wave per SIMD, 128 x 128 wave tiles, 256 accumulators, every MFMA followed
// by one fragment read or copy), parity-green.  Mixtral-shaped prefill,
// alternating runs on one box: GEMM1 1574-1579 us against 1568 us with the
// ping-pong core, GEMM2 872-873 against 852-853 us.  Its 128 KB of LDS reads
// per K-step (192 KB for eight 128 x 64 waves) lift the clock (1.79 against
// 1.74 GHz) but leave the matrix cores busy 64-65 % against 67 %; timing
// probes of it: without its copies GEMM1 takes 1411 us, without its
// fragment reads 1630 us, without its barrier and copy waits unchanged,
// with neither reads nor copies 1370 us (68 % busy; 82 % busy when each
// tile's loop runs four times as long, so about a fifth of that probe's
// time is per-tile start and epilogue).  Forms that carry the copy ring
// from one tile into the next, so that a tile after the first starts
// without waiting for memory, were slower still: persistent workgroups
// (1721 against 1562-1568 us; a static walk of equal shares leaves the CUs
// unbalanced, since an expert's last block costs less), four weight tiles
// of one token block per workgroup (1706-1712 against 1555-1573 us: 32
// token blocks resident per XCD instead of 8), two token blocks of one
// weight tile (1611-1623 against 1544-1551 us).
// The 256-row bf16 tiles of both GEMMs run the ping-pong core (two wave
// groups a phase apart, 3 weight + 2 token ring slots).  Against the shared
// core on one box, Mixtral-shaped prefill (alternating runs): GEMM1 1621-1626
// against 1705-1712 us, GEMM2 849-854 against 947 us, step 2.62 against
// 2.79 ms; counters: matrix cores busy 68 % (GEMM1) / 67 % (GEMM2) against
// 62 / 57 %, at a lower clock (1.63 / 1.53 GHz against 1.70 / 1.59), L2 hit
// rate 65 / 68 % against 58 / 66 %.  With the ping-pong core, tile groups of
// 2 and 4 weight tiles are equal for GEMM1 (1625 us), 8 slower (1685); GEMM2
// 4 best (849-854 us against 878 with 2, 890 with 8).
// (Before the ping-pong core, the shared core's rings measured best at 3 + 2
// slots for GEMM1 and 2 + 3 for GEMM2: 933-935 us against 946-950 with 3 + 2.)
// Tried on the ping-pong core and dropped:
// * the token rows as the ring copied two steps ahead (2 weight + 3 token
//   slots): GEMM1 1612-1618 against 1619-1659 us, GEMM2 907 against
//   851-878, e4m3 GEMM1 1018 against 975;
// * for an expert's last block with at most 128 (64) valid rows, all 8
//   waves on those rows with a quarter of the weight rows each: GEMM1
//   1623-1627 against 1611 us, GEMM2 850-854 against 847-850 (e4m3
//   993 / 522 against 983 / 526).  Skipping those blocks' tiles outright
//   (a timing probe) takes GEMM1 from 1640 to 1380 us: they cost about 70 %
//   of a full tile whatever their MFMA count.
// * (probes) all experts reading expert 0's weights: GEMM1 1600 against
//   1690 us on one box, L2 hit rate 71 % against 65 %, clock 1.67 against
//   1.56 GHz, matrix cores busy 68.6 % in both: fewer bytes from beyond L2
//   buy clock, not utilisation.
// the e4m3 full tiles (same bytes per K-step as the bf16 ones).  GEMM1
// group, rings (weight + token slots), us on the Mixtral shape with 4096
// tokens / the DeepSeek shape with 4096 tokens (two runs where given):
// 2, 3+2: 983-1011 / 1679-1733; 4, 3+2: 1003 / 2163; 4, 2+3: 990 / 2330;
// 8, 2+3: 1001 / 2327; 1, 3+2: 1031 / 1791; 1, 2+2: 1059 / 1750;
// 2, 2+3: 1016 / 1844; 3, 3+2: 1014 / 2267.  GEMM2: 4, 2+3: 520 / 1148;
// 4, 3+2: 555 / 1112; 2, 3+2: 582 / 1216; 2, 2+3: 542 / 1326; 8, 2+2:
// 593 / 1440; 8, 2+3: 579 / 1564.
// The e4m3 256-row tiles run the ping-pong core too (3 + 2 slots): Mixtral
// shape with e4m3 weights, alternating runs against the shared core (3 + 2
// for GEMM1, 3 + 2 for GEMM2): GEMM1 971-972 against 986-998 us, GEMM2
// 526-529 against 552-555 us, step 1.766-1.775 against 1.799-1.809 ms.
constexpr int kPrefillFp8Gemm1Group = 2, kPrefillFp8Gemm2Group = 4;
// MXFP4 weights on the full tiles (256-row blocks, the ping-pong core).
// GEMM1 / GEMM2 us, Mixtral shape with 4096 tokens / DeepSeek shape with
// 4096 tokens, for groups (GEMM1, GEMM2): (1, 4) 949/1608, 522/1160;
// (2, 4) 944/1594, 521/1151; (4, 4) 928/2309, 522/1150; (2, 2) 944/1593,
// 529/1169; (2, 8) 945/1610, 538/1474.
constexpr int kPrefillMxGemm1Group = 2, kPrefillMxGemm2Group = 4;

// ---- two-launch decode of one or two tokens (bf16) -----------------------------
// every workgroup recomputes all router logits, M*E pairs of K-long fp64 dot
// products, so the fused kernel is taken only while they stay few
constexpr int kFusedDecodeMaxPairs = 32;

// ---- router -------------------------------------------------------------------
// fp64-MFMA logits: split K until the tiles x splits cover every CU (the
// DeepSeek shape's 128 tiles in 2 splits: its logits + e4m3-rows stage
// 32 -> 23 us)
constexpr long kRouterSplitTargetTiles = 256;
// up to this many tokens (of at most this width) the FP8 token quantisation
// runs inside the single-workgroup top-k + align launch (a wave per token)
constexpr int kLateQuantRows = 16;
constexpr int kLateQuantCols = 1024;

}  // namespace tune
}  // namespace moe
