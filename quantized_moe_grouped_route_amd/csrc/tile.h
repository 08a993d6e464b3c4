// Shared geometry of the MFMA-tiled (prefill) grouped GEMMs.
//
// A workgroup of 256 threads (4 waves) owns a 128 x 128 output tile.  Each
// K step stages 128 bytes of every A row and every B row in LDS (for FP8:
// 128 e4m3 values; for INT4: 128 int4 values widened to int8; for NVFP4:
// 64 bf16 values), so all three formats share one LDS geometry:
//   [128 rows][kPitch bytes], kPitch = 128 + 16 padding bytes, which keeps
//   the 16-byte fragment reads of 8 consecutive rows on distinct banks.
// Waves sit on a 2 x 2 grid; wave (wm, wn) owns rows [64wm, 64wm+64) and
// two 32-column sub-tiles, i.e. 2 x 2 MFMA 32x32 sub-tiles.
//
// Loads from global memory: thread t moves 16 bytes of row (t/8 + 32i),
// byte (t%8)*16 of the step, i = 0..3, so 8 consecutive threads read one
// row's 128 contiguous bytes.
#pragma once

#include "common.h"

namespace moeq {

constexpr int kTileM = 128;
constexpr int kTileN = 128;
constexpr int kThreadsT = 256;
constexpr int kStepBytes = 128;
constexpr int kPitch = kStepBytes + 16;
constexpr int kMaxExperts = 1024;

// LDS row base (in the B tile) of the 32-row sub-tile `sn` of wave column
// `wn`.  NONE: contiguous 64-column halves.  SILU_MUL: B rows [0, 64) are
// gate rows and [64, 128) the matching up rows, and wave column wn takes
// gate sub-tile rows [32wn, 32wn+32) (sn = 0) and the up rows of the same
// columns (sn = 1), so gate and up values of one output meet in one lane.
__device__ __forceinline__ int b_lds_row(bool silu, int wn, int sn) {
  return silu ? (32 * wn + 64 * sn) : (64 * wn + 32 * sn);
}

// Global weight row (within the expert) of LDS B row j for n-tile nt.
__device__ __forceinline__ int b_global_row(bool silu, int nt, int j, int I) {
  if (!silu) return nt * kTileN + j;
  return j < 64 ? nt * 64 + j : I + nt * 64 + (j - 64);
}

// Activation row of sorted position s (clamped inside [0, rows_a) so that a
// corrupt table can never address outside the operand).
__device__ __forceinline__ int64_t a_row_of(int s, const int* __restrict__ sorted_ids, int a_sorted,
                                            int topk, int64_t rows_a) {
  int64_t r = (a_sorted || sorted_ids == nullptr) ? (int64_t)s : (int64_t)(sorted_ids[s] / topk);
  return (r < 0 || r >= rows_a) ? 0 : r;
}

// Number of output columns written per tile row, and tiles along N.
__device__ __forceinline__ int n_tiles_of(int N) { return N / kTileN; }

}  // namespace moeq
