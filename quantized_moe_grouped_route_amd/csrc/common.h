// Device-side building blocks shared by the gfx950 kernels: vector types,
// MFMA wrappers with their register layouts, conversions, and the
// persistent grouped-tile scheduler.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned u32;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads and stores through native vector types (arrays of these
// stay in registers; arrays of HIP's uint4 struct can end up in scratch).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

constexpr int kWave = 64;

// ---------------------------------------------------------------- MFMA
// All 32x32 MFMAs below share one register layout (wave64):
//   A operand: lane l holds row (l % 32) and the k-slice (l / 32) of the step
//   B operand: lane l holds col (l % 32) and the same k-slice (l / 32)
//   C/D (16 values): value i of lane l is C[8*(i/4) + 4*(l/32) + (i%4)][l%32]
// Which K elements sit in which (slice, register) slot is free as long as
// A and B use the same assignment: the instruction sums over all slots.

// int8 x int8 -> int32, K = 32 per step (16 bytes per lane per operand).
__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
// OCP e4m3 x e4m3 -> fp32, K = 64 per step (32 bytes per lane per operand).
// The block-scale operands of the instruction are fixed at 2^0 (E8M0 127).
__device__ __forceinline__ v16f mfma_f8_32x32x64(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// bf16 x bf16 -> fp32, K = 16 per step (8 bf16 per lane per operand).
__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16 bf16 MFMA (wave64): A lane l: row l%16, k-slice l/16 (4 slices of
// 8); B lane l: col l%16, same k-slice; D (4 values): value i of lane l is
// D[4*(l/16) + i][l%16].
__device__ __forceinline__ v4f mfma_bf16_16x16x32(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// binary16 forms of the two bf16 MFMAs above (same operand layouts).
__device__ __forceinline__ v16f mfma_f16_32x32x16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f16_16x16x32(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 output held in accumulator value i by lane l.
__device__ __forceinline__ int c32_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
// OCP e4m3fn byte -> fp32 (exact), via the gfx950 conversion.
__device__ __forceinline__ float e4m3_to_f32(u32 byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// Element storage helpers for the epilogues.
enum OutKind { OUT_F16 = 1, OUT_BF16 = 2, OUT_F32 = 3, OUT_I32 = 4 };

template <int KIND>
struct OutT;
template <>
struct OutT<OUT_F16> {
  typedef uint16_t T;
  static __device__ __forceinline__ T from(float v) { return f32_to_f16_bits(v); }
};
template <>
struct OutT<OUT_BF16> {
  typedef uint16_t T;
  static __device__ __forceinline__ T from(float v) { return f32_to_bf16_bits(v); }
};
template <>
struct OutT<OUT_F32> {
  typedef float T;
  static __device__ __forceinline__ T from(float v) { return v; }
};

template <int KIND>
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<OUT_F16>(const void* p, int64_t i) {
  return f16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <>
__device__ __forceinline__ float load_as_f32<OUT_BF16>(const void* p, int64_t i) {
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <>
__device__ __forceinline__ float load_as_f32<OUT_F32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}

// ---------------------------------------------------------------- scheduler
// Persistent grouped-tile scheduler.  The per-expert row counts come from
// expert_offsets on the device (no host round trip).  Work item w maps to
// (expert e, m-tile mt, n-tile nt); experts with no rows own no items.  The
// item space is ordered expert-major, and inside an expert in groups of
// GROUP_M m-tiles so that consecutive items share weight columns (and
// activation rows) while they are resident in L2.
//
// The table lives in LDS: tile_start[e] = first item of expert e,
// tile_start[E] = total.  Built by one workgroup-wide scan.
// Rows [lo, hi) of expert e, clamped to [0, P] so that a malformed offsets
// table can never address past the P output rows.
__device__ __forceinline__ void expert_range(const int* __restrict__ offsets, int e, int P, int& lo,
                                             int& hi) {
  lo = min(max(offsets[e], 0), P);
  hi = min(max(offsets[e + 1], lo), P);
}

// Builds tile_start in LDS.  Needs blockDim.x threads, E+1 ints of LDS in
// `tile_start` and 2*kMaxWaves ints in `scratch`.  Ends with a barrier.
constexpr int kMaxWaves = 16;
__device__ inline void sched_build(int* tile_start, int* scratch, const int* __restrict__ offsets,
                                   int E, int P, int bm, int n_tiles) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & 63, wid = tid >> 6, nw = nt >> 6;
  // Each thread owns a contiguous run of experts.
  const int per = (E + nt - 1) / nt;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) {
    int lo, hi;
    expert_range(offsets, e, P, lo, hi);
    const int m = hi - lo;
    local += m > 0 ? ((m + bm - 1) / bm) * n_tiles : 0;
  }
  // Inclusive scan of `local` across the workgroup.
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) scratch[wid] = incl;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < nw; ++w) {
      const int v = scratch[w];
      scratch[kMaxWaves + w] = s;
      s += v;
    }
  }
  __syncthreads();
  int run = incl - local + scratch[kMaxWaves + wid];
  for (int e = e0; e < e1; ++e) {
    tile_start[e] = run;
    int lo, hi;
    expert_range(offsets, e, P, lo, hi);
    const int m = hi - lo;
    run += m > 0 ? ((m + bm - 1) / bm) * n_tiles : 0;
  }
  if (tid == nt - 1) tile_start[E] = run;
  __syncthreads();
}

struct Tile {
  int e;      // expert
  int row0;   // first sorted position of the tile
  int rows;   // valid rows in the tile (1..bm)
  int nt;     // n-tile index
};

// Maps item w (< tile_start[E]) to its tile.  GROUP_M m-tiles of one expert
// are visited for each n-tile before moving to the next n-tile.
template <int GROUP_M>
__device__ __forceinline__ Tile sched_tile(const int* tile_start, const int* __restrict__ offsets,
                                           int E, int P, int bm, int n_tiles, int w) {
  // Binary search for the last e with tile_start[e] <= w.  An empty expert
  // has tile_start[e] == tile_start[e+1], so the last such e owns item w.
  int bl = 0, bh = E - 1;
  while (bl < bh) {
    const int mid = (bl + bh + 1) >> 1;
    if (tile_start[mid] <= w) bl = mid; else bh = mid - 1;
  }
  const int e = bl;
  const int local = w - tile_start[e];
  int lo, hi;
  expert_range(offsets, e, P, lo, hi);
  const int m = hi - lo;
  const int mtiles = (m + bm - 1) / bm;
  const int group = local / (GROUP_M * n_tiles);
  const int in_group = local - group * GROUP_M * n_tiles;
  const int gm = min(GROUP_M, mtiles - group * GROUP_M);
  const int mt = group * GROUP_M + in_group % gm;
  const int ntile = in_group / gm;
  Tile t;
  t.e = e;
  t.row0 = lo + mt * bm;
  t.rows = min(bm, m - mt * bm);
  t.nt = ntile;
  return t;
}

// Logical workgroup id with the XCD round robin undone: hardware places
// workgroup b on XCD (b % 8); this returns an id such that the 8 XCDs each
// own a contiguous range of logical ids (neighbouring tiles share an L2).
__device__ __forceinline__ int xcd_logical_id(int b, int nb) {
  constexpr int kXcd = 8;
  if (nb % kXcd != 0) return b;
  return (b % kXcd) * (nb / kXcd) + b / kXcd;
}

}  // namespace moeq
