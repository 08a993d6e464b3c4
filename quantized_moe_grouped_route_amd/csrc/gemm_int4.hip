// W4A4 INT4 grouped GEMM with the per-token x per-channel dequantization
// fused into the epilogue (CUTLASS discussion #2855 asks for exactly this
// epilogue, scale_act * scale_weight * accumulator, instead of a separate
// dequantization pass over an int32 buffer).
//
// CDNA4 has no int4 MFMA.  Each packed 32-bit word w holding 8 nibbles is
// split into two int8 words: (w << 4) & 0xF0F0F0F0 holds the even elements
// and w & 0xF0F0F0F0 the odd ones, each byte being 16 * value as a signed
// int8.  A and W get the same split, so the int8 MFMA sums the same
// products, each scaled by 256; |acc| <= K * 64 * 256 < 2^31 for K <= 2^17,
// and acc >> 8 is the exact int4 dot product.
#include <algorithm>

#include "kernels.h"
#include "tile.h"

namespace moeq {
namespace {

__device__ __forceinline__ void split_nibbles(u32x4 p, u32x4& lo, u32x4& hi) {
  lo = (p << 4) & 0xF0F0F0F0u;
  hi = p & 0xF0F0F0F0u;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Each K step covers 128 int4 values: 64 packed bytes per row from global
// memory (thread t: row t/4 + 64i, bytes (t%4)*16, i = 0, 1), widened to
// 128 int8 bytes per row in LDS.
template <int OUT, bool SILU>
__global__ __launch_bounds__(kThreadsT, 1) void int4_prefill(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scale, int64_t rows_a, int a_sorted,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_ids, int topk, int E, int P, int N,
    int K, void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kTileM * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[kTileN * kPitch];
  __shared__ __attribute__((aligned(16))) float lds_sa[kTileM];
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int n_tiles = N / kTileN;
  const int I = N / 2;
  const int steps = K / 128;
  const int64_t row_bytes = K / 2;
  sched_build(tile_start, sched_scratch, offsets, E, P, kTileM, n_tiles);
  const int total = tile_start[E];

  const int lrow = tid >> 2, lchunk = (tid & 3) * 16;

  for (int item = xcd_logical_id(blockIdx.x, gridDim.x); item < total; item += gridDim.x) {
    const Tile t = sched_tile<4>(tile_start, offsets, E, P, kTileM, n_tiles, item);
    __syncthreads();  // the previous tile's epilogue has read lds_sa
    const uint8_t* pa[2];
    const uint8_t* pb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = lrow + 64 * i;
      const int s = t.row0 + min(j, t.rows - 1);
      pa[i] = a + a_row_of(s, sorted_ids, a_sorted, topk, rows_a) * row_bytes + lchunk;
      pb[i] = w + ((int64_t)t.e * N + b_global_row(SILU, t.nt, j, I)) * row_bytes + lchunk;
    }
    if (tid < kTileM)
      lds_sa[tid] = a_scale[a_row_of(t.row0 + min(tid, t.rows - 1), sorted_ids, a_sorted, topk, rows_a)];

    v16i acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = v16i{};

    u32x4 ra[2], rb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i] = ld16(pa[i]);
      rb[i] = ld16(pb[i]);
    }
    for (int st = 0; st < steps; ++st) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        u32x4 lo, hi;
        uint8_t* da = lds_a + (lrow + 64 * i) * kPitch + 2 * lchunk;
        split_nibbles(ra[i], lo, hi);
        st16(da, lo);
        st16(da + 16, hi);
        uint8_t* db = lds_b + (lrow + 64 * i) * kPitch + 2 * lchunk;
        split_nibbles(rb[i], lo, hi);
        st16(db, lo);
        st16(db + 16, hi);
      }
      __syncthreads();
      if (st + 1 < steps) {
        const int64_t off = (int64_t)(st + 1) * 64;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          ra[i] = ld16(pa[i] + off);
          rb[i] = ld16(pb[i] + off);
        }
      }
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int koff = kq * 32 + (lane >> 5) * 16;
        v4i fa[2], fb[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          fa[x] = *reinterpret_cast<const v4i*>(lds_a + (64 * wm + 32 * x + (lane & 31)) * kPitch + koff);
        }
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          fb[y] = *reinterpret_cast<const v4i*>(lds_b + (b_lds_row(SILU, wn, y) + (lane & 31)) * kPitch + koff);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y) acc[x][y] = mfma_i8_32x32x32(fa[x], fb[y], acc[x][y]);
      }
    }

    // Epilogue.
    if (OUT == OUT_I32) {
      int* o = static_cast<int*>(out);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const int col = t.nt * kTileN + b_lds_row(false, wn, y) + (lane & 31);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int rr = 64 * wm + 32 * x + c32_row(i, lane);
            if (rr < t.rows) o[(int64_t)(t.row0 + rr) * N + col] = acc[x][y][i] >> 8;
          }
        }
    } else {
      typedef typename OutT<(OUT == OUT_I32 ? OUT_F32 : OUT)>::T T;
      T* o = static_cast<T*>(out);
      if (SILU) {
        const int col = t.nt * 64 + 32 * wn + (lane & 31);  // output column in [0, I)
        const float swg = w_scale[(int64_t)t.e * N + col];
        const float swu = w_scale[(int64_t)t.e * N + I + col];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int rr = 64 * wm + 32 * x + c32_row(i, lane);
            const float sa = lds_sa[rr];
            const float g = sa * swg * (float)(acc[x][0][i] >> 8);
            const float u = sa * swu * (float)(acc[x][1][i] >> 8);
            if (rr < t.rows)
              o[(int64_t)(t.row0 + rr) * I + col] = OutT<(OUT == OUT_I32 ? OUT_F32 : OUT)>::from(silu(g) * u);
          }
      } else {
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const int col = t.nt * kTileN + b_lds_row(false, wn, y) + (lane & 31);
          const float sw = w_scale[(int64_t)t.e * N + col];
#pragma unroll
          for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int rr = 64 * wm + 32 * x + c32_row(i, lane);
              const float v = lds_sa[rr] * sw * (float)(acc[x][y][i] >> 8);
              if (rr < t.rows)
                o[(int64_t)(t.row0 + rr) * N + col] = OutT<(OUT == OUT_I32 ? OUT_F32 : OUT)>::from(v);
            }
        }
      }
    }
  }
}

template <int OUT, bool SILU>
hipError_t go(const GroupedArgs& g, int grid, const uint8_t* a, const float* a_scale,
              const uint8_t* w, const float* w_scale, hipStream_t stream) {
  hipLaunchKernelGGL((int4_prefill<OUT, SILU>), dim3(grid), dim3(kThreadsT), 0, stream, a, a_scale,
                     g.rows_a, g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P, g.N,
                     g.K, g.out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_int4(const GroupedArgs& g, const uint8_t* a, const float* a_scale,
                            const uint8_t* w, const float* w_scale, hipStream_t stream) {
  const int64_t mt_ub = (g.P + kTileM - 1) / kTileM + std::min<int64_t>(g.E, g.P);
  const int64_t items_ub = mt_ub * (g.N / kTileN);
  if (items_ub == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(items_ub, (int64_t)g.num_cus * 2);
  if (g.silu_mul) {
    switch (g.out_kind) {
      case OUT_F16: return go<OUT_F16, true>(g, grid, a, a_scale, w, w_scale, stream);
      case OUT_BF16: return go<OUT_BF16, true>(g, grid, a, a_scale, w, w_scale, stream);
      default: return go<OUT_F32, true>(g, grid, a, a_scale, w, w_scale, stream);
    }
  }
  switch (g.out_kind) {
    case OUT_F16: return go<OUT_F16, false>(g, grid, a, a_scale, w, w_scale, stream);
    case OUT_BF16: return go<OUT_BF16, false>(g, grid, a, a_scale, w, w_scale, stream);
    case OUT_I32: return go<OUT_I32, false>(g, grid, a, a_scale, w, w_scale, stream);
    default: return go<OUT_F32, false>(g, grid, a, a_scale, w, w_scale, stream);
  }
}

}  // namespace moeq
