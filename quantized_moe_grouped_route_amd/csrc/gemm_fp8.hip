// FP8 e4m3 block-scaled grouped GEMM (CUTLASS issue #2087: A scaled per
// token per 128 columns of K with the scales stored M-contiguous, B scaled
// per 128x128 block, fp32 accumulation).
//
// Per 128-wide K group g the MFMAs accumulate the group's partial sums from
// zero, then the partial is promoted into the fp32 result with the
// combined scale a_scale[g][row] * w_scale[e][n/128][g].  A 128-column tile
// lies inside one weight scale block, so w_scale is one scalar per (tile,
// group) and a_scale one value per output row.
#include <algorithm>

#include "kernels.h"
#include "tile.h"

namespace moeq {
namespace {

template <int OUT>
__global__ __launch_bounds__(kThreadsT, 1) void fp8_prefill(
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
  const int n_tiles = n_tiles_of(N);
  const int G = K / 128;
  sched_build(tile_start, sched_scratch, offsets, E, P, kTileM, n_tiles);
  const int total = tile_start[E];

  const int lrow = tid >> 3, lchunk = (tid & 7) * 16;  // global->LDS mapping

  for (int item = xcd_logical_id(blockIdx.x, gridDim.x); item < total; item += gridDim.x) {
    const Tile t = sched_tile<4>(tile_start, offsets, E, P, kTileM, n_tiles, item);

    // This thread's four A rows and four B rows.
    const uint8_t* pa[4];
    const uint8_t* pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = lrow + 32 * i;
      const int s = t.row0 + min(j, t.rows - 1);
      pa[i] = a + a_row_of(s, sorted_ids, a_sorted, topk, rows_a) * (int64_t)K + lchunk;
      pb[i] = w + ((int64_t)t.e * N + (int64_t)t.nt * kTileN + j) * (int64_t)K + lchunk;
    }
    int64_t sa_row = 0;
    if (tid < kTileM) sa_row = a_row_of(t.row0 + min(tid, t.rows - 1), sorted_ids, a_sorted, topk, rows_a);
    const float* sb_ptr = w_scale + ((int64_t)t.e * (N / 128) + t.nt) * G;

    v16f acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = v16f{};

    u32x4 ra[4], rb[4];
    float rsa = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(pa[i]);
      rb[i] = ld16(pb[i]);
    }
    if (tid < kTileM) rsa = a_scale[sa_row];

    for (int g = 0; g < G; ++g) {
      __syncthreads();  // previous step's fragment reads are done
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st16(lds_a + (lrow + 32 * i) * kPitch + lchunk, ra[i]);
        st16(lds_b + (lrow + 32 * i) * kPitch + lchunk, rb[i]);
      }
      if (tid < kTileM) lds_sa[tid] = rsa;
      const float sb = sb_ptr[g];
      __syncthreads();
      if (g + 1 < G) {  // prefetch the next group while this one computes
        const int64_t off = (int64_t)(g + 1) * 128;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ra[i] = ld16(pa[i] + off);
          rb[i] = ld16(pb[i] + off);
        }
        if (tid < kTileM) rsa = a_scale[(int64_t)(g + 1) * rows_a + sa_row];
      }

      v16f part[2][2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) part[x][y] = v16f{};
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int koff = kh * 64 + (lane >> 5) * 32;
        v8i fa[2], fb[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const uint8_t* p = lds_a + (64 * wm + 32 * x + (lane & 31)) * kPitch + koff;
          fa[x] = *reinterpret_cast<const v8i*>(p);
        }
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const uint8_t* p = lds_b + (b_lds_row(false, wn, y) + (lane & 31)) * kPitch + koff;
          fb[y] = *reinterpret_cast<const v8i*>(p);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y) part[x][y] = mfma_f8_32x32x64(fa[x], fb[y], part[x][y]);
      }
      // Promote: acc += part * a_scale[g][row] * w_scale[tile][g].
#pragma unroll
      for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 s4 = *reinterpret_cast<const float4*>(
              lds_sa + 64 * wm + 32 * x + 8 * q + 4 * (lane >> 5));
          const float sc[4] = {s4.x * sb, s4.y * sb, s4.z * sb, s4.w * sb};
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int y = 0; y < 2; ++y)
              acc[x][y][4 * q + r] = __builtin_fmaf(part[x][y][4 * q + r], sc[r], acc[x][y][4 * q + r]);
        }
      }
    }

    // Epilogue: rounded stores of the valid rows.
    typedef typename OutT<OUT>::T T;
    T* o = static_cast<T*>(out);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const int col = t.nt * kTileN + b_lds_row(false, wn, y) + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rr = 64 * wm + 32 * x + c32_row(i, lane);
          if (rr < t.rows) o[(int64_t)(t.row0 + rr) * N + col] = OutT<OUT>::from(acc[x][y][i]);
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm_fp8(const GroupedArgs& g, const uint8_t* a, const float* a_scale,
                           const uint8_t* w, const float* w_scale, hipStream_t stream) {
  // Upper bound on tiles: every expert adds at most one partial m-tile.
  const int64_t mt_ub = (g.P + kTileM - 1) / kTileM + std::min<int64_t>(g.E, g.P);
  const int64_t items_ub = mt_ub * (g.N / kTileN);
  if (items_ub == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(items_ub, (int64_t)g.num_cus);
  switch (g.out_kind) {
    case OUT_BF16:
      hipLaunchKernelGGL(fp8_prefill<OUT_BF16>, dim3(grid), dim3(kThreadsT), 0, stream, a, a_scale,
                         g.rows_a, g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                         g.N, g.K, g.out);
      break;
    case OUT_F16:
      hipLaunchKernelGGL(fp8_prefill<OUT_F16>, dim3(grid), dim3(kThreadsT), 0, stream, a, a_scale,
                         g.rows_a, g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                         g.N, g.K, g.out);
      break;
    default:
      hipLaunchKernelGGL(fp8_prefill<OUT_F32>, dim3(grid), dim3(kThreadsT), 0, stream, a, a_scale,
                         g.rows_a, g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                         g.N, g.K, g.out);
      break;
  }
  return hipGetLastError();
}

}  // namespace moeq
