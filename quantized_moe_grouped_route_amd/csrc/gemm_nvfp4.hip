// NVFP4 W4A16 grouped GEMM (tilelang_kernels.py's grouped_gemm_fp4 with the
// per-expert global scale of megamoe_rm.cu): bf16 activations times E2M1
// weights with UE4M3 per-16 block scales, fp32 accumulation, the global
// scale and the optional SiLU-gated product applied in the epilogue.
//
// Two schedules over one weight layout ([E][N][K/2] codes, [E][N][K/16]
// scales), as megamoe_rm.cu keeps one copy of the weights for its decode
// kernel and for prefill:
//   prefill  128x128 MFMA tiles; weights dequantized once per tile while
//            they are staged into LDS, bf16 MFMA 32x32x16.
//   decode   few rows per expert: each workgroup streams a block of weight
//            rows in long contiguous runs and runs 16x16x32 bf16 MFMAs with
//            the weights as the 16-row operand and the (at most 16) routed
//            rows as the other, so no cross-lane reduction is needed.
#include <algorithm>

#include "kernels.h"
#include "nvfp4.h"
#include "tile.h"

namespace moeq {
namespace {

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// ------------------------------------------------------------------ prefill
// K step = 64 values: A rows 128 bytes of bf16 (thread t: row t/8 + 32i,
// bytes (t%8)*16), B rows 32 packed bytes + 4 scale bytes (thread t: row
// t/2, packed bytes (t%2)*16 = 32 codes = 2 scale blocks), dequantized to
// 128 bytes of bf16 per row in LDS.
template <int OUT, bool SILU>
__global__ __launch_bounds__(kThreadsT, 1) void nvfp4_prefill(
    const uint16_t* __restrict__ x, int64_t rows_a, int a_sorted, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ w_sf, const float* __restrict__ w_gscale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_ids, int topk, int E, int P, int N,
    int K, void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kTileM * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[kTileN * kPitch];
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int n_tiles = N / kTileN;
  const int I = N / 2;
  const int steps = K / 64;
  const int64_t wrow_bytes = K / 2, srow_bytes = K / 16;
  sched_build(tile_start, sched_scratch, offsets, E, P, kTileM, n_tiles);
  const int total = tile_start[E];

  const int arow = tid >> 3, achunk = (tid & 7) * 16;  // A: bytes of bf16
  const int brow = tid >> 1, bhalf = tid & 1;          // B: 16 packed bytes

  for (int item = xcd_logical_id(blockIdx.x, gridDim.x); item < total; item += gridDim.x) {
    const Tile t = sched_tile<4>(tile_start, offsets, E, P, kTileM, n_tiles, item);
    const uint8_t* pa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = t.row0 + min(arow + 32 * i, t.rows - 1);
      pa[i] = reinterpret_cast<const uint8_t*>(x) +
              a_row_of(s, sorted_ids, a_sorted, topk, rows_a) * (int64_t)K * 2 + achunk;
    }
    const int64_t wr = (int64_t)t.e * N + b_global_row(SILU, t.nt, brow, I);
    const uint8_t* pw = w + wr * wrow_bytes + bhalf * 16;
    const uint8_t* ps = w_sf + wr * srow_bytes + bhalf * 2;

    v16f acc[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[p][q] = v16f{};

    u32x4 ra[4], rw;
    uint32_t rs;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ld16(pa[i]);
    rw = ld16(pw);
    rs = *reinterpret_cast<const uint16_t*>(ps);

    for (int st = 0; st < steps; ++st) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st16(lds_a + (arow + 32 * i) * kPitch + achunk, ra[i]);
      {
        const float s0 = e4m3_to_f32(rs & 0xffu), s1 = e4m3_to_f32((rs >> 8) & 0xffu);
        uint8_t* db = lds_b + brow * kPitch + bhalf * 64;
        st16(db, dequant8_bf16(rw.x, s0));
        st16(db + 16, dequant8_bf16(rw.y, s0));
        st16(db + 32, dequant8_bf16(rw.z, s1));
        st16(db + 48, dequant8_bf16(rw.w, s1));
      }
      __syncthreads();
      if (st + 1 < steps) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ra[i] = ld16(pa[i] + (int64_t)(st + 1) * 128);
        rw = ld16(pw + (int64_t)(st + 1) * 32);
        rs = *reinterpret_cast<const uint16_t*>(ps + (int64_t)(st + 1) * 4);
      }
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int koff = kq * 32 + (lane >> 5) * 16;
        v8bf fa[2], fb[2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
          fa[p] = *reinterpret_cast<const v8bf*>(lds_a + (64 * wm + 32 * p + (lane & 31)) * kPitch + koff);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          fb[q] = *reinterpret_cast<const v8bf*>(lds_b + (b_lds_row(SILU, wn, q) + (lane & 31)) * kPitch + koff);
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int q = 0; q < 2; ++q) acc[p][q] = mfma_bf16_32x32x16(fa[p], fb[q], acc[p][q]);
      }
    }

    const float gs = w_gscale[t.e];
    typedef typename OutT<OUT>::T T;
    T* o = static_cast<T*>(out);
    if (SILU) {
      const int col = t.nt * 64 + 32 * wn + (lane & 31);
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rr = 64 * wm + 32 * p + c32_row(i, lane);
          const float g = gs * acc[p][0][i], u = gs * acc[p][1][i];
          if (rr < t.rows) o[(int64_t)(t.row0 + rr) * I + col] = OutT<OUT>::from(silu(g) * u);
        }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = t.nt * kTileN + b_lds_row(false, wn, q) + (lane & 31);
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int rr = 64 * wm + 32 * p + c32_row(i, lane);
            if (rr < t.rows) o[(int64_t)(t.row0 + rr) * N + col] = OutT<OUT>::from(gs * acc[p][q][i]);
          }
      }
    }
  }
}

// ------------------------------------------------------------------ decode
// Work item = (expert, 16-row m-tile, 64-column n-block); 4 waves, wave v
// computes output columns [16v, 16v+16) of the block.  For SILU_MUL a block
// covers 32 output columns: waves 0,1 the gate rows, waves 2,3 the up rows
// of the same columns, met through LDS in the epilogue.
//
// Weights are the MFMA's 16-row operand: lane l owns weight row (l % 16) of
// the wave's 16 rows and, in K chunk c (128 values = 64 bytes per row), the
// 16 bytes at (l / 16) * 16, i.e. 32 codes.  Those feed 4 MFMAs; MFMA i
// takes codes [8i, 8i+8) of every lane's 32, so its K slot (l/16, 0..7)
// holds K index 128c + 32(l/16) + 8i + (0..7).  The activation operand uses
// the same slots: lane l (routed row l % 16) loads x[row][that K range].
constexpr int kDecM = 16;
constexpr int kDecNB = 64;  // weight rows per work item

template <int OUT, bool SILU>
__global__ __launch_bounds__(256) void nvfp4_decode(
    const uint16_t* __restrict__ x, int64_t rows_a, int a_sorted, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ w_sf, const float* __restrict__ w_gscale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_ids, int topk, int E, int P, int N,
    int K, void* __restrict__ out) {
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];
  __shared__ float lds_up[2][kDecM][16 + 1];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int I = N / 2;
  // n-blocks: NONE covers 64 columns per item, SILU 32 output columns.
  const int n_blocks = SILU ? (I / 32) : (N / kDecNB);
  sched_build(tile_start, sched_scratch, offsets, E, P, kDecM, n_blocks);
  const int total = tile_start[E];
  const int64_t wrow_bytes = K / 2, srow_bytes = K / 16;
  const int chunks = K / 128;

  for (int item = xcd_logical_id(blockIdx.x, gridDim.x); item < total; item += gridDim.x) {
    const Tile t = sched_tile<1>(tile_start, offsets, E, P, kDecM, n_blocks, item);
    // Weight row of this lane.
    int wrow;
    if (SILU) wrow = (wv < 2 ? 0 : I) + t.nt * 32 + (wv & 1) * 16 + (lane & 15);
    else wrow = t.nt * kDecNB + wv * 16 + (lane & 15);
    const int g = lane >> 4;
    const uint8_t* pw = w + ((int64_t)t.e * N + wrow) * wrow_bytes + g * 16;
    const uint8_t* ps = w_sf + ((int64_t)t.e * N + wrow) * srow_bytes + g * 2;
    // Activation row of this lane (routed row lane % 16), or none.
    const int mr = lane & 15;
    const bool has_row = mr < t.rows;
    const uint8_t* px = reinterpret_cast<const uint8_t*>(x) +
                        a_row_of(t.row0 + (has_row ? mr : 0), sorted_ids, a_sorted, topk, rows_a) *
                            (int64_t)K * 2 + g * 64;

    v4f acc = v4f{};
    for (int c = 0; c < chunks; ++c) {
      const u32x4 wq = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pw + (int64_t)c * 64));
      const uint32_t sq = *reinterpret_cast<const uint16_t*>(ps + (int64_t)c * 8);
      const float s0 = e4m3_to_f32(sq & 0xffu), s1 = e4m3_to_f32(sq >> 8);
      u32x4 xa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xa[i] = has_row ? ld16(px + (int64_t)c * 256 + i * 16) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 wd = dequant8_bf16(wq[i], i < 2 ? s0 : s1);
        acc = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, wd), __builtin_bit_cast(v8bf, xa[i]), acc);
      }
    }
    // acc value i of lane l: weight row 4*(l/16) + i of the wave's 16, routed
    // row l % 16.
    const float gs = w_gscale[t.e];
    typedef typename OutT<OUT>::T T;
    T* o = static_cast<T*>(out);
    if (SILU) {
      __syncthreads();
      if (wv >= 2)
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_up[wv - 2][lane & 15][4 * (lane >> 4) + i] = gs * acc[i];
      __syncthreads();
      if (wv < 2 && has_row)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = t.nt * 32 + wv * 16 + 4 * (lane >> 4) + i;
          const float gv = gs * acc[i], uv = lds_up[wv][lane & 15][4 * (lane >> 4) + i];
          o[(int64_t)(t.row0 + mr) * I + col] = OutT<OUT>::from(silu(gv) * uv);
        }
    } else if (has_row) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = t.nt * kDecNB + wv * 16 + 4 * (lane >> 4) + i;
        o[(int64_t)(t.row0 + mr) * N + col] = OutT<OUT>::from(gs * acc[i]);
      }
    }
  }
}

template <int OUT, bool SILU>
hipError_t go(const GroupedArgs& g, bool decode, const uint16_t* x, const uint8_t* w,
              const uint8_t* sf, const float* gsc, hipStream_t stream) {
  if (decode) {
    const int64_t mt_ub = (g.P + kDecM - 1) / kDecM + std::min<int64_t>(g.E, g.P);
    const int64_t items_ub = mt_ub * (SILU ? g.N / 64 : g.N / kDecNB);
    const int grid = (int)std::min<int64_t>(items_ub, (int64_t)g.num_cus * 8);
    hipLaunchKernelGGL((nvfp4_decode<OUT, SILU>), dim3(grid), dim3(256), 0, stream, x, g.rows_a,
                       g.a_sorted, w, sf, gsc, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P, g.N, g.K,
                       g.out);
  } else {
    const int64_t mt_ub = (g.P + kTileM - 1) / kTileM + std::min<int64_t>(g.E, g.P);
    const int64_t items_ub = mt_ub * (g.N / kTileN);
    const int grid = (int)std::min<int64_t>(items_ub, (int64_t)g.num_cus * 2);
    hipLaunchKernelGGL((nvfp4_prefill<OUT, SILU>), dim3(grid), dim3(kThreadsT), 0, stream, x,
                       g.rows_a, g.a_sorted, w, sf, gsc, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                       g.N, g.K, g.out);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nvfp4(const GroupedArgs& g, const uint16_t* x, const uint8_t* w,
                             const uint8_t* w_sf, const float* w_gscale, hipStream_t stream) {
  if (g.P == 0) return hipSuccess;
  // AUTO: the streaming schedule while experts average fewer than 16 rows.
  const bool decode = g.sched == 1 || (g.sched == 0 && g.P < (int64_t)16 * g.E);
  if (g.silu_mul) {
    switch (g.out_kind) {
      case OUT_F16: return go<OUT_F16, true>(g, decode, x, w, w_sf, w_gscale, stream);
      case OUT_BF16: return go<OUT_BF16, true>(g, decode, x, w, w_sf, w_gscale, stream);
      default: return go<OUT_F32, true>(g, decode, x, w, w_sf, w_gscale, stream);
    }
  }
  switch (g.out_kind) {
    case OUT_F16: return go<OUT_F16, false>(g, decode, x, w, w_sf, w_gscale, stream);
    case OUT_BF16: return go<OUT_BF16, false>(g, decode, x, w, w_sf, w_gscale, stream);
    default: return go<OUT_F32, false>(g, decode, x, w, w_sf, w_gscale, stream);
  }
}

}  // namespace moeq
