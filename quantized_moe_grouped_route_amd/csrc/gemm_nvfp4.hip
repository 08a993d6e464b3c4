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
#include "pipeline.h"
#include "tile.h"

namespace moeq {
namespace {

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// ------------------------------------------------------------------ prefill
// CU work unit: a workgroup of 4 waves owns a 128 (activation rows) x 256
// (weight rows; for SILU_MUL 128 gate rows + the 128 matching up rows)
// tile and walks K in steps of 64 through a 3-stage LDS ring (75 KB), so
// two workgroups share a CU and their phases (dequantization on the VALU,
// MFMAs) interleave.  Stage layout (25 KB):
//   A  128 rows x 128 bytes (64 bf16), 16-byte chunks swizzled as in the
//      FP8 kernel;
//   B  256 rows x 32 packed bytes (64 E2M1 codes), the 16-byte chunk c of
//      row r at position c ^ ((r >> 3) & 1);
//   S  256 rows x 4 scale bytes.
// Wave wn owns 64 weight rows (two 32-row MFMA operands) against all 128
// activation rows, so every weight code is dequantized once per tile.
//
// K slots: in a K step, MFMA lane l (slice l/32) takes the codes
// [32*slice, +32) of its weight row - one 16-byte LDS read, two scale bytes
// - and sub-step s uses codes [32*slice + 8s, +8).  The activation operand
// uses the same slots: slice `slice`, sub-step s = logical chunk 4*slice+s
// of the row's 128 bytes.
namespace pf {
constexpr int kM = 128, kN = 256;
constexpr int kStages = 3;
constexpr int kABytes = kM * 128;
constexpr int kBBytes = kN * 32;
constexpr int kSBytes = kN * 4;
constexpr int kStageBytes = kABytes + kBBytes + kSBytes;
constexpr int kThreads = 256;
}  // namespace pf

template <int OUT, bool SILU>
__global__ __launch_bounds__(pf::kThreads, 2) void nvfp4_prefill(
    const uint16_t* __restrict__ x, int64_t rows_a, int a_sorted, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ w_sf, const float* __restrict__ w_gscale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_ids, int topk, int E, int P, int N,
    int K, void* __restrict__ out) {
  using namespace pf;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];

  const int tid = threadIdx.x, lane = tid & 63, wn = tid >> 6;
  const int I = N / 2;
  const int n_tiles = SILU ? I / 128 : N / kN;
  const int G = K / 64;
  const int64_t xrow_bytes = (int64_t)K * 2, wrow_bytes = K / 2, srow_bytes = K / 16;
  sched_build(tile_start, sched_scratch, offsets, E, P, kM, n_tiles);
  const int total = tile_start[E];

  const int slice = lane >> 5, l32 = lane & 31;
  const int key = frag_key(lane);
  // Weight rows of this lane's two operands (row index in the B tile).
  const int brow0 = SILU ? 32 * wn + l32 : 64 * wn + l32;
  const int brow1 = SILU ? 128 + 32 * wn + l32 : 64 * wn + 32 + l32;
  const int boff0 = kABytes + brow0 * 32 + ((slice ^ ((brow0 >> 3) & 1)) << 4);
  const int boff1 = kABytes + brow1 * 32 + ((slice ^ ((brow1 >> 3) & 1)) << 4);
  const int soff0 = kABytes + kBBytes + brow0 * 4 + slice * 2;
  const int soff1 = kABytes + kBBytes + brow1 * 4 + slice * 2;
  int aoff[4];  // activation chunk offsets for sub-step s (logical chunk 4*slice + s)
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = (((4 * slice + s) ^ key) << 4);

  for (int item = xcd_logical_id(blockIdx.x, gridDim.x); item < total; item += gridDim.x) {
    const Tile t = sched_tile<4>(tile_start, offsets, E, P, kM, n_tiles, item);
    // DMA sources.  A: wave wn moves rows 8q + lane/8 for q = 4wn + j.
    const uint8_t* pa[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = 4 * wn + j;
      const int r = 8 * q + (lane >> 3);
      const int s = t.row0 + min(r, t.rows - 1);
      pa[j] = reinterpret_cast<const uint8_t*>(x) + a_row_of(s, sorted_ids, a_sorted, topk, rows_a) * xrow_bytes +
              dma_chunk(lane, q);
    }
    auto grow = [&](int r) __attribute__((always_inline)) {
      if (!SILU) return (int64_t)t.e * N + (int64_t)t.nt * kN + r;
      return (int64_t)t.e * N + (r < 128 ? (int64_t)t.nt * 128 + r : (int64_t)I + t.nt * 128 + (r - 128));
    };
    // B: wave wn moves rows 64wn + 32j + lane/2 (chunk position lane%2);
    // S: rows 64wn + lane.
    const uint8_t* pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rb = 64 * wn + 32 * j + (lane >> 1);
      pb[j] = w + grow(rb) * wrow_bytes + (((lane & 1) ^ ((rb >> 3) & 1)) << 4);
    }
    const uint8_t* ps = w_sf + grow(64 * wn + lane) * srow_bytes;
    const uint32_t lds_a = lds_addr(smem + wn * 4096);
    const uint32_t lds_b = lds_addr(smem + kABytes + wn * 2048);
    const uint32_t lds_s = lds_addr(smem + kABytes + kBBytes + wn * 256);
    auto issue = [&](int g) __attribute__((always_inline)) {
      const uint32_t st = (uint32_t)((g % kStages) * kStageBytes);
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16(pa[j] + (int64_t)g * 128, lds_a + st + j * 1024);
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16(pb[j] + (int64_t)g * 32, lds_b + st + j * 1024);
      dma4(ps + (int64_t)g * 4, lds_s + st);
    };
    constexpr int kPer = 7;  // loads per wave per stage

    v16f acc[2][4];
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[a2][y] = v16f{};

    raw_barrier();  // the previous tile's LDS reads are done
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
      if (s < G) issue(s);
    int last_issued = min(G, kStages - 1) - 1;

    for (int g = 0; g < G; ++g) {
      if (last_issued - g >= 1) wait_vmcnt<kPer>();
      else wait_vmcnt<0>();
      raw_barrier();  // stage g visible to all waves; stage g-1 is free
      if (g + kStages - 1 < G) {
        issue(g + kStages - 1);
        last_issued = g + kStages - 1;
      }
      const uint8_t* st = smem + (g % kStages) * kStageBytes;
      // Dequantize this lane's 2 x 32 weight codes (exact in bf16).
      const u32x4 q0 = ld16(st + boff0), q1 = ld16(st + boff1);
      const uint32_t sc0 = *reinterpret_cast<const uint16_t*>(st + soff0);
      const uint32_t sc1 = *reinterpret_cast<const uint16_t*>(st + soff1);
      const float s00 = e4m3_to_f32(sc0 & 0xffu), s01 = e4m3_to_f32(sc0 >> 8);
      const float s10 = e4m3_to_f32(sc1 & 0xffu), s11 = e4m3_to_f32(sc1 >> 8);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v8bf wf0 = __builtin_bit_cast(v8bf, dequant8_bf16(q0[s], s < 2 ? s00 : s01));
        const v8bf wf1 = __builtin_bit_cast(v8bf, dequant8_bf16(q1[s], s < 2 ? s10 : s11));
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const v8bf xf = *reinterpret_cast<const v8bf*>(st + (32 * y + l32) * 128 + aoff[s]);
          acc[0][y] = mfma_bf16_32x32x16(wf0, xf, acc[0][y]);
          acc[1][y] = mfma_bf16_32x32x16(wf1, xf, acc[1][y]);
        }
      }
    }

    // Epilogue: global scale (and the SiLU-gated product), output tile
    // through LDS, then 16-byte stores along output rows.
    typedef typename OutT<OUT>::T T;
    constexpr int kCols = SILU ? 128 : 256;
    constexpr int kOutPitch = kCols * (int)sizeof(T) + 16;
    constexpr bool kStaged = kM * kOutPitch <= kStages * kStageBytes;  // else: f32, direct stores
    raw_barrier();  // all waves are done with the ring
    uint8_t* otile = smem;
    const float gs = w_gscale[t.e];
    const int ldo = SILU ? I : N;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      uint8_t* orow = otile + (32 * y + l32) * kOutPitch;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[2][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * q + r;
          if (SILU) {
            v[0][r] = silu(gs * acc[0][y][i]) * (gs * acc[1][y][i]);
            v[1][r] = 0.f;
          } else {
            v[0][r] = gs * acc[0][y][i];
            v[1][r] = gs * acc[1][y][i];
          }
        }
        // weight columns 8q + 4*slice + r of the lane's 32-row operand(s)
        const int col0 = (SILU ? 32 * wn : 64 * wn) + 8 * q + 4 * slice;
#pragma unroll
        for (int a2 = 0; a2 < (SILU ? 1 : 2); ++a2) {
          if constexpr (!kStaged) {
            const int rr = 32 * y + l32;
            if (rr < t.rows)
              *reinterpret_cast<float4*>(static_cast<float*>(out) + (int64_t)(t.row0 + rr) * ldo +
                                         (int64_t)t.nt * kCols + col0 + 32 * a2) =
                  make_float4(v[a2][0], v[a2][1], v[a2][2], v[a2][3]);
            continue;
          }
          uint8_t* dst = orow + (col0 + 32 * a2) * (int)sizeof(T);
          if (sizeof(T) == 2) {
            const u32 lo = pack2<OUT>(v[a2][0], v[a2][1]);
            const u32 hi = pack2<OUT>(v[a2][2], v[a2][3]);
            *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(v[a2][0], v[a2][1], v[a2][2], v[a2][3]);
          }
        }
      }
    }
    raw_barrier();
    if constexpr (kStaged) {
      constexpr int kChunksPerRow = kCols * (int)sizeof(T) / 16;
      uint8_t* obase = static_cast<uint8_t*>(out) + ((int64_t)t.row0 * ldo + (int64_t)t.nt * kCols) * (int)sizeof(T);
#pragma unroll 4
      for (int i = 0; i < kM * kChunksPerRow / kThreads; ++i) {
        const int ci = tid + kThreads * i;
        const int r = ci / kChunksPerRow, c = ci % kChunksPerRow;
        if (r < t.rows)
          st16(obase + (int64_t)r * ldo * (int)sizeof(T) + c * 16, ld16(otile + r * kOutPitch + c * 16));
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
//
// The weight stream is what bounds this schedule: each lane keeps kPre
// chunks (kPre x 16 bytes of codes, their scales) in flight in registers,
// so a CU has enough bytes outstanding to cover the HBM latency.
constexpr int kDecM = 16;
constexpr int kDecNB = 64;  // weight rows per work item
constexpr int kPre = 8;     // weight chunks in flight per lane

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
    // Activation row of this lane (routed row lane % 16).  Lanes past the
    // tile's rows read a valid row too: their MFMA columns are never stored.
    const int mr = lane & 15;
    const bool has_row = mr < t.rows;
    const uint8_t* px = reinterpret_cast<const uint8_t*>(x) +
                        a_row_of(t.row0 + (has_row ? mr : 0), sorted_ids, a_sorted, topk, rows_a) *
                            (int64_t)K * 2 + g * 64;

    v4f acc0 = v4f{}, acc1 = v4f{};
    // One K chunk: 32 codes of this lane's weight row against the matching
    // activation values; two accumulators keep the MFMA chain short.
    auto consume = [&](const u32x4& wq, uint32_t sq, int c) __attribute__((always_inline)) {
      const float s0 = e4m3_to_f32(sq & 0xffu), s1 = e4m3_to_f32(sq >> 8);
      const u32x4 x0 = ld16(px + (int64_t)c * 256), x1 = ld16(px + (int64_t)c * 256 + 16);
      const u32x4 x2 = ld16(px + (int64_t)c * 256 + 32), x3 = ld16(px + (int64_t)c * 256 + 48);
      acc0 = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, dequant8_bf16(wq[0], s0)), __builtin_bit_cast(v8bf, x0), acc0);
      acc1 = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, dequant8_bf16(wq[1], s0)), __builtin_bit_cast(v8bf, x1), acc1);
      acc0 = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, dequant8_bf16(wq[2], s1)), __builtin_bit_cast(v8bf, x2), acc0);
      acc1 = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, dequant8_bf16(wq[3], s1)), __builtin_bit_cast(v8bf, x3), acc1);
    };
    auto wload = [&](int c) __attribute__((always_inline)) {
      return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pw + (int64_t)c * 64));
    };
    auto sload = [&](int c) __attribute__((always_inline)) {
      return (uint32_t)*reinterpret_cast<const uint16_t*>(ps + (int64_t)c * 8);
    };

    u32x4 wbuf[kPre];
    uint32_t sbuf[kPre];
    int c0 = 0;
    if (chunks >= kPre) {
#pragma unroll
      for (int i = 0; i < kPre; ++i) {
        wbuf[i] = wload(i);
        sbuf[i] = sload(i);
      }
      // Steady state: every slot is consumed and refilled kPre chunks ahead.
      for (; c0 + 2 * kPre <= chunks; c0 += kPre) {
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
          const u32x4 wq = wbuf[i];
          const uint32_t sq = sbuf[i];
          wbuf[i] = wload(c0 + kPre + i);
          sbuf[i] = sload(c0 + kPre + i);
          consume(wq, sq, c0 + i);
        }
      }
      // Drain: chunks c0 .. c0+kPre-1 are in the slots; the rest (< kPre)
      // is loaded as slots free up.
#pragma unroll
      for (int i = 0; i < kPre; ++i) {
        const u32x4 wq = wbuf[i];
        const uint32_t sq = sbuf[i];
        if (c0 + kPre + i < chunks) {
          wbuf[i] = wload(c0 + kPre + i);
          sbuf[i] = sload(c0 + kPre + i);
        }
        consume(wq, sq, c0 + i);
      }
      c0 += kPre;
#pragma unroll
      for (int i = 0; i < kPre; ++i)
        if (c0 + i < chunks) consume(wbuf[i], sbuf[i], c0 + i);
    } else {
      for (int c = 0; c < chunks; ++c) consume(wload(c), sload(c), c);
    }
    const v4f acc = acc0 + acc1;
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
    const int grid = (int)std::min<int64_t>(items_ub, (int64_t)g.num_cus * 4);
    hipLaunchKernelGGL((nvfp4_decode<OUT, SILU>), dim3(grid), dim3(256), 0, stream, x, g.rows_a,
                       g.a_sorted, w, sf, gsc, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P, g.N, g.K,
                       g.out);
  } else {
    const int64_t mt_ub = (g.P + pf::kM - 1) / pf::kM + std::min<int64_t>(g.E, g.P);
    const int64_t items_ub = mt_ub * (g.N / pf::kN);
    const int grid = (int)std::min<int64_t>(items_ub, (int64_t)g.num_cus * 2);
    hipLaunchKernelGGL((nvfp4_prefill<OUT, SILU>), dim3(grid), dim3(pf::kThreads), 0, stream, x,
                       g.rows_a, g.a_sorted, w, sf, gsc, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                       g.N, g.K, g.out);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nvfp4(const GroupedArgs& g, const uint16_t* x, const uint8_t* w,
                             const uint8_t* w_sf, const float* w_gscale, hipStream_t stream) {
  if (g.P == 0) return hipSuccess;
  // The streaming schedule when asked for, under AUTO while experts average
  // fewer than 16 rows, and whenever N is not a multiple of the prefill
  // tile (256), which the prefill schedule cannot cover.
  const bool decode = g.sched == 1 || g.N % pf::kN != 0 || (g.sched == 0 && g.P < (int64_t)16 * g.E);
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
