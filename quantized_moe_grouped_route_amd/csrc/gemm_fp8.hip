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
#include <type_traits>

#include "kernels.h"
#include "pipeline.h"
#include "tile.h"

namespace moeq {
namespace {

// Pipeline geometry: kStages stages of (A tile, B tile, scales), each A/B
// tile 128 rows x 128 bytes (one 128-wide K group of e4m3), swizzled.
constexpr int kStages = 4;
constexpr int kWaves8 = 8;
constexpr int kThreads8 = 64 * kWaves8;
constexpr int kTileBytes = 128 * 128;
constexpr int kScaleBytes = kWaves8 * 256;  // per wave: 16 row scales, 1 block scale
constexpr int kStageBytes = 2 * kTileBytes + kScaleBytes;
constexpr int kDmaPerStage = 5;             // per wave: 2 (A) + 2 (B) + 1 (scales)

// Eight waves in two K groups of four: group kg = w / 4 takes the K groups
// of parity kg, so each barrier step covers two 128-wide K groups and each
// SIMD runs one wave of each group; one wave's LDS reads and VALU work
// overlap the other wave's MFMAs.  Inside a group wave (nh, mh) owns weight
// rows [64nh, +64) and activation rows [64mh, +64) of the tile.  The MFMA's
// 32-row operand is the weights and its 32-column operand the activations,
// so each lane's accumulators belong to two activation rows and the
// per-row scale of a K group is two values per lane.  The two groups'
// sums are added through LDS at the end.
template <int OUT>
__global__ __launch_bounds__(kThreads8, 1) void fp8_prefill(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scale, int64_t rows_a, int a_sorted,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_ids, int topk, int E, int P, int N,
    int K, void* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int kg = wid >> 2, nh = (wid >> 1) & 1, mh = wid & 1;
  const int n_tiles = n_tiles_of(N);
  const int G = K / 128;
  sched_build(tile_start, sched_scratch, offsets, E, P, kTileM, n_tiles);
  const int total = tile_start[E];

  const int crow = lane >> 3;
  const int key = frag_key(lane);
  // This lane's two 16-byte chunks of each K half, and its fragment rows.
  const int c0a = (lane >> 5) * 2, c0b = 4 + (lane >> 5) * 2;
  const int oa0 = (c0a ^ key) << 4, oa1 = ((c0a + 1) ^ key) << 4;
  const int ob0 = (c0b ^ key) << 4, ob1 = ((c0b + 1) ^ key) << 4;
  const int rw0 = (64 * nh + (lane & 31)) * 128, rw1 = rw0 + 32 * 128;
  const int mrow0 = 64 * mh + (lane & 31), mrow1 = mrow0 + 32;
  const int rx0 = mrow0 * 128, rx1 = mrow1 * 128;
  const int sidx0 = (mrow0 >> 4) * 64 + (mrow0 & 15), sidx1 = (mrow1 >> 4) * 64 + (mrow1 & 15);

  for (int item = xcd_logical_id(blockIdx.x, gridDim.x); item < total; item += gridDim.x) {
    const Tile t = sched_tile<4>(tile_start, offsets, E, P, kTileM, n_tiles, item);
    // Copies: wave w moves tile rows 8q + lane/8 for q = 2w, 2w+1.
    const uint8_t* pa[2];
    const uint8_t* pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = 2 * wid + j;
      const int r = 8 * q + crow;
      const int s = t.row0 + min(r, t.rows - 1);
      const int ch = dma_chunk(lane, q);
      pa[j] = a + a_row_of(s, sorted_ids, a_sorted, topk, rows_a) * (int64_t)K + ch;
      pb[j] = w + ((int64_t)t.e * N + (int64_t)t.nt * kTileN + r) * (int64_t)K + ch;
    }
    // Scales: wave w moves the 16 row scales of rows [16w, 16w+16) (lanes
    // 0..15) and lane 16 the tile's weight-block scale of the group; the
    // other lanes repeat lane 0's load.
    const int srow = 16 * wid + (lane & 15);
    const float* sb_ptr = w_scale + ((int64_t)t.e * (N / 128) + t.nt) * G;
    const float* psa = a_scale + a_row_of(t.row0 + min(lane < 16 ? srow : 16 * wid, t.rows - 1), sorted_ids,
                                          a_sorted, topk, rows_a);
    const bool sb_lane = lane == 16;

    const uint32_t lds_w = lds_addr(smem + wid * 2048);  // this wave's 2 KB of each tile
    const uint32_t lds_s = lds_addr(smem + 2 * kTileBytes + wid * 256);
    auto issue = [&](int g) __attribute__((always_inline)) {
      const uint32_t st = (uint32_t)((g % kStages) * kStageBytes);
      const int64_t ko = (int64_t)g * 128;
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16(pa[j] + ko, lds_w + st + j * 1024);
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16(pb[j] + ko, lds_w + st + kTileBytes + j * 1024);
      dma4(sb_lane ? sb_ptr + g : psa + (int64_t)g * rows_a, lds_s + st);
    };

    v16f acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = v16f{};

    raw_barrier();  // the previous tile's LDS reads are done
    // Prologue: stages 0 .. 3 in flight.
#pragma unroll
    for (int s = 0; s < kStages; ++s)
      if (s < G) issue(s);
    int last_issued = min(G, kStages) - 1;

    const int steps = (G + 1) / 2;
    auto step_start = [&](int j) __attribute__((always_inline)) {
      // Stages 2j and 2j+1 must have landed; at most the stages after them
      // (issued one step ago) may be in flight.
      const int need = min(2 * j + 1, G - 1);
      const int after = last_issued - need;
      if (after >= 2) wait_vmcnt<2 * kDmaPerStage>();
      else if (after == 1) wait_vmcnt<kDmaPerStage>();
      else wait_vmcnt<0>();
      raw_barrier();  // every wave's share is in LDS; stages 2j-2, 2j-1 are free
      if (j > 0 && 2 * j + 2 < G) {
        issue(2 * j + 2);
        last_issued = 2 * j + 2;
        if (2 * j + 3 < G) {
          issue(2 * j + 3);
          last_issued = 2 * j + 3;
        }
      }
    };
    // The 8 MFMAs of K group g into fresh partials, and the group's scales.
    auto group_mma = [&](int g, v16f (&p)[2][2], float& sc0, float& sc1) __attribute__((always_inline)) {
      const uint8_t* As = smem + (g % kStages) * kStageBytes;
      const uint8_t* Bs = As + kTileBytes;
      const float* Ss = reinterpret_cast<const float*>(As + 2 * kTileBytes);
#define MOEQ_LD8(p, o0, o1) \
  __builtin_bit_cast(v8i, __builtin_shufflevector(ld16((p) + (o0)), ld16((p) + (o1)), 0, 1, 2, 3, 4, 5, 6, 7))
      const v8i w00 = MOEQ_LD8(Bs + rw0, oa0, oa1), w01 = MOEQ_LD8(Bs + rw1, oa0, oa1);
      const v8i x00 = MOEQ_LD8(As + rx0, oa0, oa1), x01 = MOEQ_LD8(As + rx1, oa0, oa1);
      const v8i w10 = MOEQ_LD8(Bs + rw0, ob0, ob1), w11 = MOEQ_LD8(Bs + rw1, ob0, ob1);
      const v8i x10 = MOEQ_LD8(As + rx0, ob0, ob1), x11 = MOEQ_LD8(As + rx1, ob0, ob1);
#undef MOEQ_LD8
      const float sb = Ss[16];
      sc0 = Ss[sidx0] * sb;
      sc1 = Ss[sidx1] * sb;
      p[0][0] = mfma_f8_32x32x64(w00, x00, v16f{});
      p[0][1] = mfma_f8_32x32x64(w00, x01, v16f{});
      p[1][0] = mfma_f8_32x32x64(w01, x00, v16f{});
      p[1][1] = mfma_f8_32x32x64(w01, x01, v16f{});
      p[0][0] = mfma_f8_32x32x64(w10, x10, p[0][0]);
      p[0][1] = mfma_f8_32x32x64(w10, x11, p[0][1]);
      p[1][0] = mfma_f8_32x32x64(w11, x10, p[1][0]);
      p[1][1] = mfma_f8_32x32x64(w11, x11, p[1][1]);
    };
    // Promotion of a group's partials into the fp32 result.
    auto promote = [&](const v16f (&p)[2][2], float sc0, float sc1) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[0][0][i] = __builtin_fmaf(p[0][0][i], sc0, acc[0][0][i]);
        acc[0][1][i] = __builtin_fmaf(p[0][1][i], sc1, acc[0][1][i]);
        acc[1][0][i] = __builtin_fmaf(p[1][0][i], sc0, acc[1][0][i]);
        acc[1][1][i] = __builtin_fmaf(p[1][1][i], sc1, acc[1][1][i]);
      }
    };
    // The two waves on a SIMD belong to different K groups (w and w + 4).
    // Group 0 promotes each group's partials right after its MFMAs; group 1
    // promotes them after the next barrier, before its next fragment reads,
    // so one wave's promotion overlaps the other's reads and MFMAs instead
    // of both leaving the MFMA unit idle at the same time.  The two loops
    // pass the same barriers.
    if (kg == 0) {
      for (int j = 0; j < steps; ++j) {
        step_start(j);
        const int g = 2 * j;
        v16f p[2][2];
        float sc0, sc1;
        group_mma(g, p, sc0, sc1);
        promote(p, sc0, sc1);
      }
    } else {
      v16f p[2][2];
      float sc0 = 0.f, sc1 = 0.f;
      bool held = false;
      for (int j = 0; j < steps; ++j) {
        step_start(j);
        if (held) promote(p, sc0, sc1);
        // keep the held partials' live range from overlapping the next ones
        __builtin_amdgcn_sched_barrier(0);
        const int g = 2 * j + 1;
        held = g < G;
        if (held) group_mma(g, p, sc0, sc1);
      }
      if (held) promote(p, sc0, sc1);
    }

    // Epilogue.  Group 1 parks its fp32 sums in LDS (the ring is idle now);
    // group 0 adds them, rounds, and writes the output tile into LDS rows;
    // then every thread stores 16-byte chunks, 16 lanes per 256-byte row.
    typedef typename OutT<OUT>::T T;
    constexpr int kOutPitch = 128 * (int)sizeof(T) + 16;  // bytes per LDS output row
    raw_barrier();
    float* red = reinterpret_cast<float*>(smem);           // [4 waves][4 sub-tiles][16][64]
    uint8_t* otile = smem + 65536;                         // [128 rows][kOutPitch]
    const int wg = wid & 3;
    if (kg == 1) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int i = 0; i < 16; ++i) red[((wg * 4 + 2 * x + y) * 16 + i) * 64 + lane] = acc[x][y][i];
    }
    raw_barrier();
    if (kg == 0) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[x][y][i] += red[((wg * 4 + 2 * x + y) * 16 + i) * 64 + lane];
      // lane: activation rows mrow0, mrow1; weight columns
      // 64nh + 32x + 8q + 4(lane/32) + r.
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        uint8_t* orow = otile + (y ? mrow1 : mrow0) * kOutPitch + (64 * nh + 4 * (lane >> 5)) * (int)sizeof(T);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint8_t* dst = orow + (32 * x + 8 * q) * (int)sizeof(T);
            if (sizeof(T) == 2) {
              const u32 lo = (u32)OutT<OUT>::from(acc[x][y][4 * q]) | ((u32)OutT<OUT>::from(acc[x][y][4 * q + 1]) << 16);
              const u32 hi = (u32)OutT<OUT>::from(acc[x][y][4 * q + 2]) | ((u32)OutT<OUT>::from(acc[x][y][4 * q + 3]) << 16);
              *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
            } else {
              *reinterpret_cast<float4*>(dst) = make_float4(acc[x][y][4 * q], acc[x][y][4 * q + 1],
                                                            acc[x][y][4 * q + 2], acc[x][y][4 * q + 3]);
            }
          }
      }
    }
    raw_barrier();
    {
      constexpr int kChunksPerRow = 128 * (int)sizeof(T) / 16;
      uint8_t* obase = static_cast<uint8_t*>(out) + ((int64_t)t.row0 * N + (int64_t)t.nt * kTileN) * (int)sizeof(T);
#pragma unroll
      for (int i = 0; i < 128 * kChunksPerRow / kThreads8; ++i) {
        const int ci = tid + kThreads8 * i;
        const int r = ci / kChunksPerRow, c = ci % kChunksPerRow;
        if (r < t.rows)
          st16(obase + (int64_t)r * N * (int)sizeof(T) + c * 16, ld16(otile + r * kOutPitch + c * 16));
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
      hipLaunchKernelGGL(fp8_prefill<OUT_BF16>, dim3(grid), dim3(kThreads8), 0, stream, a, a_scale,
                         g.rows_a, g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                         g.N, g.K, g.out);
      break;
    case OUT_F16:
      hipLaunchKernelGGL(fp8_prefill<OUT_F16>, dim3(grid), dim3(kThreads8), 0, stream, a, a_scale,
                         g.rows_a, g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                         g.N, g.K, g.out);
      break;
    default:
      hipLaunchKernelGGL(fp8_prefill<OUT_F32>, dim3(grid), dim3(kThreads8), 0, stream, a, a_scale,
                         g.rows_a, g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                         g.N, g.K, g.out);
      break;
  }
  return hipGetLastError();
}

}  // namespace moeq
