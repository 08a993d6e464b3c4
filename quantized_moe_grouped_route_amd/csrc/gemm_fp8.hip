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


// ------------------------------------------------------------------ decode
// Few routed rows per expert (decode): the weight stream is the whole cost,
// so the wave is the unit of work and every operand arrives through a
// per-wave direct-to-LDS ring, as in the NVFP4 decode schedule.
//
// Item = (tile of at most 4 routed rows of one expert, 16 weight rows).
// Per 128-wide K group the ring slot holds the 16 weight rows (two whole-
// line copies of 8 rows x 128 bytes, piece p of row r at position
// p ^ ((r >> 1) & 7)), the tile's activation rows (one copy: 4 rows x 128
// bytes; the upper 32 lanes repeat them) and the scales (one 4-byte copy:
// lanes 0..3 the rows' activation scales of the group, lane 4 the weight
// block scale).  One v_mfma_scale_f32_16x16x128_f8f6f4 per group takes the
// weights as the 16-row operand (lane l: row l % 16, K bytes [32(l/16),
// +32)) and the activation rows as the 16 columns (columns past the tile
// are discarded); its partial is promoted with sa[g][row] * sw[e][n/128][g]
// as in the prefill schedule.
namespace fd {
constexpr int kM = 4;                       // routed rows per item
constexpr int kWaves = 4;                   // waves per workgroup, independent
constexpr int kDepth = 4;                   // K groups in flight per wave
constexpr int kW = 0, kX = 2048, kS = 3072;  // slot regions
constexpr int kSlot = 3328;
constexpr int kCopies = 4;                  // per K group: 2 weight, 1 activation, 1 scale
}  // namespace fd

typedef __attribute__((address_space(4))) const int cint8_t_;
__device__ __forceinline__ int ld_uniform8(const int* p, int i) { return ((cint8_t_*)(p))[i]; }

// vmcnt(n * fd::kCopies) for n in [0, kDepth - 1]
__device__ __forceinline__ void wait_groups(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<fd::kCopies>(); break;
    case 2: wait_vmcnt<2 * fd::kCopies>(); break;
    default: wait_vmcnt<3 * fd::kCopies>(); break;
  }
  asm volatile("" ::: "memory");
}

template <int OUT>
__global__ __launch_bounds__(64 * fd::kWaves) void fp8_decode(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scale, int64_t rows_a, int a_sorted,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_ids, int topk, int E, int P, int N,
    int K, void* __restrict__ out) {
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];
  __shared__ __attribute__((aligned(1024))) uint8_t ring[fd::kWaves][fd::kDepth][fd::kSlot];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_blocks = N / 16;
  sched_build(tile_start, sched_scratch, offsets, E, P, fd::kM, n_blocks);
  const int total = __builtin_amdgcn_readfirstlane(tile_start[E]);
  // Items are dealt round robin over all waves (as in the INT4 and NVFP4
  // streaming schedules; equal to dealing them to the fewest waves here).
  const int active = gridDim.x * fd::kWaves;
  const int wid = blockIdx.x * fd::kWaves + wv;
  if (wid >= total) return;
  const int G = K / 128;
  uint8_t* myring = &ring[wv][0][0];
  const uint32_t lb = lds_addr(myring);
  const int l16 = lane & 15, quarter = lane >> 4;
  // weight copy h: lane -> row 8h + lane/8, piece (lane % 8) ^ ((row >> 1) & 7)
  const int wr0 = lane >> 3, wr1 = 8 + (lane >> 3);
  const int wp0 = ((lane & 7) ^ ((wr0 >> 1) & 7)) << 4, wp1 = ((lane & 7) ^ ((wr1 >> 1) & 7)) << 4;
  // fragment reads: row l16, pieces 2*quarter and 2*quarter + 1
  const int wkey = (l16 >> 1) & 7;
  const int wf0 = fd::kW + l16 * 128 + (((2 * quarter) ^ wkey) << 4);
  const int wf1 = fd::kW + l16 * 128 + (((2 * quarter + 1) ^ wkey) << 4);
  const int xslot = l16 < fd::kM ? l16 : 0;
  const int xf0 = fd::kX + xslot * 128 + ((2 * quarter) << 4);
  const int xf1 = xf0 + 16;

  for (int item = wid; item < total; item += active) {
    // Tile of the item, every field wave-uniform (m-tile major, then n-blocks).
    int bl = 0, bh = E - 1;
    while (bl < bh) {
      const int mid = (bl + bh + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(tile_start[mid]) <= item) bl = mid; else bh = mid - 1;
    }
    const int e = __builtin_amdgcn_readfirstlane(bl);
    const int local = item - __builtin_amdgcn_readfirstlane(tile_start[e]);
    const int lo = min(max(ld_uniform8(offsets, e), 0), P);
    const int hi = min(max(ld_uniform8(offsets, e + 1), lo), P);
    const int mt = local / n_blocks;
    const int nb = local - mt * n_blocks;
    const int row0 = lo + mt * fd::kM;
    const int rows = min(fd::kM, hi - row0);
    int arow[fd::kM];
#pragma unroll
    for (int j = 0; j < fd::kM; ++j) {
      const int sp = row0 + min(j, rows - 1);
      const int64_t r = (a_sorted || sorted_ids == nullptr) ? (int64_t)sp : (int64_t)(ld_uniform8(sorted_ids, sp) / topk);
      arow[j] = (r < 0 || r >= rows_a) ? 0 : (int)r;
    }
    const int64_t wrow = (int64_t)e * N + (int64_t)nb * 16;
    const uint8_t* sw0 = w + (wrow + wr0) * K + wp0;
    const uint8_t* sw1 = w + (wrow + wr1) * K + wp1;
    const int xr = (lane >> 3) & 3;
    const int xrow = xr == 0 ? arow[0] : xr == 1 ? arow[1] : xr == 2 ? arow[2] : arow[3];
    const uint8_t* sx = a + (int64_t)xrow * K + ((lane & 7) << 4);
    const int srow = lane < fd::kM ? (lane == 0 ? arow[0] : lane == 1 ? arow[1] : lane == 2 ? arow[2] : arow[3]) : arow[0];
    const float* ssa = a_scale + srow;                                          // + g * rows_a
    const float* ssw = w_scale + ((int64_t)e * (N / 128) + (nb * 16) / 128) * G;  // + g
    auto issue = [&](int g) __attribute__((always_inline)) {
      const uint32_t sl = lb + (uint32_t)((g % fd::kDepth) * fd::kSlot);
      const int64_t ko = (int64_t)g * 128;
      dma16_nt(sw0 + ko, sl + fd::kW);
      dma16_nt(sw1 + ko, sl + fd::kW + 1024);
      dma16(sx + ko, sl + fd::kX);
      dma4(lane == fd::kM ? ssw + g : ssa + (int64_t)g * rows_a, sl + fd::kS);
    };
    const int npre = G < fd::kDepth ? G : fd::kDepth;
    for (int g = 0; g < npre; ++g) issue(g);
    v4f acc = v4f{};
    for (int g = 0; g < G; ++g) {
      const int after = G - 1 - g;
      wait_groups(after < fd::kDepth - 1 ? after : fd::kDepth - 1);
      const uint8_t* sp = myring + (g % fd::kDepth) * fd::kSlot;
      const v8i wfr = __builtin_bit_cast(v8i, __builtin_shufflevector(ld16(sp + wf0), ld16(sp + wf1), 0, 1, 2, 3, 4, 5, 6, 7));
      const v8i xfr = __builtin_bit_cast(v8i, __builtin_shufflevector(ld16(sp + xf0), ld16(sp + xf1), 0, 1, 2, 3, 4, 5, 6, 7));
      const float* ss = reinterpret_cast<const float*>(sp + fd::kS);
      const float sc = ss[xslot] * ss[fd::kM];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot is read; it may be refilled
      if (g + fd::kDepth < G) issue(g + fd::kDepth);
      const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wfr, xfr, v4f{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(p[i], sc, acc[i]);
    }
    // value i of lane l: weight row 4 * quarter + i, routed row l16 of the tile
    if (l16 < rows) {
      typedef typename OutT<OUT>::T T;
      T* o = static_cast<T*>(out) + (int64_t)(row0 + l16) * N + nb * 16 + 4 * quarter;
      if constexpr (sizeof(T) == 2) {
        const u32 v0 = (u32)OutT<OUT>::from(acc[0]) | ((u32)OutT<OUT>::from(acc[1]) << 16);
        const u32 v1 = (u32)OutT<OUT>::from(acc[2]) | ((u32)OutT<OUT>::from(acc[3]) << 16);
        *reinterpret_cast<uint2*>(o) = make_uint2(v0, v1);
      } else {
        *reinterpret_cast<v4f*>(o) = acc;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_fp8(const GroupedArgs& g, const uint8_t* a, const float* a_scale,
                           const uint8_t* w, const float* w_scale, hipStream_t stream) {
  // AUTO takes the decode schedule when experts hold few rows on average.
  const bool decode = g.sched == 1 || (g.sched == 0 && g.P < (int64_t)16 * g.E);
  if (decode) {
    if (g.P == 0) return hipSuccess;
    const int grid = g.num_cus * 2;
#define MOEQ_FD(OK)                                                                                              \
  hipLaunchKernelGGL(fp8_decode<OK>, dim3(grid), dim3(64 * fd::kWaves), 0, stream, a, a_scale, g.rows_a,         \
                     g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P, g.N, g.K, g.out)
    switch (g.out_kind) {
      case OUT_BF16: MOEQ_FD(OUT_BF16); break;
      case OUT_F16: MOEQ_FD(OUT_F16); break;
      default: MOEQ_FD(OUT_F32); break;
    }
#undef MOEQ_FD
    return hipGetLastError();
  }
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
