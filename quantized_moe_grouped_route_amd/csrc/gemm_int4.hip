// W4A4 INT4 grouped GEMM with the per-token x per-channel dequantization
// fused into the epilogue (CUTLASS discussion #2855 asks for exactly this
// epilogue, scale_act * scale_weight * accumulator, instead of a separate
// dequantization pass over an int32 buffer).
//
// CDNA4 has no int4 MFMA.  Each packed 32-bit word w holding 8 nibbles is
// split into two int8 words: (w << 4) & 0xF0F0F0F0 holds the even elements
// and w & 0xF0F0F0F0 the odd ones, each byte being 16 * value as a signed
// int8.  A and W get the same split, so the int8 MFMA sums the same
// products, each scaled by 256; |acc| <= K * 64 * 256 < 2^31 for K < 2^17
// (the host rejects larger K), and acc >> 8 is the exact int4 dot product.
//
// Data movement.  A workgroup of 8 waves owns a tile of 256 routed rows x
// 256 weight rows.  K advances in stages of 128 int4 values (64 packed
// bytes of every row), copied global -> LDS by the direct-to-LDS loads into
// a ring of four stages that runs on across tiles: the next tile's first
// stages load during this tile's last steps and its epilogue.  Nibbles stay
// packed in LDS (half the bytes of int8) and each wave splits its fragments
// after reading them; two waves per SIMD let one wave's LDS reads and
// splits overlap the other's MFMAs.  A tile's first stage also copies the
// tile's activation and weight scales into a per-tile LDS buffer for the
// epilogue (one buffer per ring stage, so none is overwritten before its
// epilogue).  Every global load of the main loop is one of these copies, so
// waiting for a stage is an exact vmcnt count (pipeline.h); a tile's row
// gather reads sorted_ids with scalar loads, counted in lgkmcnt instead.
//
// Wave (wm, wn) = (w / 4, w % 4) owns routed rows [128wm, +128) (four
// 32-row MFMA B operands) and weight rows [64wn, +64) (two 32-row A
// operands): 8 accumulators, 6 fragment reads per 16 MFMAs.  The MFMA's C
// layout gives each lane one routed row (l % 32) and runs of 4 consecutive
// weight rows, so the epilogue stores 4 adjacent outputs per lane.
// SILU_MUL: tile rows [64wn, 64wn+32) are the gate rows and [64wn+32,
// 64wn+64) the up rows of output columns [32wn, 32wn+32) of the tile, so
// the gate and up values of one output meet in one lane.
#include <algorithm>

#include "kernels.h"
#include "pipeline.h"
#include "tile.h"

namespace moeq {
namespace {

constexpr int kBM = 256;                                     // routed rows per tile
constexpr int kBN = 256;                                     // weight rows per tile
constexpr int kWaves4 = 8;
constexpr int kThreads4 = 64 * kWaves4;
constexpr int kRowBytes = 64;                                // packed bytes per row per stage
constexpr int kStages4 = 4;
constexpr int kATileBytes = kBM * kRowBytes;                 // 16 KB
constexpr int kStageBytes4 = kATileBytes + kBN * kRowBytes;  // 32 KB
constexpr int kScaleBytes4 = 4096;  // [8 waves][64] activation scales | [8 waves][64] weight scales
constexpr int kCopiesA = kATileBytes / 1024 / kWaves4;       // 1 KB copies per wave per stage
constexpr int kCopiesB = kBN * kRowBytes / 1024 / kWaves4;
constexpr int kCopiesStage = kCopiesA + kCopiesB;
constexpr int kCopiesScale = 2;                              // extra, in a tile's first stage
// Tile t's scales are read at its epilogue, which for half the waves comes
// one stage after its last stage; tile t+5's first stage is issued later.
constexpr int kScaleBufs = 5;
constexpr int kGroupM = 4;                                   // m-tiles per n-tile sweep
static_assert(kCopiesA == 2 && kCopiesB == 2, "copy mapping assumes 2 + 2 copies per wave");

typedef __attribute__((address_space(4))) const int cint4_t;
typedef int i32x16_a4 __attribute__((ext_vector_type(16), aligned(4)));
typedef __attribute__((address_space(4))) const i32x16_a4 ci32x16_t;
// Wave-uniform reads through the constant address space (scalar loads).
__device__ __forceinline__ int ld_uniform_i32(const int* p, int i) { return ((cint4_t*)(p))[i]; }
__device__ __forceinline__ i32x16_a4 ld_uniform_i32x16(const int* p) { return *(ci32x16_t*)(p); }

__device__ __forceinline__ v4i lo_nibbles(u32x4 p) { return __builtin_bit_cast(v4i, (p << 4) & 0xF0F0F0F0u); }
__device__ __forceinline__ v4i hi_nibbles(u32x4 p) { return __builtin_bit_cast(v4i, p & 0xF0F0F0F0u); }

// g * sigmoid(g) with the hardware reciprocal (about 1 ulp) in place of an
// IEEE division: the epilogue's largest VALU cost, and its error stays far
// below the output's own rounding.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// LDS tiles: rows of 64 bytes (four 16-byte chunks), chunk c of row r at
// position c ^ ((r >> 2) & 3).  The LDS serves 16 lanes of a 16-byte read
// per pass from 256 bytes of banks (4 rows); 16 consecutive rows reading
// one logical chunk then land on 16 distinct bank groups.  Fragment rows
// are 32k + lane % 32, so the key is (lane >> 2) & 3.
__device__ __forceinline__ int frag_off(int lane, int c) { return ((c ^ ((lane >> 2) & 3)) << 4); }
// A 1 KB copy moves 16 rows: lane l lands at row l/4, position l%4, so it
// fetches logical chunk (l % 4) ^ ((l / 16) % 4) of its row.
__device__ __forceinline__ int copy_chunk(int lane) { return ((lane & 3) ^ ((lane >> 4) & 3)) << 4; }

struct Tile4 {
  int e, row0, rows, nt;
};

// Work item -> tile with every field wave-uniform.  Same numbering as
// sched_tile: expert-major, and inside an expert kGroupM m-tiles are
// visited for each n-tile before the next n-tile.
__device__ __forceinline__ Tile4 tile_of(const int* tile_start, const int* __restrict__ offsets, int E, int P,
                                         int n_tiles, int item) {
  int bl = 0, bh = E - 1;
  while (bl < bh) {
    const int mid = (bl + bh + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(tile_start[mid]) <= item) bl = mid; else bh = mid - 1;
  }
  const int e = __builtin_amdgcn_readfirstlane(bl);
  const int local = item - __builtin_amdgcn_readfirstlane(tile_start[e]);
  const int lo = min(max(ld_uniform_i32(offsets, e), 0), P);
  const int hi = min(max(ld_uniform_i32(offsets, e + 1), lo), P);
  const int m = hi - lo;
  const int mtiles = (m + kBM - 1) / kBM;
  const int group = local / (kGroupM * n_tiles);
  const int in_group = local - group * kGroupM * n_tiles;
  const int gm = min(kGroupM, mtiles - group * kGroupM);
  const int mt = group * kGroupM + in_group % gm;
  Tile4 t;
  t.e = e;
  t.row0 = lo + mt * kBM;
  t.rows = min(kBM, m - mt * kBM);
  t.nt = in_group / gm;
  return t;
}

// Expert-local weight row of tile row rb (clamped into the matrix for the
// columns past N of a partial last n-tile; those outputs are not stored).
template <bool SILU>
__device__ __forceinline__ int weight_row(const Tile4& t, int rb, int N) {
  if (SILU) {
    const int I = N / 2;
    int col = t.nt * 128 + 32 * (rb >> 6) + (rb & 31);
    if (col >= I) col = t.nt * 128;
    return ((rb >> 5) & 1) * I + col;
  }
  const int r = t.nt * kBN + rb;
  return r < N ? r : t.nt * kBN;
}

// Split fragments of one 32-K substep j of a stage (two per stage): lane
// half h reads chunk 2j + h of its row; the chunk's low nibbles feed one
// MFMA and its high nibbles another.
struct Frag {
  v4i w[2][2];  // [weight operand][low, high nibbles]
  v4i x[4][2];  // [routed-row operand][low, high nibbles]
};

__device__ __forceinline__ Frag read_split(const uint8_t* As, const uint8_t* Bs, int wm, int wn, int lane, int j) {
  const int off = frag_off(lane, 2 * j + (lane >> 5)), l32 = lane & 31;
  u32x4 pw[2], px[4];
#pragma unroll
  for (int o = 0; o < 2; ++o) pw[o] = ld16(Bs + (64 * wn + 32 * o + l32) * kRowBytes + off);
#pragma unroll
  for (int o = 0; o < 4; ++o) px[o] = ld16(As + (128 * wm + 32 * o + l32) * kRowBytes + off);
  Frag f;
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    f.w[o][0] = lo_nibbles(pw[o]);
    f.w[o][1] = hi_nibbles(pw[o]);
  }
#pragma unroll
  for (int o = 0; o < 4; ++o) {
    f.x[o][0] = lo_nibbles(px[o]);
    f.x[o][1] = hi_nibbles(px[o]);
  }
  return f;
}

// 16 MFMAs: the low-nibble pass over the 8 accumulators, then the high pass.
__device__ __forceinline__ void mma_frag(const Frag& f, v16i (&acc)[2][4]) {
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int wo = 0; wo < 2; ++wo)
#pragma unroll
      for (int xo = 0; xo < 4; ++xo) acc[wo][xo] = mfma_i8_32x32x32(f.w[wo][p], f.x[xo][p], acc[wo][xo]);
}

template <int OUT>
__device__ __forceinline__ void store4(void* out, int64_t idx, const float (&o)[4]) {
  typedef typename OutT<OUT>::T T;
  T* dst = static_cast<T*>(out) + idx;
  if constexpr (sizeof(T) == 2) {
    const u32 lo = (u32)OutT<OUT>::from(o[0]) | ((u32)OutT<OUT>::from(o[1]) << 16);
    const u32 hi = (u32)OutT<OUT>::from(o[2]) | ((u32)OutT<OUT>::from(o[3]) << 16);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<v4f*>(dst) = v4f{o[0], o[1], o[2], o[3]};
  }
}

// Epilogue of one tile: value i of accumulator [wo][xo] in lane l is
// weight row 64wn + 32wo + 8(i/4) + 4(l/32) + i%4 and routed row
// 128wm + 32xo + l%32 of the tile.  Scale tables: routed row r at
// float (r / 32) * 64 + r % 32, weight row r at 512 + the same.
template <int OUT, bool SILU>
__device__ __forceinline__ void epilogue(const Tile4& t, const float* sb, int wm, int wn, int lane, int N,
                                         const v16i (&acc)[2][4], void* __restrict__ out) {
  const int h = lane >> 5, l32 = lane & 31;
  const int I = N / 2;
#pragma unroll
  for (int xo = 0; xo < 4; ++xo) {
    const int r = 128 * wm + 32 * xo + l32;
    if (r >= t.rows) continue;
    const int64_t orow = t.row0 + r;
    const float sa = sb[(4 * wm + xo) * 64 + l32];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int m0 = 8 * qq + 4 * h;  // operand row of values 4qq .. 4qq+3
      if constexpr (SILU) {
        const int col0 = t.nt * 128 + 32 * wn + m0;
        if (col0 >= I) continue;
        const v4f sg = *reinterpret_cast<const v4f*>(sb + 512 + (2 * wn) * 64 + m0);
        const v4f su = *reinterpret_cast<const v4f*>(sb + 512 + (2 * wn + 1) * 64 + m0);
        float o[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float g = sa * sg[rr] * (float)(acc[0][xo][4 * qq + rr] >> 8);
          const float u = sa * su[rr] * (float)(acc[1][xo][4 * qq + rr] >> 8);
          o[rr] = silu(g) * u;
        }
        store4<OUT>(out, orow * I + col0, o);
      } else {
#pragma unroll
        for (int wo = 0; wo < 2; ++wo) {
          const int col0 = t.nt * kBN + 64 * wn + 32 * wo + m0;
          if (col0 >= N) continue;
          if constexpr (OUT == OUT_I32) {
            int* dst = static_cast<int*>(out) + orow * N + col0;
            *reinterpret_cast<v4i*>(dst) = v4i{acc[wo][xo][4 * qq] >> 8, acc[wo][xo][4 * qq + 1] >> 8,
                                               acc[wo][xo][4 * qq + 2] >> 8, acc[wo][xo][4 * qq + 3] >> 8};
          } else {
            const v4f sw = *reinterpret_cast<const v4f*>(sb + 512 + (2 * wn + wo) * 64 + m0);
            float o[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) o[rr] = sa * sw[rr] * (float)(acc[wo][xo][4 * qq + rr] >> 8);
            store4<OUT>(out, orow * N + col0, o);
          }
        }
      }
    }
  }
}

template <int OUT, bool SILU>
__global__ __launch_bounds__(kThreads4, 1) void int4_prefill(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scale, int64_t rows_a, int a_sorted,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_ids, int topk, int E, int P, int N,
    int K, void* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages4 * kStageBytes4];
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[kScaleBufs * kScaleBytes4];
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wid >> 2, wn = wid & 3;
  const int l32 = lane & 31;
  const int n_tiles = SILU ? (N / 2 + 127) / 128 : (N + kBN - 1) / kBN;
  const int64_t rowb = K / 2;
  const int steps = K / 128;
  sched_build(tile_start, sched_scratch, offsets, E, P, kBM, n_tiles);
  const int total = __builtin_amdgcn_readfirstlane(tile_start[E]);
  const int G = gridDim.x;
  const int first = xcd_logical_id(blockIdx.x, G);
  if (first >= total) return;
  const int nq = ((total - first + G - 1) / G) * steps;

  // ---- issue cursor: sources of the next stage to copy.  Wave w copies
  // tile rows [32w, 32w+32) of both operands: copy i moves rows
  // 32w + 16i + lane/4.
  const uint8_t* pa[kCopiesA];
  const uint8_t* pb[kCopiesB];
  const float* psa = a_scale;
  const float* psw = w_scale;
  const int cch = copy_chunk(lane);
  int is_item = first, is_step = 0, is_sbuf = 0;
  auto set_tile = [&](int item) __attribute__((always_inline)) {
    const Tile4 t = tile_of(tile_start, offsets, E, P, n_tiles, item);
    int arow[kCopiesA];
#pragma unroll
    for (int i = 0; i < kCopiesA; ++i) {
      const int r0 = 32 * wid + 16 * i;
      int r;
      if (a_sorted || sorted_ids == nullptr) {
        r = t.row0 + min(r0 + (lane >> 2), t.rows - 1);
      } else {
        // the copy's 16 sorted ids (one 64-byte scalar load when all 16
        // rows are in the tile); each lane picks its own
        i32x16_a4 ids;
        if (r0 + 16 <= t.rows) {
          ids = ld_uniform_i32x16(sorted_ids + t.row0 + r0);
        } else {
#pragma unroll
          for (int g = 0; g < 16; ++g) ids[g] = ld_uniform_i32(sorted_ids, t.row0 + min(r0 + g, t.rows - 1));
        }
        int v = ids[0];
#pragma unroll
        for (int g = 1; g < 16; ++g) v = (lane >> 2) == g ? ids[g] : v;
        r = v / topk;
      }
      arow[i] = (r < 0 || r >= rows_a) ? 0 : r;
      pa[i] = a + (int64_t)arow[i] * rowb + cch;
      pb[i] = w + ((int64_t)t.e * N + weight_row<SILU>(t, r0 + (lane >> 2), N)) * rowb + cch;
    }
    // scales of tile rows 32w + l32: copy l32 / 16 holds the routed row in
    // lanes 4 (l32 % 16) .. +3
    const int src = 4 * (l32 & 15);
    const int s0 = __shfl(arow[0], src, 64), s1 = __shfl(arow[1], src, 64);
    psa = a_scale + ((l32 >> 4) ? s1 : s0);
    psw = w_scale + (int64_t)t.e * N + weight_row<SILU>(t, 32 * wid + l32, N);
  };
  const uint32_t ring_lds = lds_addr(ring), sbuf_lds = lds_addr(sbuf);
  auto issue = [&](int slot) __attribute__((always_inline)) {
    const uint32_t base = ring_lds + slot * kStageBytes4;
    const int64_t ko = (int64_t)is_step * kRowBytes;
#pragma unroll
    for (int i = 0; i < kCopiesA; ++i) dma16(pa[i] + ko, base + (kCopiesA * wid + i) * 1024);
#pragma unroll
    for (int i = 0; i < kCopiesB; ++i) dma16(pb[i] + ko, base + kATileBytes + (kCopiesB * wid + i) * 1024);
    if (is_step == 0) {
      const uint32_t sb = sbuf_lds + is_sbuf * kScaleBytes4;
      dma4(psa, sb + wid * 256);
      dma4(psw, sb + 2048 + wid * 256);
      is_sbuf = is_sbuf == kScaleBufs - 1 ? 0 : is_sbuf + 1;
    }
    if (++is_step == steps) {
      is_step = 0;
      is_item += G;
      if (is_item < total) set_tile(is_item);
    }
  };

  set_tile(first);
#pragma nounroll
  for (int s = 0; s < kStages4 && s < nq; ++s) issue(s);

  v16i acc[2][4];
#pragma unroll
  for (int wo = 0; wo < 2; ++wo)
#pragma unroll
    for (int xo = 0; xo < 4; ++xo) acc[wo][xo] = v16i{};

  // The two waves on a SIMD (w and w + 4, i.e. wm = 0 and 1) run half a
  // stage apart: after a barrier a wave with wm = 0 reads and splits its
  // first substep while its partner (wm = 1) runs the MFMAs of the substep
  // it split before the barrier, so one wave's LDS reads and splits overlap
  // the other's MFMAs instead of both waiting on the same phase.
  int ep_item = first, ep_sbuf = 0;
  auto finish_tile = [&]() __attribute__((always_inline)) {
    const Tile4 t = tile_of(tile_start, offsets, E, P, n_tiles, ep_item);
    epilogue<OUT, SILU>(t, reinterpret_cast<const float*>(sbuf + ep_sbuf * kScaleBytes4), wm, wn, lane, N, acc,
                        out);
    // Let the tile's stores (and the copies in flight) complete before the
    // next stage: measured 1-3 % faster on the SiLU GEMM of the Mixtral
    // layer, no change on the other.  A wait for more than the stage needs
    // only makes the later stage waits conservative.
    wait_vmcnt<0>();
#pragma unroll
    for (int wo = 0; wo < 2; ++wo)
#pragma unroll
      for (int xo = 0; xo < 4; ++xo) acc[wo][xo] = v16i{};
    ep_item += G;
    ep_sbuf = ep_sbuf == kScaleBufs - 1 ? 0 : ep_sbuf + 1;
  };
  // Both loops pass the same nq barriers; they are separate so that the
  // held substep is live only in the second.
  auto stage_start = [&](int q) __attribute__((always_inline)) {
    // Stage q must have landed.  The stages issued after it (q+1, q+2, and
    // at q = 0 also q+3) may stay in flight: each is at least kCopiesStage
    // copies (a tile's first stage has kCopiesScale more, which this count
    // leaves out, so the wait is at most a little early-conservative).
    if (q == 0 && nq > 3) wait_vmcnt<3 * kCopiesStage>();
    else if (q + 2 < nq) wait_vmcnt<2 * kCopiesStage>();
    else if (q + 1 < nq) wait_vmcnt<kCopiesStage>();
    else wait_vmcnt<0>();
    raw_barrier();  // every wave's part of stage q is in LDS; stage q-1's slot is free
    if (q >= 1 && q + kStages4 - 1 < nq) issue((unsigned)(q + kStages4 - 1) % kStages4);
    return ring + ((unsigned)q % kStages4) * kStageBytes4;
  };
  if (wm == 0) {
    for (int q = 0, st = 0; q < nq; ++q) {
      const uint8_t* As = stage_start(q);
      mma_frag(read_split(As, As + kATileBytes, wm, wn, lane, 0), acc);
      mma_frag(read_split(As, As + kATileBytes, wm, wn, lane, 1), acc);
      if (++st == steps) {
        st = 0;
        finish_tile();
      }
    }
  } else {
    Frag held;
    for (int q = 0, st = 0; q < nq; ++q) {
      const uint8_t* As = stage_start(q);
      if (q > 0) {
        mma_frag(held, acc);
        if (st == 0) finish_tile();
      }
      mma_frag(read_split(As, As + kATileBytes, wm, wn, lane, 0), acc);
      held = read_split(As, As + kATileBytes, wm, wn, lane, 1);
      if (++st == steps) st = 0;
    }
    mma_frag(held, acc);
    finish_tile();
  }
}

// ------------------------------------------------------------------ decode
// Few routed rows per expert (decode): the weight stream is the whole cost,
// so the wave is the unit of work and every operand arrives through a
// per-wave direct-to-LDS ring, as in the FP8 and NVFP4 streaming schedules.
// The arithmetic is the tiled schedule's: nibble planes scaled by 16, int8
// MFMA, acc >> 8, and the same fp32 epilogue expression, so both schedules
// give identical outputs.
//
// Item = (at most 8 routed rows of one expert) x (32 weight rows): with
// SILU_MUL the 16 gate rows and the 16 up rows of 16 output columns, else
// 32 consecutive rows.  Per K group of 256 values (128 packed bytes of a
// row, one cache line) a ring slot holds the 32 weight rows as four whole-
// line copies of 8 rows (16-byte piece p of row r at position
// p ^ ((r >> 1) & 7)) and the item's 8 activation rows (one copy).  An
// expert with up to 8 rows thus streams its weights once.  The item's
// scales ride in group 0's slot: one 4-byte-per-lane copy, lanes 0..7 the
// rows' activation scales and lanes 8..39 the 32 weight scales, read into
// registers at group 0.
//
// v_mfma_i32_16x16x64_i8 takes the weights as the 16-row operand and the
// routed rows as the 16 columns (columns past the item's rows are
// discarded).  Lane l supplies row l % 16 and 16 bytes of its K quarter
// l / 16: it reads pieces 2q and 2q + 1 of its weight row and of its routed
// row, and each piece gives a low- and a high-nibble plane, so a group is 4
// MFMAs per 16-row block.  Value i of lane l is weight row 4(l/16) + i of
// the block and routed row l % 16.
namespace dd {
constexpr int kM = 8;                                  // routed rows per item
constexpr int kRowsW = 32;                             // weight rows per item
constexpr int kWaves = 4;                              // waves per workgroup, independent
constexpr int kDepth = 3;                              // K groups in flight per wave
constexpr int kW = 0, kX = 4096, kS = 5120;            // slot regions
constexpr int kSlot = 5376;
constexpr int kCopies = 5;                             // per K group: 4 weight, 1 activation
constexpr int kGroupK = 256;
}  // namespace dd

// vmcnt(n * dd::kCopies) for n in [0, kDepth - 1]
__device__ __forceinline__ void wait_groups4(int n) {
  static_assert(dd::kDepth == 3, "wait table");
  if (n <= 0) wait_vmcnt<0>();
  else if (n == 1) wait_vmcnt<dd::kCopies>();
  else wait_vmcnt<2 * dd::kCopies>();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ v4i mfma_i8_16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

template <int OUT, bool SILU>
__global__ __launch_bounds__(64 * dd::kWaves) void int4_decode(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scale, int64_t rows_a, int a_sorted,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_ids, int topk, int E, int P, int N,
    int K, void* __restrict__ out) {
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];
  __shared__ __attribute__((aligned(1024))) uint8_t ring[dd::kWaves][dd::kDepth][dd::kSlot];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_blocks = N / dd::kRowsW;
  sched_build(tile_start, sched_scratch, offsets, E, P, dd::kM, n_blocks);
  const int total = __builtin_amdgcn_readfirstlane(tile_start[E]);
  // Items are dealt round robin over all waves (measured 3 % faster on the
  // Mixtral decode FC1 than dealing them to the fewest waves that need the
  // same number of rounds, and equal on FC2).
  const int active = gridDim.x * dd::kWaves;
  const int wid = blockIdx.x * dd::kWaves + wv;
  const int G = K / dd::kGroupK;
  const int64_t rowb = K / 2;
  const int I = N / 2;
  uint8_t* myring = &ring[wv][0][0];
  const uint32_t lb = lds_addr(myring);
  const int l16 = lane & 15, quarter = lane >> 4;
  // weight copy c (0..3): block c / 2, block row 8 (c % 2) + lane / 8, piece
  // fetched (lane % 8) ^ ((row >> 1) & 7) so that LDS position lane % 8
  // holds it
  const int crow = lane >> 3;  // + 8 (c % 2)
  const int cp0 = ((lane & 7) ^ ((crow >> 1) & 7)) << 4;
  const int cp1 = ((lane & 7) ^ (((crow + 8) >> 1) & 7)) << 4;
  // fragment reads: block row l16, pieces 2 quarter and 2 quarter + 1
  const int wkey = (l16 >> 1) & 7;
  const int wf0 = dd::kW + l16 * 128 + (((2 * quarter) ^ wkey) << 4);
  const int wf1 = dd::kW + l16 * 128 + (((2 * quarter + 1) ^ wkey) << 4);
  const int xslot = l16 < dd::kM ? l16 : 0;
  const int xf0 = dd::kX + xslot * 128 + ((2 * quarter) << 4);
  const int xf1 = xf0 + 16;

  for (int item = wid; item < total; item += active) {
    // Tile of the item, every field wave-uniform (m-tile major, then blocks).
    int bl = 0, bh = E - 1;
    while (bl < bh) {
      const int mid = (bl + bh + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(tile_start[mid]) <= item) bl = mid; else bh = mid - 1;
    }
    const int e = __builtin_amdgcn_readfirstlane(bl);
    const int local = item - __builtin_amdgcn_readfirstlane(tile_start[e]);
    const int lo = min(max(ld_uniform_i32(offsets, e), 0), P);
    const int hi = min(max(ld_uniform_i32(offsets, e + 1), lo), P);
    const int mt = local / n_blocks;
    const int nb = local - mt * n_blocks;
    const int row0 = lo + mt * dd::kM;
    const int rows = min(dd::kM, hi - row0);
    int arow[dd::kM];
#pragma unroll
    for (int j = 0; j < dd::kM; ++j) {
      const int sp = row0 + min(j, rows - 1);
      const int r = (a_sorted || sorted_ids == nullptr) ? sp : ld_uniform_i32(sorted_ids, sp) / topk;
      arow[j] = (r < 0 || r >= rows_a) ? 0 : r;
    }
    // expert-local weight row of item row rb (block rb / 16)
    auto wrow = [&](int rb) __attribute__((always_inline)) {
      if (SILU) return (rb < 16 ? 0 : I) + nb * 16 + (rb & 15);
      return nb * dd::kRowsW + rb;
    };
    const uint8_t* wbase = w + (int64_t)e * N * rowb;
    const uint8_t* sw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      sw[c] = wbase + (int64_t)wrow(16 * (c >> 1) + 8 * (c & 1) + crow) * rowb + ((c & 1) ? cp1 : cp0);
    // per-lane pick among the wave-uniform rows (a select chain, no
    // indexed register array)
    auto pick = [&](int i) __attribute__((always_inline)) {
      int v = arow[0];
#pragma unroll
      for (int j = 1; j < dd::kM; ++j) v = i == j ? arow[j] : v;
      return v;
    };
    const uint8_t* sx = a + (int64_t)pick(lane >> 3) * rowb + ((lane & 7) << 4);
    const float* ss;
    if (lane < dd::kM) ss = a_scale + pick(lane);
    else if (lane < dd::kM + dd::kRowsW) ss = w_scale + (int64_t)e * N + wrow(lane - dd::kM);
    else ss = a_scale + arow[0];
    auto issue = [&](int g) __attribute__((always_inline)) {
      const uint32_t sl = lb + (uint32_t)((g % dd::kDepth) * dd::kSlot);
      const int64_t ko = (int64_t)g * (dd::kGroupK / 2);
#pragma unroll
      for (int c = 0; c < 4; ++c) dma16_nt(sw[c] + ko, sl + dd::kW + c * 1024);
      dma16(sx + ko, sl + dd::kX);
      if (g == 0) dma4(ss, sl + dd::kS);
    };
    const int npre = G < dd::kDepth ? G : dd::kDepth;
    for (int g = 0; g < npre; ++g) issue(g);
    v4i acc[2] = {v4i{}, v4i{}};
    float sa = 0.f;
    v4f sw0 = v4f{}, sw1 = v4f{};
    for (int g = 0; g < G; ++g) {
      const int after = G - 1 - g;
      wait_groups4(after < dd::kDepth - 1 ? after : dd::kDepth - 1);
      const uint8_t* sp = myring + (g % dd::kDepth) * dd::kSlot;
      const u32x4 w00 = ld16(sp + wf0), w01 = ld16(sp + wf1);
      const u32x4 w10 = ld16(sp + 2048 + wf0), w11 = ld16(sp + 2048 + wf1);
      const u32x4 x0 = ld16(sp + xf0), x1 = ld16(sp + xf1);
      if (g == 0) {
        const float* s = reinterpret_cast<const float*>(sp + dd::kS);
        sa = s[xslot];
        sw0 = *reinterpret_cast<const v4f*>(s + dd::kM + 4 * quarter);
        sw1 = *reinterpret_cast<const v4f*>(s + dd::kM + 16 + 4 * quarter);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot is read; it may be refilled
      if (g + dd::kDepth < G) issue(g + dd::kDepth);
      const v4i xl0 = lo_nibbles(x0), xh0 = hi_nibbles(x0), xl1 = lo_nibbles(x1), xh1 = hi_nibbles(x1);
      acc[0] = mfma_i8_16x16x64(lo_nibbles(w00), xl0, acc[0]);
      acc[1] = mfma_i8_16x16x64(lo_nibbles(w10), xl0, acc[1]);
      acc[0] = mfma_i8_16x16x64(hi_nibbles(w00), xh0, acc[0]);
      acc[1] = mfma_i8_16x16x64(hi_nibbles(w10), xh0, acc[1]);
      acc[0] = mfma_i8_16x16x64(lo_nibbles(w01), xl1, acc[0]);
      acc[1] = mfma_i8_16x16x64(lo_nibbles(w11), xl1, acc[1]);
      acc[0] = mfma_i8_16x16x64(hi_nibbles(w01), xh1, acc[0]);
      acc[1] = mfma_i8_16x16x64(hi_nibbles(w11), xh1, acc[1]);
    }
    if (l16 < rows) {
      const int64_t orow = row0 + l16;
      if constexpr (SILU) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gt = sa * sw0[i] * (float)(acc[0][i] >> 8);
          const float up = sa * sw1[i] * (float)(acc[1][i] >> 8);
          o[i] = silu(gt) * up;
        }
        store4<OUT>(out, orow * I + nb * 16 + 4 * quarter, o);
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int64_t idx = orow * N + nb * dd::kRowsW + 16 * b + 4 * quarter;
          if constexpr (OUT == OUT_I32) {
            *reinterpret_cast<v4i*>(static_cast<int*>(out) + idx) =
                v4i{acc[b][0] >> 8, acc[b][1] >> 8, acc[b][2] >> 8, acc[b][3] >> 8};
          } else {
            const v4f s = b ? sw1 : sw0;
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = sa * s[i] * (float)(acc[b][i] >> 8);
            store4<OUT>(out, idx, o);
          }
        }
      }
    }
  }
}

template <int OUT, bool SILU>
hipError_t go_decode(const GroupedArgs& g, const uint8_t* a, const float* a_scale, const uint8_t* w,
                     const float* w_scale, hipStream_t stream) {
  hipLaunchKernelGGL((int4_decode<OUT, SILU>), dim3(g.num_cus * 2), dim3(64 * dd::kWaves), 0, stream, a,
                     a_scale, g.rows_a, g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                     g.N, g.K, g.out);
  return hipGetLastError();
}

template <int OUT, bool SILU>
hipError_t go(const GroupedArgs& g, int grid, const uint8_t* a, const float* a_scale,
              const uint8_t* w, const float* w_scale, hipStream_t stream) {
  hipLaunchKernelGGL((int4_prefill<OUT, SILU>), dim3(grid), dim3(kThreads4), 0, stream, a, a_scale,
                     g.rows_a, g.a_sorted, w, w_scale, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P, g.N,
                     g.K, g.out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_int4(const GroupedArgs& g, const uint8_t* a, const float* a_scale,
                            const uint8_t* w, const float* w_scale, hipStream_t stream) {
  // Upper bound on tiles: every expert adds at most one partial m-tile.
  const int64_t mt_ub = (g.P + kBM - 1) / kBM + std::min<int64_t>(g.E, g.P);
  const int64_t n_tiles = g.silu_mul ? (g.N / 2 + 127) / 128 : (g.N + kBN - 1) / kBN;
  const int64_t items_ub = mt_ub * n_tiles;
  // AUTO takes the streaming schedule when experts hold few rows on average,
  // or when the tiles would leave most compute units idle, and K fills whole
  // 256-value groups (the host rejects DECODE otherwise).
  const bool decode = g.sched == 1 || (g.sched == 0 && g.K % dd::kGroupK == 0 &&
                                       (g.P < (int64_t)16 * g.E || 2 * items_ub < g.num_cus));
  if (decode) {
    if (g.P == 0) return hipSuccess;
    if (g.silu_mul) {
      switch (g.out_kind) {
        case OUT_F16: return go_decode<OUT_F16, true>(g, a, a_scale, w, w_scale, stream);
        case OUT_BF16: return go_decode<OUT_BF16, true>(g, a, a_scale, w, w_scale, stream);
        default: return go_decode<OUT_F32, true>(g, a, a_scale, w, w_scale, stream);
      }
    }
    switch (g.out_kind) {
      case OUT_F16: return go_decode<OUT_F16, false>(g, a, a_scale, w, w_scale, stream);
      case OUT_BF16: return go_decode<OUT_BF16, false>(g, a, a_scale, w, w_scale, stream);
      case OUT_I32: return go_decode<OUT_I32, false>(g, a, a_scale, w, w_scale, stream);
      default: return go_decode<OUT_F32, false>(g, a, a_scale, w, w_scale, stream);
    }
  }
  if (items_ub == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(items_ub, (int64_t)g.num_cus);
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
