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
//   decode   few rows per expert: each wave streams 32 weight rows through
//            a direct-to-LDS ring and runs 16x16x32 bf16 MFMAs with the
//            weights as the 16-row operand and the (at most 4) routed rows
//            as the other, so no cross-lane reduction is needed.
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "nvfp4.h"
#include "pipeline.h"
#include "tile.h"

namespace moeq {
namespace {

// g * sigmoid(g) with the hardware reciprocal (about 1 ulp) in place of an
// IEEE division: the epilogue's largest VALU cost, and its error stays far
// below the output's own rounding.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// SiLU-gated product of the scaled gate and up outputs.  A finite limit
// applies the clamp of megamoe_rm.cu's fc1_rm epilogue first: the gate is
// bounded above only, the up projection on both sides.  The limit is
// uniform, so the branch costs no divergence.
__device__ __forceinline__ float swiglu(float g, float u, float limit) {
  if (limit < __builtin_inff()) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  return silu(g) * u;
}

// ------------------------------------------------------------------ prefill
// CU work unit: a workgroup of NW waves owns a 128 (activation rows) x
// 64*NW (weight rows; for SILU_MUL 32*NW gate rows + the matching up rows)
// tile and walks K in steps of 64 through an LDS ring.  Stage layout:
//   A  128 rows x 128 bytes (64 bf16), 16-byte chunks swizzled as in the
//      FP8 kernel;
//   B  64*NW rows x 32 packed bytes (64 E2M1 codes), the 16-byte chunk c
//      of row r at position c ^ ((r >> 3) & 1);
//   S  64*NW rows x 4 scale bytes.
// Wave wn owns 64 weight rows (two 32-row MFMA operands) against all 128
// activation rows, so every weight code is dequantized once per tile.
//   NW = 8 (N % 512 == 0): 512 weight rows, a 4-stage ring (136 KB), one
//          workgroup per CU.  The gathered activation tile, two thirds of
//          a 256-row tile's copy stream, feeds twice the MFMA work.
//   NW = 4: 256 weight rows, a 3-stage ring (75 KB), two workgroups per CU
//          whose phases (dequantization on the VALU, MFMAs) interleave.
//
// K slots: in a K step, MFMA lane l (slice l/32) takes the codes
// [32*slice, +32) of its weight row - one 16-byte LDS read, two scale bytes
// - and sub-step s uses codes [32*slice + 8s, +8).  The activation operand
// uses the same slots: slice `slice`, sub-step s = logical chunk 4*slice+s
// of the row's 128 bytes.
namespace pf {
constexpr int kM = 128;
constexpr int kABytes = kM * 128;
template <int NW> struct Geo {
  static constexpr int kN = 64 * NW;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kStages = NW == 8 ? 4 : 3;
  static constexpr int kBBytes = kN * 32;
  static constexpr int kSBytes = kN * 4;
  static constexpr int kStageBytes = kABytes + kBBytes + kSBytes;
  static constexpr int kACopies = 16 / NW;  // A copies (8 rows each) per wave and stage
  static constexpr int kPer = kACopies + 3;  // copies per wave and stage
};
}  // namespace pf

// PAIR (act NONE only): megamoe_rm.cu's fc2_rm epilogue.  Sorted row s is
// scaled by the top-k weight of its pair p = sorted_ids[s] and written to
// output row p instead of s.
// H16: the activations are binary16 (dequant and MFMA in fp16), else bf16.
template <int OUT, bool SILU, bool PAIR, bool H16, int NW>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : 2) void nvfp4_prefill(
    const uint16_t* __restrict__ x, int64_t rows_a, int a_sorted, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ w_sf, const float* __restrict__ w_gscale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_ids, int topk, int E, int P, int N,
    int K, void* __restrict__ out, float limit, const float* __restrict__ pair_w, int sf_quads, int w_tiled,
    int* __restrict__ queue) {
  static_assert(!(SILU && PAIR), "pair-ordered output is for act NONE");
  static_assert(NW == 4 || NW == 8, "tile widths");
  using pf::kM;
  using pf::kABytes;
  using G_ = pf::Geo<NW>;
  constexpr int kN = G_::kN, kThreads = G_::kThreads, kStages = G_::kStages;
  constexpr int kBBytes = G_::kBBytes, kStageBytes = G_::kStageBytes;
  constexpr int kACopies = G_::kACopies, kPer = G_::kPer;
  constexpr int kHalf = kN / 2;  // SILU_MUL: gate rows of the tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];

  const int tid = threadIdx.x, lane = tid & 63, wn = tid >> 6;
  const int I = N / 2;
  const int n_tiles = SILU ? I / kHalf : N / kN;
  const int G = K / 64;
  const int64_t xrow_bytes = (int64_t)K * 2, wrow_bytes = K / 2, srow_bytes = K / 16;
  sched_build(tile_start, sched_scratch, offsets, E, P, kM, n_tiles);
  const int total = tile_start[E];

  const int slice = lane >> 5, l32 = lane & 31;
  const int key = frag_key(lane);
  // Weight rows of this lane's two operands (row index in the B tile).
  const int brow0 = SILU ? 32 * wn + l32 : 64 * wn + l32;
  const int brow1 = SILU ? kHalf + 32 * wn + l32 : 64 * wn + 32 + l32;
  const int boff0 = kABytes + brow0 * 32 + ((slice ^ ((brow0 >> 3) & 1)) << 4);
  const int boff1 = kABytes + brow1 * 32 + ((slice ^ ((brow1 >> 3) & 1)) << 4);
  const int soff0 = kABytes + kBBytes + brow0 * 4 + slice * 2;
  const int soff1 = kABytes + kBBytes + brow1 * 4 + slice * 2;
  int aoff[4];  // activation chunk offsets for sub-step s (logical chunk 4*slice + s)
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = (((4 * slice + s) ^ key) << 4);

  // Tile order.  Without a queue, workgroup b takes every gridDim-th tile
  // from its XCD-first logical id, so an XCD holds a contiguous block of
  // each round of gridDim tiles.  With a queue, the workgroups of an XCD
  // claim that same block of each round through the XCD's counter, in
  // order, each taking the next tile when it finishes one; the last
  // workgroup to finish zeroes the counters for the next call.
  const int nxcd = gridDim.x % 8 == 0 ? 8 : 1;
  const int xq = blockIdx.x % nxcd, per = gridDim.x / nxcd;
  __shared__ int s_item;
  auto claim = [&]() __attribute__((always_inline)) {
    if (threadIdx.x == 0) {
      const int c = atomicAdd(&queue[xq], 1);
      s_item = (c / per) * (int)gridDim.x + per * xq + c % per;
    }
    __syncthreads();  // also: every thread has read the previous claim
    return s_item;
  };
  for (int item = queue ? claim() : xcd_logical_id(blockIdx.x, gridDim.x); item < total;
       item = queue ? claim() : item + (int)gridDim.x) {
    // two m-tiles per n-tile sweep: measured 1-3 % faster than four on the
    // Zipf prefill (FC1 and FC2), equal to one within the noise
    const Tile t = sched_tile<2>(tile_start, offsets, E, P, kM, n_tiles, item);
    // DMA sources.  A: wave wn moves rows 8q + lane/8 for q = kACopies*wn + j.
    const uint8_t* pa[kACopies];
#pragma unroll
    for (int j = 0; j < kACopies; ++j) {
      const int q = kACopies * wn + j;
      const int r = 8 * q + (lane >> 3);
      const int s = t.row0 + min(r, t.rows - 1);
      pa[j] = reinterpret_cast<const uint8_t*>(x) + a_row_of(s, sorted_ids, a_sorted, topk, rows_a) * xrow_bytes +
              dma_chunk(lane, q);
    }
    auto grow = [&](int r) __attribute__((always_inline)) {
      if (!SILU) return (int64_t)t.e * N + (int64_t)t.nt * kN + r;
      return (int64_t)t.e * N + (r < kHalf ? (int64_t)t.nt * kHalf + r : (int64_t)I + t.nt * kHalf + (r - kHalf));
    };
    // B: wave wn moves rows 64wn + 32j + lane/2 (chunk position lane%2);
    // S: rows 64wn + lane.
    // Row-major codes: 32 bytes at row stride K/2.  Tiled codes (16-row x
    // 64-K blocks of 512 bytes, a row group's blocks consecutive along K):
    // the K step's 32 bytes of a row sit in its group's block, so a wave's
    // 32 rows read two whole 512-byte blocks.
    const uint8_t* pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rb = 64 * wn + 32 * j + (lane >> 1);
      const int64_t wr = grow(rb);
      const int c16 = (((lane & 1) ^ ((rb >> 3) & 1)) << 4);
      const int64_t n = wr - (int64_t)t.e * N;
      pb[j] = w_tiled ? w + (int64_t)t.e * N * wrow_bytes + ((n >> 4) * (K / 64)) * 512 + (n & 15) * 32 + c16
                      : w + wr * wrow_bytes + c16;
    }
    const int64_t b_step = w_tiled ? 512 : 32;
    // S: row 64wn + lane, its 4 scale bytes of the K step.  Row-major
    // scales: 4 bytes at row stride K/16; K-quad-major ([K/64][N][4]): the
    // step's bytes of consecutive rows are consecutive (a whole-line copy).
    const int64_t s_row = grow(64 * wn + lane);
    const uint8_t* ps = sf_quads ? w_sf + (int64_t)t.e * N * srow_bytes + (s_row - (int64_t)t.e * N) * 4
                                 : w_sf + s_row * srow_bytes;
    const int64_t s_step = sf_quads ? (int64_t)N * 4 : 4;
    const uint32_t lds_a = lds_addr(smem + wn * (kACopies * 1024));
    const uint32_t lds_b = lds_addr(smem + kABytes + wn * 2048);
    const uint32_t lds_s = lds_addr(smem + kABytes + kBBytes + wn * 256);
    auto issue = [&](int g) __attribute__((always_inline)) {
      const uint32_t st = (uint32_t)((g % kStages) * kStageBytes);
#pragma unroll
      for (int j = 0; j < kACopies; ++j) dma16(pa[j] + (int64_t)g * 128, lds_a + st + j * 1024);
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16(pb[j] + (int64_t)g * b_step, lds_b + st + j * 1024);
      dma4(ps + (int64_t)g * s_step, lds_s + st);
    };

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

    // K loop over the tile's first NY 32-row groups of routed rows: the last
    // m-tile of an expert is usually partial (with skewed routing most
    // experts have fewer than 128 rows), and its MFMAs stop at the smallest
    // multiple of 32 rows that covers it.
    auto k_loop = [&](auto ny_c) __attribute__((always_inline)) {
      constexpr int NY = decltype(ny_c)::value;
      for (int g = 0; g < G; ++g) {
        // stage g has landed once at most the stages issued after it remain
        if (kStages > 3 && last_issued - g >= 2) wait_vmcnt<2 * kPer>();
        else if (last_issued - g >= 1) wait_vmcnt<kPer>();
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
        if constexpr (H16) {
          const v2h h0 = ue4m3x2_f16(sc0), h1 = ue4m3x2_f16(sc1);
          const v2h s00 = {h0.x, h0.x}, s01 = {h0.y, h0.y}, s10 = {h1.x, h1.x}, s11 = {h1.y, h1.y};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const v8h wf0 = __builtin_bit_cast(v8h, dequant8_f16(q0[s], s < 2 ? s00 : s01));
            const v8h wf1 = __builtin_bit_cast(v8h, dequant8_f16(q1[s], s < 2 ? s10 : s11));
#pragma unroll
            for (int y = 0; y < NY; ++y) {
              const v8h xf = *reinterpret_cast<const v8h*>(st + (32 * y + l32) * 128 + aoff[s]);
              acc[0][y] = mfma_f16_32x32x16(wf0, xf, acc[0][y]);
              acc[1][y] = mfma_f16_32x32x16(wf1, xf, acc[1][y]);
            }
          }
        } else {
          const float s00 = e4m3_to_f32(sc0 & 0xffu), s01 = e4m3_to_f32(sc0 >> 8);
          const float s10 = e4m3_to_f32(sc1 & 0xffu), s11 = e4m3_to_f32(sc1 >> 8);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const v8bf wf0 = __builtin_bit_cast(v8bf, dequant8_bf16(q0[s], s < 2 ? s00 : s01));
            const v8bf wf1 = __builtin_bit_cast(v8bf, dequant8_bf16(q1[s], s < 2 ? s10 : s11));
#pragma unroll
            for (int y = 0; y < NY; ++y) {
              const v8bf xf = *reinterpret_cast<const v8bf*>(st + (32 * y + l32) * 128 + aoff[s]);
              acc[0][y] = mfma_bf16_32x32x16(wf0, xf, acc[0][y]);
              acc[1][y] = mfma_bf16_32x32x16(wf1, xf, acc[1][y]);
            }
          }
        }
      }
    };
    switch ((t.rows + 31) >> 5) {
      case 1: k_loop(std::integral_constant<int, 1>{}); break;
      case 2: k_loop(std::integral_constant<int, 2>{}); break;
      case 3: k_loop(std::integral_constant<int, 3>{}); break;
      default: k_loop(std::integral_constant<int, 4>{}); break;
    }

    // Epilogue: global scale (and the SiLU-gated product), output tile
    // through LDS, then 16-byte stores along output rows.
    typedef typename OutT<OUT>::T T;
    constexpr int kCols = SILU ? kHalf : kN;
    constexpr int kOutPitch = kCols * (int)sizeof(T) + 16;
    constexpr bool kStaged = kM * kOutPitch <= kStages * kStageBytes;  // else: f32, direct stores
    raw_barrier();  // all waves are done with the ring
    uint8_t* otile = smem;
    const float gs = w_gscale[t.e];
    const int ldo = SILU ? I : N;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      uint8_t* orow = otile + (32 * y + l32) * kOutPitch;
      float gy = gs;
      if (PAIR) gy *= pair_w[sorted_ids[t.row0 + min(32 * y + l32, t.rows - 1)]];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[2][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * q + r;
          if (SILU) {
            v[0][r] = swiglu(gs * acc[0][y][i], gs * acc[1][y][i], limit);
            v[1][r] = 0.f;
          } else {
            v[0][r] = gy * acc[0][y][i];
            v[1][r] = gy * acc[1][y][i];
          }
        }
        // weight columns 8q + 4*slice + r of the lane's 32-row operand(s)
        const int col0 = (SILU ? 32 * wn : 64 * wn) + 8 * q + 4 * slice;
#pragma unroll
        for (int a2 = 0; a2 < (SILU ? 1 : 2); ++a2) {
          if constexpr (!kStaged) {
            const int rr = 32 * y + l32;
            if (rr < t.rows) {
              const int64_t orow_i = PAIR ? (int64_t)sorted_ids[t.row0 + rr] : (int64_t)(t.row0 + rr);
              *reinterpret_cast<float4*>(static_cast<float*>(out) + orow_i * ldo + (int64_t)t.nt * kCols + col0 +
                                         32 * a2) = make_float4(v[a2][0], v[a2][1], v[a2][2], v[a2][3]);
            }
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
      uint8_t* obase = static_cast<uint8_t*>(out) + (int64_t)t.nt * kCols * (int)sizeof(T);
#pragma unroll 4
      for (int i = 0; i < kM * kChunksPerRow / kThreads; ++i) {
        const int ci = tid + kThreads * i;
        const int r = ci / kChunksPerRow, c = ci % kChunksPerRow;
        if (r < t.rows) {
          const int64_t orow_i = PAIR ? (int64_t)sorted_ids[t.row0 + r] : (int64_t)(t.row0 + r);
          st16(obase + orow_i * ldo * (int)sizeof(T) + c * 16, ld16(otile + r * kOutPitch + c * 16));
        }
      }
    }
  }
  if (queue && threadIdx.x == 0 && atomicAdd(&queue[8], 1) == (int)gridDim.x - 1) {
    // every workgroup has made its last claim
    for (int x = 0; x < 8; ++x) atomicExch(&queue[x], 0);
    atomicExch(&queue[8], 0);
  }
}

// ------------------------------------------------------------------ decode
// Weight streaming for few rows per expert.  The wave is the unit of work:
// item = (tile of at most 4 routed rows of one expert, 16 output columns).
// For SILU_MUL the wave's two 16-row weight groups are the gate rows
// [16n, 16n+16) and the matching up rows [I+16n, ...), so both halves of an
// output element meet in the same lane; without an activation the groups
// are 32 consecutive weight rows.
//
// Every operand reaches the wave through LDS buffers filled by
// direct-to-LDS copies issued kDepth steps ahead and waited for with vmcnt
// waits counted from the copies actually issued: nothing the compiler waits
// for sits in the stream, so no wait drains it.  The number of memory
// requests in flight per CU is what bounds this stream, so copies read
// whole 128-byte lines where the layout allows.
//   WIDE (K % 512 == 0), a step is 2 chunks of K = 128:
//     weights      per step and group, two copies of 8 rows x 128 bytes;
//                  16-byte piece p of row r stored at position
//                  p ^ ((r >> 1) & 7), so the 16 rows read by one MFMA
//                  operand fall in distinct LDS banks;
//     activations  per 4 chunks ("superchunk", double buffered, parity from
//                  a running count so it alternates across items too): one
//                  1 KB copy per routed row of the tile, piece p of row r at
//                  position p ^ r;
//     scales       per superchunk, one 1 KB copy of 32 rows x 32 bytes.
//   otherwise, a step is one chunk: 16 rows x 64 weight bytes per group,
//     4 rows x 256 activation bytes (rows past the tile repeat its last
//     row), 32 rows x 8 scale bytes.
// The stream runs across item boundaries.  Item metadata is looked up for
// 64 items at a time (one per lane) and read from a lane at each switch.
//
// MFMA 16x16x32 bf16 with the weights as the 16-row operand: lane l holds
// weight row l%16, K slots [8(l/16), +8) of each sub-step; the activation
// operand (16 columns, the tile's <= 4 rows; other columns are discarded)
// uses the same K slots.  Sub-step j of chunk c covers K = 128c + 32(l/16)
// + 8j + (0..7), codes [8j, 8j+8) of the lane's 16 bytes of that chunk.
namespace dc {
constexpr int kM = 4;          // routed rows per item
constexpr int kWaves = 4;      // waves per workgroup (independent)
template <bool WIDE> constexpr int cps() { return WIDE ? 2 : 1; }            // chunks per step
template <bool WIDE> constexpr int depth() { return WIDE ? 2 : 3; }          // steps in flight
template <bool WIDE> constexpr int slot_bytes() { return WIDE ? 4096 : 3328; }
// WIDE: + activation buffers [2][4 rows][1 KB] + scale buffers [2][1 KB]
template <bool WIDE>
constexpr int wave_bytes() { return depth<WIDE>() * slot_bytes<WIDE>() + (WIDE ? 8192 + 2048 : 0); }
}  // namespace dc

// s_waitcnt vmcnt(n) for a run-time n in [0, 15]
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
  }
  asm volatile("" ::: "memory");
}

template <int OUT, bool SILU, bool WIDE, bool PAIR, bool H16>
__global__ __launch_bounds__(dc::kWaves * 64) void nvfp4_decode(
    const uint16_t* __restrict__ x, int64_t rows_a, int a_sorted, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ w_sf, const float* __restrict__ w_gscale, const int* __restrict__ offsets,
    const int* __restrict__ sorted_ids, int topk, int E, int P, int N, int K, void* __restrict__ out,
    float limit, const float* __restrict__ pair_w, int sf_quads, int w_tiled) {
  static_assert(!(SILU && PAIR), "pair-ordered output is for act NONE");
  constexpr int CPS = dc::cps<WIDE>();
  constexpr int D = dc::depth<WIDE>();
  constexpr int kSlot = dc::slot_bytes<WIDE>();
  constexpr int kWave = dc::wave_bytes<WIDE>();
  // a superchunk buffer is refilled D steps before its next use; the
  // previous superchunk (2 steps) must be consumed by then
  static_assert(!WIDE || D <= 2, "superchunk double buffer");
  __shared__ int tile_start[kMaxExperts + 1];
  __shared__ int sched_scratch[2 * kMaxWaves];
  __shared__ __attribute__((aligned(1024))) uint8_t ring[dc::kWaves * kWave];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int I = N / 2;
  const int n_blocks = SILU ? (I / 16) : (N / 32);
  sched_build(tile_start, sched_scratch, offsets, E, P, dc::kM, n_blocks);
  const int total = tile_start[E];
  // Items are dealt round robin over all waves (measured 4-8 % faster on the
  // 8-token FC1 than dealing them to the fewest waves that need the same
  // number of rounds: more waves stream at once).
  const int active = gridDim.x * dc::kWaves;
  const int wid = blockIdx.x * dc::kWaves + wv;
  if (wid >= total) return;
  const int steps = K / (128 * CPS);                                 // per item
  const int n_items = (total - wid + active - 1) / active;          // items of this wave
  const int nq = n_items * steps;                                    // steps of this wave
  const int64_t wrow = K / 2, srow = K / 16;
  // scale bytes per copy step: a superchunk (WIDE, 8 quads) or a step (2 quads)
  const int64_t s_adv = sf_quads ? (WIDE ? 8 : 2) * (int64_t)N * 4 : (WIDE ? 32 : 8);
  // code bytes per copy step and row group: 128 or 64 per row (row-major),
  // 4 or 2 blocks of 512 bytes (tiled)
  const int64_t w_adv = w_tiled ? (WIDE ? 2048 : 1024) : (WIDE ? 128 : 64);
  const int g = lane >> 4, l16 = lane & 15;
  uint8_t* myring = ring + wv * kWave;
  const uint32_t lb = lds_addr(myring);
  const uint8_t* xbuf = myring + D * kSlot;  // WIDE: [2][4 rows][1 KB]
  const uint8_t* sbuf = xbuf + 8192;          // WIDE: [2][1 KB]
  const uint32_t lxb = lb + D * kSlot, lsb = lxb + 8192;

  // ---- item metadata.  The wave's j-th item is wid + j * active.  Lane l
  // of table (b & 1) holds item 64b + l: its expert, first sorted row, row
  // count, column block, activation rows and global scale, found by all
  // lanes at once (a binary search over tile_start, then vector loads).  An
  // item switch then reads one lane instead of waiting on a search and
  // dependent loads while the copy ring drains.  The copy cursor runs
  // at most D steps (so at most D items) ahead of the compute cursor, so two
  // tables suffice; a wave with more than 64 items reloads one per 64.
  struct Meta {
    int e, row0, rows, nt, ar[dc::kM];
    float gs;
  };
  Meta tab0, tab1;
  auto load_meta = [&](int b) __attribute__((always_inline)) {
    Meta m;
    m.e = 0, m.row0 = 0, m.rows = 1, m.nt = 0, m.gs = 0.f;
#pragma unroll
    for (int r = 0; r < dc::kM; ++r) m.ar[r] = 0;
    const int j = 64 * b + lane;
    if (j < n_items) {
      const int item = wid + j * active;
      int bl = 0, bh = E - 1;
      while (bl < bh) {
        const int mid = (bl + bh + 1) >> 1;
        if (tile_start[mid] <= item) bl = mid; else bh = mid - 1;
      }
      const int local = item - tile_start[bl];
      const int lo = min(max(offsets[bl], 0), P);
      const int hi = min(max(offsets[bl + 1], lo), P);
      const int mt = local / n_blocks;
      m.e = bl;
      m.nt = local - mt * n_blocks;
      m.row0 = lo + mt * dc::kM;
      m.rows = min(dc::kM, hi - lo - mt * dc::kM);
#pragma unroll
      for (int r = 0; r < dc::kM; ++r) {
        const int sp = m.row0 + (r < m.rows ? r : m.rows - 1);
        const int64_t a = (a_sorted || sorted_ids == nullptr) ? (int64_t)sp : (int64_t)(sorted_ids[sp] / topk);
        m.ar[r] = (a < 0 || a >= rows_a) ? 0 : (int)a;
      }
      m.gs = w_gscale[bl];
    }
    if (b & 1) tab1 = m; else tab0 = m;
  };
  // item j's metadata, wave-uniform
  auto meta = [&](int j) __attribute__((always_inline)) {
    const int l = j & 63;
    const bool odd = (j >> 6) & 1;
    Meta m;
    m.e = __builtin_amdgcn_readlane(odd ? tab1.e : tab0.e, l);
    m.row0 = __builtin_amdgcn_readlane(odd ? tab1.row0 : tab0.row0, l);
    m.rows = __builtin_amdgcn_readlane(odd ? tab1.rows : tab0.rows, l);
    m.nt = __builtin_amdgcn_readlane(odd ? tab1.nt : tab0.nt, l);
#pragma unroll
    for (int r = 0; r < dc::kM; ++r) m.ar[r] = __builtin_amdgcn_readlane(odd ? tab1.ar[r] : tab0.ar[r], l);
    m.gs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, odd ? tab1.gs : tab0.gs), l));
    return m;
  };
  load_meta(0);

  // ---- copy cursor: sources of the next (item, step) to copy
  int is_j = 0, is_st = 0, is_rows = 0, is_sc = 0;
  // WIDE: weight row base of group grp, half h at wsrc[2 grp + h]
  const uint8_t* wsrc[4];
  const uint8_t *sx = nullptr, *ss = nullptr;
  int64_t xrow[dc::kM];
  auto set_sources = [&](int j) __attribute__((always_inline)) {
    if (j > 0 && (j & 63) == 0) load_meta(j >> 6);
    const Meta t = meta(j);
    const int b0 = SILU ? t.nt * 16 : t.nt * 32;
    const int b1 = SILU ? I + t.nt * 16 : t.nt * 32 + 16;
    const int64_t e0 = (int64_t)t.e * N;
    if (WIDE) {
      // copy h of a group: lane l -> row 8h + l/8, piece (l%8) ^ ((row >> 1) & 7)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + (lane >> 3);
        const int p = (lane & 7) ^ ((r >> 1) & 7);
        if (w_tiled) {
          // piece p of the step's 128 bytes: block p/2 of the step, half p%2
          const int64_t in = (int64_t)(p >> 1) * 512 + r * 32 + (p & 1) * 16;
          wsrc[h] = w + e0 * wrow + (int64_t)(b0 >> 4) * (K / 64) * 512 + in;
          wsrc[2 + h] = w + e0 * wrow + (int64_t)(b1 >> 4) * (K / 64) * 512 + in;
        } else {
          wsrc[h] = w + (e0 + b0 + r) * wrow + (p << 4);
          wsrc[2 + h] = w + (e0 + b1 + r) * wrow + (p << 4);
        }
      }
    } else if (w_tiled) {
      const int64_t in = (int64_t)(g >> 1) * 512 + l16 * 32 + (g & 1) * 16;
      wsrc[0] = w + e0 * wrow + (int64_t)(b0 >> 4) * (K / 64) * 512 + in;
      wsrc[2] = w + e0 * wrow + (int64_t)(b1 >> 4) * (K / 64) * 512 + in;
    } else {
      wsrc[0] = w + (e0 + b0 + l16) * wrow + g * 16;
      wsrc[2] = w + (e0 + b1 + l16) * wrow + g * 16;
    }
    const int* ar = t.ar;
    is_rows = t.rows;
    if (WIDE) {
#pragma unroll
      for (int r = 0; r < dc::kM; ++r) xrow[r] = (int64_t)ar[r] * K * 2 + ((lane ^ r) << 4);
    } else {
      const int r = lane >> 4;
      const int arow = r == 0 ? ar[0] : r == 1 ? ar[1] : r == 2 ? ar[2] : ar[3];
      sx = reinterpret_cast<const uint8_t*>(x) + (int64_t)arow * K * 2 + (((lane & 15) ^ r) << 4);
    }
    // scales: lane -> weight group lane/32, row (lane/2)%16, half lane%2
    const int sr = (lane >> 1) & 15;
    if (sf_quads) {
      // K-quad-major scales, LDS [group][quad][16 rows][4 bytes].  WIDE:
      // lane -> group lane/32, quad (lane/4)%8 of the superchunk, rows
      // 4(lane%4) .. +3 (16 bytes); otherwise lane -> group lane/32, quad
      // (lane/16)%2 of the step, row lane%16 (4 bytes).
      const int gb = (lane >> 5) ? b1 : b0;
      const int64_t eb = (int64_t)t.e * N * srow;
      ss = WIDE ? w_sf + eb + ((lane >> 2) & 7) * (int64_t)N * 4 + (int64_t)(gb + 4 * (lane & 3)) * 4
                : w_sf + eb + ((lane >> 4) & 1) * (int64_t)N * 4 + (int64_t)(gb + (lane & 15)) * 4;
    } else {
      ss = w_sf + (e0 + ((lane >> 5) ? b1 : b0) + sr) * srow + (lane & 1) * (WIDE ? 16 : 4);
    }
  };
  uint32_t ops_ring = 0;  // copies issued per slot, 4 bits each
  auto issue = [&](int slot) __attribute__((always_inline)) {
    const uint32_t l = lb + slot * kSlot;
    int ops;
    if (WIDE) {
      ops = 4;
      if ((is_st & 1) == 0) {  // first step of a superchunk
        const int bsel = is_sc & 1;
        const int64_t sc = is_st >> 1;
        dma16(ss + sc * s_adv, lsb + bsel * 1024);
        const uint8_t* xs = reinterpret_cast<const uint8_t*>(x) + sc * 1024;
        for (int r = 0; r < is_rows; ++r) dma16(xs + xrow[r], lxb + bsel * 4096 + r * 1024);
        ops += 1 + is_rows;
        ++is_sc;
      }
      const int64_t o = (int64_t)is_st * w_adv;
      dma16_nt(wsrc[0] + o, l);
      dma16_nt(wsrc[1] + o, l + 1024);
      dma16_nt(wsrc[2] + o, l + 2048);
      dma16_nt(wsrc[3] + o, l + 3072);
    } else {
      ops = 4;
      const int64_t o = (int64_t)is_st * w_adv;
      dma16_nt(wsrc[0] + o, l);
      dma16_nt(wsrc[2] + o, l + 1024);
      dma16(sx + (int64_t)is_st * 256, l + 2048);
      dma4(ss + (int64_t)is_st * s_adv, l + 3072);
    }
    ops_ring = (ops_ring & ~(15u << (4 * slot))) | ((uint32_t)ops << (4 * slot));
    if (++is_st == steps) {
      is_st = 0;
      if (++is_j < n_items) set_sources(is_j);
    }
  };

  set_sources(is_j);
  const int npre = nq < D ? nq : D;
  for (int i = 0; i < npre; ++i) issue(i);

  // ---- compute cursor
  int cs_j = 0, st = 0, cs_sc = 0, cbuf = 0;
  v4f acc0 = v4f{}, acc1 = v4f{};
  const int xr = l16 & 3;                 // activation row of MFMA column l16
  const int wkey = (l16 >> 1) & 7;        // WIDE weight swizzle of row l16
  for (int q = 0; q < nq; ++q) {
    // copies issued after step q's: those of steps q+1 .. min(q+D-1, nq-1)
    int after = 0;
#pragma unroll
    for (int j = 1; j < D; ++j)
      if (q + j < nq) after += (ops_ring >> (4 * ((q + j) % D))) & 15;
    wait_vm(after);
    const int slot = q % D;
    const uint8_t* sp = myring + slot * kSlot;
    u32x4 w0[CPS], w1[CPS], xv[CPS][4];
    uint32_t q0[CPS], q1[CPS];
    if (WIDE) {
      if ((st & 1) == 0) cbuf = cs_sc++ & 1;
      const uint8_t* xb = xbuf + cbuf * 4096 + xr * 1024;
#pragma unroll
      for (int cp = 0; cp < CPS; ++cp) {
        const int pos = ((4 * cp + g) ^ wkey) << 4;
        w0[cp] = *reinterpret_cast<const u32x4*>(sp + l16 * 128 + pos);
        w1[cp] = *reinterpret_cast<const u32x4*>(sp + 2048 + l16 * 128 + pos);
        const int cc = 2 * (st & 1) + cp;  // chunk within the superchunk
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xv[cp][j] = *reinterpret_cast<const u32x4*>(xb + (((16 * cc + 4 * g + j) ^ xr) << 4));
        const uint8_t* sb = sbuf + cbuf * 1024 +
                            (sf_quads ? (2 * cc + (g >> 1)) * 64 + l16 * 4 + 2 * (g & 1) : l16 * 32 + cc * 8 + 2 * g);
        q0[cp] = *reinterpret_cast<const uint16_t*>(sb);
        q1[cp] = *reinterpret_cast<const uint16_t*>(sb + 512);
      }
    } else {
      w0[0] = *reinterpret_cast<const u32x4*>(sp + lane * 16);
      w1[0] = *reinterpret_cast<const u32x4*>(sp + 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xv[0][j] = *reinterpret_cast<const u32x4*>(sp + 2048 + xr * 256 + (((4 * g + j) ^ xr) << 4));
      const int so = sf_quads ? (g >> 1) * 64 + l16 * 4 + 2 * (g & 1) : l16 * 8 + 2 * g;
      q0[0] = *reinterpret_cast<const uint16_t*>(sp + 3072 + so);
      q1[0] = *reinterpret_cast<const uint16_t*>(sp + 3072 + 128 + so);
    }
    // the slot is refilled once its reads have landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (q + D < nq) issue(slot);
#pragma unroll
    for (int cp = 0; cp < CPS; ++cp) {
      if constexpr (H16) {
        const v2h ha = ue4m3x2_f16(q0[cp]), hb = ue4m3x2_f16(q1[cp]);
        const v2h a0 = {ha.x, ha.x}, a1 = {ha.y, ha.y}, b0 = {hb.x, hb.x}, b1 = {hb.y, hb.y};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0 = mfma_f16_16x16x32(__builtin_bit_cast(v8h, dequant8_f16(w0[cp][j], j < 2 ? a0 : a1)),
                                   __builtin_bit_cast(v8h, xv[cp][j]), acc0);
          acc1 = mfma_f16_16x16x32(__builtin_bit_cast(v8h, dequant8_f16(w1[cp][j], j < 2 ? b0 : b1)),
                                   __builtin_bit_cast(v8h, xv[cp][j]), acc1);
        }
      } else {
        const float a0 = e4m3_to_f32(q0[cp] & 0xffu), a1 = e4m3_to_f32(q0[cp] >> 8);
        const float b0 = e4m3_to_f32(q1[cp] & 0xffu), b1 = e4m3_to_f32(q1[cp] >> 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0 = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, dequant8_bf16_hi(w0[cp][j], j < 2 ? a0 : a1)),
                                    __builtin_bit_cast(v8bf, xv[cp][j]), acc0);
          acc1 = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, dequant8_bf16_hi(w1[cp][j], j < 2 ? b0 : b1)),
                                    __builtin_bit_cast(v8bf, xv[cp][j]), acc1);
        }
      }
    }
    if (++st == steps) {
      // acc value i of lane l: weight row 4(l/16)+i of each 16-row group,
      // routed row l%16 of the tile.
      const Meta t = meta(cs_j);
      const float gs = t.gs;
      typedef typename OutT<OUT>::T T;
      T* o = static_cast<T*>(out);
      if (l16 < t.rows) {
        const int64_t row = t.row0 + l16;
        if (SILU) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[row * I + t.nt * 16 + 4 * g + i] = OutT<OUT>::from(swiglu(gs * acc0[i], gs * acc1[i], limit));
        } else {
          float gy = gs;
          int64_t orow_i = row;
          if (PAIR) {
            orow_i = sorted_ids[row];
            gy *= pair_w[orow_i];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[orow_i * N + t.nt * 32 + 4 * g + i] = OutT<OUT>::from(gy * acc0[i]);
            o[orow_i * N + t.nt * 32 + 16 + 4 * g + i] = OutT<OUT>::from(gy * acc1[i]);
          }
        }
      }
      acc0 = v4f{};
      acc1 = v4f{};
      st = 0;
      ++cs_j;
    }
  }
}

template <int OUT, bool SILU, bool PAIR, bool H16>
hipError_t go(const GroupedArgs& g, bool decode, const uint16_t* x, const uint8_t* w,
              const uint8_t* sf, const float* gsc, hipStream_t stream) {
  if (decode) {
    // two workgroups (8 independent waves) per CU; the kernel deals the
    // items over the waves itself
    const int grid = g.num_cus * 2;
    if (g.K % 512 == 0)
      hipLaunchKernelGGL((nvfp4_decode<OUT, SILU, true, PAIR, H16>), dim3(grid), dim3(dc::kWaves * 64), 0, stream, x,
                         g.rows_a, g.a_sorted, w, sf, gsc, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P, g.N,
                         g.K, g.out, g.act_limit, g.pair_weights, g.sf_quads, g.w_tiled);
    else
      hipLaunchKernelGGL((nvfp4_decode<OUT, SILU, false, PAIR, H16>), dim3(grid), dim3(dc::kWaves * 64), 0, stream, x,
                         g.rows_a, g.a_sorted, w, sf, gsc, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P, g.N,
                         g.K, g.out, g.act_limit, g.pair_weights, g.sf_quads, g.w_tiled);
  } else {
    // 512-row tiles (one 8-wave workgroup per CU) when N allows, else
    // 256-row tiles (two 4-wave workgroups per CU)
    const int64_t mt_ub = (g.P + pf::kM - 1) / pf::kM + std::min<int64_t>(g.E, g.P);
    if (g.N % pf::Geo<8>::kN == 0) {
      const int64_t items_ub = mt_ub * (g.N / pf::Geo<8>::kN);
      const int grid = (int)std::min<int64_t>(items_ub, (int64_t)g.num_cus);
      hipLaunchKernelGGL((nvfp4_prefill<OUT, SILU, PAIR, H16, 8>), dim3(grid), dim3(pf::Geo<8>::kThreads), 0, stream,
                         x, g.rows_a, g.a_sorted, w, sf, gsc, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                         g.N, g.K, g.out, g.act_limit, g.pair_weights, g.sf_quads, g.w_tiled, g.queue);
    } else {
      const int64_t items_ub = mt_ub * (g.N / pf::Geo<4>::kN);
      const int grid = (int)std::min<int64_t>(items_ub, (int64_t)g.num_cus * 2);
      hipLaunchKernelGGL((nvfp4_prefill<OUT, SILU, PAIR, H16, 4>), dim3(grid), dim3(pf::Geo<4>::kThreads), 0, stream,
                         x, g.rows_a, g.a_sorted, w, sf, gsc, g.offsets, g.sorted_ids, g.topk, g.E, (int)g.P,
                         g.N, g.K, g.out, g.act_limit, g.pair_weights, g.sf_quads, g.w_tiled, g.queue);
    }
  }
  return hipGetLastError();
}

template <bool H16>
hipError_t dispatch(const GroupedArgs& g, const uint16_t* x, const uint8_t* w, const uint8_t* w_sf,
                    const float* w_gscale, hipStream_t stream) {
  // The streaming schedule when asked for, under AUTO while experts average
  // fewer than 16 rows, and whenever N is not a multiple of the prefill
  // tile (256), which the prefill schedule cannot cover.
  const bool decode = g.sched == 1 || g.N % pf::Geo<4>::kN != 0 || (g.sched == 0 && g.P < (int64_t)16 * g.E);
  if (g.silu_mul) {
    switch (g.out_kind) {
      case OUT_F16: return go<OUT_F16, true, false, H16>(g, decode, x, w, w_sf, w_gscale, stream);
      case OUT_BF16: return go<OUT_BF16, true, false, H16>(g, decode, x, w, w_sf, w_gscale, stream);
      default: return go<OUT_F32, true, false, H16>(g, decode, x, w, w_sf, w_gscale, stream);
    }
  }
  if (g.pair_weights) {
    switch (g.out_kind) {
      case OUT_F16: return go<OUT_F16, false, true, H16>(g, decode, x, w, w_sf, w_gscale, stream);
      case OUT_BF16: return go<OUT_BF16, false, true, H16>(g, decode, x, w, w_sf, w_gscale, stream);
      default: return go<OUT_F32, false, true, H16>(g, decode, x, w, w_sf, w_gscale, stream);
    }
  }
  switch (g.out_kind) {
    case OUT_F16: return go<OUT_F16, false, false, H16>(g, decode, x, w, w_sf, w_gscale, stream);
    case OUT_BF16: return go<OUT_BF16, false, false, H16>(g, decode, x, w, w_sf, w_gscale, stream);
    default: return go<OUT_F32, false, false, H16>(g, decode, x, w, w_sf, w_gscale, stream);
  }
}
}  // namespace

hipError_t launch_gemm_nvfp4(const GroupedArgs& g, const uint16_t* x, const uint8_t* w,
                             const uint8_t* w_sf, const float* w_gscale, hipStream_t stream) {
  if (g.P == 0) return hipSuccess;
  return g.x_f16 ? dispatch<true>(g, x, w, w_sf, w_gscale, stream)
                 : dispatch<false>(g, x, w, w_sf, w_gscale, stream);
}

}  // namespace moeq
