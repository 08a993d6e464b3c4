// One-shot repack of NVFP4 expert weights from the layout that megamoe_rm.cu
// reads in place (the header comment of that file and its scale_off
// function: w13 with the up rows first, UE4M3 block scales in 128x4 swizzled
// tiles) into the layout of grouped_gemm_qnvfp4 (gate rows first, scales
// [N][K/16] row-major, or K-quad-major [K/64][N][4 bytes]).
//
// Weights.  With the halves swapped, output rows [0, R/2) of an expert are
// input rows [R/2, R) and the other way round; both halves are contiguous,
// so the copy of one expert is a rotation of its bytes by half their count.
// Each thread moves one 16-byte vector.  Tiled output (16-row x 64-K blocks
// of 512 bytes, a row group's blocks consecutive along K) gathers each
// block's 16 rows x 32 bytes instead.
//
// Scales.  The swizzled matrix of an expert is a run of 512-byte tiles, one
// per (128-row block, 4-column quad), row block major.  The 16-byte group i
// of a tile holds, in its four words, the quad's four scale bytes of rows
// i, i+32, i+64, i+96 of the block.  A workgroup takes 16 consecutive tiles
// of one row block (8 KB, read with 16-byte loads), transposes them through
// LDS to [128 rows][16 words], and writes each row's 64 bytes contiguously.
//
// One launch does both (workgroups split by blockIdx.x); an HBM-bound
// streaming copy.  Every byte is touched once, so all global loads and
// stores are nontemporal (no reuse to keep in the caches).
#include "common.h"
#include "kernels.h"

namespace moeq {
namespace {

constexpr int kThreads = 256;
constexpr int kTilesPerGroup = 16;         // scale tiles per workgroup
constexpr int kLdsStride = kTilesPerGroup + 1;

struct RepackArgs {
  const u32x4* w_in;
  u32x4* w_out;
  const u32x4* sf_in;
  uint32_t* sf_out;
  uint32_t chunks;      // 16-byte weight vectors per expert
  uint32_t rot;         // chunks / 2 when the halves swap, else 0
  uint32_t wblocks;     // workgroups per expert on the weights
  uint32_t R;           // rows per expert
  uint32_t quads;       // 4-byte scale words per linear row = K / 64
  uint32_t groups;      // workgroups per 128-row block on the scales
  uint32_t half_rows;   // R / 2 when the halves swap, else 0
  uint32_t out_quads;   // scales out as [K/64][R][4 bytes] (else [R][K/16])
  uint32_t w_tiled;     // codes out in 16-row x 64-K blocks of 512 bytes (else [R][K/2])
  uint32_t kblocks;     // 64-K blocks per row = K / 64
};

__device__ __forceinline__ void weights_part(const RepackArgs& a, uint32_t bx) {
  const size_t base = (size_t)blockIdx.y * a.chunks;
  const uint32_t j = bx * kThreads + threadIdx.x;
  if (j >= a.chunks) return;
  uint32_t s;
  if (a.w_tiled) {
    // output chunk j: block j/32 = (row group, 64-K block), row j%32/2 of
    // the group, half j%2 of the row's 32 bytes
    const uint32_t blk = j >> 5, rg = blk / a.kblocks, kb = blk - rg * a.kblocks;
    uint32_t r = rg * 16 + ((j & 31) >> 1) + a.half_rows;
    if (r >= a.R) r -= a.R;
    s = r * (a.kblocks * 2) + kb * 2 + (j & 1);
  } else {
    s = j + a.rot;
    if (s >= a.chunks) s -= a.chunks;
  }
  __builtin_nontemporal_store(__builtin_nontemporal_load(a.w_in + base + s), a.w_out + base + j);
}

__device__ __forceinline__ void scales_part(const RepackArgs& a, uint32_t bx, uint32_t* t) {
  const uint32_t rb = bx / a.groups;
  const uint32_t cq0 = (bx - rb * a.groups) * kTilesPerGroup;
  const size_t words = (size_t)a.R * a.quads;           // words per expert
  const u32x4* s = a.sf_in + ((size_t)blockIdx.y * words + ((size_t)rb * a.quads + cq0) * 128) / 4;
  uint32_t* d = a.sf_out + (size_t)blockIdx.y * words;
  // 16 tiles x 32 vectors; vector i of tile tt = rows i + 32q, column tt.
#pragma unroll
  for (int u = 0; u < kTilesPerGroup * 32 / kThreads; ++u) {
    const uint32_t v = threadIdx.x + u * kThreads;
    const uint32_t tt = v >> 5, i = v & 31;
    if (cq0 + tt < a.quads) {
      const u32x4 x = __builtin_nontemporal_load(s + v);
      t[(i + 0) * kLdsStride + tt] = x.x;
      t[(i + 32) * kLdsStride + tt] = x.y;
      t[(i + 64) * kLdsStride + tt] = x.z;
      t[(i + 96) * kLdsStride + tt] = x.w;
    }
  }
  __syncthreads();
  if (a.out_quads) {
    // quad-major: a quad's words of consecutive rows are consecutive, so
    // 128 consecutive lanes write one quad's 128 rows (512 bytes)
#pragma unroll
    for (int u = 0; u < 128 * kTilesPerGroup / kThreads; ++u) {
      const uint32_t m = threadIdx.x + u * kThreads;
      const uint32_t col = m >> 7, row = m & 127;
      if (cq0 + col < a.quads) {
        uint32_t r = rb * 128 + row + a.half_rows;
        if (r >= a.R) r -= a.R;
        __builtin_nontemporal_store(t[row * kLdsStride + col], d + (size_t)(cq0 + col) * a.R + r);
      }
    }
    return;
  }
  // 128 rows x 16 words; 16 consecutive lanes write one row's words.
#pragma unroll
  for (int u = 0; u < 128 * kTilesPerGroup / kThreads; ++u) {
    const uint32_t m = threadIdx.x + u * kThreads;
    const uint32_t row = m >> 4, col = m & 15;
    if (cq0 + col < a.quads) {
      uint32_t r = rb * 128 + row + a.half_rows;
      if (r >= a.R) r -= a.R;
      __builtin_nontemporal_store(t[row * kLdsStride + col], d + (size_t)r * a.quads + cq0 + col);
    }
  }
}

// grid (wblocks + R/128 * groups, E): the first wblocks workgroups of an
// expert copy its weights, the rest its scales (a workgroup-uniform split).
__global__ __launch_bounds__(kThreads) void repack_nvfp4(RepackArgs a) {
  __shared__ uint32_t t[128 * kLdsStride];
  if (blockIdx.x < a.wblocks)
    weights_part(a, blockIdx.x);
  else
    scales_part(a, blockIdx.x - a.wblocks, t);
}

}  // namespace

hipError_t launch_repack_nvfp4(const uint8_t* w_in, const uint8_t* sf_in, int64_t E, int64_t N, int64_t K,
                               int swap_halves, int w_tiled, int out_quads, uint8_t* w_out, uint8_t* sf_out,
                               hipStream_t stream) {
  RepackArgs a;
  a.w_in = reinterpret_cast<const u32x4*>(w_in);
  a.w_out = reinterpret_cast<u32x4*>(w_out);
  a.sf_in = reinterpret_cast<const u32x4*>(sf_in);
  a.sf_out = reinterpret_cast<uint32_t*>(sf_out);
  a.chunks = (uint32_t)(N * K / 32);                    // N rows x K/2 bytes / 16
  a.rot = swap_halves ? a.chunks / 2 : 0u;
  a.wblocks = (a.chunks + kThreads - 1) / kThreads;
  a.R = (uint32_t)N;
  a.quads = (uint32_t)(K / 64);
  a.groups = (a.quads + kTilesPerGroup - 1) / kTilesPerGroup;
  a.half_rows = swap_halves ? a.R / 2 : 0u;
  a.out_quads = out_quads ? 1u : 0u;
  a.w_tiled = w_tiled ? 1u : 0u;
  a.kblocks = (uint32_t)(K / 64);
  const uint32_t sblocks = (a.R / 128) * a.groups;
  hipLaunchKernelGGL(repack_nvfp4, dim3(a.wblocks + sblocks, (uint32_t)E), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moeq
