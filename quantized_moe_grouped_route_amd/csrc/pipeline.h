// Multi-stage global -> LDS pipeline for the tiled grouped GEMMs.
//
// Tiles are copied by the gfx950 direct-to-LDS loads (global_load_lds,
// 16 bytes per lane): a wave instruction writes 1 KB of LDS contiguously,
// lane l at byte 16*l, while each lane reads its own global address, so a
// row gather (token -> row) costs nothing extra and no registers hold data
// in flight.  A ring of stages keeps several K steps in flight per wave.
//
// LDS tile layout: 128 rows x 128 bytes, no padding; the 16-byte chunk c of
// row r is stored at chunk position c ^ ((r >> 1) & 7).  The LDS has 64
// banks (256 bytes), so a 16-byte-per-lane read serves 16 lanes at a time;
// 16 consecutive rows reading the same logical chunk then cover all 16
// bank groups once (even rows the low 128 bytes, odd rows the high 128).
//
// Completion: the loads count in the wave's vmcnt.  Waiting for a stage is
// an explicit s_waitcnt vmcnt(n) (n = loads issued after it), then a plain
// s_barrier so that every wave's part of the stage has landed.  The
// workgroup barrier of __syncthreads() would wait for all loads in flight.
#pragma once

#include "common.h"

namespace moeq {

typedef __attribute__((address_space(3))) void lds_void_t;

// The loads are issued through inline assembly: the compiler's own
// bookkeeping would otherwise make every LDS read wait for all of them
// (vmcnt(0)), serializing the ring.  Their completion is tracked by the
// explicit wait_vmcnt below.  M0 holds the wave's LDS base; one wait state
// separates the M0 write from the load.
// LDS address of `p` as a wave-uniform (scalar) value; `p` must be the same
// for every lane of the wave.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)p);
}
// 16 bytes per lane from `src` to LDS at byte address `lds` + 16 * lane.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds) : "memory", "m0");
}
// The same with the nontemporal hint, for bytes read once (the weight
// streams of the decode schedules): measured 7-15 % faster there than the
// plain copy (NVFP4 FC1 of 8 tokens 166 -> 141 us, FP8 decode 290 -> 253 us,
// INT4 FC1 of 8 tokens 85 -> 77 us).
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(src), "s"(lds) : "memory", "m0");
}
// 4 bytes per lane to LDS at byte address `lds` + 4 * lane.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds) : "memory", "m0");
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence; the compiler may not move
// memory accesses across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Byte offset of logical 16-byte chunk c of row r in a swizzled tile.
__device__ __forceinline__ int swz_key(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ swz_key(r)) << 4); }

// Copy mapping of one 1 KB wave instruction (tile rows 8q .. 8q+7): lane l
// lands at row 8q + l/8, chunk position l%8, so it must fetch logical chunk
// (l%8) ^ swz_key(8q + l/8) = (l%8) ^ (4*(q&1) + l/16).
__device__ __forceinline__ int dma_chunk(int lane, int q) {
  return ((lane & 7) ^ (((q & 1) << 2) | (lane >> 4))) << 4;
}
// Swizzle key of the fragment row 32k + (lane % 32) read by this lane.
__device__ __forceinline__ int frag_key(int lane) { return (lane >> 1) & 7; }

}  // namespace moeq
