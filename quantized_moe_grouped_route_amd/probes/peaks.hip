// Peak probes for one MI355X (gfx950): what the chip sustains for the two
// resources the grouped GEMMs are bound by, measured on the GPU at hand instead
// of taken from the data sheet.
//   moeq_peak_read  streams a buffer from HBM with 16-byte nontemporal loads
//                   into registers (every byte read once).
//   moeq_peak_read_lds  streams it with nontemporal direct-to-LDS copies, 16
//                   in flight per wave, each wave its own contiguous share,
//                   the way the weight-streaming decode schedules read; the
//                   faster of the two is the bound (measured 7.0 against
//                   6.0 TB/s for the register loads).
//   moeq_peak_mfma  runs back-to-back MFMAs of one kind on register operands
//                   (no memory traffic), the bound of the tiled schedules.
// Each call only enqueues one kernel on `stream`; the caller times it.
// Separate from libmoeq.so: nothing in the library calls these.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_stream(const u32x4* __restrict__ src, int64_t n16,
                                                   unsigned* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 x = {0, 0, 0, 0};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) x ^= __builtin_nontemporal_load(src + i);
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x.x ^ x.y ^ x.z ^ x.w;
}

// Wave w of the W in the grid copies its own contiguous share of the
// buffer, 1 KB at a time, into a 16-slot LDS ring of its own (W concurrent
// sequential streams, as the decode schedules' waves each stream their own
// rows); a slot is reused once the copy 16 before it has landed (vmcnt 15).
// The LDS bytes are never read.
__global__ __launch_bounds__(256) void read_lds(const uint8_t* __restrict__ src, int64_t n1k) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4][16][1024];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * 4, w = (int64_t)blockIdx.x * 4 + wv;
  const int64_t per = (n1k + W - 1) / W;
  const int64_t c0 = w * per, c1 = c0 + per < n1k ? c0 + per : n1k;
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&ring[wv][0][0]);
  int slot = 0, issued = 0;
  for (int64_t c = c0; c < c1; ++c) {
    if (issued >= 16) __builtin_amdgcn_s_waitcnt((15 & 15) | (7 << 4) | (15 << 8) | ((15 >> 4) << 14));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(src + c * 1024 + lane * 16), "s"(base + slot * 1024) : "memory", "m0");
    slot = (slot + 1) & 15;
    ++issued;
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

// Kinds: 0 int8 32x32x32, 1 fp8 e4m3 32x32x64, 2 bf16 32x32x16,
// 3 fp16 32x32x16, 4 fp6 e3m2 32x32x64, 5 fp4 e2m1 32x32x64.
// Four independent accumulators per wave.  The operands are read once from
// `src` (64 bytes per thread, finite values of the kind's format drawn by
// the caller: the switching activity, and so the power and the clock, then
// resembles real data); the accumulators are stored at the end.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop(int iters, const v8i* __restrict__ src, float* __restrict__ sink) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  v16f f[4];
  v16i n[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = v16f{};
    n[j] = v16i{};
  }
  const v8i a8 = src[2 * t], b8 = src[2 * t + 1];
  const v4i a4 = {a8[0], a8[1], a8[2], a8[3]};
  const v4i b4 = {b8[0], b8[1], b8[2], b8[3]};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (KIND == 0) {
        n[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, n[j], 0, 0, 0);
      } else if constexpr (KIND == 1) {
        f[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, f[j], 0, 0, 0, 127, 0, 127);
      } else if constexpr (KIND == 2) {
        f[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a4), __builtin_bit_cast(v8bf, b4),
                                                       f[j], 0, 0, 0);
      } else if constexpr (KIND == 3) {
        f[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a4), __builtin_bit_cast(v8h, b4),
                                                      f[j], 0, 0, 0);
      } else if constexpr (KIND == 4) {
        f[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, f[j], 3, 3, 0, 127, 0, 127);
      } else {
        f[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, f[j], 4, 4, 0, 127, 0, 127);
      }
    }
  }
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += f[j][i] + (float)n[j][i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <int KIND>
hipError_t go(int grid, int iters, const v8i* src, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(mfma_loop<KIND>, dim3(grid), dim3(256), 0, st, iters, src, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from `src`; sink: grid * 256 uint32.
int moeq_peak_read(const void* src, int64_t bytes, void* sink, int grid, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 || grid <= 0) return 1;
  hipLaunchKernelGGL(read_stream, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<unsigned*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Reads `bytes` (a multiple of 1024) from `src` with direct-to-LDS copies;
// grid workgroups of 4 waves.
int moeq_peak_read_lds(const void* src, int64_t bytes, int grid, void* stream) {
  if (!src || bytes <= 0 || bytes % 1024 || grid <= 0) return 1;
  hipLaunchKernelGGL(read_lds, dim3(grid), dim3(256), 0, (hipStream_t)stream, static_cast<const uint8_t*>(src),
                     bytes / 1024);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// grid workgroups of 4 waves, each wave `iters` x 4 MFMAs of `kind`;
// src: grid * 256 * 64 bytes of operands (A then B, 32 bytes each per
// thread); sink: grid * 256 floats.  Flops (ops) per MFMA: 2 * 32 * 32 * K
// with K = 32 (int8), 64 (fp8, fp6, fp4), 16 (bf16, fp16).
int moeq_peak_mfma(int kind, int grid, int iters, const void* src, void* sink, void* stream) {
  if (!src || !sink || grid <= 0 || iters <= 0) return 1;
  const v8i* o = static_cast<const v8i*>(src);
  float* s = static_cast<float*>(sink);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  switch (kind) {
    case 0: e = go<0>(grid, iters, o, s, st); break;
    case 1: e = go<1>(grid, iters, o, s, st); break;
    case 2: e = go<2>(grid, iters, o, s, st); break;
    case 3: e = go<3>(grid, iters, o, s, st); break;
    case 4: e = go<4>(grid, iters, o, s, st); break;
    case 5: e = go<5>(grid, iters, o, s, st); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 4;
}

}  // extern "C"
