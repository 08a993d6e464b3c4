// Per-row symmetric INT4 quantization of activations.  CUTLASS discussion
// #2855 quantizes the fp16 activations per token to int4 and applies the
// token's scale with the channel scale in the GEMM epilogue; its rounding
// rule is not given.  Rule used: amax = max |x|, s = amax / 7,
// q = clamp(rne(x * (7 / amax)), -8, 7), each step one fp32 operation (the
// fp32 product decides the integer code); a row with amax < 2^-120 becomes
// zeros with scale 1.  Codes are packed two per byte, element 2b in the low
// nibble of byte b, the layout grouped_gemm_qint4 reads.
//
// HBM-bound.  Rows of up to 16384 elements: one workgroup per row holds the
// row in registers, so it is read once.  When x is larger than the 256 MB
// Infinity Cache (it then streams from HBM) the 16-bit inputs are read and
// the codes written with nontemporal accesses, measured 10 % faster than
// ordinary ones on 16384 x 14336 fp16 rows (5.9 against 5.2 TB/s).  Longer rows: one wave per row,
// pass 1 reads the row for its amax (one wave max), pass 2 reads it again
// and writes the packed codes.
// Each lane moves 8 elements per step: 16 input bytes (32 for f32), 4 output
// bytes, so a wave reads 1 KB and writes 256 contiguous bytes per step.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moeq {
namespace {

constexpr int kWavesQ = 4;

// 8 input elements as raw bits (16 bytes; 32 for f32) and their values.
template <int XK>
struct Raw8 {
  u32x4 w[XK == OUT_F32 ? 2 : 1];
};
template <int XK, bool NT = false>
__device__ __forceinline__ Raw8<XK> load8(const void* x, int64_t i) {
  Raw8<XK> r;
  if (XK == OUT_F32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + i);
    r.w[0] = p[0];
    r.w[XK == OUT_F32 ? 1 : 0] = p[1];
  } else if (NT) {
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + i));
  } else {
    r.w[0] = ld16(static_cast<const uint16_t*>(x) + i);
  }
  return r;
}
template <int XK>
__device__ __forceinline__ void values8(const Raw8<XK>& r, float v[8]) {
  if (XK == OUT_F32) {
    // the float view of the raw words (a bit-cast of single elements of an
    // integer vector is not used: this compiler keeps only element 0)
    const v4f a = __builtin_bit_cast(v4f, r.w[0]), b = __builtin_bit_cast(v4f, r.w[XK == OUT_F32 ? 1 : 0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32 lo = r.w[0][j] & 0xffffu, hi = r.w[0][j] >> 16;
      if (XK == OUT_BF16) {
        v[2 * j] = bf16_bits_to_f32(lo);
        v[2 * j + 1] = bf16_bits_to_f32(hi);
      } else {
        v[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)lo);
        v[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)hi);
      }
    }
  }
}
template <int XK>
__device__ __forceinline__ void load8f(const void* x, int64_t i, float v[8]) {
  values8<XK>(load8<XK>(x, i), v);
}

template <int XK>
__global__ __launch_bounds__(64 * kWavesQ) void quant_int4_rows(const void* __restrict__ x, int64_t rows, int K,
                                                               uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * kWavesQ;
  for (int64_t row = (int64_t)blockIdx.x * kWavesQ + (threadIdx.x >> 6); row < rows; row += waves) {
    const int64_t base = row * K;
    float m = 0.0f;
    for (int k = lane * 8; k < K; k += 512) {
      float v[8];
      load8f<XK>(x, base + k, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const bool tiny = m < 0x1p-120f;
    const float s = tiny ? 1.0f : m / 7.0f;
    const float r = tiny ? 0.0f : 7.0f / m;
    uint8_t* qrow = q + row * (K / 2);
    for (int k = lane * 8; k < K; k += 512) {
      float v[8];
      load8f<XK>(x, base + k, v);
      u32 packed = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = fminf(fmaxf(__builtin_rintf(v[j] * r), -8.0f), 7.0f);
        packed |= ((u32)(int)t & 15u) << (4 * j);
      }
      *reinterpret_cast<u32*>(qrow + k / 2) = packed;
    }
    if (lane == 0) scale[row] = s;
  }
}

// Rows of at most 256 * 8 * kRegLoads = 16384 elements: one workgroup per row keeps
// its part of the row in registers (kRegLoads loads of 8 elements per
// thread, all issued before any is used), so the row is read once.
constexpr int kRegLoads = 8;
constexpr int kRowThreads = 256;

template <int XK, bool NT>
__global__ __launch_bounds__(kRowThreads) void quant_int4_rows_reg(const void* __restrict__ x, int64_t rows, int K,
                                                                  uint8_t* __restrict__ q,
                                                                  float* __restrict__ scale) {
  __shared__ float wmax[kRowThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t base = row * K;
    Raw8<XK> raw[kRegLoads];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kRegLoads; ++i) {
      const int k = (i * kRowThreads + tid) * 8;
      if (k < K) raw[i] = load8<XK, NT>(x, base + k);
    }
#pragma unroll
    for (int i = 0; i < kRegLoads; ++i) {
      const int k = (i * kRowThreads + tid) * 8;
      if (k < K) {
        float v[8];
        values8<XK>(raw[i], v);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) wmax[wid] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kRowThreads / 64; ++w) m = fmaxf(m, wmax[w]);
    __syncthreads();  // wmax is reused by the next row
    const bool tiny = m < 0x1p-120f;
    const float s = tiny ? 1.0f : m / 7.0f;
    const float r = tiny ? 0.0f : 7.0f / m;
    uint8_t* qrow = q + row * (K / 2);
#pragma unroll
    for (int i = 0; i < kRegLoads; ++i) {
      const int k = (i * kRowThreads + tid) * 8;
      if (k < K) {
        float v[8];
        values8<XK>(raw[i], v);
        u32 packed = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float t = fminf(fmaxf(__builtin_rintf(v[j] * r), -8.0f), 7.0f);
          packed |= ((u32)(int)t & 15u) << (4 * j);
        }
        if (NT) __builtin_nontemporal_store(packed, reinterpret_cast<u32*>(qrow + k / 2));
        else *reinterpret_cast<u32*>(qrow + k / 2) = packed;
      }
    }
    if (tid == 0) scale[row] = s;
  }
}

}  // namespace

hipError_t launch_quant_int4(const void* x, int x_kind, int64_t rows, int K, uint8_t* q, float* scale,
                             int num_cus, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (K <= kRowThreads * 8 * kRegLoads) {
    const int grid = (int)std::min<int64_t>(rows, (int64_t)num_cus * 8);
    const bool nt = rows * K * 2 >= (int64_t(256) << 20);  // 16-bit inputs past the Infinity Cache
#define MOEQ_QREG(XK, NT) \
  hipLaunchKernelGGL((quant_int4_rows_reg<XK, NT>), dim3(grid), dim3(kRowThreads), 0, stream, x, rows, K, q, scale)
    switch (x_kind) {
      case OUT_F16:
        if (nt) MOEQ_QREG(OUT_F16, true); else MOEQ_QREG(OUT_F16, false);
        break;
      case OUT_BF16:
        if (nt) MOEQ_QREG(OUT_BF16, true); else MOEQ_QREG(OUT_BF16, false);
        break;
      default:
        MOEQ_QREG(OUT_F32, false);
        break;
    }
#undef MOEQ_QREG
    return hipGetLastError();
  }
  const int64_t wgs = (rows + kWavesQ - 1) / kWavesQ;
  const int grid = (int)std::min<int64_t>(wgs, (int64_t)num_cus * 8);
  switch (x_kind) {
    case OUT_F16:
      hipLaunchKernelGGL(quant_int4_rows<OUT_F16>, dim3(grid), dim3(64 * kWavesQ), 0, stream, x, rows, K, q, scale);
      break;
    case OUT_BF16:
      hipLaunchKernelGGL(quant_int4_rows<OUT_BF16>, dim3(grid), dim3(64 * kWavesQ), 0, stream, x, rows, K, q, scale);
      break;
    default:
      hipLaunchKernelGGL(quant_int4_rows<OUT_F32>, dim3(grid), dim3(64 * kWavesQ), 0, stream, x, rows, K, q, scale);
      break;
  }
  return hipGetLastError();
}

}  // namespace moeq
