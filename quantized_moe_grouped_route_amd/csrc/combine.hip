// Top-k weighted scatter back to token rows (megamoe_rm.cu's combine: a
// token's pairs that have an expert, summed in slot order in fp32 and
// rounded once; tilelang_kernels.py: zero output plus weighted rows).
// PAIRS: the rows are already weighted and in pair order (the output of
// fc2_rm's epilogue), so token t's rows are t*topk .. t*topk+topk-1.
//
// One thread owns 8 consecutive columns of one token row: it reads the
// pair table entries of its token, then 8 elements (16 or 32 bytes) of each
// routed expert row, so every wave reads and writes contiguous runs.
// When y is larger than the 256 MB Infinity Cache it streams from HBM, and
// nontemporal loads and stores measured 17 % faster (bf16 y of 32768 x
// 7168: 107 -> 89 us); a y that fits may still sit in the cache from the
// GEMM that wrote it, and there ordinary accesses measured 9 % faster
// (f16 y of 16384 x 4096: 29.8 against 32.4 us).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moeq {
namespace {

constexpr int kThreads = 256;

constexpr int64_t kStreamBytes = int64_t(256) << 20;

template <bool NT>
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return ld16(p);
}
template <bool NT>
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  if (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else st16(p, v);
}

template <int YK, bool NT>
__device__ __forceinline__ void load8(const void* y, int64_t off, float v[8]) {
  if (YK == OUT_F32) {
    const float* p = static_cast<const float*>(y) + off;
    const v4f a = __builtin_bit_cast(v4f, ld16_nt<NT>(p)), b = __builtin_bit_cast(v4f, ld16_nt<NT>(p + 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  } else {
    const u32x4 q = ld16_nt<NT>(static_cast<const uint16_t*>(y) + off);
    const u32 w[4] = {q[0], q[1], q[2], q[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (YK == OUT_BF16) {
        v[2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
        v[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      } else {
        v[2 * j] = f16_bits_to_f32((uint16_t)(w[j] & 0xffffu));
        v[2 * j + 1] = f16_bits_to_f32((uint16_t)(w[j] >> 16));
      }
    }
  }
}

template <int OK, bool NT>
__device__ __forceinline__ void store8(void* out, int64_t off, const float v[8]) {
  if (OK == OUT_F32) {
    float* p = static_cast<float*>(out) + off;
    st16_nt<NT>(p, __builtin_bit_cast(u32x4, v4f{v[0], v[1], v[2], v[3]}));
    st16_nt<NT>(p + 4, __builtin_bit_cast(u32x4, v4f{v[4], v[5], v[6], v[7]}));
  } else {
    u32 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (u32)OutT<OK>::from(v[2 * j]) | ((u32)OutT<OK>::from(v[2 * j + 1]) << 16);
    st16_nt<NT>(static_cast<uint16_t*>(out) + off, u32x4{w[0], w[1], w[2], w[3]});
  }
}

template <int YK, int OK, bool PAIRS, bool NT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void* __restrict__ y,
                                                           const int* __restrict__ p2s,
                                                           const float* __restrict__ tw, int T,
                                                           int topk, int N, int64_t P,
                                                           void* __restrict__ out) {
  const int cblocks = (N / 8 + kThreads - 1) / kThreads;
  const int t = blockIdx.x / cblocks;
  const int c = ((blockIdx.x - t * cblocks) * kThreads + threadIdx.x) * 8;
  if (c >= N) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const int64_t p = (int64_t)t * topk + j;
    const int s = p2s[p];
    if (s < 0 || s >= P) continue;
    float v[8];
    load8<YK, NT>(y, (PAIRS ? p : (int64_t)s) * N + c, v);
    if (PAIRS) {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += v[q];
    } else {
      const float w = tw[p];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(w, v[q], acc[q]);
    }
  }
  store8<OK, NT>(out, (int64_t)t * N + c, acc);
}

template <int YK, bool PAIRS, bool NT>
hipError_t launch_nt(const void* y, const int* p2s, const float* tw, int T, int topk, int N,
                     int64_t P, int out_kind, void* out, hipStream_t stream) {
  const dim3 grid(((N / 8 + kThreads - 1) / kThreads) * T);
  switch (out_kind) {
    case OUT_F16:
      hipLaunchKernelGGL((combine_kernel<YK, OUT_F16, PAIRS, NT>), grid, dim3(kThreads), 0, stream, y, p2s, tw,
                         T, topk, N, P, out);
      break;
    case OUT_BF16:
      hipLaunchKernelGGL((combine_kernel<YK, OUT_BF16, PAIRS, NT>), grid, dim3(kThreads), 0, stream, y, p2s,
                         tw, T, topk, N, P, out);
      break;
    default:
      hipLaunchKernelGGL((combine_kernel<YK, OUT_F32, PAIRS, NT>), grid, dim3(kThreads), 0, stream, y, p2s, tw,
                         T, topk, N, P, out);
      break;
  }
  return hipGetLastError();
}

template <int YK, bool PAIRS>
hipError_t launch_y(const void* y, const int* p2s, const float* tw, int T, int topk, int N,
                    int64_t P, int out_kind, void* out, hipStream_t stream) {
  // the rows actually read: T * topk of them at most
  const int64_t y_bytes = std::min<int64_t>(P, (int64_t)T * topk) * N * (YK == OUT_F32 ? 4 : 2);
  if (y_bytes >= kStreamBytes)
    return launch_nt<YK, PAIRS, true>(y, p2s, tw, T, topk, N, P, out_kind, out, stream);
  return launch_nt<YK, PAIRS, false>(y, p2s, tw, T, topk, N, P, out_kind, out, stream);
}

template <bool PAIRS>
hipError_t launch_kind(const void* y, int y_kind, const int* p2s, const float* tw, int T, int topk, int N,
                       int64_t P, int out_kind, void* out, hipStream_t stream) {
  switch (y_kind) {
    case OUT_F16: return launch_y<OUT_F16, PAIRS>(y, p2s, tw, T, topk, N, P, out_kind, out, stream);
    case OUT_BF16: return launch_y<OUT_BF16, PAIRS>(y, p2s, tw, T, topk, N, P, out_kind, out, stream);
    default: return launch_y<OUT_F32, PAIRS>(y, p2s, tw, T, topk, N, P, out_kind, out, stream);
  }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_kind, const int* p2s, const float* tw, int T,
                          int topk, int N, int64_t P, int out_kind, void* out,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (tw == nullptr) return launch_kind<true>(y, y_kind, p2s, tw, T, topk, N, P, out_kind, out, stream);
  return launch_kind<false>(y, y_kind, p2s, tw, T, topk, N, P, out_kind, out, stream);
}

}  // namespace moeq
