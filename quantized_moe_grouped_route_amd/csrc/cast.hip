// bf16 -> binary16 conversion of activations for the binary16 form of the
// NVFP4 GEMM (megamoe_rm.cu converts its bf16 input to fp16 the same way,
// in its route_prep).  Each bf16 value is widened to fp32 exactly and
// rounded once to the nearest binary16 (ties to even, overflow to +-inf),
// so values of magnitude in [2^-14, 65504] convert exactly.
// One thread converts 8 values (16-byte nontemporal load and store): an
// HBM-bound stream.
#include "common.h"
#include "kernels.h"

namespace moeq {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void cast_bf16_f16(const u32x4* __restrict__ x, u32x4* __restrict__ y,
                                                          int64_t n8) {
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kThreads) {
    const u32x4 v = __builtin_nontemporal_load(x + i);
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __builtin_bit_cast(float, v[j] << 16), hi = __builtin_bit_cast(float, v[j] & 0xffff0000u);
      r[j] = __builtin_bit_cast(u32, __builtin_convertvector(v2f{lo, hi}, v2h));
    }
    __builtin_nontemporal_store(r, y + i);
  }
}

}  // namespace

hipError_t launch_cast_bf16_f16(const uint16_t* x, int64_t n, uint16_t* y, int num_cus, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t n8 = n / 8;
  const int64_t blocks = (n8 + kThreads - 1) / kThreads;
  const int grid = (int)(blocks < (int64_t)num_cus * 16 ? blocks : (int64_t)num_cus * 16);
  hipLaunchKernelGGL(cast_bf16_f16, dim3(grid), dim3(kThreads), 0, stream, reinterpret_cast<const u32x4*>(x),
                     reinterpret_cast<u32x4*>(y), n8);
  return hipGetLastError();
}

}  // namespace moeq
