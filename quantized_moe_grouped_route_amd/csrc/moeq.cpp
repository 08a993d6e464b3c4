// C ABI of the library: host-side validation and asynchronous launch on the
// caller's stream.  Nothing here allocates device memory, synchronizes, or
// copies between host and device.  The argument checks mirror the pages'
// conventions (CUTLASS discussion #2855 rejects K or N not multiples of 32
// before launching; megamoe_rm.cu checks every shape before its launches),
// reported as status codes because the boundary is C.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/moeq.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

moeq_status fail(moeq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxE = 1024;
constexpr int kMaxTopk = 64;

// Compute units of the current device, looked up once per device.  Calls
// may come from several host threads at once; each stores the same value.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

moeq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOEQ_OK;
  return fail(MOEQ_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// Checks shared by the three grouped GEMMs.  n_align is the multiple N
// must be: 32 for INT4 and NVFP4 (CUTLASS discussion #2855's launcher
// checks N % 32; the INT4 epilogue masks partial column tiles and the NVFP4
// streaming schedule works in 16- and 32-row weight blocks), 128 for FP8,
// whose weight scales cover 128 x 128 blocks.
moeq_status check_grouped(const char* fn, const void* a, int64_t rows_a, int a_row, const void* w,
                          const int32_t* offsets, int64_t P, int32_t topk, int32_t E, int64_t N,
                          int64_t K, const void* out, int64_t n_align) {
  if (E < 1 || E > kMaxE) return fail(MOEQ_EINVAL, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (topk < 1 || topk > kMaxTopk) return fail(MOEQ_EINVAL, "%s: topk=%d outside [1, %d]", fn, topk, kMaxTopk);
  if (P < 0 || P >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: P=%lld out of range", fn, (long long)P);
  if (rows_a < 0 || rows_a >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: rows_a=%lld out of range", fn, (long long)rows_a);
  if (P > 0 && rows_a == 0) return fail(MOEQ_EINVAL, "%s: rows_a=0 with P>0", fn);
  if (N <= 0 || K <= 0 || N > (1 << 20) || K > (1 << 17))
    return fail(MOEQ_EINVAL, "%s: N=%lld K=%lld out of range", fn, (long long)N, (long long)K);
  if (K % 128 != 0) return fail(MOEQ_EALIGN, "%s: K=%lld must be a multiple of 128", fn, (long long)K);
  if (N % n_align != 0)
    return fail(MOEQ_EALIGN, "%s: N=%lld must be a multiple of %lld", fn, (long long)N, (long long)n_align);
  if (a_row != MOEQ_AROW_TOKEN && a_row != MOEQ_AROW_SORTED) return fail(MOEQ_EINVAL, "%s: bad a_row %d", fn, a_row);
  if (!a || !w || !offsets || !out) return fail(MOEQ_EINVAL, "%s: null pointer", fn);
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(out, 16) || !aligned(offsets, 4))
    return fail(MOEQ_EALIGN, "%s: pointers must be 16-byte aligned", fn);
  return MOEQ_OK;
}

moeq::GroupedArgs make_args(const int32_t* offsets, const int32_t* sorted, int64_t rows_a,
                            moeq_arow a_row, int64_t P, int32_t topk, int32_t E, int64_t N,
                            int64_t K, bool silu, moeq_dtype od, void* out, moeq_sched sched) {
  moeq::GroupedArgs g;
  g.offsets = offsets;
  g.sorted_ids = sorted;
  g.rows_a = rows_a;
  g.a_sorted = (a_row == MOEQ_AROW_SORTED) ? 1 : 0;
  g.topk = topk;
  g.E = E;
  g.P = P;
  g.N = (int)N;
  g.K = (int)K;
  g.silu_mul = silu ? 1 : 0;
  g.act_limit = INFINITY;
  g.pair_weights = nullptr;
  g.x_f16 = 0;
  g.sf_quads = 0;
  g.w_tiled = 0;
  g.out_kind = (int)od;
  g.out = out;
  g.sched = (int)sched;
  g.queue = nullptr;
  g.num_cus = device_cus();
  return g;
}

}  // namespace

extern "C" {

const char* moeq_last_error(void) { return g_err.c_str(); }

int32_t moeq_abi_version(void) { return 3; }

size_t moe_route_prep_workspace_bytes(int64_t T, int32_t topk, int32_t E) {
  // T is bounded before the product so that T*topk cannot overflow
  if (T < 0 || T >= (int64_t(1) << 31) || topk < 1 || topk > kMaxTopk || E < 1 || E > kMaxE) return 0;
  const int64_t P = T * (int64_t)topk;
  if (P >= (int64_t(1) << 31)) return 0;
  return moeq::route_workspace_bytes(P, E);
}

moeq_status moe_route_prep(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                           int32_t* expert_offsets, int32_t* sorted_pair_ids,
                           int32_t* pair_to_sorted, int32_t* n_invalid, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const char* fn = "moe_route_prep";
  if (T < 0 || T >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: T=%lld outside [0, 2^31)", fn, (long long)T);
  if (topk < 1 || topk > kMaxTopk) return fail(MOEQ_EINVAL, "%s: topk=%d outside [1, %d]", fn, topk, kMaxTopk);
  if (E < 1 || E > kMaxE) return fail(MOEQ_EINVAL, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  const int64_t P = T * (int64_t)topk;
  if (P >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: T*topk too large", fn);
  if (!expert_offsets || !n_invalid || (P > 0 && (!topk_ids || !sorted_pair_ids || !pair_to_sorted)))
    return fail(MOEQ_EINVAL, "%s: null pointer", fn);
  if (!aligned(topk_ids, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_pair_ids, 4) ||
      !aligned(pair_to_sorted, 4) || !aligned(n_invalid, 4) || !aligned(workspace, 4))
    return fail(MOEQ_EALIGN, "%s: int32 arrays must be 4-byte aligned", fn);
  const size_t need = moeq::route_workspace_bytes(P, E);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(MOEQ_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
  return hip_status(moeq::launch_route(topk_ids, (int)P, E, expert_offsets, sorted_pair_ids,
                                       pair_to_sorted, n_invalid, workspace, (hipStream_t)stream),
                    fn);
}

moeq_status moe_route_prep_noalloc(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                                   int32_t* expert_offsets, int32_t* sorted_pair_ids,
                                   int32_t* pair_to_sorted, int32_t* n_invalid, void* stream) {
  const char* fn = "moe_route_prep_noalloc";
  static_assert(moeq::kRouteNoallocScratchBytes == MOEQ_ROUTE_NOALLOC_SCRATCH_BYTES, "header and library agree");
  if (T < 0 || T >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: T=%lld outside [0, 2^31)", fn, (long long)T);
  if (topk < 1 || topk > kMaxTopk) return fail(MOEQ_EINVAL, "%s: topk=%d outside [1, %d]", fn, topk, kMaxTopk);
  if (E < 1 || E > kMaxE) return fail(MOEQ_EINVAL, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  const int64_t P = T * (int64_t)topk;
  if (P >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: T*topk too large", fn);
  if (!expert_offsets || !n_invalid || (P > 0 && (!topk_ids || !sorted_pair_ids || !pair_to_sorted)))
    return fail(MOEQ_EINVAL, "%s: null pointer", fn);
  if (!aligned(topk_ids, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_pair_ids, 4) ||
      !aligned(pair_to_sorted, 4) || !aligned(n_invalid, 4))
    return fail(MOEQ_EALIGN, "%s: int32 arrays must be 4-byte aligned", fn);
  const size_t need = moeq::route_workspace_bytes(P, E);
  if (need > moeq::kRouteNoallocScratchBytes)
    return fail(MOEQ_EINVAL, "%s: T*topk=%lld with E=%d needs %zu bytes of scratch, above the fixed %zu", fn,
                (long long)P, E, need, moeq::kRouteNoallocScratchBytes);
  return hip_status(moeq::launch_route_noalloc(topk_ids, (int)P, E, expert_offsets, sorted_pair_ids,
                                               pair_to_sorted, n_invalid, (hipStream_t)stream),
                    fn);
}

moeq_status grouped_gemm_qint4(const uint8_t* a, const float* a_scale, int64_t rows_a,
                               moeq_arow a_row, const uint8_t* w, const float* w_scale,
                               const int32_t* expert_offsets, const int32_t* sorted_pair_ids,
                               int64_t P, int32_t topk, int32_t E, int64_t N, int64_t K,
                               moeq_act act, moeq_dtype out_dtype, void* out, moeq_sched sched,
                               void* stream) {
  const char* fn = "grouped_gemm_qint4";
  moeq_status st = check_grouped(fn, a, rows_a, a_row, w, expert_offsets, P, topk, E, N, K, out, 32);
  if (st != MOEQ_OK) return st;
  // The int8 MFMA sums products of nibbles scaled by 16, at most 2^14 each:
  // K < 2^17 keeps every int32 partial sum below 2^31.
  if (K >= (int64_t(1) << 17))
    return fail(MOEQ_EINVAL, "%s: K=%lld must be below 131072 (int32 accumulator range)", fn, (long long)K);
  if (!a_scale || !w_scale) return fail(MOEQ_EINVAL, "%s: null scale pointer", fn);
  if (!aligned(a_scale, 4) || !aligned(w_scale, 4)) return fail(MOEQ_EALIGN, "%s: scales must be 4-byte aligned", fn);
  if (act != MOEQ_ACT_NONE && act != MOEQ_ACT_SILU_MUL) return fail(MOEQ_EUNSUPPORTED, "%s: act %d", fn, act);
  if (out_dtype != MOEQ_F16 && out_dtype != MOEQ_BF16 && out_dtype != MOEQ_F32 && out_dtype != MOEQ_I32)
    return fail(MOEQ_EUNSUPPORTED, "%s: out dtype %d", fn, out_dtype);
  if (out_dtype == MOEQ_I32 && act != MOEQ_ACT_NONE)
    return fail(MOEQ_EUNSUPPORTED, "%s: I32 output needs act NONE", fn);
  if (a_row == MOEQ_AROW_TOKEN && !sorted_pair_ids && rows_a < P)
    return fail(MOEQ_EINVAL, "%s: identity rows need rows_a >= P", fn);
  if (sched < MOEQ_SCHED_AUTO || sched > MOEQ_SCHED_PREFILL) return fail(MOEQ_EINVAL, "%s: sched %d", fn, sched);
  if (sched == MOEQ_SCHED_DECODE && K % 256 != 0)
    return fail(MOEQ_EALIGN, "%s: the streaming schedule needs K %% 256 == 0 (K=%lld)", fn, (long long)K);
  moeq::GroupedArgs g = make_args(expert_offsets, sorted_pair_ids, rows_a, a_row, P, topk, E, N, K,
                                  act == MOEQ_ACT_SILU_MUL, out_dtype, out, sched);
  return hip_status(moeq::launch_gemm_int4(g, a, a_scale, w, w_scale, (hipStream_t)stream), fn);
}

moeq_status grouped_gemm_qfp8_block(const uint8_t* a, const float* a_scale, int64_t rows_a,
                                    moeq_arow a_row, const uint8_t* w, const float* w_scale,
                                    const int32_t* expert_offsets,
                                    const int32_t* sorted_pair_ids, int64_t P, int32_t topk,
                                    int32_t E, int64_t N, int64_t K, moeq_dtype out_dtype,
                                    void* out, moeq_sched sched, void* stream) {
  const char* fn = "grouped_gemm_qfp8_block";
  moeq_status st = check_grouped(fn, a, rows_a, a_row, w, expert_offsets, P, topk, E, N, K, out, 128);
  if (st != MOEQ_OK) return st;
  if (!a_scale || !w_scale) return fail(MOEQ_EINVAL, "%s: null scale pointer", fn);
  if (!aligned(a_scale, 4) || !aligned(w_scale, 4)) return fail(MOEQ_EALIGN, "%s: scales must be 4-byte aligned", fn);
  if (out_dtype != MOEQ_F16 && out_dtype != MOEQ_BF16 && out_dtype != MOEQ_F32)
    return fail(MOEQ_EUNSUPPORTED, "%s: out dtype %d", fn, out_dtype);
  if (a_row == MOEQ_AROW_TOKEN && !sorted_pair_ids && rows_a < P)
    return fail(MOEQ_EINVAL, "%s: identity rows need rows_a >= P", fn);
  if (sched < MOEQ_SCHED_AUTO || sched > MOEQ_SCHED_PREFILL) return fail(MOEQ_EINVAL, "%s: sched %d", fn, sched);
  moeq::GroupedArgs g = make_args(expert_offsets, sorted_pair_ids, rows_a, a_row, P, topk, E, N, K,
                                  false, out_dtype, out, sched);
  return hip_status(moeq::launch_gemm_fp8(g, a, a_scale, w, w_scale, (hipStream_t)stream), fn);
}

moeq_status grouped_gemm_qnvfp4(const void* x, moeq_dtype x_dtype, int64_t rows_a, moeq_arow a_row, const uint8_t* w,
                                moeq_w_layout w_layout, const uint8_t* w_sf, moeq_sf_layout sf_layout,
                                const float* w_gscale,
                                const int32_t* expert_offsets, const int32_t* sorted_pair_ids,
                                int64_t P, int32_t topk, int32_t E, int64_t N, int64_t K,
                                moeq_act act, float act_limit, const float* pair_weights,
                                moeq_dtype out_dtype, void* out, int32_t* work_queue, moeq_sched sched,
                                void* stream) {
  const char* fn = "grouped_gemm_qnvfp4";
  moeq_status st = check_grouped(fn, x, rows_a, a_row, w, expert_offsets, P, topk, E, N, K, out, 32);
  if (st != MOEQ_OK) return st;
  if (!w_sf || !w_gscale) return fail(MOEQ_EINVAL, "%s: null scale pointer", fn);
  if (!aligned(w_sf, 16) || !aligned(w_gscale, 4)) return fail(MOEQ_EALIGN, "%s: scales misaligned", fn);
  if (x_dtype != MOEQ_BF16 && x_dtype != MOEQ_F16) return fail(MOEQ_EUNSUPPORTED, "%s: x dtype %d", fn, x_dtype);
  if (sf_layout != MOEQ_SF_ROWS && sf_layout != MOEQ_SF_KQUADS)
    return fail(MOEQ_EINVAL, "%s: sf_layout %d", fn, sf_layout);
  if (w_layout != MOEQ_W_ROWS && w_layout != MOEQ_W_TILED) return fail(MOEQ_EINVAL, "%s: w_layout %d", fn, w_layout);
  if (act != MOEQ_ACT_NONE && act != MOEQ_ACT_SILU_MUL && act != MOEQ_ACT_SILU_MUL_LIMIT)
    return fail(MOEQ_EUNSUPPORTED, "%s: act %d", fn, act);
  if (act == MOEQ_ACT_SILU_MUL_LIMIT && !(act_limit > 0.0f))
    return fail(MOEQ_EINVAL, "%s: act_limit %g must be > 0", fn, (double)act_limit);
  if (pair_weights) {
    if (act != MOEQ_ACT_NONE) return fail(MOEQ_EUNSUPPORTED, "%s: pair_weights need act NONE", fn);
    if (!sorted_pair_ids) return fail(MOEQ_EINVAL, "%s: pair_weights need sorted_pair_ids", fn);
    if (!aligned(pair_weights, 4)) return fail(MOEQ_EALIGN, "%s: pair_weights misaligned", fn);
  }
  if (out_dtype != MOEQ_F16 && out_dtype != MOEQ_BF16 && out_dtype != MOEQ_F32)
    return fail(MOEQ_EUNSUPPORTED, "%s: out dtype %d", fn, out_dtype);
  if (a_row == MOEQ_AROW_TOKEN && !sorted_pair_ids && rows_a < P)
    return fail(MOEQ_EINVAL, "%s: identity rows need rows_a >= P", fn);
  if (sched < MOEQ_SCHED_AUTO || sched > MOEQ_SCHED_PREFILL) return fail(MOEQ_EINVAL, "%s: sched %d", fn, sched);
  static_assert(moeq::kWorkQueueInts == MOEQ_WORK_QUEUE_INTS, "header and library agree");
  if (work_queue && !aligned(work_queue, 4)) return fail(MOEQ_EALIGN, "%s: work_queue misaligned", fn);
  moeq::GroupedArgs g = make_args(expert_offsets, sorted_pair_ids, rows_a, a_row, P, topk, E, N, K,
                                  act != MOEQ_ACT_NONE, out_dtype, out, sched);
  g.queue = work_queue;
  if (act == MOEQ_ACT_SILU_MUL_LIMIT) g.act_limit = act_limit;
  g.pair_weights = pair_weights;
  g.x_f16 = x_dtype == MOEQ_F16 ? 1 : 0;
  g.sf_quads = sf_layout == MOEQ_SF_KQUADS ? 1 : 0;
  g.w_tiled = w_layout == MOEQ_W_TILED ? 1 : 0;
  return hip_status(moeq::launch_gemm_nvfp4(g, static_cast<const uint16_t*>(x), w, w_sf, w_gscale,
                                            (hipStream_t)stream),
                    fn);
}

moeq_status moe_scatter_combine(const void* y, moeq_dtype y_dtype, const int32_t* pair_to_sorted,
                                const float* topk_weights, int64_t T, int32_t topk, int64_t N,
                                moeq_dtype out_dtype, void* out, void* stream) {
  const char* fn = "moe_scatter_combine";
  if (T < 0 || T >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: T=%lld outside [0, 2^31)", fn, (long long)T);
  if (topk < 1 || topk > kMaxTopk) return fail(MOEQ_EINVAL, "%s: topk=%d outside [1, %d]", fn, topk, kMaxTopk);
  if (N <= 0 || N > (1 << 24)) return fail(MOEQ_EINVAL, "%s: N=%lld out of range", fn, (long long)N);
  if (N % 8 != 0) return fail(MOEQ_EALIGN, "%s: N=%lld must be a multiple of 8", fn, (long long)N);
  if (T * (int64_t)topk >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: T*topk too large", fn);
  if (y_dtype != MOEQ_F16 && y_dtype != MOEQ_BF16 && y_dtype != MOEQ_F32)
    return fail(MOEQ_EUNSUPPORTED, "%s: y dtype %d", fn, y_dtype);
  if (out_dtype != MOEQ_F16 && out_dtype != MOEQ_BF16 && out_dtype != MOEQ_F32)
    return fail(MOEQ_EUNSUPPORTED, "%s: out dtype %d", fn, out_dtype);
  if (T > 0 && (!y || !pair_to_sorted || !topk_weights || !out)) return fail(MOEQ_EINVAL, "%s: null pointer", fn);
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(pair_to_sorted, 4) || !aligned(topk_weights, 4))
    return fail(MOEQ_EALIGN, "%s: pointers misaligned", fn);
  return hip_status(moeq::launch_combine(y, (int)y_dtype, pair_to_sorted, topk_weights, (int)T, topk,
                                         (int)N, T * (int64_t)topk, (int)out_dtype, out,
                                         (hipStream_t)stream),
                    fn);
}

moeq_status moe_sum_pairs(const void* y_pairs, moeq_dtype y_dtype, const int32_t* pair_to_sorted, int64_t T,
                          int32_t topk, int64_t N, moeq_dtype out_dtype, void* out, void* stream) {
  const char* fn = "moe_sum_pairs";
  if (T < 0 || T >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: T=%lld outside [0, 2^31)", fn, (long long)T);
  if (topk < 1 || topk > kMaxTopk) return fail(MOEQ_EINVAL, "%s: topk=%d outside [1, %d]", fn, topk, kMaxTopk);
  if (N <= 0 || N > (1 << 24)) return fail(MOEQ_EINVAL, "%s: N=%lld out of range", fn, (long long)N);
  if (N % 8 != 0) return fail(MOEQ_EALIGN, "%s: N=%lld must be a multiple of 8", fn, (long long)N);
  if (T * (int64_t)topk >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: T*topk too large", fn);
  if (y_dtype != MOEQ_F16 && y_dtype != MOEQ_BF16 && y_dtype != MOEQ_F32)
    return fail(MOEQ_EUNSUPPORTED, "%s: y dtype %d", fn, y_dtype);
  if (out_dtype != MOEQ_F16 && out_dtype != MOEQ_BF16 && out_dtype != MOEQ_F32)
    return fail(MOEQ_EUNSUPPORTED, "%s: out dtype %d", fn, out_dtype);
  if (T > 0 && (!y_pairs || !pair_to_sorted || !out)) return fail(MOEQ_EINVAL, "%s: null pointer", fn);
  if (!aligned(y_pairs, 16) || !aligned(out, 16) || !aligned(pair_to_sorted, 4))
    return fail(MOEQ_EALIGN, "%s: pointers misaligned", fn);
  return hip_status(moeq::launch_combine(y_pairs, (int)y_dtype, pair_to_sorted, nullptr, (int)T, topk, (int)N,
                                         T * (int64_t)topk, (int)out_dtype, out, (hipStream_t)stream),
                    fn);
}

moeq_status moe_cast_bf16_to_f16(const uint16_t* x, int64_t n, uint16_t* y, void* stream) {
  const char* fn = "moe_cast_bf16_to_f16";
  if (n < 0 || n >= (int64_t(1) << 40)) return fail(MOEQ_EINVAL, "%s: n=%lld out of range", fn, (long long)n);
  if (n % 8 != 0) return fail(MOEQ_EALIGN, "%s: n=%lld must be a multiple of 8", fn, (long long)n);
  if (n > 0 && (!x || !y)) return fail(MOEQ_EINVAL, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(MOEQ_EALIGN, "%s: pointers must be 16-byte aligned", fn);
  const uintptr_t a = (uintptr_t)x, b = (uintptr_t)y, nb = (uintptr_t)(2 * n);
  if (n > 0 && a != b && a < b + nb && b < a + nb)
    return fail(MOEQ_EINVAL, "%s: x and y overlap (only exact in-place is allowed)", fn);
  return hip_status(moeq::launch_cast_bf16_f16(x, n, y, device_cus(), (hipStream_t)stream), fn);
}

moeq_status moe_quantize_int4(const void* x, moeq_dtype x_dtype, int64_t rows, int64_t K, uint8_t* q,
                              float* scale, void* stream) {
  const char* fn = "moe_quantize_int4";
  if (rows < 0 || rows >= (int64_t(1) << 31)) return fail(MOEQ_EINVAL, "%s: rows=%lld out of range", fn, (long long)rows);
  if (K <= 0 || K > (1 << 24)) return fail(MOEQ_EINVAL, "%s: K=%lld out of range", fn, (long long)K);
  if (K % 16 != 0) return fail(MOEQ_EALIGN, "%s: K=%lld must be a multiple of 16", fn, (long long)K);
  if (x_dtype != MOEQ_F16 && x_dtype != MOEQ_BF16 && x_dtype != MOEQ_F32)
    return fail(MOEQ_EUNSUPPORTED, "%s: x dtype %d", fn, x_dtype);
  if (rows > 0 && (!x || !q || !scale)) return fail(MOEQ_EINVAL, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return fail(MOEQ_EALIGN, "%s: pointers misaligned", fn);
  return hip_status(moeq::launch_quant_int4(x, (int)x_dtype, rows, (int)K, q, scale, device_cus(), (hipStream_t)stream),
                    fn);
}

moeq_status moe_nvfp4_repack(const uint8_t* w_in, const uint8_t* sf_in, int64_t E, int64_t N, int64_t K,
                             int32_t swap_halves, moeq_w_layout w_out_layout, moeq_sf_layout out_layout,
                             uint8_t* w_out, uint8_t* sf_out, void* stream) {
  const char* fn = "moe_nvfp4_repack";
  if (E < 1 || E > kMaxE) return fail(MOEQ_EINVAL, "%s: E=%lld outside [1, %d]", fn, (long long)E, kMaxE);
  if (N <= 0 || K <= 0 || N > (1 << 20) || K > (1 << 17))
    return fail(MOEQ_EINVAL, "%s: N=%lld K=%lld out of range", fn, (long long)N, (long long)K);
  if (N * K >= (int64_t(1) << 36)) return fail(MOEQ_EINVAL, "%s: N*K=%lld too large", fn, (long long)(N * K));
  if (N % 128 != 0 || K % 64 != 0)
    return fail(MOEQ_EALIGN, "%s: N=%lld must be a multiple of 128 and K=%lld of 64 (128x4 scale tiles)", fn,
                (long long)N, (long long)K);
  if (swap_halves != 0 && swap_halves != 1) return fail(MOEQ_EINVAL, "%s: swap_halves=%d", fn, swap_halves);
  if (out_layout != MOEQ_SF_ROWS && out_layout != MOEQ_SF_KQUADS)
    return fail(MOEQ_EINVAL, "%s: out_layout %d", fn, out_layout);
  if (w_out_layout != MOEQ_W_ROWS && w_out_layout != MOEQ_W_TILED)
    return fail(MOEQ_EINVAL, "%s: w_out_layout %d", fn, w_out_layout);
  if (!w_in || !sf_in || !w_out || !sf_out) return fail(MOEQ_EINVAL, "%s: null pointer", fn);
  if (!aligned(w_in, 16) || !aligned(sf_in, 16) || !aligned(w_out, 16) || !aligned(sf_out, 16))
    return fail(MOEQ_EALIGN, "%s: pointers must be 16-byte aligned", fn);
  const uintptr_t wb = (uintptr_t)(E * N * (K / 2)), sb = (uintptr_t)(E * N * (K / 16));
  auto overlap = [](const void* a, uintptr_t na, const void* b, uintptr_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  if (overlap(w_out, wb, w_in, wb) || overlap(w_out, wb, sf_in, sb) || overlap(w_out, wb, sf_out, sb) ||
      overlap(sf_out, sb, w_in, wb) || overlap(sf_out, sb, sf_in, sb))
    return fail(MOEQ_EINVAL, "%s: an output overlaps an input or the other output (no in-place repack)", fn);
  return hip_status(moeq::launch_repack_nvfp4(w_in, sf_in, E, N, K, swap_halves, w_out_layout == MOEQ_W_TILED,
                                              out_layout == MOEQ_SF_KQUADS,
                                              w_out, sf_out,
                                              (hipStream_t)stream),
                    fn);
}

}  // extern "C"
