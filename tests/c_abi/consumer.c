/* A plain C99 program that uses the library through include/moeq.h only:
 * no Python, no PyTorch.  It shows that the boundary needs nothing beyond
 * the header, the shared library and the HIP runtime.
 *
 *   moeq_consumer host
 *       Host-only calls: the ABI version, route-prep workspace sizes, and
 *       argument checks that the library rejects before any device work.
 *       One "key value ..." line each.
 *   moeq_consumer gpu DIR
 *       One W4A4 MoE layer step on device 0, on inputs read from DIR:
 *       route prep -> INT4 grouped GEMM (activation rows gathered by token,
 *       act NONE, f32 out) -> top-k weighted combine (f32).  DIR holds
 *       meta.txt ("T topk E N K") and the raw little-endian arrays
 *       topk_ids.bin (int32 [T][topk]), a.bin (uint8 [T][K/2]),
 *       a_scale.bin (f32 [T]), w.bin (uint8 [E][N][K/2]), w_scale.bin
 *       (f32 [E][N]) and topk_weights.bin (f32 [T][topk]).  It writes
 *       offsets.bin, sorted.bin, p2s.bin, n_invalid.bin (int32), y.bin
 *       (f32 [T*topk][N], rows past the routed ones untouched zeros) and
 *       out.bin (f32 [T][N]) to DIR.
 * Exit status 0 on success; otherwise a message on stderr. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moeq.h"

static int fail_hip(const char* what, hipError_t e) {
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 1;
}

static int fail_moeq(const char* what, moeq_status s) {
  fprintf(stderr, "%s: status %d (%s)\n", what, (int)s, moeq_last_error());
  return 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  size_t put = fwrite(p, 1, bytes, f);
  fclose(f);
  return put != bytes;
}

/* Host-only checks.  Every rejected call below fails a documented argument
 * check, which the library applies before touching the device; the
 * pointers passed are never dereferenced. */
static int run_host(void) {
  static int32_t ids[64] __attribute__((aligned(16)));
  static unsigned char buf[4096] __attribute__((aligned(16)));
  printf("abi %d\n", (int)moeq_abi_version());
  printf("ws 64 2 4 %zu\n", moe_route_prep_workspace_bytes(64, 2, 4));
  printf("ws 8192 2 8 %zu\n", moe_route_prep_workspace_bytes(8192, 2, 8));
  printf("ws 4096 8 256 %zu\n", moe_route_prep_workspace_bytes(4096, 8, 256));
  /* null topk_ids with T > 0 */
  moeq_status s = moe_route_prep(NULL, 4, 2, 4, (int32_t*)buf, (int32_t*)buf, (int32_t*)buf,
                                 (int32_t*)buf, NULL, 0, NULL);
  printf("route_null %d\n", (int)s);
  /* E outside [1, 1024] */
  s = moe_route_prep(ids, 4, 2, 0, (int32_t*)buf, (int32_t*)buf, (int32_t*)buf, (int32_t*)buf, NULL, 0,
                     NULL);
  printf("route_e0 %d\n", (int)s);
  /* INT4: N not a multiple of 32 */
  s = grouped_gemm_qint4(buf, (const float*)buf, 8, MOEQ_AROW_TOKEN, buf, (const float*)buf, ids, ids, 8, 2, 4,
                         48, 256, MOEQ_ACT_NONE, MOEQ_F32, buf, MOEQ_SCHED_AUTO, NULL);
  printf("int4_n48 %d\n", (int)s);
  /* INT4: the streaming schedule needs K % 256 == 0 */
  s = grouped_gemm_qint4(buf, (const float*)buf, 8, MOEQ_AROW_TOKEN, buf, (const float*)buf, ids, ids, 8, 2, 4,
                         64, 384, MOEQ_ACT_NONE, MOEQ_F32, buf, MOEQ_SCHED_DECODE, NULL);
  printf("int4_decode_k384 %d\n", (int)s);
  /* INT4: K at the int32 accumulator's limit */
  s = grouped_gemm_qint4(buf, (const float*)buf, 8, MOEQ_AROW_TOKEN, buf, (const float*)buf, ids, ids, 8, 2, 4,
                         64, 131072, MOEQ_ACT_NONE, MOEQ_F32, buf, MOEQ_SCHED_AUTO, NULL);
  printf("int4_k131072 %d\n", (int)s);
  /* T*topk beyond int64: T is rejected before the product is formed */
  const int64_t huge = (int64_t)1 << 62;
  printf("ws_huge %zu\n", moe_route_prep_workspace_bytes(huge, 4, 256));
  s = moe_route_prep(ids, huge, 4, 4, (int32_t*)buf, (int32_t*)buf, (int32_t*)buf, (int32_t*)buf, NULL, 0, NULL);
  printf("route_huge %d\n", (int)s);
  s = moe_route_prep_noalloc(ids, huge, 4, 4, (int32_t*)buf, (int32_t*)buf, (int32_t*)buf, (int32_t*)buf, NULL);
  printf("noalloc_huge %d\n", (int)s);
  s = moe_scatter_combine(buf, MOEQ_F32, ids, (const float*)buf, huge, 4, 64, MOEQ_F32, buf, NULL);
  printf("combine_huge %d\n", (int)s);
  s = moe_sum_pairs(buf, MOEQ_F32, ids, huge, 4, 64, MOEQ_F32, buf, NULL);
  printf("sum_pairs_huge %d\n", (int)s);
  /* FP8: N not a multiple of 128 */
  s = grouped_gemm_qfp8_block(buf, (const float*)buf, 8, MOEQ_AROW_TOKEN, buf, (const float*)buf, ids, ids, 8, 1,
                              1, 64, 256, MOEQ_BF16, buf, MOEQ_SCHED_AUTO, NULL);
  printf("fp8_n64 %d\n", (int)s);
  /* NVFP4: activations must be bf16 or f16 */
  s = grouped_gemm_qnvfp4(buf, MOEQ_F32, 8, MOEQ_AROW_TOKEN, buf, MOEQ_W_ROWS, buf, MOEQ_SF_ROWS,
                          (const float*)buf, ids, ids, 8, 2, 4, 64, 256, MOEQ_ACT_NONE, 0.0f, NULL, MOEQ_BF16, buf,
                          NULL, MOEQ_SCHED_AUTO, NULL);
  printf("nvfp4_x_f32 %d\n", (int)s);
  /* quantizer: K not a multiple of 16 */
  s = moe_quantize_int4(buf, MOEQ_F16, 8, 40, buf, (float*)buf, NULL);
  printf("quant_k40 %d\n", (int)s);
  /* repack: an output overlapping an input */
  s = moe_nvfp4_repack(buf, buf + 2048, 1, 128, 64, 0, MOEQ_W_ROWS, MOEQ_SF_ROWS, buf, buf + 3072, NULL);
  printf("repack_overlap %d\n", (int)s);
  /* cast: a partial overlap of x and y */
  s = moe_cast_bf16_to_f16((const uint16_t*)buf, 64, (uint16_t*)(buf + 16), NULL);
  printf("cast_overlap %d\n", (int)s);
  /* combine: N not a multiple of 8 */
  s = moe_scatter_combine(buf, MOEQ_F32, ids, (const float*)buf, 4, 2, 12, MOEQ_F32, buf, NULL);
  printf("combine_n12 %d\n", (int)s);
  printf("last_error %s\n", moeq_last_error());
  return 0;
}

static int run_gpu(const char* dir) {
  long long T, topk, E, N, K;
  char path[4096];
  snprintf(path, sizeof path, "%s/meta.txt", dir);
  FILE* f = fopen(path, "r");
  if (!f || fscanf(f, "%lld %lld %lld %lld %lld", &T, &topk, &E, &N, &K) != 5) {
    fprintf(stderr, "cannot read %s\n", path);
    if (f) fclose(f);
    return 1;
  }
  fclose(f);
  if (T < 1 || topk < 1 || E < 1 || N < 1 || K < 2 || T * topk >= (1LL << 31)) {
    fprintf(stderr, "bad sizes in %s\n", path);
    return 1;
  }
  const size_t P = (size_t)(T * topk);
  const size_t b_ids = P * 4, b_a = (size_t)T * (size_t)(K / 2), b_sa = (size_t)T * 4;
  const size_t b_w = (size_t)E * (size_t)N * (size_t)(K / 2), b_sw = (size_t)E * (size_t)N * 4;
  const size_t b_y = P * (size_t)N * 4, b_out = (size_t)T * (size_t)N * 4;
  void* h_ids = read_file(dir, "topk_ids.bin", b_ids);
  void* h_a = read_file(dir, "a.bin", b_a);
  void* h_sa = read_file(dir, "a_scale.bin", b_sa);
  void* h_w = read_file(dir, "w.bin", b_w);
  void* h_sw = read_file(dir, "w_scale.bin", b_sw);
  void* h_tw = read_file(dir, "topk_weights.bin", b_ids);
  if (!h_ids || !h_a || !h_sa || !h_w || !h_sw || !h_tw) {
    fprintf(stderr, "missing or short input file in %s\n", dir);
    return 1;
  }

  hipError_t e = hipSetDevice(0);
  if (e != hipSuccess) return fail_hip("hipSetDevice", e);
  const size_t ws = moe_route_prep_workspace_bytes(T, (int32_t)topk, (int32_t)E);
  void *d_ids, *d_a, *d_sa, *d_w, *d_sw, *d_tw, *d_off, *d_srt, *d_p2s, *d_inv, *d_y, *d_out, *d_ws = NULL;
  void** bufs[] = {&d_ids, &d_a, &d_sa, &d_w, &d_sw, &d_tw, &d_off, &d_srt, &d_p2s, &d_inv, &d_y, &d_out};
  const size_t sizes[] = {b_ids, b_a, b_sa, b_w, b_sw, b_ids, (size_t)(E + 1) * 4, b_ids, b_ids, 4, b_y, b_out};
  for (size_t i = 0; i < sizeof sizes / sizeof sizes[0]; ++i)
    if ((e = hipMalloc(bufs[i], sizes[i])) != hipSuccess) return fail_hip("hipMalloc", e);
  if (ws && (e = hipMalloc(&d_ws, ws)) != hipSuccess) return fail_hip("hipMalloc workspace", e);
  const void* srcs[] = {h_ids, h_a, h_sa, h_w, h_sw, h_tw};
  for (size_t i = 0; i < 6; ++i)
    if ((e = hipMemcpy(*bufs[i], srcs[i], sizes[i], hipMemcpyHostToDevice)) != hipSuccess)
      return fail_hip("hipMemcpy in", e);
  if ((e = hipMemset(d_y, 0, b_y)) != hipSuccess) return fail_hip("hipMemset", e);

  moeq_status s = moe_route_prep((const int32_t*)d_ids, T, (int32_t)topk, (int32_t)E, (int32_t*)d_off,
                                 (int32_t*)d_srt, (int32_t*)d_p2s, (int32_t*)d_inv, d_ws, ws, NULL);
  if (s != MOEQ_OK) return fail_moeq("moe_route_prep", s);
  s = grouped_gemm_qint4((const uint8_t*)d_a, (const float*)d_sa, T, MOEQ_AROW_TOKEN, (const uint8_t*)d_w,
                         (const float*)d_sw, (const int32_t*)d_off, (const int32_t*)d_srt, (int64_t)P,
                         (int32_t)topk, (int32_t)E, N, K, MOEQ_ACT_NONE, MOEQ_F32, d_y, MOEQ_SCHED_AUTO, NULL);
  if (s != MOEQ_OK) return fail_moeq("grouped_gemm_qint4", s);
  s = moe_scatter_combine(d_y, MOEQ_F32, (const int32_t*)d_p2s, (const float*)d_tw, T, (int32_t)topk, N, MOEQ_F32,
                          d_out, NULL);
  if (s != MOEQ_OK) return fail_moeq("moe_scatter_combine", s);
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail_hip("hipDeviceSynchronize", e);

  const char* names[] = {"offsets.bin", "sorted.bin", "p2s.bin", "n_invalid.bin", "y.bin", "out.bin"};
  void* outs[] = {d_off, d_srt, d_p2s, d_inv, d_y, d_out};
  const size_t out_sizes[] = {(size_t)(E + 1) * 4, b_ids, b_ids, 4, b_y, b_out};
  for (size_t i = 0; i < 6; ++i) {
    void* h = malloc(out_sizes[i]);
    if (!h) return 1;
    if ((e = hipMemcpy(h, outs[i], out_sizes[i], hipMemcpyDeviceToHost)) != hipSuccess)
      return fail_hip("hipMemcpy out", e);
    if (write_file(dir, names[i], h, out_sizes[i])) {
      fprintf(stderr, "cannot write %s/%s\n", dir, names[i]);
      return 1;
    }
    free(h);
  }
  for (size_t i = 0; i < sizeof sizes / sizeof sizes[0]; ++i) hipFree(*bufs[i]);
  if (d_ws) hipFree(d_ws);
  free(h_ids), free(h_a), free(h_sa), free(h_w), free(h_sw), free(h_tw);
  printf("gpu ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "host") == 0) return run_host();
  if (argc == 3 && strcmp(argv[1], "gpu") == 0) return run_gpu(argv[2]);
  fprintf(stderr, "usage: %s host | gpu DIR\n", argv[0]);
  return 2;
}
