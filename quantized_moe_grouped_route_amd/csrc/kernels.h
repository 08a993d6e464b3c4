// Internal launchers (host side of each kernel file).  Arguments are
// validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq {

// Route prep.
size_t route_workspace_bytes(int64_t P, int E);
hipError_t launch_route(const int* ids, int P, int E, int* offsets, int* sorted_ids,
                        int* pair_to_sorted, int* n_invalid, void* ws, hipStream_t stream);
// Route prep with its per-chunk counts in the library's fixed device array
// (kRouteNoallocScratchBytes per device) instead of a caller's workspace.
constexpr size_t kRouteNoallocScratchBytes = size_t(1) << 20;
// Counters of the NVFP4 tiled schedule's work queue: one claim counter per
// XCD (8) and one count of finished workgroups.
constexpr int kWorkQueueInts = 16;
hipError_t launch_route_noalloc(const int* ids, int P, int E, int* offsets, int* sorted_ids,
                                int* pair_to_sorted, int* n_invalid, hipStream_t stream);

// Combine.  y_kind / out_kind are OutKind values.  tw == null: y holds
// pre-weighted rows in pair order (row t*topk + j), summed unweighted.
hipError_t launch_combine(const void* y, int y_kind, const int* p2s, const float* tw, int T,
                          int topk, int N, int64_t P, int out_kind, void* out, hipStream_t stream);

// Per-row symmetric INT4 quantization (x_kind: OutKind of the input).
hipError_t launch_quant_int4(const void* x, int x_kind, int64_t rows, int K, uint8_t* q, float* scale,
                             int num_cus, hipStream_t stream);

// Arguments common to the grouped GEMMs.
struct GroupedArgs {
  const int* offsets;       // [E+1]
  const int* sorted_ids;    // [P] or null (identity rows)
  int64_t rows_a;           // rows of the activation operand
  int a_sorted;             // 1: row = s, 0: row = sorted_ids[s] / topk
  int topk;
  int E;
  int64_t P;
  int N;                    // GEMM columns (2I for SILU_MUL)
  int K;
  int silu_mul;             // 1: write I = N/2 columns silu(gate) * up
  float act_limit;          // SwiGLU clamp (NVFP4 only); +inf: none
  const float* pair_weights;  // [P] or null: write w[p] * y to row p = sorted_ids[s] (NVFP4 only)
  int x_f16;                // NVFP4: activations are binary16 (else bf16)
  int sf_quads;             // NVFP4: scales [E][K/64][N][4] (else [E][N][K/16])
  int w_tiled;              // NVFP4: codes in 16-row x 64-K blocks (else [E][N][K/2])
  int out_kind;             // OutKind
  void* out;
  int sched;                // 0 auto, 1 decode, 2 prefill
  int* queue;               // NVFP4 tiled schedule: [kWorkQueueInts] zeroed counters, or null
  int num_cus;              // compute units of the current device
};

hipError_t launch_gemm_int4(const GroupedArgs& g, const uint8_t* a, const float* a_scale,
                            const uint8_t* w, const float* w_scale, hipStream_t stream);
hipError_t launch_gemm_fp8(const GroupedArgs& g, const uint8_t* a, const float* a_scale,
                           const uint8_t* w, const float* w_scale, hipStream_t stream);
hipError_t launch_gemm_nvfp4(const GroupedArgs& g, const uint16_t* x, const uint8_t* w,
                             const uint8_t* w_sf, const float* w_gscale, hipStream_t stream);

// bf16 -> binary16 (round to nearest even), n values, n % 8 == 0.
hipError_t launch_cast_bf16_f16(const uint16_t* x, int64_t n, uint16_t* y, int num_cus, hipStream_t stream);

// NVFP4 weight repack: megamoe_rm.cu layout (swizzled scales, optionally up
// rows first) -> grouped_gemm_qnvfp4's, E experts of N rows and K columns.
hipError_t launch_repack_nvfp4(const uint8_t* w_in, const uint8_t* sf_in, int64_t E, int64_t N, int64_t K,
                               int swap_halves, int w_tiled, int out_quads, uint8_t* w_out, uint8_t* sf_out,
                               hipStream_t stream);

}  // namespace moeq
