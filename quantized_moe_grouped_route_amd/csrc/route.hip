// Route / sort-by-expert preparation (megamoe_rm.cu's route_prep: pairs
// grouped by expert in ascending pair-id order, id -1 skipped; CUTLASS
// discussion #2855's [E+1] per-expert row-offset table).
//
// The pairs are cut into chunks of kChunk (one per workgroup thread).  The
// sorted position of a valid pair p with expert e is
//   offsets[e] + (pairs of e in earlier chunks) + (pairs of e earlier in the
//   same chunk),
// which is the pair's rank among all earlier pairs of its expert: the unique
// stable order.  Inside a chunk the rank is built per wave (ballots, one
// round per distinct expert, for E <= 16; otherwise a 64-step comparison
// with every lane's expert) plus the counts of earlier waves.  One chunk
// needs one workgroup:
//   * P <= kChunk: a single fused kernel counts, scans and scatters (with
//                  4 waves when P <= 256).
//   * otherwise:   route_count writes per-chunk counts to the workspace and
//                  route_scatter (one workgroup per chunk) derives every
//                  prefix it needs from them.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moeq {

// Device memory of moe_route_prep_noalloc: the per-chunk counts that
// route_count writes and route_scatter reads, in a fixed array instead of a
// caller's workspace.  Every GPU the library runs on holds its own copy
// until the process ends.  Host code must not pass `scratch` itself to a
// kernel (in host code it names a host-side stand-in); it uses the device
// address that static_scratch() looks up once per device.
static __device__ __align__(256) unsigned char scratch[kRouteNoallocScratchBytes];

namespace {

constexpr int kChunk = 1024;
constexpr int kWaves = kChunk / 64;

__device__ __forceinline__ bool valid_id(int e, int E) { return e >= 0 && e < E; }

// Rank of this lane's pair among earlier lanes of its wave with the same
// expert; the wave's count of each expert present goes to wcnt_w[e].
__device__ __forceinline__ int wave_rank(int e, bool valid, unsigned char* wcnt_w, int lane) {
  unsigned long long active = __ballot(valid);
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
  while (active) {
    const int leader = __ffsll((long long)active) - 1;
    const int le = __shfl(e, leader, 64);
    const bool mine = valid && e == le;
    const unsigned long long m = __ballot(mine);
    if (mine) rank = __popcll(m & lt);
    if (lane == leader) wcnt_w[le] = (unsigned char)__popcll(m);
    active &= ~m;
  }
  return rank;
}

// The same rank and counts by comparing the lane's expert with every lane's
// expert, read as a wave-uniform value: 64 steps whatever the number of
// distinct experts in the wave, where the ballot form takes one round (with
// a cross-lane shuffle) per distinct expert.  The first lane of each expert
// writes its count.
__device__ __forceinline__ int wave_rank_scan(int e, bool valid, unsigned char* wcnt_w, int lane) {
  const int key = valid ? e : -1;
  int rank = 0, cnt = 0;
#pragma unroll 16
  for (int j = 0; j < 64; ++j) {
    const int ej = __builtin_amdgcn_readlane(key, j);
    const int same = ej == key;
    rank += (j < lane) & same;
    cnt += same;
  }
  if (valid && rank == 0) wcnt_w[e] = (unsigned char)cnt;
  return rank;
}

// Exclusive scan over E values held in LDS `v`, result in `out`; returns the
// total.  All NT threads of the workgroup must call.
template <int NT>
__device__ int block_exclusive_scan(const int* v, int* out, int E, int* scratch) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int per = (E + NT - 1) / NT;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += v[e];
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) scratch[wid] = incl;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < NW; ++w) {
      const int t = scratch[w];
      scratch[NW + w] = s;
      s += t;
    }
    scratch[2 * NW] = s;
  }
  __syncthreads();
  int run = incl - local + scratch[NW + wid];
  for (int e = e0; e < e1; ++e) {
    out[e] = run;
    run += v[e];
  }
  const int total = scratch[2 * NW];
  __syncthreads();
  return total;
}

// Per-chunk expert counts (+ invalid count in column E) -> ws[chunk][E+1].
__global__ __launch_bounds__(kChunk) void route_count(const int* __restrict__ ids, int P, int E,
                                                      int* __restrict__ ws) {
  extern __shared__ int sm[];
  int* cnt = sm;  // [E+1]
  for (int e = threadIdx.x; e <= E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  const int i = blockIdx.x * kChunk + threadIdx.x;
  if (i < P) {
    const int e = ids[i];
    if (valid_id(e, E)) atomicAdd(&cnt[e], 1);
    else if (e != -1) atomicAdd(&cnt[E], 1);
  }
  __syncthreads();
  int* dst = ws + (size_t)blockIdx.x * (E + 1);
  for (int e = threadIdx.x; e <= E; e += kChunk) dst[e] = cnt[e];
}

// FUSED: one workgroup of NT threads, P <= NT, counts computed here.
// Otherwise (NT == kChunk): workgroup b handles chunk b and reads all chunk
// counts from ws.
template <bool FUSED, int NT>
__global__ __launch_bounds__(NT) void route_scatter(const int* __restrict__ ids, int P, int E,
                                                        const int* __restrict__ ws,
                                                        int* __restrict__ offsets,
                                                        int* __restrict__ sorted_ids,
                                                        int* __restrict__ pair_to_sorted,
                                                        int* __restrict__ n_invalid) {
  extern __shared__ int sm[];
  int* base = sm;                        // [E+1] first sorted position of e in this chunk
  int* tot = base + (E + 1);             // [E+1] pairs per expert (+ invalid count at E)
  int* offs = tot + (E + 1);             // [E]   exclusive scan of tot
  constexpr int NW = NT / 64;
  static_assert(FUSED || NT == kChunk, "chunks of kChunk pairs");
  int* scratch = offs + E;               // [2*NW+1]
  unsigned char* wcnt = reinterpret_cast<unsigned char*>(scratch + 2 * NW + 1);  // [NW][E]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x, nchunks = (P + NT - 1) / NT;

  __shared__ int winv[NW];  // per wave: ids outside [0, E) other than -1
  for (int j = tid; j < NW * E; j += NT) wcnt[j] = 0;
  const int i = b * NT + tid;
  const int e = i < P ? ids[i] : -1;
  const bool valid = i < P && valid_id(e, E);
  __syncthreads();  // wcnt cleared

  // Rank in the wave and the wave's count of each expert (few experts: one
  // ballot round each; many: the fixed 64-step scan), and the wave's
  // invalid ids.
  const int r_wave = E <= 16 ? wave_rank(e, valid, wcnt + wid * E, lane)
                             : wave_rank_scan(e, valid, wcnt + wid * E, lane);
  const unsigned long long bad = __ballot(!valid && e != -1);
  if (lane == 0) winv[wid] = (int)__popcll(bad);
  __syncthreads();  // wcnt and winv complete

  if (FUSED) {
    // Expert counts as sums of the wave counts: no atomics on shared
    // counters (with one expert every pair would hit the same one).
    for (int x = tid; x < E; x += NT) {
      int sum = 0;
      for (int w = 0; w < NW; ++w) sum += wcnt[w * E + x];
      tot[x] = sum;
      base[x] = 0;  // no earlier chunks
    }
    if (tid == 0) {
      int sum = 0;
      for (int w = 0; w < NW; ++w) sum += winv[w];
      tot[E] = sum;
      base[E] = 0;
    }
  } else {
    // tot[x] = sum over all chunks, base[x] = sum over chunks before b.
    for (int x = tid; x <= E; x += NT) {
      int all = 0, before = 0;
      for (int c = 0; c < nchunks; ++c) {
        const int v = ws[(size_t)c * (E + 1) + x];
        all += v;
        before += c < b ? v : 0;
      }
      tot[x] = all;
      base[x] = before;
    }
  }
  __syncthreads();
  const int nvalid = block_exclusive_scan<NT>(tot, offs, E, scratch);
  for (int x = tid; x < E; x += NT) {
    base[x] += offs[x];
    if (b == 0) offsets[x] = offs[x];
  }
  if (b == 0 && tid == 0) {
    offsets[E] = nvalid;
    *n_invalid = tot[E];
  }

  // Rank inside the chunk: rank in the wave plus the counts of earlier waves.
  __syncthreads();
  if (i < P) {
    int pos = -1;
    if (valid) {
      int r = base[e] + r_wave;
      for (int w = 0; w < wid; ++w) r += wcnt[w * E + e];
      pos = r;
      sorted_ids[pos] = i;
    }
    pair_to_sorted[i] = pos;
  }
  // Positions past the valid pairs hold -1; each chunk clears its own range.
  if (i < P && i >= nvalid) sorted_ids[i] = -1;
}

}  // namespace

size_t route_workspace_bytes(int64_t P, int E) {
  if (P <= kChunk) return 0;
  const int64_t nchunks = (P + kChunk - 1) / kChunk;
  return (size_t)(nchunks * (E + 1) * sizeof(int));
}

// dynamic LDS of route_scatter with nw waves
static size_t route_lds_bytes(int E, int nw) {
  return sizeof(int) * (size_t)(2 * (E + 1) + E + 2 * nw + 1) + (size_t)nw * E;
}

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept per device.
static hipError_t static_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_route_noalloc(const int* ids, int P, int E, int* offsets, int* sorted_ids,
                                int* pair_to_sorted, int* n_invalid, hipStream_t stream) {
  if (route_workspace_bytes(P, E) > kRouteNoallocScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_route(ids, P, E, offsets, sorted_ids, pair_to_sorted, n_invalid, ws, stream);
}

hipError_t launch_route(const int* ids, int P, int E, int* offsets, int* sorted_ids,
                        int* pair_to_sorted, int* n_invalid, void* ws, hipStream_t stream) {
  // P <= 256 (decode batches): one 4-wave workgroup, so fewer waves meet
  // at each barrier; P <= kChunk: one 16-wave workgroup
  if (P <= 256) {
    hipLaunchKernelGGL((route_scatter<true, 256>), dim3(1), dim3(256), route_lds_bytes(E, 4), stream, ids, P, E,
                       (const int*)nullptr, offsets, sorted_ids, pair_to_sorted, n_invalid);
    return hipGetLastError();
  }
  const size_t lds = route_lds_bytes(E, kWaves);
  if (P <= kChunk) {
    hipLaunchKernelGGL((route_scatter<true, kChunk>), dim3(1), dim3(kChunk), lds, stream, ids, P, E,
                       (const int*)nullptr, offsets, sorted_ids, pair_to_sorted, n_invalid);
    return hipGetLastError();
  }
  const int nchunks = (P + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(route_count, dim3(nchunks), dim3(kChunk), sizeof(int) * (E + 1), stream, ids,
                     P, E, (int*)ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((route_scatter<false, kChunk>), dim3(nchunks), dim3(kChunk), lds, stream, ids, P, E,
                     (const int*)ws, offsets, sorted_ids, pair_to_sorted, n_invalid);
  return hipGetLastError();
}

}  // namespace moeq
