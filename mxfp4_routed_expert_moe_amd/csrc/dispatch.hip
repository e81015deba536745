// Dispatch of the MoE layer: a stable counting sort of the (token, slot)
// pairs by expert, followed by the shared-expert group of every token in
// order.  The experts call of the DeepSeek-V4-Flash sparse block takes the
// flattened tokens together with the routed ids ("Model techniques map --
// DeepSeek-V4-Flash", row "Shared expert"); the row order chosen here,
// (expert, token, slot), makes every later step deterministic.
//
// Three kernels, no host synchronisation and no ordering atomics:
//  1. per chunk of 32 tokens: the rank of each pair among the earlier pairs
//     of the chunk with the same expert, and the chunk's per-expert counts;
//  2. per expert (one wave): exclusive scan of its counts over the chunks;
//  3. per chunk: exclusive scan of the expert totals -> offsets, then every
//     pair's row = offsets[e] + chunk base + rank, and the shared rows.
// Small batches (T * k <= 2048, E <= 256) take one single-block kernel with
// the same result (ranks from wave ballots and per-chunk prefix counts).
#include <atomic>
#include <mutex>

#include "moe_internal.h"

// Scratch of moe_dispatch_noalloc: the per-pair ranks and per-chunk counts
// that moe_dispatch keeps in its workspace argument, in a static device array
// instead (every GPU the library runs on holds its own copy until the process
// ends).  Host code never passes this name to a kernel: it is a host-side
// stand-in for the device symbol.  Its device address, per device, comes from
// hipGetSymbolAddress (dispatch_noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MOE_DISPATCH_NOALLOC_SCRATCH_BYTES];

namespace moe {

namespace {

constexpr int kChunk = 32;  // tokens per chunk

struct DispatchWs {
  int32_t* rank;   // [T*k]
  int32_t* cnt;    // [E][nch] counts, then exclusive chunk bases
  int32_t* total;  // [E]
};

__host__ __device__ inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

__host__ __device__ inline DispatchWs carve(void* ws, int T, int E, int k) {
  const int nch = (T + kChunk - 1) / kChunk;
  char* p = static_cast<char*>(ws);
  DispatchWs w;
  w.rank = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * static_cast<size_t>(T) * k);
  w.cnt = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * static_cast<size_t>(E) * nch);
  w.total = reinterpret_cast<int32_t*>(p);
  return w;
}

__global__ __launch_bounds__(256) void dispatch_rank_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                            int nch, DispatchWs w) {
  __shared__ int sid[kChunk * 8];
  __shared__ int hist[1024];
  const int c = blockIdx.x;
  const int t0 = c * kChunk;
  const int n = min(kChunk, T - t0) * k;
  for (int i = threadIdx.x; i < E; i += 256) hist[i] = 0;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int e = ids[static_cast<size_t>(t0) * k + i];
    sid[i] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 256) {
    const int e = sid[i];
    if (e < 0) continue;
    int r = 0;
    for (int j = 0; j < i; ++j) r += (sid[j] == e) ? 1 : 0;
    w.rank[static_cast<size_t>(t0) * k + i] = r;
    atomicAdd(&hist[e], 1);  // integer counts: the result does not depend on order
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += 256) w.cnt[static_cast<size_t>(i) * nch + c] = hist[i];
}

// grid E, 64 threads: exclusive scan of cnt[e][0..nch) in place, total[e].
__global__ __launch_bounds__(64) void dispatch_chunk_scan_kernel(int nch, DispatchWs w) {
  const int e = blockIdx.x;
  const int lane = threadIdx.x;
  int32_t* row = w.cnt + static_cast<size_t>(e) * nch;
  int carry = 0;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    const int v = c < nch ? row[c] : 0;
    const int incl = wave_incl_scan(v);
    if (c < nch) row[c] = carry + incl - v;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) w.total[e] = carry;
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                               int nch, DispatchWs w, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ row_token,
                                                               int32_t* __restrict__ slot_row) {
  __shared__ int off[1024];
  __shared__ int tmp[4];
  for (int i = threadIdx.x; i < E; i += 256) off[i] = w.total[i];
  __syncthreads();
  const int n_routed = block_excl_scan_256(off, E, tmp);
  const int c = blockIdx.x;
  if (c == 0) {
    for (int i = threadIdx.x; i < E; i += 256) offsets[i] = off[i];
    if (threadIdx.x == 0) {
      offsets[E] = n_routed;
      offsets[E + 1] = n_routed + T;
    }
  }
  const int t0 = c * kChunk;
  const int nt = min(kChunk, T - t0);
  for (int i = threadIdx.x; i < nt * k; i += 256) {
    const int t = t0 + i / k, j = i % k;
    const int e = ids[static_cast<size_t>(t0) * k + i];
    int32_t row = -1;
    if (e >= 0 && e < E) {
      row = off[e] + w.cnt[static_cast<size_t>(e) * nch + c] + w.rank[static_cast<size_t>(t0) * k + i];
      row_token[row] = t;
    }
    slot_row[static_cast<size_t>(t) * (k + 1) + j] = row;
  }
  for (int i = threadIdx.x; i < nt; i += 256) {
    const int t = t0 + i;
    row_token[n_routed + t] = t;
    slot_row[static_cast<size_t>(t) * (k + 1) + k] = n_routed + t;
  }
}

constexpr int kSmallPairs = 2048;
constexpr int kSmallExperts = 256;
constexpr int kSmallChunks = kSmallPairs / 64;

// One 1024-thread block, T * k <= 2048 pairs, E <= 256.  Pair i is handled by
// thread i mod 1024 and belongs to 64-pair chunk i / 64, one wave's worth.
// Its rank among the earlier pairs of its expert = (pairs of that expert in
// earlier chunks) + (lanes below it in its own chunk with the same expert).
// The second term comes from ballots: the wave repeatedly takes the expert of
// its lowest unmatched lane and matches all lanes holding it, so the loop runs
// once per distinct expert of the chunk.  The first lane of each match writes
// the chunk's count of that expert; per-expert prefix sums over the chunks
// then give the first term.  No atomics, no order-dependent step.
__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ row_token,
                                                              int32_t* __restrict__ slot_row) {
  __shared__ int cnt[kSmallExperts];
  __shared__ unsigned short pre[kSmallChunks][kSmallExperts];
  __shared__ int tmp[16];
  const int n = T * k;
  const int nch = (n + 63) / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < nch * kSmallExperts; i += 1024) (&pre[0][0])[i] = 0;
  __syncthreads();

  int ex[2], rk[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int i = tid + 1024 * p;
    const int c = wave + 16 * p;
    ex[p] = -1;
    rk[p] = 0;
    if (c >= nch) continue;  // wave-uniform
    int e = i < n ? ids[i] : -1;
    if (e >= E) e = -1;
    ex[p] = e;
    // Branch-free body: every lane evaluates the match; only the matched
    // lanes keep its rank and count.
    uint64_t todo = __ballot(e >= 0);
    int r = 0, cm = 0;
    while (todo) {
      const int leader = __builtin_ctzll(todo);
      const int el = __builtin_amdgcn_readlane(e, leader);
      const uint64_t m = __ballot(e == el);
      const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
      const bool mine = e == el;
      r = mine ? below : r;
      cm = mine ? __builtin_popcountll(m) : cm;
      todo &= ~m;
    }
    rk[p] = r;
    if (e >= 0 && r == 0) pre[c][e] = static_cast<unsigned short>(cm);
  }
  __syncthreads();
  if (tid < E) {
    int run = 0;
    for (int c = 0; c < nch; ++c) {
      const int v = pre[c][tid];
      pre[c][tid] = static_cast<unsigned short>(run);
      run += v;
    }
    cnt[tid] = run;
  }
  __syncthreads();
  const int n_routed = block_excl_scan_1024(cnt, E, tmp);
  for (int i = tid; i < E; i += 1024) offsets[i] = cnt[i];
  if (tid == 0) {
    offsets[E] = n_routed;
    offsets[E + 1] = n_routed + T;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int i = tid + 1024 * p;
    if (i >= n) continue;
    const int t = i / k, j = i - t * k;
    int32_t row = -1;
    if (ex[p] >= 0) {
      row = cnt[ex[p]] + pre[wave + 16 * p][ex[p]] + rk[p];
      row_token[row] = t;
    }
    slot_row[static_cast<size_t>(t) * (k + 1) + j] = row;
  }
  for (int t = tid; t < T; t += 1024) {
    row_token[n_routed + t] = t;
    slot_row[static_cast<size_t>(t) * (k + 1) + k] = n_routed + t;
  }
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of `scratch` on the device that owns stream s (the
// current device for the null stream), looked up once per device with that
// device current and kept for later calls.
hipError_t dispatch_noalloc_scratch(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = 0;
      e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      const hipError_t eg = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return e;
      if (eg != hipSuccess) return eg;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

size_t dispatch_ws_bytes(int T, int E, int k) {
  const int nch = (T + kChunk - 1) / kChunk;
  return align256(sizeof(int32_t) * static_cast<size_t>(T) * k) +
         align256(sizeof(int32_t) * static_cast<size_t>(E) * nch) + align256(sizeof(int32_t) * static_cast<size_t>(E));
}

hipError_t launch_dispatch(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* row_token,
                           int32_t* slot_row, void* ws, hipStream_t s) {
  if (T * k <= kSmallPairs && E <= kSmallExperts) {
    dispatch_small_kernel<<<1, 1024, 0, s>>>(ids, T, E, k, offsets, row_token, slot_row);
    return hipGetLastError();
  }
  const int nch = (T + kChunk - 1) / kChunk;
  DispatchWs w = carve(ws, T, E, k);
  dispatch_rank_kernel<<<nch, 256, 0, s>>>(ids, T, E, k, nch, w);
  dispatch_chunk_scan_kernel<<<E, 64, 0, s>>>(nch, w);
  dispatch_scatter_kernel<<<nch, 256, 0, s>>>(ids, T, E, k, nch, w, offsets, row_token, slot_row);
  return hipGetLastError();
}

hipError_t launch_dispatch_noalloc(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* row_token,
                                   int32_t* slot_row, hipStream_t s) {
  // Every word of the scratch the kernels read is written earlier in the same
  // call, so nothing needs clearing between calls.
  void* ws = nullptr;
  const hipError_t e = dispatch_noalloc_scratch(s, &ws);
  if (e != hipSuccess) return e;
  return launch_dispatch(ids, T, E, k, offsets, row_token, slot_row, ws, s);
}

}  // namespace moe
