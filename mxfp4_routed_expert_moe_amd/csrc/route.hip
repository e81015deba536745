// Router of the MoE layer: float64 logits, sqrt-softplus scores, wave-level
// top-k with a selection-only bias, normalised weights x route scale; or the
// token-id hash table.  ("Model techniques map -- DeepSeek-V4-Flash", Checked
// in its code, rows "Mixture of experts" and "Auxiliary-loss-free load
// balancing"; "DeepSeek-V4-Flash export design", Source configuration.)
//
// The logits accumulate in float64 so that the chosen ids do not depend on
// the summation order: a bf16 x float32 product is exact in float64 and the
// remaining rounding (~1e-16 relative) is far below the gaps between scores.
#include <math.h>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kTokTile = 32;  // tokens per logits block
constexpr int kHStage = 32;   // h values staged in LDS per step

// part[hs][t][e] = sum over h in slice hs of x[t,h] * W[h,e], float64.
// grid (ceil(T/32), hsplit), 256 threads: thread e owns expert e and keeps the
// 32 token sums in registers; x is staged in LDS already widened to float64.
__global__ __launch_bounds__(256) void route_logits_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                           const float* __restrict__ W, int E, int hsplit,
                                                           double* __restrict__ part) {
  __shared__ double xs[kHStage][kTokTile];
  const int e = threadIdx.x;
  const int t0 = blockIdx.x * kTokTile;
  const int hlen = H / hsplit;
  const int h0 = blockIdx.y * hlen;
  double acc[kTokTile];
#pragma unroll
  for (int i = 0; i < kTokTile; ++i) acc[i] = 0.0;

  for (int hc = h0; hc < h0 + hlen; hc += kHStage) {
    __syncthreads();
    for (int i = threadIdx.x; i < kTokTile * kHStage; i += 256) {
      const int tt = i / kHStage, hh = i % kHStage;
      const int t = t0 + tt;
      xs[hh][tt] = (t < T) ? static_cast<double>(bf16_bits_to_float(x[static_cast<size_t>(t) * H + hc + hh])) : 0.0;
    }
    __syncthreads();
    if (e < E) {
#pragma unroll 4
      for (int hh = 0; hh < kHStage; ++hh) {
        const double w = static_cast<double>(W[static_cast<size_t>(hc + hh) * E + e]);
#pragma unroll
        for (int i = 0; i < kTokTile; ++i) acc[i] = fma(xs[hh][i], w, acc[i]);
      }
    }
  }
  if (e < E) {
    for (int i = 0; i < kTokTile; ++i) {
      const int t = t0 + i;
      if (t < T) part[(static_cast<size_t>(blockIdx.y) * T + t) * E + e] = acc[i];
    }
  }
}

// One wave per token: z = sum of the hsplit partial sums (fixed order),
// s = sqrt(softplus(z)), key = s + bias, k rounds of a wave-wide argmax over
// (key descending, expert id ascending), then weights from the unbiased s.
__global__ __launch_bounds__(256) void route_topk_kernel(const double* __restrict__ part, int T, int E, int hsplit,
                                                         const float* __restrict__ bias, int k, float scale,
                                                         int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  double key[4], sc[4];
  bool live[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    live[q] = e < E;
    key[q] = -INFINITY;
    sc[q] = 0.0;
    if (live[q]) {
      double z = 0.0;
      for (int hs = 0; hs < hsplit; ++hs) z += part[(static_cast<size_t>(hs) * T + t) * E + e];
      const double sp = fmax(z, 0.0) + log1p(exp(-fabs(z)));
      sc[q] = sqrt(sp);
      key[q] = sc[q] + (bias ? static_cast<double>(bias[e]) : 0.0);
    }
  }
  int sel_id[8];
  double sel_s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel_id[j] = 0x7fffffff;
    sel_s[j] = 0.0;
    if (j >= k) continue;
    double bk = -INFINITY, bs = 0.0;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (live[q] && (key[q] > bk || (key[q] == bk && e < be))) {
        bk = key[q];
        be = e;
        bs = sc[q];
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ok = __shfl_xor(bk, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      const double os = __shfl_xor(bs, off, 64);
      if (ok > bk || (ok == bk && oe < be)) {
        bk = ok;
        be = oe;
        bs = os;
      }
    }
    sel_id[j] = be;
    sel_s[j] = bs;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (be == lane + 64 * q) live[q] = false;
  }
  if (lane == 0) {
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) sum += sel_s[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) continue;
      const bool ok = sel_id[j] != 0x7fffffff;
      ids[static_cast<size_t>(t) * k + j] = ok ? sel_id[j] : -1;
      weights[static_cast<size_t>(t) * k + j] = ok ? static_cast<float>(static_cast<double>(scale) * sel_s[j] / sum) : 0.0f;
    }
  }
}

__global__ __launch_bounds__(256) void route_hash_kernel(const int32_t* __restrict__ tok, int T,
                                                         const int32_t* __restrict__ table, int V, int k, float w,
                                                         int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int v = tok[t];
  const bool ok = v >= 0 && v < V;
  for (int j = 0; j < k; ++j) {
    ids[static_cast<size_t>(t) * k + j] = ok ? table[static_cast<size_t>(v) * k + j] : -1;
    weights[static_cast<size_t>(t) * k + j] = w;
  }
}

}  // namespace

// Number of h slices of the logits: enough blocks to cover the chip, each
// slice a multiple of the LDS stage and a divisor of H.
int route_hsplit(int T, int H) {
  const int ntb = (T + kTokTile - 1) / kTokTile;
  const int max_split = H / kHStage;
  int hs = 1;
  while (hs * 2 <= max_split && (max_split % (hs * 2)) == 0 && ntb * hs * 2 <= 512) hs *= 2;
  return hs;
}

hipError_t launch_route_learned(const uint16_t* x, int T, int H, const float* w, const float* bias, int E, int k,
                                float scale, int32_t* ids, float* weights, double* part, hipStream_t s) {
  const int hs = route_hsplit(T, H);
  dim3 g1((T + kTokTile - 1) / kTokTile, hs);
  route_logits_kernel<<<g1, 256, 0, s>>>(x, T, H, w, E, hs, part);
  route_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(part, T, E, hs, bias, k, scale, ids, weights);
  return hipGetLastError();
}

hipError_t launch_route_hash(const int32_t* tok, int T, const int32_t* table, int V, int k, float scale,
                             int32_t* ids, float* weights, hipStream_t s) {
  route_hash_kernel<<<(T + 255) / 256, 256, 0, s>>>(tok, T, table, V, k, scale / static_cast<float>(k), ids, weights);
  return hipGetLastError();
}

}  // namespace moe
