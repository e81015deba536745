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

constexpr int kExpBlock = 64;   // experts per logits block (one per lane)
constexpr int kHStage = 16;     // h values per LDS stage

// part[hs][t][e] = sum over h in slice hs of x[t,h] * W[h,e], float64.
// grid (E/64, ceil(T/TB), hsplit), 256 threads.  Lane l owns expert
// 64*blockIdx.x + l and keeps TB token sums in registers; wave w sums a
// quarter of the block's h slice (x staged in LDS already widened to
// float64); the four wave sums meet in LDS, added in wave order.
template <int TB>
__global__ __launch_bounds__(256) void route_logits_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                           const float* __restrict__ W, int E, int hsplit,
                                                           double* __restrict__ part) {
  __shared__ double xs[4][kHStage][TB];
  __shared__ double red[4][TB][kExpBlock];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * kExpBlock + lane;
  const int t0 = blockIdx.y * TB;
  const int hlen = H / hsplit;
  const int hw = hlen / 4;
  const int h0 = blockIdx.z * hlen + wave * hw;
  double acc[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) acc[i] = 0.0;
  const bool live = e < E;
  const int ec = live ? e : 0;

  for (int hc = h0; hc < h0 + hw; hc += kHStage) {
    // each wave stages its own x[t0..t0+TB)[hc..hc+16) (one element per lane per pass)
    for (int i = lane; i < TB * kHStage; i += 64) {
      const int tt = i / kHStage, hh = i % kHStage;
      const int t = t0 + tt;
      xs[wave][hh][tt] = (t < T) ? static_cast<double>(bf16_bits_to_float(x[static_cast<size_t>(t) * H + hc + hh])) : 0.0;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll 4
    for (int hh = 0; hh < kHStage; ++hh) {
      const double w = static_cast<double>(W[static_cast<size_t>(hc + hh) * E + ec]);
#pragma unroll
      for (int i = 0; i < TB; ++i) acc[i] = fma(xs[wave][hh][i], w, acc[i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
#pragma unroll
  for (int i = 0; i < TB; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  for (int i = wave; i < TB; i += 4) {
    const int t = t0 + i;
    if (t < T && live) {
      const double z = ((red[0][i][lane] + red[1][i][lane]) + red[2][i][lane]) + red[3][i][lane];
      part[(static_cast<size_t>(blockIdx.z) * T + t) * E + e] = z;
    }
  }
}

// TPB tokens per block of 256 threads.  Thread e sums the hsplit partial
// logits of expert e (fixed order) and writes s = sqrt(softplus(z)) and the
// selection key s + bias to LDS; then wave w runs the top-k of token w: k
// rounds of a wave-wide argmax over (key descending, expert id ascending),
// and the weights from the unbiased s.
template <int TPB>
__global__ __launch_bounds__(256) void route_topk_kernel(const double* __restrict__ part, int T, int E, int hsplit,
                                                         const float* __restrict__ bias, int k, float scale,
                                                         int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ double s_key[TPB][256];
  __shared__ double s_sc[TPB][256];
  const int e = threadIdx.x;
  const int tb = blockIdx.x * TPB;
  if (e < E) {
    const double b = bias ? static_cast<double>(bias[e]) : 0.0;
#pragma unroll
    for (int q = 0; q < TPB; ++q) {
      const int t = tb + q;
      if (t >= T) break;
      double z = 0.0;
      const double* pp = part + static_cast<size_t>(t) * E + e;
      const size_t stride = static_cast<size_t>(T) * E;
      int hs = 0;
      for (; hs + 8 <= hsplit; hs += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pp[(hs + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) z += v[u];
      }
      for (; hs < hsplit; ++hs) z += pp[hs * stride];
      const double sc = sqrt(fmax(z, 0.0) + log1p(exp(-fabs(z))));
      s_sc[q][e] = sc;
      s_key[q][e] = sc + b;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  if (q >= TPB) return;
  const int t = tb + q;
  if (t >= T) return;
  double key[4], sc[4];
  bool live[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ee = lane + 64 * u;
    live[u] = ee < E;
    key[u] = live[u] ? s_key[q][ee] : -INFINITY;
    sc[u] = live[u] ? s_sc[q][ee] : 0.0;
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
    for (int u = 0; u < 4; ++u) {
      const int ee = lane + 64 * u;
      if (live[u] && (key[u] > bk || (key[u] == bk && ee < be))) {
        bk = key[u];
        be = ee;
        bs = sc[u];
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
    for (int u = 0; u < 4; ++u)
      if (be == lane + 64 * u) live[u] = false;
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

inline int route_tb(int T) { return T <= 256 ? 8 : 32; }

// Number of h slices of the logits: enough blocks to cover the chip while
// every wave keeps at least one LDS stage of h; always a divisor of H/64.
int route_hsplit(int T, int H) {
  const int ntb = (T + route_tb(T) - 1) / route_tb(T);
  const int blocks = ntb * 4;  // E = 256 -> 4 expert blocks
  const int max_split = H / (4 * kHStage);
  int hs = 1;
  while (hs * 2 <= max_split && (max_split % (hs * 2)) == 0 && blocks * hs * 2 <= 512) hs *= 2;
  return hs;
}

hipError_t launch_route_learned(const uint16_t* x, int T, int H, const float* w, const float* bias, int E, int k,
                                float scale, int32_t* ids, float* weights, double* part, hipStream_t s) {
  const int hs = route_hsplit(T, H);
  const int tb = route_tb(T);
  dim3 g1((E + kExpBlock - 1) / kExpBlock, (T + tb - 1) / tb, hs);
  if (tb == 8) route_logits_kernel<8><<<g1, 256, 0, s>>>(x, T, H, w, E, hs, part);
  else route_logits_kernel<32><<<g1, 256, 0, s>>>(x, T, H, w, E, hs, part);
  if (T <= 256) route_topk_kernel<1><<<T, 256, 0, s>>>(part, T, E, hs, bias, k, scale, ids, weights);
  else route_topk_kernel<4><<<(T + 3) / 4, 256, 0, s>>>(part, T, E, hs, bias, k, scale, ids, weights);
  return hipGetLastError();
}

hipError_t launch_route_hash(const int32_t* tok, int T, const int32_t* table, int V, int k, float scale,
                             int32_t* ids, float* weights, hipStream_t s) {
  route_hash_kernel<<<(T + 255) / 256, 256, 0, s>>>(tok, T, table, V, k, scale / static_cast<float>(k), ids, weights);
  return hipGetLastError();
}

}  // namespace moe
