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

// part[hs][t][e] = sum over h in slice hs of x[t,h] * W[h,e], float64.
// grid (E/64, ceil(T/TB), hsplit), 256 threads.  Lane l owns expert
// 64*blockIdx.x + l and keeps TB token sums in registers; wave w sums a
// quarter of the block's h slice in chunks of HC: for each chunk it first
// issues every load (HC router weights per lane into registers, TB x values
// per lane into LDS widened to float64), then runs the HC x TB fused
// multiply-adds, so a chunk costs one memory round trip.  The four wave sums
// meet in LDS (reusing the x buffer), added in wave order.
template <int TB, int HC>
__global__ __launch_bounds__(256) void route_logits_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                           const float* __restrict__ W, int E, int hsplit,
                                                           double* __restrict__ part) {
  constexpr int kBuf = (HC > 64 ? HC : 64) * TB;
  __shared__ double buf[4][kBuf];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * kExpBlock + lane;
  const int t0 = blockIdx.y * TB;
  const int hw = H / hsplit / 4;
  const int h0 = blockIdx.z * (H / hsplit) + wave * hw;
  const bool live = e < E;
  const int ec = live ? e : 0;
  double* xs = buf[wave];  // [HC][TB]
  double acc[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) acc[i] = 0.0;

  for (int hc = h0; hc < h0 + hw; hc += HC) {
    float wv[HC];
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) wv[hh] = W[static_cast<size_t>(hc + hh) * E + ec];
    uint16_t xv[TB];
    const bool xl = lane < HC;
#pragma unroll
    for (int t = 0; t < TB; ++t)
      xv[t] = (xl && t0 + t < T) ? x[static_cast<size_t>(t0 + t) * H + hc + lane] : static_cast<uint16_t>(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (xl) {
#pragma unroll
      for (int t = 0; t < TB; ++t) xs[lane * TB + t] = static_cast<double>(bf16_bits_to_float(xv[t]));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
      const double w = static_cast<double>(wv[hh]);
#pragma unroll
      for (int i = 0; i < TB; ++i) acc[i] = fma(xs[hh * TB + i], w, acc[i]);
    }
  }
  __syncthreads();
  double* red = &buf[0][0];  // [4][TB][64]
#pragma unroll
  for (int i = 0; i < TB; ++i) red[(wave * TB + i) * 64 + lane] = acc[i];
  __syncthreads();
  for (int i = wave; i < TB; i += 4) {
    const int t = t0 + i;
    if (t < T && live) {
      const double z = ((red[(0 * TB + i) * 64 + lane] + red[(1 * TB + i) * 64 + lane]) +
                        red[(2 * TB + i) * 64 + lane]) + red[(3 * TB + i) * 64 + lane];
      part[(static_cast<size_t>(blockIdx.z) * T + t) * E + e] = z;
    }
  }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Many-token regime on the float64 matrix cores (v_mfma_f64_16x16x4_f64).
// part[hs][t][e] as above; grid (ceil(T/32), hsplit), 64 * E/64 threads
// (E a multiple of 64).  Wave w owns experts 64w .. 64w+63 of 32 tokens: two
// row tiles of 16 tokens x four column tiles of 16 experts, where column c of
// tile j is expert 64w + 4c + j, so one 16-byte load gives a lane its four
// tiles' router weights of one h.  The sum over h runs in chunks of 32: at
// step s of a chunk, the lanes of k group g (lane / 16) supply
// h = chunk + 8g + s for both operands (any assignment of h to (step, k) that
// A and B share gives the same sum), so a lane loads its token's 8
// consecutive x values with one 16-byte load and its experts' weights of
// 8 rows with eight.  Products of bf16 x and float32 weights are exact in
// float64.  Result layout of the instruction: lane l holds rows
// 4r + l / 16, r = 0..3, of column l % 16.
template <int MT>
__global__ __launch_bounds__(256) void route_logits_mfma_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                                const float* __restrict__ W, int E, int hsplit,
                                                                double* __restrict__ part) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * (16 * MT);
  const int hlen = H / hsplit;
  const int h0 = blockIdx.y * hlen + 8 * g;
  const int e0 = 64 * wave + 4 * c;
  const uint16_t* xr[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xr[m] = x + static_cast<size_t>(min(t0 + 16 * m + c, T - 1)) * H + h0;
  const float* wr = W + static_cast<size_t>(h0) * E + e0;

  f64x4 acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = f64x4{0.0, 0.0, 0.0, 0.0};

  u32x4 xv[2][MT];
  f32x4 wv[2][8];
  auto load = [&](int b, int hc) {
#pragma unroll
    for (int m = 0; m < MT; ++m) xv[b][m] = ld16(xr[m] + hc);
#pragma unroll
    for (int s = 0; s < 8; ++s) wv[b][s] = *reinterpret_cast<const f32x4*>(wr + static_cast<size_t>(hc + s) * E);
  };
  auto compute = [&](int b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      double a[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t word = xv[b][m][s >> 1];
        a[m] = static_cast<double>(__uint_as_float((s & 1) ? (word & 0xffff0000u) : (word << 16)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double bw = static_cast<double>(wv[b][s][j]);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[m], bw, acc[m][j], 0, 0, 0);
      }
    }
  };
  // Two register buffers: the loads of chunk n+1 are in flight while chunk n
  // is multiplied.
  load(0, 0);
  int hc = 0;
  for (; hc + 64 <= hlen; hc += 64) {
    load(1, hc + 32);
    compute(0);
    if (hc + 64 < hlen) load(0, hc + 64);
    compute(1);
  }
  if (hc < hlen) compute(0);

#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * m + 4 * r + g;
      if (t < T) {
        f64x4 v = {acc[m][0][r], acc[m][1][r], acc[m][2][r], acc[m][3][r]};
        *reinterpret_cast<f64x4*>(part + (static_cast<size_t>(blockIdx.y) * T + t) * E + e0) = v;
      }
    }
}

// One step of a wave arg-max: take the (key, id) of the lane that DPP
// control CTRL pairs with this one when it is larger, or equal with a lower
// id (the same order as the top-k).
// (ok, oe) precedes (bk, be) in the top-k order: larger key, or equal key and
// lower id.  Bitwise operators keep it branch-free (no exec-mask juggling).
__device__ __forceinline__ bool precedes(double ok, int oe, double bk, int be) {
  return (ok > bk) | ((ok == bk) & (oe < be));
}

// One step of a wave arg-max: take the (key, id) of the lane that DPP
// control CTRL pairs with this one when it precedes this lane's.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp_step(double& bk, int& be) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, bk);
  const uint32_t lo = __builtin_amdgcn_mov_dpp(static_cast<int>(bits), CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_mov_dpp(static_cast<int>(bits >> 32), CTRL, 0xF, 0xF, false);
  const int oe = __builtin_amdgcn_mov_dpp(be, CTRL, 0xF, 0xF, false);
  const double ok = __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
  const bool take = precedes(ok, oe, bk, be);
  bk = take ? ok : bk;
  be = take ? oe : be;
}

// Arg-max of (key descending, id ascending) over the 64 lanes; every lane
// gets the result.  Within each row of 16 lanes four DPP exchanges (lane ^ 1,
// lane ^ 2, then the half-row and row mirrors) leave the row's best in all its
// lanes; the four row results are then read as uniform values and compared.
// No LDS round trips, unlike a shuffle butterfly.
__device__ __forceinline__ void wave_argmax(double& bk, int& be) {
  argmax_dpp_step<0xB1>(bk, be);   // quad_perm [1,0,3,2]
  argmax_dpp_step<0x4E>(bk, be);   // quad_perm [2,3,0,1]
  argmax_dpp_step<0x141>(bk, be);  // row_half_mirror
  argmax_dpp_step<0x140>(bk, be);  // row_mirror
  const uint64_t bits = __builtin_bit_cast(uint64_t, bk);
  const uint32_t lo = static_cast<uint32_t>(bits), hi = static_cast<uint32_t>(bits >> 32);
  double rk = __builtin_bit_cast(double, (static_cast<uint64_t>(__builtin_amdgcn_readlane(hi, 0)) << 32) |
                                             static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, 0)));
  int re = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const double ok = __builtin_bit_cast(
        double, (static_cast<uint64_t>(__builtin_amdgcn_readlane(hi, 16 * r)) << 32) |
                    static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, 16 * r)));
    const int oe = __builtin_amdgcn_readlane(be, 16 * r);
    const bool take = precedes(ok, oe, rk, re);
    rk = take ? ok : rk;
    re = take ? oe : re;
  }
  bk = rk;
  be = re;
}

// TPB tokens per block of 256 * SPLIT threads.  The SPLIT threads of expert e
// sum interleaved subsets of its hsplit partial logits, which are then added
// in a fixed order; thread e writes s = sqrt(softplus(z)) and the
// selection key s + bias to LDS; then wave w runs the top-k of token w: k
// rounds of a wave-wide argmax over (key descending, expert id ascending),
// and the weights from the unbiased s of the chosen ids.
template <int TPB, int SPLIT>
__global__ __launch_bounds__(256 * SPLIT) void route_topk_kernel(const double* __restrict__ part, int T, int E,
                                                                 int hsplit, const float* __restrict__ bias, int k,
                                                                 float scale, int32_t* __restrict__ ids,
                                                                 float* __restrict__ weights) {
  __shared__ double s_key[TPB][256];
  __shared__ double s_sc[TPB][256];
  __shared__ double s_part[SPLIT][TPB][256];
  const int e = threadIdx.x & 255;
  const int qs = threadIdx.x >> 8;  // which of the SPLIT threads of expert e
  const int tb = blockIdx.x * TPB;
  const size_t stride = static_cast<size_t>(T) * E;
  if (e < E) {
#pragma unroll
    for (int q = 0; q < TPB; ++q) {
      const int t = tb + q;
      if (t >= T) break;
      // Slices qs, qs + SPLIT, ... in increasing order, eight loads in flight.
      const double* pp = part + static_cast<size_t>(qs) * stride + static_cast<size_t>(t) * E + e;
      const size_t step = static_cast<size_t>(SPLIT) * stride;
      const int cnt = qs < hsplit ? (hsplit - qs + SPLIT - 1) / SPLIT : 0;
      double z = 0.0;
      int i = 0;
      for (; i + 8 <= cnt; i += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pp[(i + u) * step];
#pragma unroll
        for (int u = 0; u < 8; ++u) z += v[u];
      }
      for (; i < cnt; ++i) z += pp[i * step];
      s_part[qs][q][e] = z;
    }
  }
  if (SPLIT > 1) __syncthreads();
  if (qs == 0 && e < E) {
    const double b = bias ? static_cast<double>(bias[e]) : 0.0;
#pragma unroll
    for (int q = 0; q < TPB; ++q) {
      const int t = tb + q;
      if (t >= T) break;
      double z = s_part[0][q][e];
#pragma unroll
      for (int r = 1; r < SPLIT; ++r) z += s_part[r][q][e];
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
  double key[4];
  bool live[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ee = lane + 64 * u;
    live[u] = ee < E;
    key[u] = live[u] ? s_key[q][ee] : -INFINITY;
  }
  int sel_id[8];
  double sel_s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel_id[j] = 0x7fffffff;
    sel_s[j] = 0.0;
    if (j >= k) continue;
    double bk = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ee = lane + 64 * u;
      const bool take = live[u] & precedes(key[u], ee, bk, be);
      bk = take ? key[u] : bk;
      be = take ? ee : be;
    }
    wave_argmax(bk, be);
    sel_id[j] = be;
    if (be != 0x7fffffff) sel_s[j] = s_sc[q][be];
#pragma unroll
    for (int u = 0; u < 4; ++u) live[u] = live[u] & (be != lane + 64 * u);
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

// Number of h slices of the vector kernel: enough blocks to cover the chip,
// with every wave's h range (H / hsplit / 4) either 16, 32 or a multiple of 64.
static int route_hsplit_vector(int T, int H) {
  const int ntb = (T + route_tb(T) - 1) / route_tb(T);
  const int blocks = ntb * 4;  // E = 256 -> 4 expert blocks
  int hs = 1;
  for (;;) {
    const int n = hs * 2;
    if ((H / 4) % n != 0 || blocks * n > 512) break;
    const int hw = H / 4 / n;
    if (!(hw == 16 || hw == 32 || hw % 64 == 0)) break;
    hs = n;
  }
  return hs;
}

constexpr int kMfmaTokens = 32;  // tokens per block of the matrix-core kernel

// Number of h slices of the matrix-core kernel: up to 1024 blocks (four
// resident per CU), every slice a multiple of 32.
static int route_hsplit_mfma(int T, int H) {
  const int ntb = (T + kMfmaTokens - 1) / kMfmaTokens;
  int hs = 1;
  while (ntb * hs * 2 <= 1024 && (H / (hs * 2)) % 32 == 0) hs *= 2;
  return hs;
}

// The matrix-core kernel takes many-token batches when E is a multiple of 64
// and the router weights are 16-byte aligned (its weight loads are 16 bytes).
static bool route_use_mfma(int T, int E, const float* w) {
  return T > 256 && E % 64 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0;
}

int route_hsplit(int T, int H) { return max(route_hsplit_vector(T, H), route_hsplit_mfma(T, H)); }

hipError_t launch_route_learned(const uint16_t* x, int T, int H, const float* w, const float* bias, int E, int k,
                                float scale, int32_t* ids, float* weights, double* part, hipStream_t s) {
  int hs;
  if (route_use_mfma(T, E, w)) {
    hs = route_hsplit_mfma(T, H);
    dim3 g1((T + kMfmaTokens - 1) / kMfmaTokens, hs);
    route_logits_mfma_kernel<kMfmaTokens / 16><<<g1, 64 * (E / 64), 0, s>>>(x, T, H, w, E, hs, part);
  } else {
    hs = route_hsplit_vector(T, H);
    const int tb = route_tb(T);
    const int hw = H / hs / 4;
    dim3 g1((E + kExpBlock - 1) / kExpBlock, (T + tb - 1) / tb, hs);
#define MOE_LOGITS(TB_, HC_) route_logits_kernel<TB_, HC_><<<g1, 256, 0, s>>>(x, T, H, w, E, hs, part)
    if (tb == 8) {
      if (hw == 16) MOE_LOGITS(8, 16);
      else if (hw == 32) MOE_LOGITS(8, 32);
      else MOE_LOGITS(8, 64);
    } else {
      MOE_LOGITS(32, 16);  // compute-bound regime: a short chunk keeps registers for the 32 token sums
    }
#undef MOE_LOGITS
  }
  // Few tokens: one token per block (many slices when very few: four threads
  // per expert share them).  Many tokens: four tokens per block.
  if (T <= 256 && hs >= 32) route_topk_kernel<1, 4><<<T, 1024, 0, s>>>(part, T, E, hs, bias, k, scale, ids, weights);
  else if (T <= 256) route_topk_kernel<1, 1><<<T, 256, 0, s>>>(part, T, E, hs, bias, k, scale, ids, weights);
  else route_topk_kernel<4, 1><<<(T + 3) / 4, 256, 0, s>>>(part, T, E, hs, bias, k, scale, ids, weights);
  return hipGetLastError();
}

hipError_t launch_route_hash(const int32_t* tok, int T, const int32_t* table, int V, int k, float scale,
                             int32_t* ids, float* weights, hipStream_t s) {
  route_hash_kernel<<<(T + 255) / 256, 256, 0, s>>>(tok, T, table, V, k, scale / static_cast<float>(k), ids, weights);
  return hipGetLastError();
}

}  // namespace moe
