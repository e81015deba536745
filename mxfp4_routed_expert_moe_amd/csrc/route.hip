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

#include <algorithm>
#include <cmath>

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

// Number of h slices of the float64 logits over a list of n tokens, whose
// partial sums [hs][n][E] must fit the region_bytes the caller set aside:
// up to 32 (parallelism for short lists), fewer for long ones.  Evaluated
// the same way by the logits and the top-k kernels of the list.
__host__ __device__ inline int list_hsplit(int n, int E, int H, size_t region_bytes) {
  int hs = 32;
  while (hs > 1 && (static_cast<size_t>(hs) * n * E * sizeof(double) > region_bytes || (H / hs) % 32 != 0)) hs >>= 1;
  return hs;
}

// The float64 logits on the matrix cores (v_mfma_f64_16x16x4_f64) of the
// tokens list[0 .. *count) (the tokens whose selection the bf16 matrix-core
// logits could not decide): part[hs][i][E] for list position i, hs =
// list_hsplit(*count, ...).  A 1-D grid of 64 * E/64-thread blocks (E a
// multiple of 64) walks the units (token block of 16 MT, slice) from
// blockIdx.x in steps of gridDim.x, so any list length spreads over the
// whole grid.  Wave w owns experts 64w .. 64w+63 of 16 MT tokens: MT row
// tiles of 16 tokens x four column tiles of 16 experts, where column c of
// tile j is expert 64w + 4c + j, so one 16-byte load gives a lane its four
// tiles' router weights of one h.  The sum over h runs in chunks of 32: at
// step s of a chunk, the lanes of k group g (lane / 16) supply h = chunk +
// 8g + s for both operands (any assignment of h to (step, k) that A and B
// share gives the same sum), so a lane loads its token's 8 consecutive x
// values with one 16-byte load and its experts' weights of 8 rows with
// eight.  Products of bf16 x and float32 weights are exact in float64.
// Result layout of the instruction: lane l holds rows 4r + l / 16, r =
// 0..3, of column l % 16.
template <int MT>
__global__ __launch_bounds__(256) void route_logits_list_kernel(const uint16_t* __restrict__ x, int H,
                                                                const float* __restrict__ W, int E,
                                                                const int32_t* __restrict__ list,
                                                                const int32_t* __restrict__ count,
                                                                size_t region_bytes, double* __restrict__ part) {
  const int n = *count;
  if (n <= 0) return;
  const int hs = list_hsplit(n, E, H, region_bytes);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int hlen = H / hs;
  const int e0 = 64 * wave + 4 * c;
  const int units = ((n + 16 * MT - 1) / (16 * MT)) * hs;

  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int tb = unit / hs, slice = unit - tb * hs;
    const int h0 = slice * hlen + 8 * g;
    const float* wr = W + static_cast<size_t>(h0) * E + e0;
    const int i0 = tb * 16 * MT;
    const uint16_t* xr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xr[m] = x + static_cast<size_t>(list[min(i0 + 16 * m + c, n - 1)]) * H + h0;

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
          for (int m = 0; m < MT; ++m)
            acc[m][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[m], bw, acc[m][j], 0, 0, 0);
        }
      }
    };
    // Two register buffers: the loads of chunk n+1 are in flight while chunk
    // n is multiplied.
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
        const int i = i0 + 16 * m + 4 * r + g;
        if (i < n) {
          f64x4 v = {acc[m][0][r], acc[m][1][r], acc[m][2][r], acc[m][3][r]};
          *reinterpret_cast<f64x4*>(part + (static_cast<size_t>(slice) * n + i) * E + e0) = v;
        }
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
// LIST: the rows of part are the tokens list[0 .. *count) (hsplit from
// list_hsplit); the grid may be smaller than the list, blocks take groups
// blockIdx.x, blockIdx.x + gridDim.x, ...
template <int TPB, int SPLIT, bool LIST>
__global__ __launch_bounds__(256 * SPLIT) void route_topk_kernel(const double* __restrict__ part, int T, int E,
                                                                 int hsplit, const float* __restrict__ bias, int k,
                                                                 float scale, int32_t* __restrict__ ids,
                                                                 float* __restrict__ weights,
                                                                 const int32_t* __restrict__ list,
                                                                 const int32_t* __restrict__ count, int H,
                                                                 size_t region_bytes) {
  __shared__ double s_key[TPB][256];
  __shared__ double s_sc[TPB][256];
  __shared__ double s_part[SPLIT][TPB][256];
  const int n = LIST ? *count : T;  // rows of part
  if (n <= 0) return;
  const int hs = LIST ? list_hsplit(n, E, H, region_bytes) : hsplit;
  const int e = threadIdx.x & 255;
  const int qs = threadIdx.x >> 8;  // which of the SPLIT threads of expert e
  const size_t stride = static_cast<size_t>(n) * E;
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  for (int i0 = blockIdx.x * TPB; i0 < n; i0 += gridDim.x * TPB) {
    if (e < E) {
#pragma unroll
      for (int qq = 0; qq < TPB; ++qq) {
        const int i = i0 + qq;
        if (i >= n) break;
        // Slices qs, qs + SPLIT, ... in increasing order, eight loads in flight.
        const double* pp = part + static_cast<size_t>(qs) * stride + static_cast<size_t>(i) * E + e;
        const size_t step = static_cast<size_t>(SPLIT) * stride;
        const int cnt = qs < hs ? (hs - qs + SPLIT - 1) / SPLIT : 0;
        double z = 0.0;
        int j = 0;
        for (; j + 8 <= cnt; j += 8) {
          double v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = pp[(j + u) * step];
#pragma unroll
          for (int u = 0; u < 8; ++u) z += v[u];
        }
        for (; j < cnt; ++j) z += pp[j * step];
        s_part[qs][qq][e] = z;
      }
    }
    if (SPLIT > 1) __syncthreads();
    if (qs == 0 && e < E) {
      const double b = bias ? static_cast<double>(bias[e]) : 0.0;
#pragma unroll
      for (int qq = 0; qq < TPB; ++qq) {
        if (i0 + qq >= n) break;
        double z = s_part[0][qq][e];
#pragma unroll
        for (int r = 1; r < SPLIT; ++r) z += s_part[r][qq][e];
        const double sc = sqrt(fmax(z, 0.0) + log1p(exp(-fabs(z))));
        s_sc[qq][e] = sc;
        s_key[qq][e] = sc + b;
      }
    }
    __syncthreads();
    if (q < TPB && i0 + q < n) {
      const int t = LIST ? list[i0 + q] : i0 + q;
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
          weights[static_cast<size_t>(t) * k + j] =
              ok ? static_cast<float>(static_cast<double>(scale) * sel_s[j] / sum) : 0.0f;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- many tokens
// The bf16 matrix cores compute the logits of every token; where their
// rounding could change the selection, the token's logits are computed again
// in float64 (route_logits_list_kernel) and its top-k taken from those.
//
// Split of the router matrix: W = W1 + W2 + W3 exactly, each term bf16 (W1 =
// bf16(W), W2 = bf16(W - W1), W3 = W - W1 - W2; a float32 significand of 24
// bits is three bf16 significands of 8), so x . W = x . W1 + x . W2 + x . W3
// with every product of bf16 x and a bf16 term exact in float32.  The kernel
// checks the identity for every weight; where it fails (a weight of
// magnitude 2^120 or more, or not finite) the expert's norm becomes
// infinite, which sends every token to the float64 path.
//
// Error bound.  A block sums a 32-long k step of all three terms in one
// float32 MFMA accumulator (96 exact products; each addition inside the
// instruction, in whatever order and however rounded, errs by at most 2^-23
// of the sum of its operands' magnitudes), adds that step sum to a float64
// running sum, and the top-k kernel adds the hs slice sums in float64.  With
// S = sum_h |x_h| |W_he| and |W1| + |W2| + |W3| <= (1 + 2^-7) |W|:
//   |z~ - z| <= ((96 * 2^-23) (1 + 2^-7) + (hs + 4) 2^-24) S,
// the second term a generous allowance for the float64 additions, and S <=
// |x_t|_2 |W_e|_2 (Cauchy-Schwarz).  The two norms are computed here (x_t
// from the same LDS tiles the MFMAs read, per slice; W_e by the split kernel,
// per 512 h), so the bound costs no pass of its own.  Products that leave
// float32's normal range (a flushed denormal) add at most 2^-100 (|x_t|_2 +
// |W_e|_2) + 1e-30 (H <= 2^16), also added.
//
// Selection.  s = sqrt(softplus(z)) has slope sigma(z) / (2 s(z)) <= 0.33
// everywhere and <= 1 / (2 sqrt(z)) for z >= 1, so a logit within d of z~
// gives a key within kd = min(0.33, 0.5 / sqrt(z~ - d)) d (the second form
// for z~ - d >= 1) of the computed key, plus 1e-12 (|key| + 1) for the
// float64 evaluation of s.  The top-k taken from the computed keys is the
// one the exact keys give, in the same order, when every chosen key's
// interval lies above every other key's and the chosen intervals are
// disjoint from each other; otherwise, or when any key or bound is not
// finite, the token goes on the float64 list.
//
// Weights.  The logits' actual rounding (about 1e-6 at most, not the bound)
// moves s by a relative sigma(z) / (2 softplus(z)) times it: below 1/8 for
// z >= 4, up to 1/2 for very negative z, which a selection bias can still
// choose.  So the top-k kernel recomputes in float64, from x and a
// transposed float32 copy of W, every chosen logit whose s is below
// sqrt(softplus(4)) (kRefineS), and takes the weights from those.

constexpr int kSplitTok = 64;   // tokens per block of the split logits kernel
constexpr int kSplitStage = 64; // k per pipeline stage

// grid (E/16, H/512), 1024 threads.  Thread (n = tid % 16, r = tid / 16)
// handles expert 16 blockIdx.x + n at the 8 h from 512 blockIdx.y + 8 r.
// The terms go to planes[p] (p = 0, 1, 2 for W1, W2, W3) in the B-operand
// order of the 16x16x32 bf16 MFMA: fragment (16-expert group eg, 32-h step
// ks) is 1 KiB at element (eg * H/32 + ks) * 512, its lane 16 g + n holding
// expert 16 eg + n at h = 32 ks + 8 g + 0..7.
// wt[e][h] = W[h][e] (float32, for the exact recompute of chosen logits).
// nw_part[blockIdx.y][e] = sum of W^2 over the block's 512 h (float64; the
// squares of float32 are exact in it), added in r order.  Block (0, 0) also
// clears the float64 list's counter.
__global__ __launch_bounds__(1024) void route_wsplit_kernel(const float* __restrict__ W, int E, int H,
                                                            uint16_t* __restrict__ planes, float* __restrict__ wt,
                                                            double* __restrict__ nw_part,
                                                            int32_t* __restrict__ fb_count) {
  __shared__ double red[64][16];
  const int n = threadIdx.x & 15, r = threadIdx.x >> 4;
  const int eg = blockIdx.x, e = 16 * eg + n;
  const int h = blockIdx.y * 512 + 8 * r;
  const size_t plane = static_cast<size_t>(E) * H;
  const int KS = H / 32;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *fb_count = 0;
  double sq = 0.0;
  bool bad = false;
  float wv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) wv[j] = W[static_cast<size_t>(h + j) * E + e];
  uint32_t pk[3][4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float w = wv[j];
    const uint16_t b1 = float_to_bf16_bits(w);
    const float r1 = w - bf16_bits_to_float(b1);
    const uint16_t b2 = float_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_float(b2);
    const uint16_t b3 = float_to_bf16_bits(r2);
    const double sum3 = (static_cast<double>(bf16_bits_to_float(b1)) + bf16_bits_to_float(b2)) +
                        static_cast<double>(bf16_bits_to_float(b3));
    bad |= !(fabsf(w) < 0x1p120f) || sum3 != static_cast<double>(w);
    sq = fma(static_cast<double>(w), static_cast<double>(w), sq);
    const uint32_t sh = (j & 1) * 16;
    if ((j & 1) == 0) {
      pk[0][j >> 1] = b1;
      pk[1][j >> 1] = b2;
      pk[2][j >> 1] = b3;
    } else {
      pk[0][j >> 1] |= static_cast<uint32_t>(b1) << sh;
      pk[1][j >> 1] |= static_cast<uint32_t>(b2) << sh;
      pk[2][j >> 1] |= static_cast<uint32_t>(b3) << sh;
    }
  }
  f32x4* wtp = reinterpret_cast<f32x4*>(wt + static_cast<size_t>(e) * H + h);
  wtp[0] = f32x4{wv[0], wv[1], wv[2], wv[3]};
  wtp[1] = f32x4{wv[4], wv[5], wv[6], wv[7]};
  const int ks = h >> 5, g = (h & 31) >> 3;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    u32x4 v = {pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
    *reinterpret_cast<u32x4*>(planes + p * plane + (static_cast<size_t>(eg) * KS + ks) * 512 + (16 * g + n) * 8) = v;
  }
  red[r][n] = bad ? INFINITY : sq;
  __syncthreads();
  if (r == 0) {
    double t = 0.0;
    for (int i = 0; i < 64; ++i) t += red[i][n];
    nw_part[static_cast<size_t>(blockIdx.y) * E + e] = t;
  }
}

// grid (ceil(T / 64), hs), 64 NW threads (NW = E / 32 waves).  Block (bx, s)
// computes the float32 logit partials of tokens 64 bx .. 64 bx + 63 over h
// slice s (L = H / hs) for all E experts: wave w owns experts 32w .. 32w+31
// (two 16-expert n tiles) of all 64 tokens (four 16-token m tiles).
// Activations (64 tokens x 64 k per stage) arrive by LDS-DMA into two stages,
// row r's 16-byte chunk c at slot c ^ (r & 7) so the 16 rows of a fragment
// read hit distinct banks; each wave's weight fragments (2 k steps x 3 terms
// x 2 n tiles per stage) go straight into a two-stage register ring.  One
// barrier per stage: drain, barrier, issue the next stage, multiply this one.
// Each k step accumulates its three terms (W3, W2, W1) into a zeroed
// float32 tile, then adds it to the float64 running sum.  The squares of x for the
// norm bound come from the same A fragments, fragment (m, k step) counted by
// wave (4 ks + m) % NW.  Outputs: part[s][t][e] (float64), nx_part[s][t].
template <int NW>
__global__ __launch_bounds__(64 * NW) void route_logits_split_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                                     const uint16_t* __restrict__ planes, int E,
                                                                     int hs, double* __restrict__ part,
                                                                     float* __restrict__ nx_part) {
  __shared__ __attribute__((aligned(1024))) uint16_t As[2][kSplitTok * kSplitStage];
  __shared__ float xs_red[NW][4][16];
  constexpr int kOps = (8 + NW - 1) / NW;  // 1 KiB DMA ops per wave per stage (8 per stage)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kSplitTok;
  const int L = H / hs;
  const int h0 = blockIdx.y * L;
  const int NS = L / kSplitStage;
  const int KS = H / 32;
  const size_t plane = static_cast<size_t>(E) * H;

  // weight fragment bases (uniform): term p, n tile j of this wave
  const uint16_t* bp[3][2];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bp[p][j] = planes + p * plane + static_cast<size_t>(2 * wave + j) * KS * 512 + static_cast<size_t>(h0 >> 5) * 512;
  const uint32_t blane = lane * 16;  // byte offset of the lane inside a fragment

  // activation DMA sources: op q of wave w covers chunk index cidx = (q NW +
  // w) * 64 + lane: row cidx / 8, LDS slot cidx % 8, global chunk slot ^ (row & 7)
  const char* asrc[4];  // kOps <= 4 (a size that depends on NW here drops the kernel's host stub)
#pragma unroll
  for (int q = 0; q < kOps; ++q) {
    const int cidx = (q * NW + wave) * 64 + lane;
    const int row = (cidx >> 3) & 63;
    const int c = (cidx & 7) ^ (row & 7);
    asrc[q] = reinterpret_cast<const char*>(x + static_cast<size_t>(min(t0 + row, T - 1)) * H + h0 + 8 * c);
  }

  u32x4 bq[2][2][3][2];  // [ring slot][k step][term][n tile]
  auto issue = [&](int slot, int st) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bq[slot][ks][p][j] = ld16(reinterpret_cast<const char*>(bp[p][j] + static_cast<size_t>(2 * st + ks) * 512) + blane);
#pragma unroll
    for (int q = 0; q < kOps; ++q)
      if (q * NW + wave < 8)
        __builtin_amdgcn_global_load_lds(asrc[q] + st * (kSplitStage * 2), &As[slot][(q * NW + wave) * 512], 16, 0, 0);
  };

  double acc[4][2][4];
  float xsq[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    xsq[m] = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][j][i] = 0.0;
  }

  auto compute = [&](int slot) {
    const uint16_t* abuf = As[slot];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 a[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = 16 * m + (lane & 15);
        const int c = 4 * ks + (lane >> 4);
        a[m] = *reinterpret_cast<const bf16x8*>(abuf + row * kSplitStage + ((c ^ (row & 7)) * 8));
        if ((4 * ks + m) % NW == wave) {
          const u32x4 u = __builtin_bit_cast(u32x4, a[m]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v0 = __uint_as_float(u[i] << 16), v1 = __uint_as_float(u[i] & 0xffff0000u);
            xsq[m] = fmaf(v0, v0, xsq[m]);
            xsq[m] = fmaf(v1, v1, xsq[m]);
          }
        }
      }
      // two m tiles at a time: 4 independent accumulations between
      // dependent MFMAs, half the float32 step registers
#pragma unroll
      for (int mh = 0; mh < 4; mh += 2) {
        f32x4 t[2][2];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int j = 0; j < 2; ++j) t[mm][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 2; p >= 0; --p)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              t[mm][j] = mfma16x16x32(a[mh + mm], __builtin_bit_cast(bf16x8, bq[slot][ks][p][j]), t[mm][j]);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mh + mm][j][i] += static_cast<double>(t[mm][j][i]);
      }
    }
  };

  issue(0, 0);
  for (int st = 0; st < NS; st += 2) {
    wait_vmcnt<0>();
    lds_barrier();
    if (st + 1 < NS) issue(1, st + 1);
    compute(0);
    if (st + 1 < NS) {
      wait_vmcnt<0>();
      lds_barrier();
      if (st + 2 < NS) issue(0, st + 2);
      compute(1);
    }
  }

  // squares: lanes l, l ^ 16, l ^ 32, l ^ 48 hold the four k groups of token
  // 16 m + l % 16; then the waves' counts in wave order
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float v = xsq[m];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (lane < 16) xs_red[wave][m][lane] = v;
  }
  __syncthreads();
  if (threadIdx.x < 64 && t0 + static_cast<int>(threadIdx.x) < T) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += xs_red[w][threadIdx.x >> 4][threadIdx.x & 15];
    nx_part[static_cast<size_t>(blockIdx.y) * T + t0 + threadIdx.x] = v;
  }
  // result layout of the 16x16 MFMA: lane l holds column l % 16, rows
  // 4 (l / 16) + i
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * m + 4 * (lane >> 4) + i;
      if (t < T) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          part[(static_cast<size_t>(blockIdx.y) * T + t) * E + 32 * wave + 16 * j + (lane & 15)] = acc[m][j][i];
      }
    }
}

// Top-k from the split logits, 4 tokens per block of 256 threads (one wave
// per token), E <= 256.  Thread e sums the hs float64 partials of its
// expert, computes s, the key, the bound d and the key's half-width kd; wave
// q then runs the same top-k as route_topk_kernel and checks that the result
// is certain.  A token whose chosen set is not certain goes on the float64
// list (whose top-k writes its ids and weights).  Otherwise the chosen
// experts whose key intervals overlap another chosen one's, and those with
// s below kRefineS, get exact logits, and the k are ordered by key.  An exact logit: lane l sums
// its 8-h chunks l, l + 64, ... in float64 (four chunks' loads in flight),
// then the wave adds the 64 lane sums pairwise; lane 0's total is the one
// used.
constexpr double kRefineS = 2.0046;  // > sqrt(softplus(4)) = 2.00453...

__global__ __launch_bounds__(256) void route_topk_split_kernel(const double* __restrict__ part,
                                                               const float* __restrict__ nx_part,
                                                               const double* __restrict__ nw_part,
                                                               const uint16_t* __restrict__ x,
                                                               const float* __restrict__ wt, int T, int E, int H,
                                                               int hs, double cbound, const float* __restrict__ bias,
                                                               int k, float scale, int32_t* __restrict__ ids,
                                                               float* __restrict__ weights,
                                                               int32_t* __restrict__ fb_count,
                                                               int32_t* __restrict__ fb_list) {
  constexpr int TPB = 4;
  __shared__ double s_key[TPB][256];
  __shared__ double s_sc[TPB][256];
  __shared__ double s_kd[TPB][256];
  __shared__ double s_nx[TPB];
  __shared__ int s_bad[TPB];
  const int e = threadIdx.x;
  const int tb = blockIdx.x * TPB;
  const int nwp = H / 512;
  if (threadIdx.x < TPB) {
    const int t = tb + threadIdx.x;
    double v = 0.0;
    if (t < T)
      for (int i = 0; i < hs; ++i) v += static_cast<double>(nx_part[static_cast<size_t>(i) * T + t]);
    // float32 sums of at most H exact squares: relative error far below 1e-3
    s_nx[threadIdx.x] = sqrt(v * 1.001) * (1.0 + 0x1p-40);
    s_bad[threadIdx.x] = 0;
  }
  double wn = 0.0;
  if (e < E) {
    for (int i = 0; i < nwp; ++i) wn += nw_part[static_cast<size_t>(i) * E + e];
    wn = sqrt(wn) * (1.0 + 0x1p-40);
  }
  __syncthreads();
  if (e < E) {
    const double b = bias ? static_cast<double>(bias[e]) : 0.0;
#pragma unroll
    for (int q = 0; q < TPB; ++q) {
      const int t = tb + q;
      if (t >= T) break;
      double z = 0.0;
      for (int i = 0; i < hs; ++i) z += part[(static_cast<size_t>(i) * T + t) * E + e];
      const double sc = sqrt(fmax(z, 0.0) + log1p(exp(-fabs(z))));
      const double key = sc + b;
      const double d = cbound * s_nx[q] * wn + 0x1p-100 * (s_nx[q] + wn) + 1e-30;
      const double lo = z - d;
      const double lip = lo >= 1.0 ? fmin(0.33, 0.5 / sqrt(lo)) : 0.33;
      const double kd = lip * d + 1e-12 * (fabs(key) + 1.0);
      if (!(fabs(key) < INFINITY) || !(kd < INFINITY)) s_bad[q] = 1;
      s_sc[q][e] = sc;
      s_key[q][e] = key;
      s_kd[q][e] = kd;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
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
  // highest upper end among the experts not chosen
  double hi = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (live[u]) hi = fmax(hi, key[u] + s_kd[q][lane + 64 * u]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) hi = fmax(hi, __shfl_xor(hi, off, 64));
  // Certainty, the same in every lane (sel_id, hi and the LDS values are):
  // the set is certain when every chosen interval lies above hi; chosen
  // experts whose intervals overlap another chosen one's get exact logits.
  bool set_ok = s_bad[q] == 0;
  int refine = 0;
  {
    double lo_min = INFINITY;
    double clo[8], chi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      clo[j] = chi[j] = 0.0;
      if (j >= k) continue;
      if (sel_id[j] == 0x7fffffff) {
        set_ok = false;
        continue;
      }
      clo[j] = s_key[q][sel_id[j]] - s_kd[q][sel_id[j]];
      chi[j] = s_key[q][sel_id[j]] + s_kd[q][sel_id[j]];
      lo_min = fmin(lo_min, clo[j]);
    }
    set_ok = set_ok && lo_min > hi;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i != j && i < k && j < k && !(clo[j] > chi[i] || clo[i] > chi[j])) refine |= 1 << j;
  }
  if (!set_ok) {
    // the float64 list decides this token (and writes its ids and weights)
    if (lane == 0) fb_list[atomicAdd(fb_count, 1)] = t;
    return;
  }
  // Exact logits of the chosen experts that overlap another chosen one, and
  // of those whose s is sensitive to rounding.  The set is the exact top-k
  // set, and each expert not recomputed has an interval apart from all the
  // others, so ordering by exact logits where recomputed (and computed keys
  // elsewhere) gives the exact order.
  const uint16_t* xr = x + static_cast<size_t>(t) * H;
  const int nch = H / 8;  // 8-h chunks, a multiple of 64
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k || (!((refine >> j) & 1) && !(sel_s[j] < kRefineS))) continue;
    const float* wr = wt + static_cast<size_t>(sel_id[j]) * H;
    double acc = 0.0;
    for (int c0 = 0; c0 < nch; c0 += 256) {
      u32x4 xv[4];
      f32x4 w0[4], w1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 64 * u + lane;
        if (c0 + 64 * u < nch) {
          xv[u] = ld16(xr + 8 * c);
          w0[u] = *reinterpret_cast<const f32x4*>(wr + 8 * c);
          w1[u] = *reinterpret_cast<const f32x4*>(wr + 8 * c + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c0 + 64 * u >= nch) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const double x0 = static_cast<double>(__uint_as_float(xv[u][i] << 16));
          const double x1 = static_cast<double>(__uint_as_float(xv[u][i] & 0xffff0000u));
          const double wa = static_cast<double>(i < 2 ? w0[u][2 * i] : w1[u][2 * i - 4]);
          const double wb = static_cast<double>(i < 2 ? w0[u][2 * i + 1] : w1[u][2 * i - 3]);
          acc = fma(x0, wa, acc);
          acc = fma(x1, wb, acc);
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    sel_s[j] = sqrt(fmax(acc, 0.0) + log1p(exp(-fabs(acc))));
  }
  if (lane == 0) {
    if (refine) {
      // order the k chosen by key (descending), equal keys by id
      double sk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) sk[j] = j < k ? sel_s[j] + (bias ? static_cast<double>(bias[sel_id[j]]) : 0.0) : 0.0;
      for (int i = 1; i < k; ++i) {
        for (int j = i; j > 0 && precedes(sk[j], sel_id[j], sk[j - 1], sel_id[j - 1]); --j) {
          const double tk = sk[j]; sk[j] = sk[j - 1]; sk[j - 1] = tk;
          const double ts = sel_s[j]; sel_s[j] = sel_s[j - 1]; sel_s[j - 1] = ts;
          const int ti = sel_id[j]; sel_id[j] = sel_id[j - 1]; sel_id[j - 1] = ti;
        }
      }
    }
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) sum += sel_s[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) continue;
      ids[static_cast<size_t>(t) * k + j] = sel_id[j];
      weights[static_cast<size_t>(t) * k + j] = static_cast<float>(static_cast<double>(scale) * sel_s[j] / sum);
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

// The split path takes many-token batches when E is a multiple of 64 (up to
// 256; E / 32 waves per block) and the router weights are 16-byte aligned
// (the float64 list kernel's weight loads are 16 bytes).
static bool route_use_split(int T, int E, const float* w) {
  return T > 256 && E % 64 == 0 && E <= 256 && (reinterpret_cast<uintptr_t>(w) & 15) == 0;
}

// h slices of the split logits: until the blocks cover the 256 CUs, up to 8
// (every slice a multiple of the 64-k stage).
static int split_hsplit(int T, int H) {
  const int ntb = (T + kSplitTok - 1) / kSplitTok;
  int hs = 1;
  while (ntb * hs < 256 && hs < 8 && (H / (hs * 2)) % kSplitStage == 0) hs *= 2;
  return hs;
}

constexpr int kListTokens = 32;  // tokens per block of the float64 list kernel

// Workspace of the split path, each part 256-byte aligned: the three weight
// planes, the transposed router, the W norm partials, the x norm partials,
// the logit partials (the float64 list's partials reuse this region once the
// top-k has read it), the list counter and the list.
struct SplitWs {
  uint16_t* planes;
  float* wt;
  double* nw_part;
  float* nx_part;
  double* part;
  size_t region;
  int32_t* fb_count;
  int32_t* fb_list;
};

static size_t split_layout(int T, int H, int E, char* base, SplitWs* w) {
  const int hs = split_hsplit(T, H);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~static_cast<size_t>(255);
    return o;
  };
  const size_t n_te = static_cast<size_t>(T) * E;
  const size_t o_pl = take(static_cast<size_t>(3) * E * H * sizeof(uint16_t));
  const size_t o_wt = take(static_cast<size_t>(E) * H * sizeof(float));
  const size_t o_nw = take(static_cast<size_t>(H / 512) * E * sizeof(double));
  const size_t o_nx = take(static_cast<size_t>(hs) * T * sizeof(float));
  const size_t region = static_cast<size_t>(std::max(hs, 2)) * n_te * sizeof(double);
  const size_t o_part = take(region);
  const size_t o_cnt = take(sizeof(int32_t));
  const size_t o_list = take(static_cast<size_t>(T) * sizeof(int32_t));
  if (w) {
    w->planes = reinterpret_cast<uint16_t*>(base + o_pl);
    w->wt = reinterpret_cast<float*>(base + o_wt);
    w->nw_part = reinterpret_cast<double*>(base + o_nw);
    w->nx_part = reinterpret_cast<float*>(base + o_nx);
    w->part = reinterpret_cast<double*>(base + o_part);
    w->region = region;
    w->fb_count = reinterpret_cast<int32_t*>(base + o_cnt);
    w->fb_list = reinterpret_cast<int32_t*>(base + o_list);
  }
  return off;
}

size_t route_ws_bytes(int T, int H, int E) {
  size_t v = static_cast<size_t>(route_hsplit_vector(T, H)) * T * E * sizeof(double);
  if (T > 256) v = std::max(v, split_layout(T, H, E, nullptr, nullptr));
  return v;
}

hipError_t launch_route_learned(const uint16_t* x, int T, int H, const float* w, const float* bias, int E, int k,
                                float scale, int32_t* ids, float* weights, void* ws, hipStream_t s) {
  if (route_use_split(T, E, w)) {
    SplitWs sw;
    split_layout(T, H, E, static_cast<char*>(ws), &sw);
    const int hs = split_hsplit(T, H);
    route_wsplit_kernel<<<dim3(E / 16, H / 512), 1024, 0, s>>>(w, E, H, sw.planes, sw.wt, sw.nw_part, sw.fb_count);
    const dim3 g1((T + kSplitTok - 1) / kSplitTok, hs);
    switch (E / 32) {
      case 2:
        route_logits_split_kernel<2><<<g1, 128, 0, s>>>(x, T, H, sw.planes, E, hs, sw.part, sw.nx_part);
        break;
      case 4:
        route_logits_split_kernel<4><<<g1, 256, 0, s>>>(x, T, H, sw.planes, E, hs, sw.part, sw.nx_part);
        break;
      case 6:
        route_logits_split_kernel<6><<<g1, 384, 0, s>>>(x, T, H, sw.planes, E, hs, sw.part, sw.nx_part);
        break;
      default:
        route_logits_split_kernel<8><<<g1, 512, 0, s>>>(x, T, H, sw.planes, E, hs, sw.part, sw.nx_part);
        break;
    }
    // the error bound's constant (see the split kernels' description)
    const double cbound =
        (std::ldexp(96.0, -23) * (1.0 + std::ldexp(1.0, -7)) + std::ldexp(static_cast<double>(hs + 4), -24)) *
        (1.0 + 1e-4);
    route_topk_split_kernel<<<(T + 3) / 4, 256, 0, s>>>(sw.part, sw.nx_part, sw.nw_part, x, sw.wt, T, E, H, hs, cbound,
                                                        bias, k, scale, ids, weights, sw.fb_count, sw.fb_list);
    route_logits_list_kernel<kListTokens / 16><<<256, 64 * (E / 64), 0, s>>>(x, H, w, E, sw.fb_list, sw.fb_count,
                                                                             sw.region, sw.part);
    route_topk_kernel<1, 4, true><<<std::min(T, 1024), 1024, 0, s>>>(sw.part, T, E, 0, bias, k, scale, ids, weights,
                                                                     sw.fb_list, sw.fb_count, H, sw.region);
    return hipGetLastError();
  }
  double* part = static_cast<double*>(ws);
  const int hs = route_hsplit_vector(T, H);
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
  // Few tokens: one token per block (many slices when very few: four threads
  // per expert share them).  Many tokens: four tokens per block.
  if (T <= 256 && hs >= 32)
    route_topk_kernel<1, 4, false><<<T, 1024, 0, s>>>(part, T, E, hs, bias, k, scale, ids, weights, nullptr, nullptr,
                                                      H, 0);
  else if (T <= 256)
    route_topk_kernel<1, 1, false><<<T, 256, 0, s>>>(part, T, E, hs, bias, k, scale, ids, weights, nullptr, nullptr, H,
                                                     0);
  else
    route_topk_kernel<4, 1, false><<<(T + 3) / 4, 256, 0, s>>>(part, T, E, hs, bias, k, scale, ids, weights, nullptr,
                                                               nullptr, H, 0);
  return hipGetLastError();
}

hipError_t launch_route_hash(const int32_t* tok, int T, const int32_t* table, int V, int k, float scale,
                             int32_t* ids, float* weights, hipStream_t s) {
  route_hash_kernel<<<(T + 255) / 256, 256, 0, s>>>(tok, T, table, V, k, scale / static_cast<float>(k), ids, weights);
  return hipGetLastError();
}

}  // namespace moe
