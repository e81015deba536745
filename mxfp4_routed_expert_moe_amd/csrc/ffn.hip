// Expert FFN of the MoE layer on gfx950: for every dispatched row p of group
// e (E routed experts, then the shared expert),
//   h = bf16( silu(min(W_gate[e] x, L)) * clamp(W_up[e] x, -L, L) )
//   out_rows[p] = W_down[e] h
// ("Model techniques map -- DeepSeek-V4-Flash", row "SwiGLU feed-forward";
// weights MXFP4 as in "ElytronAI / DeepSeek-v4-Flash", Sizes).
//
// MXFP4 bytes stream from HBM in the tiled device layout: one 16-byte load per
// lane gives the 32 codes of one column for one 128-wide k tile, and the
// hardware scaled convert turns 8 codes and their E8M0 scale into the 8 bf16
// of one 16x16x32 MFMA B fragment.  Nothing is ever dequantised to memory.
//
// Work is a device-side list of items (group, first row, row count) built
// from the dispatch offsets, so the host never learns the per-expert counts:
// the grid covers the worst case and surplus blocks return at once.
//
// Two kernel families:
//  * decode (few rows per expert, HBM bound): the four waves of a block split
//    the K axis and share one set of 16-row tiles; each wave streams its
//    quarter of the block's weight columns with 16-byte loads one k tile
//    ahead, and the partial sums meet in LDS in a fixed order;
//  * prefill (many rows per expert, MFMA bound): 128-row tiles of the
//    gathered activations go through LDS (row pitch padded so that MFMA
//    fragment reads are bank-conflict free), double buffered; each wave owns
//    a 64 x 64 output tile and reads its weight fragments straight from HBM.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kPrefillRows = 128;
constexpr int kLdsPitch = 136;  // bf16 per LDS row: 128 + 8 of padding (272 bytes)

__host__ __device__ inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

struct FfnWs {
  int32_t* n_items;  // [1]
  int4* items;       // [max_items]
  uint16_t* h;       // [rows, I] bf16
};

inline int ffn_max_items(int T, int E, int k, int bm) {
  const long rows = static_cast<long>(T) * (k + 1);
  return static_cast<int>((rows + bm - 1) / bm) + E + 1;
}

inline FfnWs ffn_carve(void* ws, int max_items) {
  char* p = static_cast<char*>(ws);
  FfnWs w;
  w.n_items = reinterpret_cast<int32_t*>(p);
  p += 256;
  w.items = reinterpret_cast<int4*>(p);
  p += align256(sizeof(int4) * static_cast<size_t>(max_items));
  w.h = reinterpret_cast<uint16_t*>(p);
  return w;
}

// Work list: every group with rows is cut into items of at most bm rows.
__global__ __launch_bounds__(256) void ffn_plan_kernel(const int32_t* __restrict__ offsets, int E, int bm,
                                                       int4* __restrict__ items, int32_t* __restrict__ n_items) {
  __shared__ int cnt[1024];
  __shared__ int tmp[4];
  const int G = E + 1;
  for (int g = threadIdx.x; g < G; g += 256) {
    const int c = offsets[g + 1] - offsets[g];
    cnt[g] = (c + bm - 1) / bm;
  }
  __syncthreads();
  const int total = block_excl_scan_256(cnt, G, tmp);
  for (int g = threadIdx.x; g < G; g += 256) {
    const int r0 = offsets[g];
    const int c = offsets[g + 1] - r0;
    const int base = cnt[g];
    for (int i = 0; i * bm < c; ++i) items[base + i] = make_int4(g, r0 + i * bm, min(bm, c - i * bm), 0);
  }
  if (threadIdx.x == 0) *n_items = total;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ------------------------------------------------------------------ decode
// grid (n blocks, max items), 256 threads, items of at most 16 rows.
// GATEUP: 64 output columns per block (4 gate + 4 up n-tiles), K = H, A = x
// rows via row_token, output h.  Otherwise 128 output columns (8 down
// n-tiles), K = I, A = h rows, output float32 rows.  Wave w owns k tiles
// [w*KTW, (w+1)*KTW) of all 8 n-tiles.  The k loop is fully unrolled over a
// ring of three register buffers, so two k tiles (8 KB per wave) of weight
// loads stay in flight while one is consumed; the activation loads of a tile
// are issued one tile ahead and before the weight loads two tiles ahead, so
// the in-order load counter never makes a tile wait for a later one.
template <bool GATEUP, int KTW>
__global__ __launch_bounds__(256, 2) void ffn_decode_kernel(const uint16_t* __restrict__ act,
                                                            const int32_t* __restrict__ row_token,
                                                            const int4* __restrict__ items,
                                                            const int32_t* __restrict__ n_items,
                                                            const uint8_t* __restrict__ blob, uint64_t expert_bytes,
                                                            int H, int I, float limit, uint16_t* __restrict__ h_out,
                                                            float* __restrict__ out_rows) {
  constexpr int KT = 4 * KTW;        // k tiles of the whole K axis
  constexpr int NSW = KTW >= 4 ? KTW / 4 : 1;  // scale words per n-tile per wave
  const int item = blockIdx.y;
  if (item >= *n_items) return;
  const int4 it = items[item];
  const int g = it.x, row0 = it.y, nrows = it.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kt0 = wave * KTW;
  const ExpertPlanes pl = expert_planes(H, I);
  const uint8_t* eb = blob + static_cast<uint64_t>(g) * expert_bytes;
  constexpr uint64_t kTileStride = static_cast<uint64_t>(KT) * 1024;  // bytes between n-tiles
  constexpr uint64_t kScStride = static_cast<uint64_t>(KT / 4) * 256;

  const uint8_t* nb0;
  const uint8_t* nb1;
  const uint8_t* sb0;
  const uint8_t* sb1;
  if (GATEUP) {
    nb0 = eb + pl.gate_nib + blockIdx.x * 4 * kTileStride;
    nb1 = eb + pl.up_nib + blockIdx.x * 4 * kTileStride;
    sb0 = eb + pl.gate_sc + blockIdx.x * 4 * kScStride;
    sb1 = eb + pl.up_sc + blockIdx.x * 4 * kScStride;
  } else {
    nb0 = eb + pl.down_nib + blockIdx.x * 8 * kTileStride;
    nb1 = nb0 + 4 * kTileStride;
    sb0 = eb + pl.down_sc + blockIdx.x * 8 * kScStride;
    sb1 = sb0 + 4 * kScStride;
  }
  nb0 += static_cast<uint64_t>(kt0) * 1024 + lane * 16;
  nb1 += static_cast<uint64_t>(kt0) * 1024 + lane * 16;
  sb0 += static_cast<uint64_t>(kt0 >> 2) * 256 + lane * 4;
  sb1 += static_cast<uint64_t>(kt0 >> 2) * 256 + lane * 4;

  // Padded lanes (rows >= nrows) re-read the item's last row; their results
  // are never stored.
  const int r = lane & 15;
  const int p = row0 + min(r, nrows - 1);
  const uint16_t* arow = (GATEUP ? act + static_cast<size_t>(row_token[p]) * H : act + static_cast<size_t>(p) * I) +
                         32 * (lane >> 4) + kt0 * 128;

  uint32_t sw[NSW][8];
#pragma unroll
  for (int d = 0; d < NSW; ++d)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sw[d][j] = *reinterpret_cast<const uint32_t*>((j < 4 ? sb0 : sb1) + (j & 3) * kScStride + d * 256);

  u32x4 bq[3][8];
  u32x4 a[2][4];
  auto load_b = [&](int buf, int i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[buf][j] = ld16((j < 4 ? nb0 : nb1) + (j & 3) * kTileStride + i * 1024);
  };
  auto load_a = [&](int buf, int i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) a[buf][q] = ld16(arow + i * 128 + 8 * q);
  };

  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_a(0, 0);
  load_b(0, 0);
  if (KTW > 1) {
    load_a(1, 1);
    load_b(1, 1);
  }
  // sched_barrier(0) keeps the compiler from sinking prefetches below the
  // MFMAs of the current tile (which would leave one tile in flight).
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < KTW; ++i) {
    if (i + 2 < KTW) load_b((i + 2) % 3, i + 2);
    __builtin_amdgcn_sched_barrier(0);
    const int kt = kt0 + i;
    const int sh = 8 * (kt & 3);
    const int d = KTW >= 4 ? (i >> 2) : 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, a[i & 1][s]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float sc = e8m0_to_float((sw[d][j] >> sh) & 255u);
        acc[j] = mfma16x16x32(av, dequant8(bq[i % 3][j][s], sc), acc[j]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (i + 2 < KTW) load_a(i & 1, i + 2);
  }

  // Split-K partial sums meet in LDS; summed in wave order 0,1,2,3.
  __shared__ f32x4 red[4][8][64];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  const int rbase = 4 * (lane >> 4);
  if (GATEUP) {
    const int jg = wave, ju = 4 + wave;
    const f32x4 gs = ((red[0][jg][lane] + red[1][jg][lane]) + red[2][jg][lane]) + red[3][jg][lane];
    const f32x4 us = ((red[0][ju][lane] + red[1][ju][lane]) + red[2][ju][lane]) + red[3][ju][lane];
    const int col = blockIdx.x * 64 + wave * 16 + (lane & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = rbase + e;
      if (rr < nrows) {
        const float gv = fminf(gs[e], limit);
        const float uv = fminf(fmaxf(us[e], -limit), limit);
        h_out[static_cast<size_t>(row0 + rr) * I + col] = float_to_bf16_bits(silu_f(gv) * uv);
      }
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * wave + jj;
      const f32x4 os = ((red[0][j][lane] + red[1][j][lane]) + red[2][j][lane]) + red[3][j][lane];
      const int col = blockIdx.x * 128 + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = rbase + e;
        if (rr < nrows) out_rows[static_cast<size_t>(row0 + rr) * H + col] = os[e];
      }
    }
  }
}

// ------------------------------------------------------------------ prefill
// grid (n blocks, max items), 256 threads = 2 x 2 waves, 128-row items.
// GATEUP: 64 output columns per block (wave column wn: gate and up n-tiles of
// output columns 32*wn .. 32*wn+31).  Otherwise 128 output columns per block
// (wave column wn: 4 down n-tiles).
template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void ffn_prefill_kernel(const uint16_t* __restrict__ act,
                                                             const int32_t* __restrict__ row_token,
                                                             const int4* __restrict__ items,
                                                             const int32_t* __restrict__ n_items,
                                                             const uint8_t* __restrict__ blob, uint64_t expert_bytes,
                                                             int H, int I, float limit, uint16_t* __restrict__ h_out,
                                                             float* __restrict__ out_rows) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kPrefillRows * kLdsPitch];
  const int item = blockIdx.y;
  if (item >= *n_items) return;
  const int4 it = items[item];
  const int g = it.x, row0 = it.y, nrows = it.z;
  const int K = GATEUP ? H : I;
  const int KT = K >> 7;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const ExpertPlanes pl = expert_planes(H, I);
  const uint8_t* eb = blob + static_cast<uint64_t>(g) * expert_bytes;

  const uint8_t* nib[4];
  const uint8_t* scl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int nt;
    uint64_t onib, osc;
    if (GATEUP) {
      nt = blockIdx.x * 4 + wn * 2 + (j & 1);
      onib = j < 2 ? pl.gate_nib : pl.up_nib;
      osc = j < 2 ? pl.gate_sc : pl.up_sc;
    } else {
      nt = blockIdx.x * 8 + wn * 4 + j;
      onib = pl.down_nib;
      osc = pl.down_sc;
    }
    nib[j] = eb + onib + static_cast<uint64_t>(nt) * KT * 1024 + lane * 16;
    scl[j] = eb + osc + static_cast<uint64_t>(nt) * (KT >> 2) * 256 + lane * 4;
  }

  // A loader: 16 threads per row (16 bytes each = one 128-wide k tile row),
  // rows tid/16 + 16*q.
  const int lc = tid & 15, lr = tid >> 4;
  const uint16_t* ldp[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = lr + 16 * q;
    ldp[q] = nullptr;
    if (r < nrows) {
      const int p = row0 + r;
      ldp[q] = (GATEUP ? act + static_cast<size_t>(row_token[p]) * H : act + static_cast<size_t>(p) * I) + lc * 8;
    }
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[8];
  u32x4 bq[4], bn[4];
  uint32_t sw[4];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int q = 0; q < 8; ++q) areg[q] = ldp[q] ? ld16(ldp[q] + kt * 128) : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *reinterpret_cast<u32x4*>(&As[buf][(lr + 16 * q) * kLdsPitch + lc * 8]) = areg[q];
  };

  load_a(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) bq[j] = ld16(nib[j]);
  store_a(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) {
      load_a(kt + 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) bn[j] = ld16(nib[j] + static_cast<size_t>(kt + 1) * 1024);
    }
    if ((kt & 3) == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sw[j] = *reinterpret_cast<const uint32_t*>(scl[j] + static_cast<size_t>(kt >> 2) * 256);
    }
    float scf[4];
    const int sh = 8 * (kt & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) scf[j] = e8m0_to_float((sw[j] >> sh) & 255u);
    const uint16_t* abase = &As[kt & 1][(wm * 64 + (lane & 15)) * kLdsPitch + 32 * (lane >> 4)];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = dequant8(bq[j][s], scf[j]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(abase + mt * 16 * kLdsPitch + 8 * s);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mt][j] = mfma16x16x32(a, b[j], acc[mt][j]);
      }
    }
    if (more) {
      store_a((kt + 1) & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) bq[j] = bn[j];
    }
    __syncthreads();
  }

#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int rbase = wm * 64 + mt * 16 + 4 * (lane >> 4);
    if (GATEUP) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = blockIdx.x * 64 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + i;
          if (r < nrows) {
            const float gv = fminf(acc[mt][j][i], limit);
            const float uv = fminf(fmaxf(acc[mt][j + 2][i], -limit), limit);
            h_out[static_cast<size_t>(row0 + r) * I + col] = float_to_bf16_bits(silu_f(gv) * uv);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = blockIdx.x * 128 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + i;
          if (r < nrows) out_rows[static_cast<size_t>(row0 + r) * H + col] = acc[mt][j][i];
        }
      }
    }
  }
}

constexpr int kDecodeRows = 16;

inline bool decode_k_ok(int K) { return K == 512 || K == 1024 || K == 2048 || K == 4096; }

// Decode kernels while the average group holds at most ~16 rows (and the K
// sizes have a compiled decode variant); prefill kernels otherwise.
inline bool use_decode(int T, int E, int k, int H, int I) {
  return static_cast<long>(T) * (k + 1) <= 16L * (E + 1) && decode_k_ok(H) && decode_k_ok(I);
}

template <bool GATEUP>
void launch_decode_phase(const uint16_t* act, const int32_t* row_token, const FfnWs& w, const uint8_t* blob,
                         uint64_t eb, int H, int I, float limit, float* out_rows, int max_items, hipStream_t s) {
  const int K = GATEUP ? H : I;
  dim3 grid(GATEUP ? I / 64 : H / 128, max_items);
  uint16_t* h = GATEUP ? w.h : nullptr;
  float* o = GATEUP ? nullptr : out_rows;
  switch (K / 512) {
    case 1: ffn_decode_kernel<GATEUP, 1><<<grid, 256, 0, s>>>(act, row_token, w.items, w.n_items, blob, eb, H, I, limit, h, o); break;
    case 2: ffn_decode_kernel<GATEUP, 2><<<grid, 256, 0, s>>>(act, row_token, w.items, w.n_items, blob, eb, H, I, limit, h, o); break;
    case 4: ffn_decode_kernel<GATEUP, 4><<<grid, 256, 0, s>>>(act, row_token, w.items, w.n_items, blob, eb, H, I, limit, h, o); break;
    default: ffn_decode_kernel<GATEUP, 8><<<grid, 256, 0, s>>>(act, row_token, w.items, w.n_items, blob, eb, H, I, limit, h, o); break;
  }
}

inline int ffn_bm(int T, int E, int k, int H, int I) { return use_decode(T, E, k, H, I) ? kDecodeRows : kPrefillRows; }

}  // namespace

size_t ffn_ws_bytes(int T, int E, int H, int I, int k) {
  const int mi = ffn_max_items(T, E, k, ffn_bm(T, E, k, H, I));
  return 256 + align256(sizeof(int4) * static_cast<size_t>(mi)) +
         align256(sizeof(uint16_t) * static_cast<size_t>(T) * (k + 1) * I);
}

hipError_t launch_ffn(const uint16_t* x, int T, const uint8_t* blob, uint64_t expert_bytes, int E, int H, int I,
                      int k, const int32_t* offsets, const int32_t* row_token, float limit, float* out_rows,
                      void* ws, int phase, hipStream_t s) {
  const int bm = ffn_bm(T, E, k, H, I);
  const int max_items = ffn_max_items(T, E, k, bm);
  const bool dec = use_decode(T, E, k, H, I);
  FfnWs w = ffn_carve(ws, max_items);
  for (int ph = 0; ph < 3; ++ph) {
    if (phase >= 0 && ph != phase) continue;
    if (ph == 0) {
      ffn_plan_kernel<<<1, 256, 0, s>>>(offsets, E, bm, w.items, w.n_items);
    } else if (dec) {
      if (ph == 1) launch_decode_phase<true>(x, row_token, w, blob, expert_bytes, H, I, limit, out_rows, max_items, s);
      else launch_decode_phase<false>(w.h, nullptr, w, blob, expert_bytes, H, I, limit, out_rows, max_items, s);
    } else if (ph == 1) {
      dim3 g1(I / 64, max_items);
      ffn_prefill_kernel<true><<<g1, 256, 0, s>>>(x, row_token, w.items, w.n_items, blob, expert_bytes, H, I, limit,
                                                  w.h, nullptr);
    } else {
      dim3 g2(H / 128, max_items);
      ffn_prefill_kernel<false><<<g2, 256, 0, s>>>(w.h, nullptr, w.items, w.n_items, blob, expert_bytes, H, I, limit,
                                                   nullptr, out_rows);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
