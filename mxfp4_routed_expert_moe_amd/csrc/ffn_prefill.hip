// Expert FFN, prefill family (many rows per expert; MFMA bound).  Same
// arithmetic as the decode family over items of up to 128 rows
// ("Model techniques map -- DeepSeek-V4-Flash", row "SwiGLU feed-forward").
#include "ffn_internal.h"

namespace moe {

namespace {

constexpr int kLdsPitch = 136;  // bf16 per LDS row: 128 + 8 of padding (272 bytes)

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

}  // namespace

void launch_ffn_prefill(bool gateup, const uint16_t* act, const int32_t* row_token, const FfnWs& w,
                        const uint8_t* blob, uint64_t eb, int H, int I, float limit, float* out_rows, int max_items,
                        hipStream_t s) {
  if (gateup) {
    dim3 g1(I / 64, max_items);
    ffn_prefill_kernel<true><<<g1, 256, 0, s>>>(act, row_token, w.items, w.n_items, blob, eb, H, I, limit, w.h,
                                                nullptr);
  } else {
    dim3 g2(H / 128, max_items);
    ffn_prefill_kernel<false><<<g2, 256, 0, s>>>(act, nullptr, w.items, w.n_items, blob, eb, H, I, limit, nullptr,
                                                 out_rows);
  }
}

}  // namespace moe
