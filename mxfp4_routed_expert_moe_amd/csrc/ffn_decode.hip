// Expert FFN, decode family (few rows per expert; HBM bound).  Computes, for
// the rows of one item (at most 16 rows of one expert),
//   phase 1: h = bf16( silu(min(W_gate x, L)) * clamp(W_up x, -L, L) )
//   phase 2: out = W_down h
// ("Model techniques map -- DeepSeek-V4-Flash", row "SwiGLU feed-forward";
// MXFP4 weights as in "ElytronAI / DeepSeek-v4-Flash", Sizes), streaming the
// expert's tiled MXFP4 bytes (or an MXFP8 shared expert's, the same page's
// dense format) once from HBM into bf16 MFMA B fragments via the hardware
// scaled FP4 / FP8 converts.
#include "ffn_internal.h"

namespace moe {

namespace {

constexpr int kWaves = 4;  // waves per block; they split the K axis

// One chunk of at most 16 rows [row0, row0 + nrows) of group g.  red: the
// block's LDS for the split-K reduction.  W8: group g is an MXFP8 expert
// (2048-byte tiles read as two 1 KiB halves; half the n-tiles per block, so
// the register ring keeps its size).
template <bool GATEUP, int KTW, bool W8>
__device__ __forceinline__ void decode_chunk(const uint16_t* __restrict__ act, const int32_t* __restrict__ row_token,
                                             int g, int row0, int nrows, const uint8_t* __restrict__ blob,
                                             uint64_t expert_bytes, int H, int I, float limit,
                                             uint16_t* __restrict__ h_out, float* __restrict__ out_rows,
                                             f32x4 (*red)[8][64]) {
  constexpr int KT = kWaves * KTW;    // k tiles of the whole K axis
  constexpr int NT = W8 ? 4 : 8;      // n-tiles per block (GATEUP: NT/2 gate + NT/2 up)
  constexpr int NH = NT / 2;
  constexpr int NQ = W8 ? 2 : 1;      // 16-byte loads per lane per n-tile per k tile
  constexpr uint64_t kTileBytes = W8 ? 2048 : 1024;
  constexpr int NSW = KTW >= 4 ? KTW / 4 : 1;  // scale words per n-tile per wave
  static_assert(KTW % 4 == 0 || 4 % KTW == 0, "a wave's k tiles tile its scale words");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kt0 = wave * KTW;
  const ExpertPlanes pl = W8 ? expert_planes8(H, I) : expert_planes(H, I);
  const uint8_t* eb = blob + static_cast<uint64_t>(g) * expert_bytes;
  constexpr uint64_t kTileStride = static_cast<uint64_t>(KT) * kTileBytes;  // bytes between n-tiles
  constexpr uint64_t kScStride = static_cast<uint64_t>(KT / 4) * 256;

  const uint8_t* nb0;
  const uint8_t* nb1;
  const uint8_t* sb0;
  const uint8_t* sb1;
  if (GATEUP) {
    nb0 = eb + pl.gate_nib + blockIdx.x * NH * kTileStride;
    nb1 = eb + pl.up_nib + blockIdx.x * NH * kTileStride;
    sb0 = eb + pl.gate_sc + blockIdx.x * NH * kScStride;
    sb1 = eb + pl.up_sc + blockIdx.x * NH * kScStride;
  } else {
    nb0 = eb + pl.down_nib + blockIdx.x * NT * kTileStride;
    nb1 = nb0 + NH * kTileStride;
    sb0 = eb + pl.down_sc + blockIdx.x * NT * kScStride;
    sb1 = sb0 + NH * kScStride;
  }
  nb0 += static_cast<uint64_t>(kt0) * kTileBytes + lane * 16;
  nb1 += static_cast<uint64_t>(kt0) * kTileBytes + lane * 16;
  sb0 += static_cast<uint64_t>(kt0 >> 2) * 256 + lane * 4;
  sb1 += static_cast<uint64_t>(kt0 >> 2) * 256 + lane * 4;

  // Padded lanes (rows >= nrows) re-read the item's last row; their results
  // are never stored.
  const int r = lane & 15;
  const int p = row0 + min(r, nrows - 1);
  const uint16_t* arow = (GATEUP ? act + static_cast<size_t>(row_token[p]) * H : act + static_cast<size_t>(p) * I) +
                         32 * (lane >> 4) + kt0 * 128;

  uint32_t sw[NSW][NT];
#pragma unroll
  for (int d = 0; d < NSW; ++d)
#pragma unroll
    for (int j = 0; j < NT; ++j)
      sw[d][j] = *reinterpret_cast<const uint32_t*>((j < NH ? sb0 : sb1) + (j % NH) * kScStride + d * 256);

  u32x4 bq[3][NT][NQ];
  u32x4 a[2][4];
  auto load_b = [&](int buf, int i) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        bq[buf][j][q] = ld16((j < NH ? nb0 : nb1) + (j % NH) * kTileStride + i * kTileBytes + q * 1024);
  };
  auto load_a = [&](int buf, int i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) a[buf][q] = ld16(arow + i * 128 + 8 * q);
  };

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

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
      for (int j = 0; j < NT; ++j) {
        const float sc = e8m0_scale_operand((sw[d][j] >> sh) & 255u);
        // MFMA s takes k = 32 (lane / 16) + 8 s + 0..7 of the tile: 8 E2M1
        // codes of word s, or 8 E4M3 codes of words 2 (s % 2), +1 of half s / 2.
        bf16x8 bv;
        if constexpr (W8) {
          const u32x4& h = bq[i % 3][j][s >> 1];
          bv = dequant8_fp8(h[2 * (s & 1)], h[2 * (s & 1) + 1], sc);
        } else {
          bv = dequant8(bq[i % 3][j][0][s], sc);
        }
        acc[j] = mfma16x16x32(av, bv, acc[j]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (i + 2 < KTW) load_a(i & 1, i + 2);
  }

  // Split-K partial sums meet in LDS; summed in wave order.
#pragma unroll
  for (int j = 0; j < NT; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  auto wave_sum = [&](int j) {
    f32x4 v = red[0][j][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += red[w][j][lane];
    return v;
  };
  const int rbase = 4 * (lane >> 4);
  if (GATEUP) {
    // output n-tile pairs (gate jg, up NH + jg), one per wave while they last
    for (int jg = wave; jg < NH; jg += kWaves) {
      const f32x4 gs = wave_sum(jg);
      const f32x4 us = wave_sum(NH + jg);
      const int col = blockIdx.x * 16 * NH + jg * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = rbase + e;
        if (rr < nrows) {
          const float gv = fminf(gs[e], limit);
          const float uv = fminf(fmaxf(us[e], -limit), limit);
          h_out[static_cast<size_t>(row0 + rr) * I + col] = float_to_bf16_bits(silu_f(gv) * uv);
        }
      }
    }
  } else {
    constexpr int kPer = NT / kWaves;
#pragma unroll
    for (int jj = 0; jj < kPer; ++jj) {
      const int j = wave * kPer + jj;
      const f32x4 os = wave_sum(j);
      const int col = blockIdx.x * 16 * NT + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = rbase + e;
        if (rr < nrows) out_rows[static_cast<size_t>(row0 + rr) * H + col] = os[e];
      }
    }
  }
}

// grid (n blocks, E + ceil(T / 16)), 64 * kWaves threads: block row y < E takes the
// rows of routed expert y (16 at a time; an expert with no rows returns at
// once), the rest take 16-row chunks of the shared group, so the decode path
// needs no work list.  W8 (MXFP8 shared expert): grid (n blocks, ceil(T / 16))
// over the shared group only, while the MXFP4 launch then has E block rows.
// GATEUP: 64 output columns per block (4 gate + 4 up n-tiles; W8: 32, 2 + 2),
// K = H, A = x rows via row_token, output h.  Otherwise 128 output columns
// (8 down n-tiles; W8: 64, 4), K = I, A = h rows, output float32 rows.  Wave
// w owns k tiles [w*KTW, (w+1)*KTW) of all the block's n-tiles.  The k loop is
// fully unrolled over a ring of three register buffers, so two k tiles (8 KB
// per wave) of weight loads stay in flight while one is consumed; the
// activation loads of a tile are issued one tile ahead and before the weight
// loads two tiles ahead, so the in-order load counter never makes a tile wait
// for a later one.
template <bool GATEUP, int KTW, bool W8>
__global__ __launch_bounds__(64 * kWaves, 2) void ffn_decode_kernel(const uint16_t* __restrict__ act,
                                                            const int32_t* __restrict__ row_token,
                                                            const int32_t* __restrict__ offsets, int E,
                                                            const uint8_t* __restrict__ blob, uint64_t expert_bytes,
                                                            int H, int I, float limit, uint16_t* __restrict__ h_out,
                                                            float* __restrict__ out_rows) {
  // blockIdx.y < E: routed expert y, all of its rows (16 at a time);
  // otherwise chunk y - E of the shared group (16 rows).  W8: chunk y of the
  // shared group.
  int g, first, end;
  if (!W8 && static_cast<int>(blockIdx.y) < E) {
    g = blockIdx.y;
    first = offsets[g];
    end = offsets[g + 1];
  } else {
    g = E;
    first = offsets[E] + (blockIdx.y - (W8 ? 0 : E)) * kDecodeRows;
    end = min(first + kDecodeRows, offsets[E + 1]);
  }
  if (first >= end) return;
  __shared__ f32x4 red[kWaves][8][64];
  decode_chunk<GATEUP, KTW, W8>(act, row_token, g, first, min(kDecodeRows, end - first), blob, expert_bytes, H, I,
                                limit, h_out, out_rows, red);
  // Experts with more than 16 rows (rare while decoding) take further chunks.
  for (int row0 = first + kDecodeRows; row0 < end; row0 += kDecodeRows) {
    __syncthreads();  // the previous chunk is done with red
    // The weight addresses do not depend on the chunk; this empty asm hides
    // that from the compiler, which would otherwise hoist dozens of them out
    // of the loop and spill.
    const uint8_t* bl = blob;
    asm volatile("" : "+s"(bl));
    decode_chunk<GATEUP, KTW, W8>(act, row_token, g, row0, min(kDecodeRows, end - row0), bl, expert_bytes, H, I,
                                  limit, h_out, out_rows, red);
  }
}

}  // namespace

void launch_ffn_decode(bool gateup, const uint16_t* act, const int32_t* row_token, const int32_t* offsets, int T,
                       int E, const uint8_t* blob, uint64_t eb, int H, int I, float limit, uint16_t* h,
                       float* out_rows, bool shared_w8, hipStream_t s) {
  const int K = gateup ? H : I;
  const int ktw = K / (128 * kWaves);  // k tiles per wave; decode_k_ok(K) keeps it in {1, 2, 4, 8}
  if (ktw * 128 * kWaves != K) return;  // never taken: decode_k_ok(K) holds for the decode path
  const int chunks = (T + kDecodeRows - 1) / kDecodeRows;
  // MXFP4 experts (and the shared one unless it is MXFP8); then the MXFP8 shared expert.
  dim3 grid(gateup ? I / 64 : H / 128, E + (shared_w8 ? 0 : chunks));
  dim3 grid8(gateup ? I / 32 : H / 64, chunks);
#define MOE_DECODE_LAUNCH(G, KTW)                                                                                    \
  do {                                                                                                             \
    ffn_decode_kernel<G, KTW, false><<<grid, 64 * kWaves, 0, s>>>(act, row_token, offsets, E, blob, eb, H, I, limit, \
                                                                  G ? h : nullptr, G ? nullptr : out_rows);        \
    if (shared_w8)                                                                                                 \
      ffn_decode_kernel<G, KTW, true><<<grid8, 64 * kWaves, 0, s>>>(act, row_token, offsets, E, blob, eb, H, I,      \
                                                                    limit, G ? h : nullptr, G ? nullptr : out_rows); \
  } while (0)
#define MOE_DECODE_SWITCH(G)                     \
  switch (ktw) {                                 \
    case 1: MOE_DECODE_LAUNCH(G, 1); break;      \
    case 2: MOE_DECODE_LAUNCH(G, 2); break;      \
    case 4: MOE_DECODE_LAUNCH(G, 4); break;      \
    case 8: MOE_DECODE_LAUNCH(G, 8); break;      \
    default: break; /* excluded by decode_k_ok */ \
  }
  if (gateup) {
    MOE_DECODE_SWITCH(true)
  } else {
    MOE_DECODE_SWITCH(false)
  }
#undef MOE_DECODE_SWITCH
#undef MOE_DECODE_LAUNCH
}

}  // namespace moe
