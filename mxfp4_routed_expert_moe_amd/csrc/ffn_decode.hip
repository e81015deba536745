// Expert FFN, decode family (few rows per expert; HBM bound).  Computes, for
// the rows of one item (at most 16 rows of one expert),
//   phase 1: h = bf16( silu(min(W_gate x, L)) * clamp(W_up x, -L, L) )
//   phase 2: out = W_down h
// ("Model techniques map -- DeepSeek-V4-Flash", row "SwiGLU feed-forward";
// MXFP4 weights as in "ElytronAI / DeepSeek-v4-Flash", Sizes), streaming the
// expert's tiled MXFP4 bytes (or an MXFP8 shared expert's, the same page's
// dense format, or 2-bit affine routed experts' codes, "OsaurusAI /
// DeepSeek-V4-Flash-0731-JANG", Dynamic affine recipe) once from HBM into
// bf16 MFMA B fragments via the hardware scaled FP4 / FP8 converts.
#include "ffn_internal.h"

namespace moe {

namespace {

constexpr int kWaves = 4;  // waves per block; they split the K axis

// One chunk of at most 16 rows [row0, row0 + nrows) of group g.  red: the
// block's LDS for the split-K reduction.  W8: group g is an MXFP8 expert
// (2048-byte tiles read as two 1 KiB halves; half the n-tiles per block, so
// the register ring keeps its size).
//
// NARROW (MXFP4): half the n-tiles per block and twice the blocks, for
// batches so small that only a few experts stream: the launch's blocks then
// finish more evenly.
template <bool GATEUP, int KTW, bool W8, bool NARROW = false>
__device__ __forceinline__ void decode_chunk(const uint16_t* __restrict__ act, const int32_t* __restrict__ row_token,
                                             int g, int row0, int nrows, const uint8_t* __restrict__ blob,
                                             uint64_t expert_bytes, int H, int I, float limit,
                                             uint16_t* __restrict__ h_out, uint16_t* __restrict__ out_rows,
                                             f32x4 (*red)[8][64]) {
  constexpr int KT = kWaves * KTW;    // k tiles of the whole K axis
  constexpr int NT = W8 || NARROW ? 4 : 8;  // n-tiles per block (GATEUP: NT/2 gate + NT/2 up)
  constexpr int NH = NT / 2;
  constexpr int NQ = W8 ? 2 : 1;      // 16-byte loads per lane per n-tile per k tile
  constexpr uint64_t kTileBytes = W8 ? 2048 : 1024;
  // Which k tiles each wave takes.  Down projection, 4 tiles per wave (K =
  // 2048): the wave pairs (0, 1) and (2, 3) each cover half the tiles, the
  // two waves of a pair alternating (wave w: tiles 8 (w / 2) + w % 2 + 2i), so
  // at each step the block reads two runs of two consecutive tiles of every
  // n-tile and a wave needs two scale words per n-tile.  Down with 1 or 2
  // tiles per wave: all four waves alternate (tile w + 4i).  Otherwise
  // (gate/up, K = 4096 down): contiguous quarters.  Measured at 64 tokens:
  // down 150 us with pairs, 151.5 all four alternating, 154 quarters; gate/up
  // with pairs 295 against 292.6 for quarters.
  constexpr bool PR = !GATEUP && KTW == 4;
  constexpr bool IL = !GATEUP && KTW <= 2;
  constexpr int KS = PR ? 2 : IL ? kWaves : 1;                       // k-tile step of a wave
  constexpr int NSW = PR ? 2 : IL ? KTW : (KTW >= 4 ? KTW / 4 : 1);  // scale words per n-tile per wave
  static_assert(KTW % 4 == 0 || 4 % KTW == 0, "a wave's k tiles tile its scale words");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kt0 = PR ? 8 * (wave >> 1) + (wave & 1) : IL ? wave : wave * KTW;
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
        bq[buf][j][q] = ld16((j < NH ? nb0 : nb1) + (j % NH) * kTileStride + i * KS * kTileBytes + q * 1024);
  };
  auto load_a = [&](int buf, int i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) a[buf][q] = ld16(arow + i * KS * 128 + 8 * q);
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
    const int kt = kt0 + i * KS;
    const int sh = 8 * (kt & 3);
    const int d = PR ? (i >> 1) : IL ? i : (KTW >= 4 ? (i >> 2) : 0);
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
        if (rr < nrows) out_rows[static_cast<size_t>(row0 + rr) * H + col] = float_to_bf16_bits(os[e]);
      }
    }
  }
}

// 2-bit affine codes -> MFMA B operand.  Word w of a tile lane holds the
// codes of two MFMAs: code i of MFMA s sits in bits 4i + 2(s%2) + 1 : +0, so
// w & 0x33333333 (s even) or (w >> 2) & 0x33333333 (s odd) is eight E2M1
// nibbles 00qq, which encode q / 2; the scaled convert with scale 2 turns them
// into the eight bf16 values q, exactly.
template <int HALF>
__device__ __forceinline__ bf16x8 affine2_operand(uint32_t w) {
  const uint32_t nib = (HALF ? (w >> 2) : w) & 0x33333333u;
  return dequant8(nib, e8m0_scale_operand(128u));
}

// One chunk of at most 16 rows of 2-bit affine routed expert g.  Per group of
// G input columns (64 for gate and up, 32 for down), with q the codes and s, b
// the group's bf16 scale and bias,
//   sum_k x_k (s q_k + b) = s * (sum_k x_k q_k) + b * sum_k x_k,
// so the MFMAs run x against the exact bf16 values q (P) and against ones (S,
// the row sums of x over the group), and each group is folded into the
// float32 accumulator with two multiply-adds per element.  (The bias term as
// MFMAs of x against the broadcast bias, instead of S and a multiply-add,
// measured slower: the matrix cores are as busy as the vector unit here.)
// MFMA s of a 128-k tile covers k = 32 s .. 32 s + 31 (lane 16 g + r: k =
// 32 s + 8 g + 0..7), so an MFMA never straddles two groups.  Same block
// shape, split-K and epilogue as the MX chunk.
template <bool GATEUP, int KTW>
__device__ __forceinline__ void decode_chunk_a2(const uint16_t* __restrict__ act,
                                                const int32_t* __restrict__ row_token, int g, int row0, int nrows,
                                                const uint8_t* __restrict__ blob, uint64_t expert_bytes, int H,
                                                int I, float limit, uint16_t* __restrict__ h_out,
                                                uint16_t* __restrict__ out_rows, f32x4 (*red)[8][64]) {
  constexpr int KT = kWaves * KTW;
  constexpr int NT = 8;
  constexpr int NH = NT / 2;
  constexpr int G = GATEUP ? 64 : 32;   // group size ("OsaurusAI / DeepSeek-V4-Flash-0731-JANG", recipe)
  constexpr int NG = 128 / G;           // groups per k tile
  constexpr int SPG = G / 32;           // MFMAs per group
  constexpr uint64_t kTileBytes = 512;  // codes of a 16-column x 128-k tile
  constexpr uint64_t kSbBytes = 16 * NG * 4;
  constexpr uint64_t kTileStride = static_cast<uint64_t>(KT) * kTileBytes;
  constexpr uint64_t kSbStride = static_cast<uint64_t>(KT) * kSbBytes;
  typedef __attribute__((__vector_size__(NG * sizeof(unsigned)))) unsigned u32xg;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kt0 = wave * KTW;
  const ExpertPlanes pl = expert_planes_a2(H, I);
  const uint8_t* eb = blob + static_cast<uint64_t>(g) * expert_bytes;

  const uint8_t* nb0;
  const uint8_t* nb1;
  const uint8_t* sb0;
  const uint8_t* sb1;
  if (GATEUP) {
    nb0 = eb + pl.gate_nib + blockIdx.x * NH * kTileStride;
    nb1 = eb + pl.up_nib + blockIdx.x * NH * kTileStride;
    sb0 = eb + pl.gate_sc + blockIdx.x * NH * kSbStride;
    sb1 = eb + pl.up_sc + blockIdx.x * NH * kSbStride;
  } else {
    nb0 = eb + pl.down_nib + blockIdx.x * NT * kTileStride;
    nb1 = nb0 + NH * kTileStride;
    sb0 = eb + pl.down_sc + blockIdx.x * NT * kSbStride;
    sb1 = sb0 + NH * kSbStride;
  }
  nb0 += static_cast<uint64_t>(kt0) * kTileBytes + lane * 8;
  nb1 += static_cast<uint64_t>(kt0) * kTileBytes + lane * 8;
  // the (scale, bias) words of output column lane % 16 (the MFMA result layout)
  sb0 += static_cast<uint64_t>(kt0) * kSbBytes + (lane & 15) * (NG * 4);
  sb1 += static_cast<uint64_t>(kt0) * kSbBytes + (lane & 15) * (NG * 4);

  const int r = lane & 15;
  const int p = row0 + min(r, nrows - 1);
  const uint16_t* arow = (GATEUP ? act + static_cast<size_t>(row_token[p]) * H : act + static_cast<size_t>(p) * I) +
                         8 * (lane >> 4) + kt0 * 128;

  // codes two tiles ahead (gate/up: three-deep ring) or one (down, whose
  // (scale, bias) words take twice the registers: two-deep); activations and
  // the (scale, bias) words one tile ahead (two-deep rings), issued together
  constexpr int RB = GATEUP ? 3 : 2;
  u32x2 bq[RB][NT];
  u32xg sq[2][NT];
  u32x4 a[2][4];
  auto load_b = [&](int buf, int i) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
      bq[buf][j] = *reinterpret_cast<const u32x2*>((j < NH ? nb0 : nb1) + (j % NH) * kTileStride + i * kTileBytes);
  };
  auto load_a = [&](int buf, int i) {
#pragma unroll
    for (int s = 0; s < 4; ++s) a[buf][s] = ld16(arow + i * 128 + 32 * s);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      sq[buf][j] = *reinterpret_cast<const u32xg*>((j < NH ? sb0 : sb1) + (j % NH) * kSbStride + i * kSbBytes);
  };

  const u32x4 ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
  const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_w);
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_a(0, 0);
  load_b(0, 0);
  if (KTW > 1) {
    load_a(1, 1);
    if (RB == 3) load_b(1, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < KTW; ++i) {
    if (i + RB - 1 < KTW) load_b((i + RB - 1) % RB, i + RB - 1);
    __builtin_amdgcn_sched_barrier(0);
    // group by group: its row sums S, then four n-tiles at a time the group's
    // MFMAs into fresh P (four independent chains, so one n-tile's fold waits
    // on no MFMA still in flight for it), then the folds
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ss = 0; ss < SPG; ++ss)
        S = mfma16x16x32(__builtin_bit_cast(bf16x8, a[i & 1][gi * SPG + ss]), ones, S);
#pragma unroll
      for (int j0 = 0; j0 < NT; j0 += 4) {
        f32x4 P[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          P[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ss = 0; ss < SPG; ++ss) {
            const int s = gi * SPG + ss;
            const uint32_t w = bq[i % RB][j0 + jj][s >> 1];
            const bf16x8 bv = (s & 1) ? affine2_operand<1>(w) : affine2_operand<0>(w);
            P[jj] = mfma16x16x32(__builtin_bit_cast(bf16x8, a[i & 1][s]), bv, P[jj]);
          }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t sbw = sq[i & 1][j0 + jj][gi];
          const float sc = __uint_as_float(sbw << 16);          // bf16 scale (low half)
          const float bc = __uint_as_float(sbw & 0xffff0000u);  // bf16 bias (high half)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[j0 + jj][e] = fmaf(bc, S[e], fmaf(sc, P[jj][e], acc[j0 + jj][e]));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (i + 2 < KTW) load_a(i & 1, i + 2);
  }

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
        if (rr < nrows) out_rows[static_cast<size_t>(row0 + rr) * H + col] = float_to_bf16_bits(os[e]);
      }
    }
  }
}

// grid (n blocks, nrouted + ceil(T / 16)), 64 * kWaves threads: block row y <
// nrouted takes the rows of routed expert y (16 at a time; an expert with no
// rows returns at once), the rest take 16-row chunks of the shared group, so
// the decode path needs no work list.  nrouted is E, or 0 in a launch of the
// shared group alone (an MXFP8 shared expert, whose other launch then has no
// chunks).  Beside 2-bit affine routed experts an MXFP4 shared expert rides in
// the affine launch (its blocks take the MXFP4 chunk code).
// GATEUP: 64 output columns per block (4 gate + 4 up n-tiles; MXFP8: 32, 2 + 2),
// K = H, A = x rows via row_token, output h.  Otherwise 128 output columns
// (8 down n-tiles; MXFP8: 64, 4), K = I, A = h rows, output float32 rows.  Wave
// w owns k tiles [w*KTW, (w+1)*KTW) of all the block's n-tiles.  The k loop is
// fully unrolled over a ring of three register buffers, so two k tiles (8 KB
// per wave) of weight loads stay in flight while one is consumed; the
// activation loads of a tile are issued one tile ahead and before the weight
// loads two tiles ahead, so the in-order load counter never makes a tile wait
// for a later one.
template <bool GATEUP, int KTW, int FMT, bool NARROW = false>
__global__ __launch_bounds__(64 * kWaves, 2) void ffn_decode_kernel(const uint16_t* __restrict__ act,
                                                            const int32_t* __restrict__ row_token,
                                                            const int32_t* __restrict__ offsets, int E, int nrouted,
                                                            const uint8_t* __restrict__ blob, uint64_t expert_bytes,
                                                            int H, int I, float limit, uint16_t* __restrict__ h_out,
                                                            uint16_t* __restrict__ out_rows) {
  int g, first, end;
  if (static_cast<int>(blockIdx.y) < nrouted) {
    g = blockIdx.y;
    first = offsets[g];
    end = offsets[g + 1];
  } else {
    g = E;
    first = offsets[E] + (blockIdx.y - nrouted) * kDecodeRows;
    end = min(first + kDecodeRows, offsets[E + 1]);
  }
  if (first >= end) return;
  __shared__ f32x4 red[kWaves][8][64];
  auto chunk = [&](int row0, const uint8_t* bl) {
    if constexpr (FMT == kFmtA2) {
      if (g < E)
        decode_chunk_a2<GATEUP, KTW>(act, row_token, g, row0, min(kDecodeRows, end - row0), bl, expert_bytes, H, I,
                                     limit, h_out, out_rows, red);
      else  // the MXFP4 shared expert beside affine routed experts
        decode_chunk<GATEUP, KTW, false>(act, row_token, g, row0, min(kDecodeRows, end - row0), bl, expert_bytes, H,
                                         I, limit, h_out, out_rows, red);
    } else
      decode_chunk<GATEUP, KTW, FMT == kFmtMx8, NARROW>(act, row_token, g, row0, min(kDecodeRows, end - row0), bl,
                                                        expert_bytes, H, I, limit, h_out, out_rows, red);
  };
  chunk(first, blob);
  // Experts with more than 16 rows (rare while decoding) take further chunks.
  for (int row0 = first + kDecodeRows; row0 < end; row0 += kDecodeRows) {
    __syncthreads();  // the previous chunk is done with red
    // The weight addresses do not depend on the chunk; this empty asm hides
    // that from the compiler, which would otherwise hoist dozens of them out
    // of the loop and spill.
    const uint8_t* bl = blob;
    asm volatile("" : "+s"(bl));
    chunk(row0, bl);
  }
}

}  // namespace

void launch_ffn_decode(bool gateup, const uint16_t* act, const int32_t* row_token, const int32_t* offsets, int T,
                       int E, int k, const uint8_t* blob, uint64_t eb, int H, int I, float limit, uint16_t* h,
                       uint16_t* out_rows, bool shared_w8, bool routed_a2, hipStream_t s) {
  const int K = gateup ? H : I;
  const int ktw = K / (128 * kWaves);  // k tiles per wave; decode_k_ok(K) keeps it in {1, 2, 4, 8}
  if (ktw * 128 * kWaves != K) return;  // never taken: decode_k_ok(K) holds for the decode path
  const int chunks = (T + kDecodeRows - 1) / kDecodeRows;
  const int nb = gateup ? I / 64 : H / 128;    // column blocks of the MXFP4 and affine launches
  const int nb8 = gateup ? I / 32 : H / 64;    // of the MXFP8 launch
  // Routed experts (MXFP4 or 2-bit affine); an MXFP4 shared group rides along
  // in the same launch, an MXFP8 one runs in a launch of its own.
  const dim3 grid(nb, E + (shared_w8 ? 0 : chunks));
  const dim3 grid_sh(nb8, chunks);
  // MXFP4 gate/up of a batch of at most 64 (token, slot) pairs: the narrow
  // blocks (measured at 4 tokens: gate/up -3 us; the down projection and
  // larger batches lose with them)
  const bool narrow = gateup && !routed_a2 && static_cast<long>(T) * k <= 64;
  const dim3 grid_n(I / 32, E + (shared_w8 ? 0 : chunks));
  uint16_t* ho = gateup ? h : nullptr;
  uint16_t* oo = gateup ? nullptr : out_rows;
#define MOE_DECODE_LAUNCH(G, KTW)                                                                                 \
  do {                                                                                                          \
    if (routed_a2)                                                                                              \
      ffn_decode_kernel<G, KTW, kFmtA2><<<grid, 64 * kWaves, 0, s>>>(act, row_token, offsets, E, E, blob, eb, H, \
                                                                     I, limit, ho, oo);                         \
    else if (G && narrow)                                                                                       \
      ffn_decode_kernel<G, KTW, kFmtMx4, true><<<grid_n, 64 * kWaves, 0, s>>>(act, row_token, offsets, E, E,    \
                                                                              blob, eb, H, I, limit, ho, oo);   \
    else                                                                                                        \
      ffn_decode_kernel<G, KTW, kFmtMx4><<<grid, 64 * kWaves, 0, s>>>(act, row_token, offsets, E, E, blob, eb,  \
                                                                      H, I, limit, ho, oo);                     \
    if (shared_w8)                                                                                              \
      ffn_decode_kernel<G, KTW, kFmtMx8><<<grid_sh, 64 * kWaves, 0, s>>>(act, row_token, offsets, E, 0, blob,   \
                                                                         eb, H, I, limit, ho, oo);              \
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
