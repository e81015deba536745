// Expert FFN, prefill family on the scaled MXFP4 matrix cores.  Same
// arithmetic as the decode family over items of up to 64 rows
// ("Model techniques map -- DeepSeek-V4-Flash", row "SwiGLU feed-forward";
// MXFP4 weights as in "ElytronAI / DeepSeek-v4-Flash", Sizes).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 takes the weights as they are stored --
// E2M1 codes with one E8M0 scale per 32 k -- but its other operand must be
// an 8-bit (or narrower) float.  A bf16 activation v is therefore carried as
// two E4M3 terms with one E8M0 scale S per 32 consecutive k:
//   v = S * hi + (S / 16) * lo,   hi = RNE_e4m3(v / S),  lo = RNE_e4m3(16 (v / S - hi)),
// with S = 2^(floor(log2 max|v|) - 7), so |v| / S < 256 and |lo| <= 128.  hi
// keeps the top 4 significant bits of v and lo the remaining 4, so the sum is
// exactly v for every element within 2^13 of the block maximum: there v / S
// >= 2^-6 and the 4 bits of 16 (v / S - hi) lie on the E4M3 grid.  Smaller
// elements lose only what falls below the E4M3 subnormal step 2^-9 of lo,
// S * 2^-14 <= 2^-21 of the block maximum.  Each 16x16x128 product is two MFMAs, hi
// then lo, at the FP8 rate -- the bf16 rate overall -- and the weights need no
// conversion instructions at all.
#include "ffn_internal.h"

namespace moe {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// The split of one 32-value block: its E8M0 scale byte from the block's
// largest magnitude (S = 2^(e - 7) for amax = 2^e * 1.m, so amax / S lies in
// [128, 256); the byte is kept >= 4 so that S / 16 is representable too), 1 / S,
// and the hi, lo E4M3 codes of two values (bytes 0 and 1 of each result).
__device__ __forceinline__ int split_scale_byte(float amax) {
  return max(static_cast<int>((__float_as_uint(amax) >> 23) & 255u) - 7, 4);
}
__device__ __forceinline__ float split_inv_scale(int sb) { return __uint_as_float(static_cast<uint32_t>(254 - sb) << 23); }
__device__ __forceinline__ void split_pair(float v0, float v1, float inv, int& hi, int& lo) {
  const float a0 = v0 * inv, a1 = v1 * inv;
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.f * (a0 - __builtin_amdgcn_cvt_f32_fp8(hi, 0)),
                                       16.f * (a1 - __builtin_amdgcn_cvt_f32_fp8(hi, 1)), 0, false);
}

// Activation split: one thread per 32 consecutive k of one row.
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ src, int rows, int K,
                                                        QAct dst) {
  const int nb = K >> 5;
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long>(rows) * nb) return;
  const long row = idx / nb;
  const int blk = static_cast<int>(idx - row * nb);
  const u32x4* p = reinterpret_cast<const u32x4*>(src + row * K + 32 * blk);
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = p[i];
  float f[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t w = v[i >> 3][(i >> 1) & 3];
    f[i] = __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    amax = fmaxf(amax, fabsf(f[i]));
  }
  const int sb = split_scale_byte(amax);  // E8M0 byte of S (lo uses sb - 4)
  const float inv = split_inv_scale(sb);
  u32x4 hi[2], lo[2];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    int h0, l0, h1, l1;
    split_pair(f[4 * w], f[4 * w + 1], inv, h0, l0);
    split_pair(f[4 * w + 2], f[4 * w + 3], inv, h1, l1);
    hi[w >> 2][w & 3] = (static_cast<uint32_t>(h0) & 0xffffu) | (static_cast<uint32_t>(h1) << 16);
    lo[w >> 2][w & 3] = (static_cast<uint32_t>(l0) & 0xffffu) | (static_cast<uint32_t>(l1) << 16);
  }
  u32x4* ph = reinterpret_cast<u32x4*>(dst.hi + row * K + 32 * blk);
  u32x4* pl = reinterpret_cast<u32x4*>(dst.lo + row * K + 32 * blk);
  ph[0] = hi[0];
  ph[1] = hi[1];
  pl[0] = lo[0];
  pl[1] = lo[1];
  dst.sc[row * nb + blk] = static_cast<uint8_t>(sb);
}

// ---------------------------------------------------------------------------
constexpr int kStages = 4;
constexpr int kWaves = 4;                         // side by side along the columns
constexpr int kThreads = 64 * kWaves;
constexpr int kNT = 4;                            // weight n-tiles (16 columns) per wave
constexpr int kRowBytes = 128;                    // one 128-k tile row of hi (or lo)
constexpr int kPlane = kPrefillRows * kRowBytes;  // hi (or lo) of one stage
constexpr int kStageBytes = 2 * kPlane + kPrefillRows * 4;
constexpr int kDmaOps = kPlane / (16 * kThreads);  // 16-byte DMA chunks per lane per plane per tile

// LDS slot of 16-byte chunk c (0..7) of tile row r: the XOR spreads the 16
// rows of an MFMA fragment read over all banks (rows are 128 bytes apart).
__device__ __forceinline__ int a_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

// grid (n blocks, max items) of 256 threads = 4 waves, two blocks per CU.  A
// block covers 64 rows x 256 weight columns, a wave 64 rows x 4 n-tiles
// (GATEUP: 2 gate + 2 up n-tiles of the same 32 output columns).  Operand
// layouts of the 16x16x128 instruction (checked on the device): A lane l holds
// row l % 16 at k = 16 (l / 16) + 0..15 and 64 + 16 (l / 16) + 0..15; B lane l
// holds column l % 16 at k = 32 (l / 16) + 0..31 -- the tiled weight layout
// as stored; the scale of A row r, k block p comes from lane 16 p + r, that
// of B column c, k block p from lane 16 p + c, byte op_sel of its register.
//
// Per stage the LDS holds the item's hi and lo rows of one 128-k tile
// (64 x 128 bytes each, chunk c of row r at slot c ^ ((r / 2) mod 8)) and their
// scales (4 bytes per row); all three arrive by LDS-DMA.  Pipeline, barriers
// and block order (with its grid slack) as in the bf16 prefill kernel.
template <bool GATEUP>
__global__ __launch_bounds__(kThreads, 2) void ffn_prefill_f8_kernel(QAct aq, const int32_t* __restrict__ row_token,
                                                                 const int4* __restrict__ items,
                                                                 const int32_t* __restrict__ n_items,
                                                                 const uint8_t* __restrict__ blob,
                                                                 uint64_t expert_bytes, int H, int I, float limit,
                                                                 QAct hq, uint16_t* __restrict__ out_rows) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages][kStageBytes];
  const int nbc = gridDim.x;
  const int nit = *n_items;
  const int total = nit * nbc;
  const int b = blockIdx.x + blockIdx.y * nbc;
  const int per = (total + 7) >> 3;
  if ((b >> 3) >= per) return;
  const int lam = (b & 7) * per + (b >> 3);
  if (lam >= total) return;
  int item, nb;
  window_unit(lam, nit, nbc, item, nb);
  const int4 it = items[item];
  const int g = it.x, row0 = it.y, nrows = it.z;
  const int K = GATEUP ? H : I;
  const int KT = K >> 7;  // a multiple of 4
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave;
  const ExpertPlanes pl = expert_planes(H, I);
  const uint8_t* eb = blob + static_cast<uint64_t>(g) * expert_bytes;
  const uint64_t tstride = static_cast<uint64_t>(KT) * 1024;  // bytes between n-tiles
  const uint64_t sstride = static_cast<uint64_t>(KT >> 2) * 256;

  const uint8_t* nb0;
  const uint8_t* nb1;
  const uint8_t* sb0;
  const uint8_t* sb1;
  if (GATEUP) {
    const int nt0 = nb * 8 + wn * 2;  // 2 gate then 2 up n-tiles of the same columns
    nb0 = eb + pl.gate_nib + nt0 * tstride;
    nb1 = eb + pl.up_nib + nt0 * tstride;
    sb0 = eb + pl.gate_sc + nt0 * sstride;
    sb1 = eb + pl.up_sc + nt0 * sstride;
  } else {
    const int nt0 = nb * 16 + wn * 4;
    nb0 = eb + pl.down_nib + nt0 * tstride;
    nb1 = nb0 + 2 * tstride;
    sb0 = eb + pl.down_sc + nt0 * sstride;
    sb1 = sb0 + 2 * sstride;
  }
  nb0 += lane * 16;
  nb1 += lane * 16;
  sb0 += lane * 4;
  sb1 += lane * 4;

  // LDS-DMA sources.  Op q of wave w fills 8 tile rows 8 (4q + w) + lane / 8
  // of a plane (1 KB per wave); the lane landing in slot s loads chunk
  // a_slot(r, s) (the XOR is its own inverse).  Rows past the item reload its
  // last row (never stored).  Wave 0 also fetches the 64 rows' 4 scale bytes.
  const int nbk = K >> 5;
  long arow_off[kDmaOps];
#pragma unroll
  for (int q = 0; q < kDmaOps; ++q) {
    const int r = 8 * (kWaves * q + wave) + (lane >> 3);
    const int p = row0 + min(r, nrows - 1);
    const long src_row = GATEUP ? static_cast<long>(row_token[p]) : static_cast<long>(p);
    arow_off[q] = src_row * K + 16 * a_slot(r, lane & 7);
  }
  const int srow = row0 + min(lane, nrows - 1);
  const uint8_t* sc_src = aq.sc + (GATEUP ? static_cast<long>(row_token[srow]) : static_cast<long>(srow)) * nbk;

  u32x4 bq[kStages][kNT];
  uint32_t sw[kNT], swn[kNT];
  auto issue_tile = [&](int stage, int kt) {
#pragma unroll
    for (int j = 0; j < kNT; ++j) bq[stage][j] = ld16((j < 2 ? nb0 : nb1) + (j & 1) * tstride + kt * 1024);
#pragma unroll
    for (int q = 0; q < kDmaOps; ++q) {
      uint8_t* dst = &smem[stage][(8 * (kWaves * q + wave)) * kRowBytes];
      __builtin_amdgcn_global_load_lds(aq.hi + arow_off[q] + kt * 128, dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(aq.lo + arow_off[q] + kt * 128, dst + kPlane, 16, 0, 0);
    }
    if (wave == 0) __builtin_amdgcn_global_load_lds(sc_src + 4 * kt, &smem[stage][2 * kPlane], 4, 0, 0);
  };
  auto issue_scales = [&](uint32_t* dst, int grp) {
#pragma unroll
    for (int j = 0; j < kNT; ++j)
      dst[j] = *reinterpret_cast<const uint32_t*>((j < 2 ? sb0 : sb1) + (j & 1) * sstride + grp * 256);
  };

  f32x4 acc[4][kNT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue_scales(sw, 0);
  issue_tile(0, 0);
  issue_tile(1, 1);
  __builtin_amdgcn_sched_barrier(0);

  const int qa = lane >> 4;  // A: k chunks qa and 4 + qa; scale block qa
  const int groups = KT >> 2;
  for (int u = 0; u < groups; ++u) {
    const bool last = u + 1 == groups;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kt = 4 * u + i;
      if ((i & 1) == 0) {
        wait_vmcnt<0>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (i == 0 && !last) issue_scales(swn, u + 1);
        if (kt + 2 < KT) issue_tile((i + 2) % kStages, kt + 2);
        if (kt + 3 < KT) issue_tile((i + 3) % kStages, kt + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint8_t* st = smem[i];
      i32x8 bv[kNT];
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const u32x4 w = bq[i][j];
        bv[j] = i32x8{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]), static_cast<int>(w[3]),
                      0, 0, 0, 0};
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r = 16 * mt + (lane & 15);
        const uint8_t* rowp = st + r * kRowBytes;
        const u32x4 h0 = *reinterpret_cast<const u32x4*>(rowp + 16 * a_slot(r, qa));
        const u32x4 h1 = *reinterpret_cast<const u32x4*>(rowp + 16 * a_slot(r, 4 + qa));
        const u32x4 l0 = *reinterpret_cast<const u32x4*>(rowp + kPlane + 16 * a_slot(r, qa));
        const u32x4 l1 = *reinterpret_cast<const u32x4*>(rowp + kPlane + 16 * a_slot(r, 4 + qa));
        const uint32_t scw = *reinterpret_cast<const uint32_t*>(st + 2 * kPlane + 4 * r);
        const int sa_hi = static_cast<int>((scw >> (8 * qa)) & 255u);
        const int sa_lo = sa_hi - 4;
        const i32x8 ahi = {static_cast<int>(h0[0]), static_cast<int>(h0[1]), static_cast<int>(h0[2]),
                           static_cast<int>(h0[3]), static_cast<int>(h1[0]), static_cast<int>(h1[1]),
                           static_cast<int>(h1[2]), static_cast<int>(h1[3])};
        const i32x8 alo = {static_cast<int>(l0[0]), static_cast<int>(l0[1]), static_cast<int>(l0[2]),
                           static_cast<int>(l0[3]), static_cast<int>(l1[0]), static_cast<int>(l1[1]),
                           static_cast<int>(l1[2]), static_cast<int>(l1[3])};
#pragma unroll
        for (int j = 0; j < kNT; ++j)
          acc[mt][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ahi, bv[j], acc[mt][j], 0, 4, 0, sa_hi, 0,
                                                                        static_cast<int>(sw[j] >> (8 * i)));
#pragma unroll
        for (int j = 0; j < kNT; ++j)
          acc[mt][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(alo, bv[j], acc[mt][j], 0, 4, 0, sa_lo, 0,
                                                                        static_cast<int>(sw[j] >> (8 * i)));
      }
      // Pin this tile's products here: left alone, the compiler sinks the
      // MFMAs of two tiles below the next barrier and holds both tiles' A
      // fragments live across it, which spills.
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < kNT; ++j) asm volatile("" : "+v"(acc[mt][j]));
    }
    if (!last) {
#pragma unroll
      for (int j = 0; j < kNT; ++j) sw[j] = swn[j];
    }
  }

  const int g4 = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int rbase = mt * 16 + 4 * g4;
    if (GATEUP) {
      // h = bf16(silu(min(gate, L)) * clamp(up, -L, L)), written straight in
      // its split form: the wave's 32 output columns are one 32-k block of
      // the down projection, spread over the 16 lanes of a row group (columns
      // lane % 16 and 16 + lane % 16), so the block maximum is a 16-lane max.
      const int c0 = nb * 128 + wn * 32;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float hv[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float gv = fminf(acc[mt][j][e], limit);
          const float uv = fminf(fmaxf(acc[mt][j + 2][e], -limit), limit);
          hv[j] = bf16_bits_to_float(float_to_bf16_bits(silu_f(gv) * uv));
        }
        float m = fmaxf(fabsf(hv[0]), fabsf(hv[1]));
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 16));
        const int sb = split_scale_byte(m);
        int hi, lo;
        split_pair(hv[0], hv[1], split_inv_scale(sb), hi, lo);
        const int r = rbase + e;
        if (r < nrows) {
          const size_t o = static_cast<size_t>(row0 + r) * I + c0 + (lane & 15);
          hq.hi[o] = static_cast<uint8_t>(hi);
          hq.hi[o + 16] = static_cast<uint8_t>(hi >> 8);
          hq.lo[o] = static_cast<uint8_t>(lo);
          hq.lo[o + 16] = static_cast<uint8_t>(lo >> 8);
          if ((lane & 15) == 0) hq.sc[static_cast<size_t>(row0 + r) * (I >> 5) + (c0 >> 5)] = static_cast<uint8_t>(sb);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int col = nb * 256 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rbase + e;
          if (r < nrows) out_rows[static_cast<size_t>(row0 + r) * H + col] = float_to_bf16_bits(acc[mt][j][e]);
        }
      }
    }
  }
}

}  // namespace

void launch_quant_act(const uint16_t* src, int rows, int K, const QAct& dst, hipStream_t s) {
  const long n = static_cast<long>(rows) * (K >> 5);
  quant_act_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(src, rows, K, dst);
}

void launch_ffn_prefill_f8(bool gateup, const QAct& aq, const int32_t* row_token, const FfnWs& w,
                           const uint8_t* blob, uint64_t eb, int H, int I, float limit, uint16_t* out_rows,
                           int max_items, hipStream_t s) {
  if (gateup) {
    dim3 g1(I / 128, max_items + kGridSlack);
    ffn_prefill_f8_kernel<true><<<g1, kThreads, 0, s>>>(aq, row_token, w.items, w.n_items, blob, eb, H, I, limit,
                                                        w.hq, nullptr);
  } else {
    dim3 g2(H / 256, max_items + kGridSlack);
    ffn_prefill_f8_kernel<false><<<g2, kThreads, 0, s>>>(aq, nullptr, w.items, w.n_items, blob, eb, H, I, limit,
                                                         QAct{nullptr, nullptr, nullptr}, out_rows);
  }
}

}  // namespace moe
