// Expert FFN, prefill family (many rows per expert; MFMA bound).  Same
// arithmetic as the decode family over items of up to 64 rows
// ("Model techniques map -- DeepSeek-V4-Flash", row "SwiGLU feed-forward").
#include "ffn_internal.h"

namespace moe {

namespace {

constexpr int kStages = 4;        // ring depth of activation (LDS) and weight (register) tiles
constexpr int kWavesM = 1, kWavesN = 4;        // 4 waves side by side along the columns
constexpr int kThreads = 64 * kWavesM * kWavesN;
constexpr int kNT4 = 16 / kWavesN;               // weight n-tiles per wave (MXFP4)
constexpr int kDmaOps = kPrefillRows * 16 / kThreads;  // 16-byte activation chunks per lane per tile

// grid (n blocks, max items) of 256 threads = 4 waves side by side, two
// blocks per CU (64 KB of LDS each), so two waves per SIMD: each wave has 4 x 4
// MFMA 16x16x32 accumulators plus a four-deep ring of its weight fragments
// within half the register file, and one block's barriers, pipeline fill and
// epilogue overlap the other block's MFMAs.  Items hold up to 64 rows of one
// expert.  A block covers 64 rows x 256 weight columns: GATEUP -> 128 output
// columns (wave wn: gate and up n-tiles of output columns 32*wn .. 32*wn+31),
// otherwise 256 down columns (wave wn: 4 n-tiles).
//
// Activation tiles (64 rows x 128 k, 16 KB) go from global memory straight
// into LDS with the LDS-DMA load (global_load_lds_dwordx4) into a ring of
// four stages.  Row r of a tile occupies 256 bytes; its 16-byte chunk c sits
// at slot c ^ (r & 15), so an MFMA fragment read (16 rows, same chunk) hits 16
// distinct bank groups.  The DMA puts each wave's 64 lanes in 1 KB of
// contiguous LDS, so the swizzle is applied on the global side: the lane that
// lands in slot s of row r loads chunk s ^ (r & 15).
//
// Pipeline, in pairs of k tiles: after the barrier before tiles kt, kt+1
// (kt even), tiles kt+2 and kt+3 (weights into registers, then activations
// into LDS) are issued into the two stages freed by tiles kt-2, kt-1, and stay
// in flight while kt and kt+1 are multiplied; one barrier per pair halves the
// block-wide synchronisation.
//
// Block order is remapped so the n blocks of one item run on the same XCD:
// blocks go to the 8 XCDs round robin, and block b takes logical work
// b % 8 * ceil(total / 8) + b / 8, so consecutive logical blocks (the column
// blocks of one item, then the next item of the same expert) share an L2.
// That covers every logical block only if the grid has at least
// 8 * ceil(total / 8) blocks: launches add kGridSlack rows of blocks.
//
// W8: the items of an MXFP8 shared expert (group skip_g of the MXFP4 launch),
// which are the last n_w8 items of the work list.  Its 2048-byte weight
// tiles are read as two 1 KiB halves into a two-stage register ring (the
// same registers as four MXFP4 stages), one tile ahead: each tile drains the
// wave's loads and passes the barrier, then issues the next tile.
template <bool GATEUP, bool W8>
__global__ __launch_bounds__(kThreads, 2) void ffn_prefill_kernel(const uint16_t* __restrict__ act,
                                                             const int32_t* __restrict__ row_token,
                                                             const int4* __restrict__ items,
                                                             const int32_t* __restrict__ n_items,
                                                             const uint8_t* __restrict__ blob, uint64_t expert_bytes,
                                                             int H, int I, float limit, int skip_g, int n_w8,
                                                             uint16_t* __restrict__ h_out,
                                                             float* __restrict__ out_rows) {
  constexpr int kNT = kNT4;           // weight n-tiles per wave
  constexpr int NQ = W8 ? 2 : 1;      // 16-byte loads per lane per n-tile per k tile
  constexpr uint64_t kTileBytes = W8 ? 2048 : 1024;
  __shared__ __attribute__((aligned(1024))) uint16_t As[kStages][kPrefillRows * 128];
  const int nbc = gridDim.x;
  const int total = (W8 ? n_w8 : *n_items) * nbc;
  const int b = blockIdx.x + blockIdx.y * nbc;
  const int per = (total + 7) >> 3;
  if ((b >> 3) >= per) return;
  const int lam = (b & 7) * per + (b >> 3);
  if (lam >= total) return;
  const int4 it = items[(W8 ? *n_items - n_w8 : 0) + lam / nbc];
  const int nb = lam % nbc;
  const int g = it.x, row0 = it.y, nrows = it.z;
  if (!W8 && g == skip_g) return;  // the MXFP8 shared expert's items run in their own launch
  const int K = GATEUP ? H : I;
  const int KT = K >> 7;  // a multiple of 4
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const ExpertPlanes pl = W8 ? expert_planes8(H, I) : expert_planes(H, I);
  const uint8_t* eb = blob + static_cast<uint64_t>(g) * expert_bytes;
  const uint64_t tstride = static_cast<uint64_t>(KT) * kTileBytes;  // bytes between n-tiles
  const uint64_t sstride = static_cast<uint64_t>(KT >> 2) * 256;

  const uint8_t* nb0;
  const uint8_t* nb1;
  const uint8_t* sb0;
  const uint8_t* sb1;
  if (GATEUP) {
    const int nt0 = nb * 2 * kNT + wn * (kNT / 2);  // kNT/2 gate then kNT/2 up n-tiles of the same columns
    nb0 = eb + pl.gate_nib + nt0 * tstride;
    nb1 = eb + pl.up_nib + nt0 * tstride;
    sb0 = eb + pl.gate_sc + nt0 * sstride;
    sb1 = eb + pl.up_sc + nt0 * sstride;
  } else {
    const int nt0 = nb * 4 * kNT + wn * kNT;
    nb0 = eb + pl.down_nib + nt0 * tstride;
    nb1 = nb0 + (kNT / 2) * tstride;
    sb0 = eb + pl.down_sc + nt0 * sstride;
    sb1 = sb0 + (kNT / 2) * sstride;
  }
  nb0 += lane * 16;
  nb1 += lane * 16;
  sb0 += lane * 4;
  sb1 += lane * 4;

  // LDS-DMA sources: op q of wave w fills rows 16q + 4w + lane/16.  Rows past
  // the item reload its last row (never stored).
  const char* asrc[kDmaOps];
#pragma unroll
  for (int q = 0; q < kDmaOps; ++q) {
    const int r = (kThreads / 16) * q + 4 * wave + (lane >> 4);
    const int p = row0 + min(r, nrows - 1);
    const uint16_t* rowp = GATEUP ? act + static_cast<size_t>(row_token[p]) * H : act + static_cast<size_t>(p) * I;
    asrc[q] = reinterpret_cast<const char*>(rowp) + 16 * ((lane & 15) ^ (r & 15));
  }

  constexpr int kH = kNT / 2;
  u32x4 bq[W8 ? 2 : kStages][kNT][NQ];  // W8: a two-stage ring (twice the bytes per tile)
  uint32_t sw[kNT], swn[kNT];
  auto issue_tile = [&](int stage, int kt) {
#pragma unroll
    for (int j = 0; j < kNT; ++j)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        bq[stage][j][q] = ld16((j < kH ? nb0 : nb1) + (j % kH) * tstride + kt * kTileBytes + q * 1024);
#pragma unroll
    for (int q = 0; q < kDmaOps; ++q)
      __builtin_amdgcn_global_load_lds(asrc[q] + kt * 256, &As[stage][((kThreads / 16) * q + 4 * wave) * 128], 16,
                                       0, 0);
  };
  auto issue_scales = [&](uint32_t* dst, int grp) {
#pragma unroll
    for (int j = 0; j < kNT; ++j)
      dst[j] = *reinterpret_cast<const uint32_t*>((j < kH ? sb0 : sb1) + (j % kH) * sstride + grp * 256);
  };

  f32x4 acc[4][kNT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int arow = wm * 64 + (lane & 15);
  const int g4 = lane >> 4;
  const int groups = KT >> 2;
  // Tile kt = 4u + i from LDS stage st and register stage sb (scale byte i).
  auto compute_tile = [&](int i, int st, int sb) {
    float scf[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) scf[j] = e8m0_scale_operand_of(sw[j], i);
    const uint16_t* abuf = As[st];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a[4];
      const int slot = ((4 * g4 + s) ^ (lane & 15)) * 8;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a[mt] = *reinterpret_cast<const bf16x8*>(abuf + (arow + 16 * mt) * 128 + slot);
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        // k = 32 (lane / 16) + 8 s + 0..7 of the tile: 8 E2M1 codes of word
        // s, or 8 E4M3 codes of words 2 (s % 2), +1 of half s / 2
        bf16x8 bv;
        if constexpr (W8) {
          const u32x4& hw = bq[sb][j][s >> 1];
          bv = dequant8_fp8(hw[2 * (s & 1)], hw[2 * (s & 1) + 1], scf[j]);
        } else {
          bv = dequant8(bq[sb][j][0][s], scf[j]);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][j] = mfma16x16x32(a[mt], bv, acc[mt][j]);
      }
    }
  };
  if constexpr (W8) {
    issue_scales(sw, 0);
    issue_tile(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    for (int u = 0; u < groups; ++u) {
      const bool last = u + 1 == groups;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kt = 4 * u + i;
        wait_vmcnt<0>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (i == 3 && !last) issue_scales(swn, u + 1);
        if (kt + 1 < KT) issue_tile((i + 1) & 1, kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute_tile(i, i & 1, i & 1);
      }
      if (!last) {
#pragma unroll
        for (int j = 0; j < kNT; ++j) sw[j] = swn[j];
      }
    }
  } else {
    issue_scales(sw, 0);
    issue_tile(0, 0);
    issue_tile(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int u = 0; u < groups; ++u) {
      const bool last = u + 1 == groups;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kt = 4 * u + i;
        // Every second tile: tiles kt and kt+1 (issued two tiles ago) are the
        // last ops issued, so the wave drains its counter; the barrier then
        // publishes all waves' DMA writes of both and frees the two stages of
        // tiles kt-2, kt-1 for tiles kt+2, kt+3.
        if ((i & 1) == 0) {
          wait_vmcnt<0>();
          lds_barrier();
          __builtin_amdgcn_sched_barrier(0);
          if (i == 0 && !last) issue_scales(swn, u + 1);
          if (kt + 2 < KT) issue_tile((i + 2) % kStages, kt + 2);
          if (kt + 3 < KT) issue_tile((i + 3) % kStages, kt + 3);
          __builtin_amdgcn_sched_barrier(0);
        }
        compute_tile(i, i, i);
      }
      if (!last) {
#pragma unroll
        for (int j = 0; j < kNT; ++j) sw[j] = swn[j];
      }
    }
  }

#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int rbase = wm * 64 + mt * 16 + 4 * g4;
    if (GATEUP) {
#pragma unroll
      for (int j = 0; j < kH; ++j) {
        const int col = nb * (64 * kH) + wn * (16 * kH) + j * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rbase + e;
          if (r < nrows) {
            const float gv = fminf(acc[mt][j][e], limit);
            const float uv = fminf(fmaxf(acc[mt][j + kH][e], -limit), limit);
            h_out[static_cast<size_t>(row0 + r) * I + col] = float_to_bf16_bits(silu_f(gv) * uv);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int col = nb * (64 * kNT) + wn * (16 * kNT) + j * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rbase + e;
          if (r < nrows) out_rows[static_cast<size_t>(row0 + r) * H + col] = acc[mt][j][e];
        }
      }
    }
  }
}

}  // namespace

void launch_ffn_prefill(bool gateup, const uint16_t* act, const int32_t* row_token, const FfnWs& w,
                        const uint8_t* blob, uint64_t eb, int H, int I, float limit, float* out_rows, int max_items,
                        int T, int E, bool shared_w8, hipStream_t s) {
  // the MXFP8 shared expert's items (the last ceil(T / 64) of the work list) in a launch of their own
  const int skip = shared_w8 ? E : -1;
  const int nsh = (T + kPrefillRows - 1) / kPrefillRows;
  const int ny = max_items + kGridSlack, ny8 = nsh + kGridSlack;
  if (gateup) {
    ffn_prefill_kernel<true, false><<<dim3(I / 128, ny), kThreads, 0, s>>>(
        act, row_token, w.items, w.n_items, blob, eb, H, I, limit, skip, 0, w.h, nullptr);
    if (shared_w8)
      ffn_prefill_kernel<true, true><<<dim3(I / 128, ny8), kThreads, 0, s>>>(act, row_token, w.items, w.n_items, blob,
                                                                           eb, H, I, limit, -1, nsh, w.h, nullptr);
  } else {
    ffn_prefill_kernel<false, false><<<dim3(H / 256, ny), kThreads, 0, s>>>(
        act, nullptr, w.items, w.n_items, blob, eb, H, I, limit, skip, 0, nullptr, out_rows);
    if (shared_w8)
      ffn_prefill_kernel<false, true><<<dim3(H / 256, ny8), kThreads, 0, s>>>(
          act, nullptr, w.items, w.n_items, blob, eb, H, I, limit, -1, nsh, nullptr, out_rows);
  }
}

}  // namespace moe
