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

// grid (column blocks / UPB, max items) of 256 threads = 4 waves side by side, two
// blocks per CU (64 KB of LDS each), so two waves per SIMD: each wave has 4 x 4
// MFMA 16x16x32 accumulators plus a four-deep ring of its weight fragments
// within half the register file, and one block's barriers, pipeline fill and
// epilogue overlap the other block's MFMAs.  Items hold up to 64 rows of one
// expert.  A block covers 64 rows x 256 weight columns: GATEUP -> 128 output
// columns (wave wn: gate and up n-tiles of output columns 32*wn .. 32*wn+31),
// otherwise 256 down columns (wave wn: 4 n-tiles).
//
// Activation tiles (64 rows x 128 k, 16 KB) go from global memory straight
// into LDS with the LDS-DMA load (buffer_load_dwordx4 ... lds) into a ring of
// four stages.  Row r of a tile occupies 256 bytes; its 16-byte chunk c sits
// at slot c ^ (r & 15), so an MFMA fragment read (16 rows, same chunk) hits 16
// distinct bank groups.  The DMA puts each wave's 64 lanes in 1 KB of
// contiguous LDS, so the swizzle is applied on the global side: the lane that
// lands in slot s of row r loads chunk s ^ (r & 15).
//
// Addresses stay scalar where they can: weight and scale loads go through one
// buffer resource per n-tile and the activation DMA through one over x (or
// over the item's rows of h), so a lane's 32-bit offset is the only vector
// operand and the k-tile advance is a scalar offset.
//
// Epilogue: the output tile is assembled in the activation ring (idle once
// the k loop is done) and written in 16-byte stores of whole rows, marked
// non-temporal: the rows are read back only by the next launch, and the L2
// keeps the weight slices and activation rows the XCD's blocks share.
//
// Pipeline, in pairs of k tiles: after the barrier before tiles kt, kt+1
// (kt even), tiles kt+2 and kt+3 (weights into registers, then activations
// into LDS) are issued into the two stages freed by tiles kt-2, kt-1, and stay
// in flight while kt and kt+1 are multiplied; one barrier per pair halves the
// block-wide synchronisation.
//
// Block order is remapped so consecutive logical blocks run on the same XCD:
// blocks go to the 8 XCDs round robin, and block b takes logical work
// b % 8 * ceil(total / 8) + b / 8; logical blocks walk windows of items x
// column blocks (window_unit), so the blocks an XCD runs at once share
// weight slices and activation rows in its L2.
// That covers every logical block only if the grid has at least
// 8 * ceil(total / 8) blocks: launches add kGridSlack rows of blocks.
//
// A launch covers the whole work list, or (n_tail > 0) only its last n_tail
// items -- the shared expert's, which come last -- and its blocks of group
// skip_g return at once (that group runs in a launch of its own).
//
// FMT kFmtMx8: an MXFP8 shared expert.  Its 2048-byte weight tiles are read
// as two 1 KiB halves into a two-stage register ring (the same registers as
// four MXFP4 stages), one tile ahead: each tile drains the wave's loads and
// passes the barrier, then issues the next tile.
//
// FMT kFmtA2: 2-bit affine routed experts ("OsaurusAI /
// DeepSeek-V4-Flash-0731-JANG", Dynamic affine recipe).  Each 512-byte code
// tile (8 bytes a lane) and its (scale, bias) words ride in the MXFP4 ring
// and pipeline; per group of G input columns (64 for gate and up, 32 for
// down) the MFMAs run x against the exact bf16 codes q (P) and against ones
// (S, the row sums of x over the group), and acc += s * P + b * S -- the
// group's sum x . (s q + b), regrouped.
// One block's unit: item (g, row0, nrows) of group g, column block nb, as MT
// 16-row tiles (MT = 4: the full 64; fewer skip the MFMAs, activation loads and
// stores of row tiles past the item's rows).  As: the block's activation ring.
// X64: x spans more than 4 GiB, so the MXFP4 gate/up instance gathers its
// token rows by 64-bit address instead of a 32-bit offset.
template <bool GATEUP, int FMT, int MT, bool X64>
__device__ __forceinline__ void prefill_unit(const uint16_t* __restrict__ act, const int32_t* __restrict__ row_token,
                                             const uint8_t* __restrict__ blob, uint64_t expert_bytes, int H, int I,
                                             float limit, uint16_t* __restrict__ h_out,
                                             uint16_t* __restrict__ out_rows, int g, int row0, int nrows,
                                             int nb_first, int nub, uint16_t (*As)[kPrefillRows * 128]) {
  constexpr bool W8 = FMT == kFmtMx8;
  constexpr bool A2 = FMT == kFmtA2;
  constexpr int kNT = kNT4;           // weight n-tiles per wave
  constexpr int NQ = W8 ? 2 : 1;      // 16-byte loads per lane per n-tile per k tile
  constexpr uint64_t kTileBytes = W8 ? 2048 : A2 ? 512 : 1024;
  constexpr int G = GATEUP ? 64 : 32;  // affine group size
  constexpr int NG = 128 / G;          // affine groups per k tile
  constexpr int SPG = G / 32;          // MFMA k steps per affine group
  constexpr uint64_t kSbBytes = 16 * NG * 4;  // affine (scale, bias) words of a 16 x 128 tile
  typedef __attribute__((__vector_size__(NG * sizeof(unsigned)))) unsigned u32xg;
  const int K = GATEUP ? H : I;
  const int KT = K >> 7;  // a multiple of 4
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const ExpertPlanes pl = W8 ? expert_planes8(H, I) : A2 ? expert_planes_a2(H, I) : expert_planes(H, I);
  const uint8_t* eb = blob + static_cast<uint64_t>(g) * expert_bytes;
  const uint64_t tstride = static_cast<uint64_t>(KT) * kTileBytes;  // bytes between n-tiles
  // bytes between n-tiles of the scale plane (MX: one 256-byte block per 4 k
  // tiles; affine: kSbBytes per k tile)
  const uint64_t sstride = A2 ? static_cast<uint64_t>(KT) * kSbBytes : static_cast<uint64_t>(KT >> 2) * 256;

  // LDS-DMA sources: op q of wave w fills rows 16q + 4w + lane/16.  Rows past
  // the item reload its last row (never stored).
  constexpr int kDmaOps = MT;  // 16-byte activation chunks per lane per tile (16 MT rows)
  // The down projection reads the item's own rows of h, the MXFP4 gate/up
  // the token rows it gathers from x (below 4 GiB), each through a buffer
  // resource, with 32-bit lane offsets and the k-tile advance scalar; the
  // other gate/up instances gather by 64-bit address.
  constexpr bool kDma64 = GATEUP && (X64 || FMT != kFmtMx4);
  const char* asrc[4];         // (a size that depends on MT here drops the kernel's host stub)
  uint32_t aoff[4];
  // (gate/up: the whole of x, whose size the host checked against 4 GiB)
  const __amdgpu_buffer_rsrc_t arc =
      raw_buffer(act + (GATEUP ? 0 : static_cast<size_t>(row0) * I), GATEUP ? -1 : nrows * I * 2);
#pragma unroll
  for (int q = 0; q < kDmaOps; ++q) {
    const int r = (kThreads / 16) * q + 4 * wave + (lane >> 4);
    const int rr = min(r, nrows - 1);
    const int p = row0 + rr;
    const uint32_t cb = 16 * ((lane & 15) ^ (r & 15));
    if constexpr (kDma64)
      asrc[q] = reinterpret_cast<const char*>(act + static_cast<size_t>(row_token[p]) * H) + cb;
    else if constexpr (GATEUP)
      aoff[q] = static_cast<uint32_t>(row_token[p]) * static_cast<uint32_t>(H * 2) + cb;
    else
      aoff[q] = static_cast<uint32_t>(rr) * (I * 2) + cb;
  }

  // One pass per column block nb_first .. nb_first + nub - 1 of the item; the
  // body (weight addressing, k loop, epilogue) runs to the end of the
  // function at this indentation.
#pragma unroll 1
  for (int u = 0; u < nub; ++u) {
  const int nb = nb_first + u;
  if (u > 0) __syncthreads();  // the previous unit's copy-out is done with the ring
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
  // The bases above are uniform; a lane adds one 32-bit offset.  MX weight
  // and scale loads go through one buffer resource per n-tile (its bytes over
  // all k: at most 1 MiB of codes, 32 KiB of scales), so the k-tile advance is
  // a scalar offset and the lane offset the only vector operand.
  const uint32_t loff = lane * (A2 ? 8 : 16);
  // affine: the (scale, bias) words of output column lane % 16 (MFMA result layout)
  const uint32_t soff = A2 ? (lane & 15) * (NG * 4) : lane * 4;
  __amdgpu_buffer_rsrc_t wrc[kNT], src[kNT];
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    wrc[j] = raw_buffer((j < kNT / 2 ? nb0 : nb1) + (j % (kNT / 2)) * tstride, static_cast<int>(tstride));
    src[j] = raw_buffer((j < kNT / 2 ? sb0 : sb1) + (j % (kNT / 2)) * sstride, static_cast<int>(sstride));
  }

  constexpr int kH = kNT / 2;
  u32x4 bq[A2 ? 1 : W8 ? 2 : kStages][kNT][NQ];  // W8: a two-stage ring (twice the bytes per tile)
  u32x2 bq2[A2 ? kStages : 1][kNT];              // affine codes
  u32xg sq2[A2 ? kStages : 1][kNT];              // affine (scale, bias) words
  uint32_t sw[kNT], swn[kNT];
  auto issue_tile = [&](int stage, int kt) {
    if constexpr (A2) {
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        bq2[stage][j] = *reinterpret_cast<const u32x2*>((j < kH ? nb0 : nb1) + (j % kH) * tstride + kt * kTileBytes + loff);
        sq2[stage][j] = *reinterpret_cast<const u32xg*>((j < kH ? sb0 : sb1) + (j % kH) * sstride + kt * kSbBytes + soff);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kNT; ++j)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          bq[stage][j][q] =
              __builtin_amdgcn_raw_buffer_load_b128(wrc[j], loff, kt * static_cast<int>(kTileBytes) + q * 1024, 0);
    }
#pragma unroll
    for (int q = 0; q < kDmaOps; ++q) {
      if constexpr (kDma64)
        __builtin_amdgcn_global_load_lds(asrc[q] + kt * 256, &As[stage][((kThreads / 16) * q + 4 * wave) * 128], 16,
                                         0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(arc, &As[stage][((kThreads / 16) * q + 4 * wave) * 128], 16, aoff[q],
                                                 kt * 256, 0, 0);
    }
  };
  auto issue_scales = [&](uint32_t* dst, int grp) {
#pragma unroll
    for (int j = 0; j < kNT; ++j)
      dst[j] = __builtin_amdgcn_raw_buffer_load_b32(src[j], soff, grp * 256, 0);
  };

  f32x4 acc[MT][kNT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
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
    // k = 32 (lane / 16) + 8 s + 0..7 of the tile: 8 E2M1 codes of word s, or
    // 8 E4M3 codes of words 2 (s % 2), +1 of half s / 2
    auto conv = [&](int s, int j) -> bf16x8 {
      if constexpr (W8) {
        const u32x4& hw = bq[sb][j][s >> 1];
        return dequant8_fp8(hw[2 * (s & 1)], hw[2 * (s & 1) + 1], scf[j]);
      } else {
        return dequant8(bq[sb][j][0][s], scf[j]);
      }
    };
    // The B operand of the next (s, j) group is converted before the current
    // group's MFMAs are issued, so its conversions overlap them.
    bf16x8 bcur = conv(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a[MT];
      const int slot = ((4 * g4 + s) ^ (lane & 15)) * 8;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[mt] = *reinterpret_cast<const bf16x8*>(abuf + (arow + 16 * mt) * 128 + slot);
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int ns = j + 1 < kNT ? s : s + 1, nj = j + 1 < kNT ? j + 1 : 0;
        bf16x8 bnext = bcur;
        if (ns < 4) bnext = conv(ns, nj);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][j] = mfma16x16x32(a[mt], bcur, acc[mt][j]);
        bcur = bnext;
      }
    }
  };
  // Affine tile kt from LDS stage st (codes and (scale, bias) words in ring
  // stage st): group by group, the row sums S of each row tile, then per
  // n-tile the group's MFMAs into fresh P (four row-tile chains) and the folds.
  auto compute_tile_a2 = [&](int st) {
    const uint16_t* abuf = As[st];
    const u32x4 ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
    const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_w);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      bf16x8 a[SPG][MT];
      f32x4 S[MT];
#pragma unroll
      for (int ss = 0; ss < SPG; ++ss) {
        const int s = gi * SPG + ss;
        // MFMA step s takes k = 32 s + 8 (lane / 16) + 0..7: 16-byte chunk 4 s + lane / 16 of the row
        const int slot = ((4 * s + g4) ^ (lane & 15)) * 8;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) a[ss][mt] = *reinterpret_cast<const bf16x8*>(abuf + (arow + 16 * mt) * 128 + slot);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ss = 0; ss < SPG; ++ss) S[mt] = mfma16x16x32(a[ss][mt], ones, S[mt]);
      }
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        f32x4 P[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) P[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ss = 0; ss < SPG; ++ss) {
          const int s = gi * SPG + ss;
          // code i of step s: bits 4i + 2 (s % 2) of word s / 2 -> E2M1 nibbles 00qq = q / 2
          const uint32_t w = bq2[st][j][s >> 1];
          const uint32_t nib = ((s & 1) ? (w >> 2) : w) & 0x33333333u;
          const bf16x8 bv = dequant8(nib, e8m0_scale_operand(128u));  // scale 2: the bf16 values q
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) P[mt] = mfma16x16x32(a[ss][mt], bv, P[mt]);
        }
        const uint32_t sbw = sq2[st][j][gi];
        const float sc = __uint_as_float(sbw << 16);          // bf16 scale (low half)
        const float bc = __uint_as_float(sbw & 0xffff0000u);  // bf16 bias (high half)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mt][j][e] = fmaf(bc, S[mt][e], fmaf(sc, P[mt][e], acc[mt][j][e]));
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
    if (!A2) issue_scales(sw, 0);
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
          if (!A2 && i == 0 && !last) issue_scales(swn, u + 1);
          if (kt + 2 < KT) issue_tile((i + 2) % kStages, kt + 2);
          if (kt + 3 < KT) issue_tile((i + 3) % kStages, kt + 3);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (A2) {
          compute_tile_a2(i);
          // keep each tile's MFMAs and folds above the next barrier (the
          // compiler otherwise sinks them and runs out of registers)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < kNT; ++j) asm volatile("" : "+v"(acc[mt][j]));
        } else {
          compute_tile(i, i, i);
        }
      }
      if (!A2 && !last) {
#pragma unroll
        for (int j = 0; j < kNT; ++j) sw[j] = swn[j];
      }
    }
  }

  // Epilogue: the block's output tile (64 rows x 128 h columns, or 64 x 256
  // down columns, bf16) is assembled in the free activation ring, rows
  // padded by 16 bytes so the 16-row MFMA result columns land on distinct
  // banks, then written out in 16-byte chunks, whole rows at a time.
  constexpr int kOutCols = GATEUP ? 16 * kH * kWavesN : 16 * kNT * kWavesN;  // 128 or 256
  constexpr int kStageLd = kOutCols + 8;                                       // uint16 elements per staged row
  static_assert(kPrefillRows * kStageLd <= kStages * kPrefillRows * 128, "staged tile fits the ring");
  uint16_t* stg = &As[0][0];
  __syncthreads();  // every wave is done with the ring's last tiles
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int rbase = wm * 64 + mt * 16 + 4 * g4;
    if (GATEUP) {
#pragma unroll
      for (int j = 0; j < kH; ++j) {
        const int c = wn * (16 * kH) + j * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gv = fminf(acc[mt][j][e], limit);
          const float uv = fminf(fmaxf(acc[mt][j + kH][e], -limit), limit);
          stg[(rbase + e) * kStageLd + c] = float_to_bf16_bits(silu_f(gv) * uv);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int c = wn * (16 * kNT) + j * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) stg[(rbase + e) * kStageLd + c] = float_to_bf16_bits(acc[mt][j][e]);
      }
    }
  }
  __syncthreads();
  constexpr int kChunks = kOutCols / 8;  // 16-byte chunks per row
  uint16_t* const dst = GATEUP ? h_out + static_cast<size_t>(row0) * I + nb * kOutCols
                               : out_rows + static_cast<size_t>(row0) * H + nb * kOutCols;
  const int ld = GATEUP ? I : H;
#pragma unroll
  for (int i = 0; i < (16 * MT * kChunks) / kThreads; ++i) {
    const int cidx = i * kThreads + tid;
    const int r = cidx / kChunks, c = cidx % kChunks;
    if (r < nrows)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stg + r * kStageLd + 8 * c),
                                  reinterpret_cast<u32x4*>(dst + static_cast<size_t>(r) * ld + 8 * c));
  }
  }
}

// grid (n blocks / UPB, max items + kGridSlack) of 256 threads; see above.
// SW: a block of an item with fewer than 64 rows runs the unit with
// ceil(rows / 16) row tiles (a launch option for work lists of many partial
// items: its register allocation is the largest unit's, and it is chosen on
// the host).  UPB: column blocks a block takes in turn (same item, adjacent
// column blocks), so the item lookup, the gathered rows' offsets and the
// block's launch are paid once per UPB units.
template <bool GATEUP, int FMT, bool SW = false, bool X64 = false, int UPB = 1>
__global__ __launch_bounds__(kThreads, 2) void ffn_prefill_kernel(const uint16_t* __restrict__ act,
                                                             const int32_t* __restrict__ row_token,
                                                             const int4* __restrict__ items,
                                                             const int32_t* __restrict__ n_items,
                                                             const uint8_t* __restrict__ blob, uint64_t expert_bytes,
                                                             int H, int I, float limit, int skip_g, int n_tail,
                                                             uint16_t* __restrict__ h_out,
                                                             uint16_t* __restrict__ out_rows) {
  __shared__ __attribute__((aligned(1024))) uint16_t As[kStages][kPrefillRows * 128];
  const int nbc = gridDim.x;  // groups of UPB column blocks
  const int nit = *n_items;
  const int total = (n_tail > 0 ? n_tail : nit) * nbc;
  const int b = blockIdx.x + blockIdx.y * nbc;
  const int per = (total + 7) >> 3;
  if ((b >> 3) >= per) return;
  const int lam = (b & 7) * per + (b >> 3);
  if (lam >= total) return;
  int item, nb;
  window_unit(lam, n_tail > 0 ? n_tail : nit, nbc, item, nb);
  const int4 it = items[(n_tail > 0 ? nit - n_tail : 0) + item];
  const int g = it.x, row0 = it.y, nrows = it.z;
  if (g == skip_g) return;  // this group's items run in a launch of their own
#define MOE_UNIT(M) \
  prefill_unit<GATEUP, FMT, M, X64>(act, row_token, blob, expert_bytes, H, I, limit, h_out, out_rows, g, row0, nrows, \
                                    UPB * nb, UPB, As)
  if constexpr (SW) {
    switch ((nrows + 15) >> 4) {
      case 1: MOE_UNIT(1); break;
      case 2: MOE_UNIT(2); break;
      case 3: MOE_UNIT(3); break;
      default: MOE_UNIT(4); break;
    }
  } else {
    MOE_UNIT(4);
  }
#undef MOE_UNIT
}

}  // namespace

void launch_ffn_prefill(bool gateup, const uint16_t* act, const int32_t* row_token, const FfnWs& w,
                        const uint8_t* blob, uint64_t eb, int H, int I, float limit, uint16_t* out_rows, int max_items,
                        int T, int E, int k, bool shared_w8, bool routed_a2, hipStream_t s) {
  // The routed experts' launch (MXFP4, with an MXFP4 shared expert riding
  // along, or 2-bit affine), then the shared expert's own launch over the last
  // ceil(T / 64) items of the work list when it has another format.
  const bool own_shared = shared_w8 || routed_a2;
  const int skip = own_shared ? E : -1;
  const int nsh = (T + kPrefillRows - 1) / kPrefillRows;
  const int ny = max_items + kGridSlack, ny_sh = nsh + kGridSlack;
  const int nbc = gateup ? I / 128 : H / 256;  // column blocks (even: I and H are multiples of 512)
  const dim3 grid(nbc, ny), grid2(nbc / 2, ny), grid2_sh(nbc / 2, ny_sh);
  uint16_t* ho = gateup ? w.h : nullptr;
  uint16_t* oo = gateup ? nullptr : out_rows;
  const int32_t* rt = gateup ? row_token : nullptr;
  // Experts averaging under two items of rows: most items are partial, and
  // the MXFP4 launch sizes each block to its item's rows (the switch costs
  // registers, so work lists of mostly full items keep the plain kernel).
  const bool sw = static_cast<long>(T) * k < 2L * kPrefillRows * E;
  // x beyond 4 GiB: the MXFP4 gate/up instances gather their rows by 64-bit
  // address (for the down projection X64 = G is the plain instance)
  const bool x64 = gateup && static_cast<uint64_t>(T) * static_cast<uint64_t>(H) * 2u > 0xffffffffull;
  // The MXFP4 and MXFP8 instances take column blocks in pairs, except the
  // row-tile switching one: its blocks end at different times, and pairs would
  // spread a window's blocks over twice the column blocks (more L2 misses).
  // The affine instances (whose registers a second unit would overflow) take
  // one at a time.
#define MOE_MX4(G, SW_, UPB_, GRID, SKIP, NTAIL)                                                                 \
  do {                                                                                                          \
    if (x64)                                                                                                    \
      ffn_prefill_kernel<G, kFmtMx4, SW_, G, UPB_><<<GRID, kThreads, 0, s>>>(act, rt, w.items, w.n_items, blob,  \
                                                                            eb, H, I, limit, SKIP, NTAIL, ho,   \
                                                                            oo);                                \
    else                                                                                                        \
      ffn_prefill_kernel<G, kFmtMx4, SW_, false, UPB_><<<GRID, kThreads, 0, s>>>(act, rt, w.items, w.n_items,    \
                                                                                blob, eb, H, I, limit, SKIP,    \
                                                                                NTAIL, ho, oo);                 \
  } while (0)
#define MOE_PREFILL(G)                                                                                            \
  do {                                                                                                          \
    if (routed_a2)                                                                                              \
      ffn_prefill_kernel<G, kFmtA2><<<grid, kThreads, 0, s>>>(act, rt, w.items, w.n_items, blob, eb, H, I, limit, \
                                                              skip, 0, ho, oo);                                 \
    else if (sw)                                                                                                \
      MOE_MX4(G, true, 1, grid, skip, 0);                                                                       \
    else                                                                                                        \
      MOE_MX4(G, false, 2, grid2, skip, 0);                                                                     \
    if (shared_w8)                                                                                              \
      ffn_prefill_kernel<G, kFmtMx8, false, false, 2><<<grid2_sh, kThreads, 0, s>>>(                            \
          act, rt, w.items, w.n_items, blob, eb, H, I, limit, -1, nsh, ho, oo);                                 \
    else if (routed_a2)                                                                                         \
      MOE_MX4(G, false, 2, grid2_sh, -1, nsh);                                                                  \
  } while (0)
  if (gateup) {
    MOE_PREFILL(true);
  } else {
    MOE_PREFILL(false);
  }
#undef MOE_PREFILL
#undef MOE_MX4
}

}  // namespace moe
