// Internal interface between the expert-FFN driver (ffn.hip) and its two
// kernel families (ffn_decode.hip, ffn_prefill.hip).
#pragma once

#include "moe_internal.h"

namespace moe {

// Activations as two scaled E4M3 terms: v = S * hi + (S / 16) * lo, with one
// E8M0 scale byte sc (S = 2^(sc - 127)) per 32 consecutive k of a row.
struct QAct {
  uint8_t* hi;  // [rows, K]
  uint8_t* lo;  // [rows, K]
  uint8_t* sc;  // [rows, K / 32]
};

// Device-side work list, the h buffer and the prefill split activations,
// carved from the FFN workspace.
struct FfnWs {
  int32_t* n_items;  // [1]
  int4* items;       // [max_items] (group, first row, row count, 0)
  uint16_t* h;       // [rows, I] bf16
  QAct xq;           // [T, H] (prefill)
  QAct hq;           // [rows, I] (prefill)
};

// Weight format of the groups a kernel instance covers: MXFP4, MXFP8 (the
// shared expert, MOE_SHARED_MXFP8), 2-bit affine (routed, MOE_ROUTED_AFFINE2).
constexpr int kFmtMx4 = 0, kFmtMx8 = 1, kFmtA2 = 2;

constexpr int kDecodeRows = 16;    // rows per decode item
constexpr int kPrefillRows = 64;   // rows per prefill item
// Extra rows of blocks in the prefill grids: their XCD-aware block order
// reaches every logical block only with at least 8 * ceil(n / 8) blocks.
constexpr int kGridSlack = 7;

// Traversal of a prefill grid of n_items x nbc (item, column block) units:
// logical unit lam belongs to the window of kWinItems consecutive items
// (the last window may hold fewer) x kWinCb consecutive column blocks, and
// walks it column block fastest.  The units of one XCD are consecutive
// logical units, so the ~64 blocks an XCD runs at once cover one window: an
// expert's weight slice of a column block is shared by the window's items of
// that expert and an item's activation rows by its column blocks, both
// streamed through one L2 by blocks that start together.
constexpr int kWinItems = 8, kWinCb = 8;

__device__ __forceinline__ void window_unit(int lam, int n_items, int nbc, int& item, int& cb) {
  const int gc = nbc % kWinCb == 0 ? kWinCb : 1;
  const int per_group = kWinItems * nbc;
  const int ig = lam / per_group;
  const int r = lam - ig * per_group;
  const int ni = min(kWinItems, n_items - ig * kWinItems);
  const int cg = r / (ni * gc);
  const int r2 = r - cg * ni * gc;
  item = ig * kWinItems + r2 / gc;
  cb = cg * gc + r2 % gc;
}

// Phase 1 (gateup = true: x rows -> h) or phase 2 (h rows -> out_rows).
// The decode family reads the dispatch offsets directly; the prefill family
// walks the work list (grid (column blocks, max_items), surplus blocks return).
void launch_ffn_decode(bool gateup, const uint16_t* act, const int32_t* row_token, const int32_t* offsets, int T,
                       int E, int k, const uint8_t* blob, uint64_t eb, int H, int I, float limit, uint16_t* h,
                       uint16_t* out_rows, bool shared_w8, bool routed_a2, hipStream_t s);
void launch_ffn_prefill(bool gateup, const uint16_t* act, const int32_t* row_token, const FfnWs& w,
                        const uint8_t* blob, uint64_t eb, int H, int I, float limit, uint16_t* out_rows, int max_items,
                        int T, int E, int k, bool shared_w8, bool routed_a2, hipStream_t s);
void launch_quant_act(const uint16_t* src, int rows, int K, const QAct& dst, hipStream_t s);
void launch_ffn_prefill_f8(bool gateup, const QAct& aq, const int32_t* row_token, const FfnWs& w,
                           const uint8_t* blob, uint64_t eb, int H, int I, float limit, uint16_t* out_rows,
                           int max_items, hipStream_t s);

}  // namespace moe
