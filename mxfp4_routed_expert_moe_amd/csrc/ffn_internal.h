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

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt[3:0] |
// expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Block barrier for the activation ring.  Unlike __syncthreads() it does not
// drain the vector-memory counter, so the prefetched tiles stay in flight
// across it.  No release fence is needed: the only LDS writes are LDS-DMA
// loads, which each wave has already waited for explicitly (wait_vmcnt), and
// every LDS read before it has been consumed by an MFMA.  The acquire fence
// keeps later LDS reads below the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}

// Phase 1 (gateup = true: x rows -> h) or phase 2 (h rows -> out_rows).
// The decode family reads the dispatch offsets directly; the prefill family
// walks the work list (grid (column blocks, max_items), surplus blocks return).
void launch_ffn_decode(bool gateup, const uint16_t* act, const int32_t* row_token, const int32_t* offsets, int T,
                       int E, const uint8_t* blob, uint64_t eb, int H, int I, float limit, uint16_t* h,
                       float* out_rows, bool shared_w8, bool routed_a2, hipStream_t s);
void launch_ffn_prefill(bool gateup, const uint16_t* act, const int32_t* row_token, const FfnWs& w,
                        const uint8_t* blob, uint64_t eb, int H, int I, float limit, float* out_rows, int max_items,
                        int T, int E, bool shared_w8, bool routed_a2, hipStream_t s);
void launch_quant_act(const uint16_t* src, int rows, int K, const QAct& dst, hipStream_t s);
void launch_ffn_prefill_f8(bool gateup, const QAct& aq, const int32_t* row_token, const FfnWs& w,
                           const uint8_t* blob, uint64_t eb, int H, int I, float limit, float* out_rows,
                           int max_items, hipStream_t s);

}  // namespace moe
