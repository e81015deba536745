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
// of one MFMA B fragment.  Nothing is ever dequantised to memory.
//
// Two kernel families (ffn_decode.hip, ffn_prefill.hip):
//  * decode (few rows per expert, HBM bound): a block takes one routed expert
//    straight from the dispatch offsets, or one 16-row chunk of the shared
//    group; its four waves split the K axis and the partial sums meet in LDS
//    in a fixed order;
//  * prefill (many rows per expert, MFMA bound): a device-side work list of
//    items (group, first row, row count) of at most 64 rows, built here from
//    the offsets so the host never learns the per-expert counts; the grid
//    covers the worst case and surplus blocks return at once.  Activation
//    tiles go to LDS by DMA, weight fragments straight to registers.
#include "ffn_internal.h"

namespace moe {

namespace {

__host__ __device__ inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

inline int ffn_max_items(int T, int E, int k, int bm) {
  const long rows = static_cast<long>(T) * (k + 1);
  return static_cast<int>((rows + bm - 1) / bm) + E + 1;
}

inline size_t qact_bytes(long rows, int K) {
  return 2 * align256(static_cast<size_t>(rows) * K) + align256(static_cast<size_t>(rows) * (K / 32));
}

inline QAct qact_carve(char*& p, long rows, int K) {
  QAct q;
  q.hi = reinterpret_cast<uint8_t*>(p);
  p += align256(static_cast<size_t>(rows) * K);
  q.lo = reinterpret_cast<uint8_t*>(p);
  p += align256(static_cast<size_t>(rows) * K);
  q.sc = reinterpret_cast<uint8_t*>(p);
  p += align256(static_cast<size_t>(rows) * (K / 32));
  return q;
}

// The prefill path (split = true) keeps x and h in split form only; the
// decode path keeps h as bf16.
inline FfnWs ffn_carve(void* ws, int max_items, int T, int k, int H, int I, bool split) {
  char* p = static_cast<char*>(ws);
  FfnWs w;
  w.n_items = reinterpret_cast<int32_t*>(p);
  p += 256;
  w.items = reinterpret_cast<int4*>(p);
  p += align256(sizeof(int4) * static_cast<size_t>(max_items));
  w.h = nullptr;
  w.xq = w.hq = QAct{nullptr, nullptr, nullptr};
  if (split) {
    w.xq = qact_carve(p, T, H);
    w.hq = qact_carve(p, static_cast<long>(T) * (k + 1), I);
  } else {
    w.h = reinterpret_cast<uint16_t*>(p);
  }
  return w;
}

// Work list: every group with rows is cut into items of at most bm rows.
// After the scan of the per-group item counts, thread t writes items t,
// t + 256, ... (consecutive threads, consecutive 16-byte items), each finding
// its group by binary search of the item bases in LDS: a hot group's hundreds
// of items are written by the whole block, not by one thread.
__global__ __launch_bounds__(256) void ffn_plan_kernel(const int32_t* __restrict__ offsets, int E, int bm,
                                                       int4* __restrict__ items, int32_t* __restrict__ n_items) {
  __shared__ int cnt[1025];
  __shared__ int off[1025];
  __shared__ int tmp[4];
  const int G = E + 1;
  for (int g = threadIdx.x; g <= G; g += 256) {
    off[g] = offsets[g];
    if (g < G) cnt[g] = (offsets[g + 1] - offsets[g] + bm - 1) / bm;
  }
  __syncthreads();
  const int total = block_excl_scan_256(cnt, G, tmp);  // cnt[g] = first item of group g
  if (threadIdx.x == 0) cnt[G] = total;
  __syncthreads();
  for (int it = threadIdx.x; it < total; it += 256) {
    // the last group g with cnt[g] <= it (empty groups share their base with the next)
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cnt[mid] <= it) lo = mid;
      else hi = mid - 1;
    }
    const int g = lo;
    const int i = it - cnt[g];
    const int c = off[g + 1] - off[g];
    items[it] = make_int4(g, off[g] + i * bm, min(bm, c - i * bm), 0);
  }
  if (threadIdx.x == 0) *n_items = total;
}

// Decode kernels while the average group holds at most ~16 rows (and both K
// sizes have a compiled decode variant, which the validation requires for
// 2-bit affine routed experts); prefill kernels otherwise.
inline bool use_decode(int T, int E, int k, int H, int I) {
  return static_cast<long>(T) * (k + 1) <= 16L * (E + 1) && decode_k_ok(H) && decode_k_ok(I);
}

inline int ffn_bm(int T, int E, int k, int H, int I) { return use_decode(T, E, k, H, I) ? kDecodeRows : kPrefillRows; }

}  // namespace

size_t ffn_ws_bytes(int T, int E, int H, int I, int k, bool split_fp8, bool routed_a2) {
  (void)routed_a2;  // same workspace as MXFP4 routed experts
  const int mi = ffn_max_items(T, E, k, ffn_bm(T, E, k, H, I));
  const size_t n = 256 + align256(sizeof(int4) * static_cast<size_t>(mi));
  if (split_fp8 && !use_decode(T, E, k, H, I))
    return n + qact_bytes(T, H) + qact_bytes(static_cast<long>(T) * (k + 1), I);
  return n + align256(sizeof(uint16_t) * static_cast<size_t>(T) * (k + 1) * I);
}

hipError_t launch_ffn(const uint16_t* x, int T, const uint8_t* blob, uint64_t expert_bytes, int E, int H, int I,
                      int k, const int32_t* offsets, const int32_t* row_token, float limit, uint16_t* out_rows,
                      void* ws, int phase, bool split_fp8, bool shared_w8, bool routed_a2, hipStream_t s) {
  const int bm = ffn_bm(T, E, k, H, I);
  const int max_items = ffn_max_items(T, E, k, bm);
  const bool dec = use_decode(T, E, k, H, I);
  const bool split = split_fp8 && !dec;
  FfnWs w = ffn_carve(ws, max_items, T, k, H, I, split);
  for (int ph = 0; ph < 3; ++ph) {
    if (phase >= 0 && ph != phase) continue;
    if (ph == 0) {
      // the decode family reads the offsets directly: no work list to build
      if (!dec) ffn_plan_kernel<<<1, 256, 0, s>>>(offsets, E, bm, w.items, w.n_items);
    } else {
      const bool gateup = ph == 1;
      const uint16_t* act = gateup ? x : w.h;
      const int32_t* rt = gateup ? row_token : nullptr;
      if (dec) {
        launch_ffn_decode(gateup, act, rt, offsets, T, E, k, blob, expert_bytes, H, I, limit, w.h, out_rows, shared_w8,
                          routed_a2, s);
      } else if (split) {
        // phase 1 splits x, then writes h split; phase 2 reads it
        if (gateup) launch_quant_act(x, T, H, w.xq, s);
        launch_ffn_prefill_f8(gateup, gateup ? w.xq : w.hq, rt, w, blob, expert_bytes, H, I, limit, out_rows,
                              max_items, s);
      } else {
        launch_ffn_prefill(gateup, act, rt, w, blob, expert_bytes, H, I, limit, out_rows, max_items, T, E, k,
                           shared_w8, routed_a2, s);
      }
    }
  }
  return hipGetLastError();
}

}  // namespace moe
