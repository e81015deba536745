// Weighted combine of the routed expert rows plus the shared expert
// ("Model techniques map -- DeepSeek-V4-Flash", row "Shared expert": the
// routed output is added to the shared expert of the same input):
//   y[t] = bf16( sum_{j<k} w[t,j] * out[slot_row[t,j]] + out[slot_row[t,k]] )
// A plain gather-reduce in a fixed order -- no atomics -- so the output is
// bit-reproducible (the deterministic reductions listed among the inference
// kernels of the same page).  HBM bound: each thread owns 8 columns of one
// token, reads 7 bf16 rows of 16 bytes and writes 16 bytes.
#include "moe_internal.h"

namespace moe {

namespace {

// All row indices and weights of a token are read first, then all of its
// row loads are issued together (16 bytes = 8 bf16 columns each), so a
// thread waits for one memory round trip, not one per slot.
__global__ __launch_bounds__(128) void combine_kernel(const uint16_t* __restrict__ out_rows,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ weights, int T, int H, int k,
                                                      uint16_t* __restrict__ y) {
  constexpr int kMaxK = 8;
  const int groups = H >> 3;
  const long idx = static_cast<long>(blockIdx.x) * 128 + threadIdx.x;
  const int t = static_cast<int>(idx / groups);
  const int c = static_cast<int>(idx % groups) * 8;
  if (t >= T) return;
  const int32_t* sr = slot_row + static_cast<size_t>(t) * (k + 1);
  int rows[kMaxK + 1];
  float w[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    rows[j] = j < k ? sr[j] : -1;
    w[j] = j < k ? weights[static_cast<size_t>(t) * k + j] : 0.f;
  }
  rows[kMaxK] = sr[k];
  u32x4 v[kMaxK + 1];
#pragma unroll
  for (int j = 0; j <= kMaxK; ++j)
    v[j] = rows[j] >= 0 ? ld16(out_rows + static_cast<size_t>(rows[j]) * H + c) : u32x4{0u, 0u, 0u, 0u};
  // element 2i of a row is the low half of word i, element 2i + 1 the high half
  auto elem = [&](const u32x4& r, int e) {
    const uint32_t word = r[e >> 1];
    return __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
  };
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (rows[j] < 0) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[j], elem(v[j], i), acc[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] += elem(v[kMaxK], i);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = static_cast<uint32_t>(float_to_bf16_bits(acc[2 * i])) |
           (static_cast<uint32_t>(float_to_bf16_bits(acc[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4*>(y + static_cast<size_t>(t) * H + c) = o;
}

}  // namespace

hipError_t launch_combine(const uint16_t* out_rows, const int32_t* slot_row, const float* weights, int T, int H, int k,
                          uint16_t* y, hipStream_t s) {
  const long threads = static_cast<long>(T) * (H / 8);
  combine_kernel<<<static_cast<unsigned>((threads + 127) / 128), 128, 0, s>>>(out_rows, slot_row, weights, T, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
