// Internal declarations of the gfx950 MoE library: device helpers shared by the
// kernels and the launch functions that moe_api.hip calls after validating.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bf16 bits, round to nearest even; NaN stays NaN.  One gfx950
// convert (v_cvt_pk_bf16_f32); on the device it gave the same bits as the
// integer form (add 0x7fff plus the kept low bit, shift by 16) for all 2^32
// non-NaN inputs, denormals included.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// ---------------------------------------------------------------- MXFP4
// Scale operand of the scaled FP4 convert for E8M0 byte e (value 2^(e-127),
// e = 255 NaN).  The convert reads only the exponent field of its float
// scale operand, as an E8M0 value: e << 23 places the byte there, and the
// convert then scales exactly for every e, including e = 0 (2^-127) and
// e = 255 (NaN) -- checked on gfx950 for all 256 bytes and all 16 codes.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t e) { return __uint_as_float(e << 23); }

// Byte i (0..3) of a word of four E8M0 scales, as a convert scale operand.
__device__ __forceinline__ float e8m0_scale_operand_of(uint32_t word, int i) {
  return __uint_as_float(((word >> (8 * i)) & 255u) << 23);
}

// Eight E2M1 codes (one 32-bit word, low nibble first) times one scale ->
// eight bf16 in k order, the B operand of one 16x16x32 bf16 MFMA.  The
// hardware convert is exact here: an E2M1 value times a power of two has two
// significant bits.
__device__ __forceinline__ bf16x8 dequant8(uint32_t codes, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  u32x4 w;
  w[0] = __builtin_bit_cast(uint32_t, p0);
  w[1] = __builtin_bit_cast(uint32_t, p1);
  w[2] = __builtin_bit_cast(uint32_t, p2);
  w[3] = __builtin_bit_cast(uint32_t, p3);
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// A raw buffer resource over `bytes` bytes at `base` (a uniform address):
// stride 0, and descriptor word 3 = 0x00020000, the 32-bit data format that
// untyped buffer loads and the buffer form of the LDS-DMA expect on gfx9.
// Loads through it take a 32-bit lane offset and a scalar offset, and reads
// past `bytes` return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Byte offsets of the six planes inside one expert (same in both layouts).
struct ExpertPlanes {
  uint64_t gate_nib, gate_sc, up_nib, up_sc, down_nib, down_sc;
};

// The planes of an MXFP8 expert: one code byte per weight, same scale planes.
__host__ __device__ inline ExpertPlanes expert_planes8(int H, int I) {
  const uint64_t nh = static_cast<uint64_t>(H) * I;
  ExpertPlanes p;
  p.gate_nib = 0;
  p.gate_sc = nh;
  p.up_nib = nh + nh / 32;
  p.up_sc = p.up_nib + nh;
  p.down_nib = 2 * (nh + nh / 32);
  p.down_sc = p.down_nib + nh;
  return p;
}

__host__ __device__ inline ExpertPlanes expert_planes(int H, int I) {
  const uint64_t nh = static_cast<uint64_t>(H) * I;
  ExpertPlanes p;
  p.gate_nib = 0;
  p.gate_sc = nh / 2;
  p.up_nib = nh / 2 + nh / 32;
  p.up_sc = p.up_nib + nh / 2;
  p.down_nib = 2 * (nh / 2 + nh / 32);
  p.down_sc = p.down_nib + nh / 2;
  return p;
}

// The planes of a 2-bit affine expert: per projection the code plane (2 bits
// per weight) then its (scale, bias) plane, 4 bytes per group of 64 (gate,
// up) or 32 (down) weights.  The *_sc fields point at the (scale, bias) planes.
__host__ __device__ inline ExpertPlanes expert_planes_a2(int H, int I) {
  const uint64_t nh = static_cast<uint64_t>(H) * I;
  ExpertPlanes p;
  p.gate_nib = 0;
  p.gate_sc = nh / 4;
  p.up_nib = nh / 4 + nh / 16;
  p.up_sc = p.up_nib + nh / 4;
  p.down_nib = 2 * (nh / 4 + nh / 16);
  p.down_sc = p.down_nib + nh / 4;
  return p;
}

// K sizes with a compiled decode variant of the expert FFN (k tiles per wave:
// K / 512 with four K-splitting waves, one of 1, 2, 4, 8).
__host__ __device__ inline bool decode_k_ok(int K) { return K == 512 || K == 1024 || K == 2048 || K == 4096; }

// Eight E4M3 codes (two 32-bit words, byte order = k order) times one scale
// -> eight bf16, the B operand of one 16x16x32 bf16 MFMA.  The hardware
// convert is exact for every code and scale byte < 255 (checked on the
// device): an E4M3 value times a power of two has four significant bits.
__device__ __forceinline__ bf16x8 dequant8_fp8(uint32_t lo, uint32_t hi, float scale) {
  u32x4 w;
  w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false));
  w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true));
  w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false));
  w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true));
  return __builtin_bit_cast(bf16x8, w);
}

// v / (1 + e^-v) from the fast exponential (relative error about |v| 2^-24)
// and the hardware reciprocal (1 ulp): for the |v| that matter, both far
// below the bf16 rounding of h that follows (2^-9 relative).
__device__ __forceinline__ float silu_f(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// ---------------------------------------------------------------- pipelines
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

// ---------------------------------------------------------------- wave / block scans
// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive scan of n <= 1024 ints in LDS buffer `a` (in place) by a 256-thread
// block; returns the total to every thread.  `tmp` needs 4 ints.
__device__ inline int block_excl_scan_256(int* a, int n, int* tmp) {
  const int tid = threadIdx.x;
  int v[4];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid * 4 + i;
    v[i] = idx < n ? a[idx] : 0;
    local += v[i];
  }
  const int incl = wave_incl_scan(local);
  const int wave = tid >> 6;
  if ((tid & 63) == 63) tmp[wave] = incl;
  __syncthreads();
  int wave_base = 0;
  for (int w = 0; w < wave; ++w) wave_base += tmp[w];
  const int total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  int run = wave_base + incl - local;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid * 4 + i;
    if (idx < n) a[idx] = run;
    run += v[i];
  }
  __syncthreads();
  return total;
}

// Exclusive scan of n <= 1024 ints in LDS buffer `a` (in place) by a
// 1024-thread block, one element per thread; returns the total to every
// thread.  `tmp` needs 16 ints.
__device__ inline int block_excl_scan_1024(int* a, int n, int* tmp) {
  const int tid = threadIdx.x;
  const int v = tid < n ? a[tid] : 0;
  const int incl = wave_incl_scan(v);
  const int wave = tid >> 6;
  if ((tid & 63) == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < 16; ++w) {
    base += (w < wave) ? tmp[w] : 0;
    total += tmp[w];
  }
  if (tid < n) a[tid] = base + incl - v;
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------- launchers
// Each returns hipGetLastError() of its launches.  Arguments are validated
// by the caller in moe_api.hip.
size_t route_ws_bytes(int T, int H, int E);
hipError_t launch_route_learned(const uint16_t* x, int T, int H, const float* w, const float* bias, int E, int k,
                                float scale, int32_t* ids, float* weights, void* ws, hipStream_t s);
hipError_t launch_route_hash(const int32_t* tok, int T, const int32_t* table, int V, int k, float scale,
                             int32_t* ids, float* weights, hipStream_t s);

size_t dispatch_ws_bytes(int T, int E, int k);
hipError_t launch_dispatch(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* row_token,
                           int32_t* slot_row, void* ws, hipStream_t s);
// The same with the library's static scratch (moe_dispatch_noalloc).
hipError_t launch_dispatch_noalloc(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* row_token,
                                   int32_t* slot_row, hipStream_t s);

// split_fp8: the prefill family on the scaled FP4 matrix cores (MOE_FFN_SPLIT_FP8);
// shared_w8: the shared expert is MXFP8 (MOE_SHARED_MXFP8); routed_a2: the
// routed experts are 2-bit affine (MOE_ROUTED_AFFINE2).
size_t ffn_ws_bytes(int T, int E, int H, int I, int k, bool split_fp8, bool routed_a2);
hipError_t launch_ffn(const uint16_t* x, int T, const uint8_t* blob, uint64_t expert_bytes, int E, int H, int I,
                      int k, const int32_t* offsets, const int32_t* row_token, float limit, uint16_t* out_rows,
                      void* ws, int phase, bool split_fp8, bool shared_w8, bool routed_a2, hipStream_t s);

hipError_t launch_combine(const uint16_t* out_rows, const int32_t* slot_row, const float* weights, int T, int H, int k,
                          uint16_t* y, hipStream_t s);

}  // namespace moe
