// Host repack of expert blobs (MXFP4, MXFP8, 2-bit affine): canonical layout
// <-> gfx950 tiled layout.
//
// Both layouts hold the same six planes (gate, up, down nibbles and scales) at
// the same offsets; the tiled layout permutes the bytes inside each plane so
// that a 64-lane wave loads one 16-column x 128-k tile with one coalesced
// 16-byte load per lane, and the E8M0 scales of four such tiles with one
// 4-byte load per lane.  Being a permutation, the repack keeps the byte count
// (the repacking "ElytronAI / DeepSeek-v4-Flash" describes under Sizes keeps
// its expert payload byte-identical in size, and its Verification section
// reports exact inversion).
#include <stdint.h>
#include <string.h>

#include "../../include/moe.h"

namespace {

// H and I: positive multiples of 512 up to MOE_MAX_DIM, so every size below
// fits 64 bits and every tile index an int.
bool shape_ok(int32_t H, int32_t I) {
  return H > 0 && I > 0 && H % 512 == 0 && I % 512 == 0 && H <= MOE_MAX_DIM && I <= MOE_MAX_DIM;
}

// Offset in the tiled nibble plane of canonical byte (n, kb) of an [N, K] projection.
inline uint64_t tiled_nib_index(int N, int K, int n, int kb) {
  (void)N;
  const int k = kb * 2;
  const int tile = (n / 16) * (K / 128) + k / 128;
  const int lane = 16 * ((k % 128) / 32) + n % 16;
  return static_cast<uint64_t>(tile) * 1024 + lane * 16 + (kb % 16);
}

// Offset in the tiled scale plane of canonical scale (n, grp) of an [N, K] projection.
inline uint64_t tiled_sc_index(int N, int K, int n, int grp) {
  (void)N;
  const int block = (n / 16) * (K / 512) + grp / 16;
  const int i = (grp % 16) / 4;  // k tile within the 512 block
  const int gq = grp % 4;        // 32-column group within the k tile
  const int lane = 16 * gq + n % 16;
  return static_cast<uint64_t>(block) * 256 + lane * 4 + i;
}

// dir = +1: canonical -> tiled; -1: tiled -> canonical.
void permute_projection(const uint8_t* src, uint8_t* dst, int N, int K, int dir) {
  const int kbytes = K / 2;
  for (int n = 0; n < N; ++n) {
    for (int kb = 0; kb < kbytes; kb += 16) {
      const uint64_t c = static_cast<uint64_t>(n) * kbytes + kb;
      const uint64_t t = tiled_nib_index(N, K, n, kb);
      if (dir > 0) memcpy(dst + t, src + c, 16);
      else memcpy(dst + c, src + t, 16);
    }
  }
  const uint64_t nib_bytes = static_cast<uint64_t>(N) * K / 2;
  const int groups = K / 32;
  for (int n = 0; n < N; ++n) {
    for (int gi = 0; gi < groups; ++gi) {
      const uint64_t c = nib_bytes + static_cast<uint64_t>(n) * groups + gi;
      const uint64_t t = nib_bytes + tiled_sc_index(N, K, n, gi);
      if (dir > 0) dst[t] = src[c];
      else dst[c] = src[t];
    }
  }
}

// Offset in the tiled MXFP8 code plane of canonical bytes (n, k .. k+15) of an
// [N, K] projection (k a multiple of 16): 2048-byte tiles of 16 rows x 128
// columns; lane 16g + r holds columns 32g .. 32g+15 in the first KiB of the
// tile and 32g+16 .. 32g+31 in the second.
inline uint64_t tiled_code8_index(int K, int n, int k) {
  const int tile = (n / 16) * (K / 128) + k / 128;
  const int g = (k % 128) / 32, half = (k % 32) / 16;
  const int lane = 16 * g + n % 16;
  return static_cast<uint64_t>(tile) * 2048 + half * 1024 + lane * 16;
}

void permute_projection8(const uint8_t* src, uint8_t* dst, int N, int K, int dir) {
  for (int n = 0; n < N; ++n) {
    for (int k = 0; k < K; k += 16) {
      const uint64_t c = static_cast<uint64_t>(n) * K + k;
      const uint64_t t = tiled_code8_index(K, n, k);
      if (dir > 0) memcpy(dst + t, src + c, 16);
      else memcpy(dst + c, src + t, 16);
    }
  }
  const uint64_t code_bytes = static_cast<uint64_t>(N) * K;
  const int groups = K / 32;
  for (int n = 0; n < N; ++n) {
    for (int gi = 0; gi < groups; ++gi) {
      const uint64_t c = code_bytes + static_cast<uint64_t>(n) * groups + gi;
      const uint64_t t = code_bytes + tiled_sc_index(N, K, n, gi);
      if (dir > 0) dst[t] = src[c];
      else dst[c] = src[t];
    }
  }
}

int repack8(const uint8_t* src, uint64_t src_bytes, int32_t H, int32_t I, uint8_t* dst, uint64_t dst_bytes, int dir) {
  if (!src || !dst) return MOE_EINVAL;
  if (!shape_ok(H, I)) return MOE_ESHAPE;
  const uint64_t need = moe_expert_bytes_mxfp8(H, I);
  if (src_bytes < need || dst_bytes < need) return MOE_EINVAL;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + need && b < a + need) return MOE_EINVAL;  // overlapping buffers
  const uint64_t pg = static_cast<uint64_t>(I) * H + static_cast<uint64_t>(I) * H / 32;
  permute_projection8(src, dst, I, H, dir);                    // gate [I, H]
  permute_projection8(src + pg, dst + pg, I, H, dir);          // up   [I, H]
  permute_projection8(src + 2 * pg, dst + 2 * pg, H, I, dir);  // down [H, I]
  return MOE_OK;
}

int repack(const uint8_t* src, uint64_t src_bytes, int32_t n_total, int32_t H, int32_t I, uint8_t* dst,
           uint64_t dst_bytes, int dir) {
  if (!src || !dst) return MOE_EINVAL;
  if (n_total <= 0) return MOE_EINVAL;
  if (!shape_ok(H, I)) return MOE_ESHAPE;
  const uint64_t eb = moe_expert_bytes(H, I);
  const uint64_t need = eb * static_cast<uint64_t>(n_total);
  if (src_bytes < need || dst_bytes < need) return MOE_EINVAL;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + need && b < a + need) return MOE_EINVAL;  // overlapping buffers
  const uint64_t pg = static_cast<uint64_t>(I) * H / 2 + static_cast<uint64_t>(I) * H / 32;
  for (int32_t x = 0; x < n_total; ++x) {
    const uint8_t* s = src + eb * x;
    uint8_t* d = dst + eb * x;
    permute_projection(s, d, I, H, dir);                    // gate [I, H]
    permute_projection(s + pg, d + pg, I, H, dir);          // up   [I, H]
    permute_projection(s + 2 * pg, d + 2 * pg, H, I, dir);  // down [H, I]
  }
  return MOE_OK;
}

// 2-bit affine experts.  Position of canonical code (n, k) of an [N, K]
// projection in the tiled code plane: byte offset and bit within that byte.
inline void tiled_code2_pos(int K, int n, int k, uint64_t* byte, int* bit) {
  const int tile = (n / 16) * (K / 128) + k / 128;
  const int kk = k % 128;
  const int s = kk / 32, g = (kk % 32) / 8, i = kk % 8;
  const int lane = 16 * g + n % 16;
  const int b = 4 * i + 2 * (s % 2);  // bit in little-endian word s / 2: nibble i, low or high half
  *byte = static_cast<uint64_t>(tile) * 512 + lane * 8 + (s / 2) * 4 + b / 8;
  *bit = b % 8;
}

// Offset (from the start of the scale plane) of the 4-byte (scale, bias)
// entry of row n, group gi in the tiled layout.
inline uint64_t tiled_sb2_index(int K, int G, int n, int gi) {
  const int k = gi * G;
  const uint64_t block = static_cast<uint64_t>(n / 16) * (K / 128) + k / 128;
  return block * (16 * (128 / G) * 4) + ((n % 16) * (128 / G) + (k % 128) / G) * 4;
}

void permute_projection2(const uint8_t* src, uint8_t* dst, int N, int K, int G, int dir) {
  const uint64_t code_bytes = static_cast<uint64_t>(N) * K / 4;
  memset(dst, 0, code_bytes);
  // (byte, bit) of column kk of a 128-k tile, relative to the tile and row
  // (lane r = n % 16 of lane group 0): one table for every row and tile
  uint16_t off[128];
  uint8_t bitpos[128];
  for (int kk = 0; kk < 128; ++kk) {
    uint64_t b;
    int bit;
    tiled_code2_pos(128, 0, kk, &b, &bit);
    off[kk] = static_cast<uint16_t>(b);
    bitpos[kk] = static_cast<uint8_t>(bit);
  }
  for (int n = 0; n < N; ++n) {
    const uint8_t* crow = (dir > 0 ? src : dst) + static_cast<uint64_t>(n) * (K / 4);
    for (int kt = 0; kt < K / 128; ++kt) {
      const uint64_t tbase = (static_cast<uint64_t>(n / 16) * (K / 128) + kt) * 512 + (n % 16) * 8;
      for (int kk = 0; kk < 128; ++kk) {
        const int k = kt * 128 + kk;
        const int cbit = 2 * (k % 4);
        const uint64_t tb = tbase + off[kk];
        if (dir > 0) dst[tb] |= static_cast<uint8_t>(((crow[k / 4] >> cbit) & 3) << bitpos[kk]);
        else dst[static_cast<uint64_t>(n) * (K / 4) + k / 4] |= static_cast<uint8_t>(((src[tb] >> bitpos[kk]) & 3) << cbit);
      }
    }
  }
  const uint64_t ng = static_cast<uint64_t>(N) * (K / G);  // groups; canonical scales then biases, 2 bytes each
  const uint8_t* s_sb = src + code_bytes;
  uint8_t* d_sb = dst + code_bytes;
  for (int n = 0; n < N; ++n) {
    for (int gi = 0; gi < K / G; ++gi) {
      const uint64_t c = static_cast<uint64_t>(n) * (K / G) + gi;
      const uint64_t t = tiled_sb2_index(K, G, n, gi);
      if (dir > 0) {
        memcpy(d_sb + t, s_sb + 2 * c, 2);
        memcpy(d_sb + t + 2, s_sb + 2 * ng + 2 * c, 2);
      } else {
        memcpy(d_sb + 2 * c, s_sb + t, 2);
        memcpy(d_sb + 2 * ng + 2 * c, s_sb + t + 2, 2);
      }
    }
  }
}

int repack2(const uint8_t* src, uint64_t src_bytes, int32_t n_experts, int32_t H, int32_t I, uint8_t* dst,
            uint64_t dst_bytes, int dir) {
  if (!src || !dst) return MOE_EINVAL;
  if (n_experts <= 0) return MOE_EINVAL;
  if (!shape_ok(H, I)) return MOE_ESHAPE;
  const uint64_t eb = moe_expert_bytes_affine2(H, I);
  const uint64_t need = eb * static_cast<uint64_t>(n_experts);
  if (src_bytes < need || dst_bytes < need) return MOE_EINVAL;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + need && b < a + need) return MOE_EINVAL;  // overlapping buffers
  const uint64_t nh = static_cast<uint64_t>(H) * I;
  const uint64_t pg = nh / 4 + 4 * (nh / 64);  // gate (and up) projection bytes
  for (int32_t x = 0; x < n_experts; ++x) {
    const uint8_t* s = src + eb * x;
    uint8_t* d = dst + eb * x;
    permute_projection2(s, d, I, H, 64, dir);                    // gate [I, H], groups of 64
    permute_projection2(s + pg, d + pg, I, H, 64, dir);          // up   [I, H], groups of 64
    permute_projection2(s + 2 * pg, d + 2 * pg, H, I, 32, dir);  // down [H, I], groups of 32
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

uint64_t moe_expert_bytes(int32_t hidden, int32_t inter) {
  if (!shape_ok(hidden, inter)) return 0;
  return 3ull * static_cast<uint64_t>(hidden) * static_cast<uint64_t>(inter) * 17ull / 32ull;
}

int moe_pack_mxfp4(const uint8_t* src_canonical, uint64_t src_bytes, int32_t n_total, int32_t hidden, int32_t inter,
                   uint8_t* dst_device_layout, uint64_t dst_bytes) {
  return repack(src_canonical, src_bytes, n_total, hidden, inter, dst_device_layout, dst_bytes, +1);
}

int moe_unpack_mxfp4(const uint8_t* src_device_layout, uint64_t src_bytes, int32_t n_total, int32_t hidden,
                     int32_t inter, uint8_t* dst_canonical, uint64_t dst_bytes) {
  return repack(src_device_layout, src_bytes, n_total, hidden, inter, dst_canonical, dst_bytes, -1);
}

uint64_t moe_expert_bytes_mxfp8(int32_t hidden, int32_t inter) {
  if (!shape_ok(hidden, inter)) return 0;
  return 3ull * static_cast<uint64_t>(hidden) * static_cast<uint64_t>(inter) * 33ull / 32ull;
}

int moe_pack_mxfp8(const uint8_t* src_canonical, uint64_t src_bytes, int32_t hidden, int32_t inter,
                   uint8_t* dst_device_layout, uint64_t dst_bytes) {
  return repack8(src_canonical, src_bytes, hidden, inter, dst_device_layout, dst_bytes, +1);
}

int moe_unpack_mxfp8(const uint8_t* src_device_layout, uint64_t src_bytes, int32_t hidden, int32_t inter,
                     uint8_t* dst_canonical, uint64_t dst_bytes) {
  return repack8(src_device_layout, src_bytes, hidden, inter, dst_canonical, dst_bytes, -1);
}

uint64_t moe_expert_bytes_affine2(int32_t hidden, int32_t inter) {
  if (!shape_ok(hidden, inter)) return 0;
  return static_cast<uint64_t>(hidden) * static_cast<uint64_t>(inter);
}

int moe_pack_affine2(const uint8_t* src_canonical, uint64_t src_bytes, int32_t n_experts, int32_t hidden,
                     int32_t inter, uint8_t* dst_device_layout, uint64_t dst_bytes) {
  return repack2(src_canonical, src_bytes, n_experts, hidden, inter, dst_device_layout, dst_bytes, +1);
}

int moe_unpack_affine2(const uint8_t* src_device_layout, uint64_t src_bytes, int32_t n_experts, int32_t hidden,
                       int32_t inter, uint8_t* dst_canonical, uint64_t dst_bytes) {
  return repack2(src_device_layout, src_bytes, n_experts, hidden, inter, dst_canonical, dst_bytes, -1);
}

}  // extern "C"
