// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer around the repack code and the argument
// validation (tests/test_host_sanitizers.py builds and runs this).
//
// Everything here runs on the host: the repack is pure host code, and every
// device-side call below is one the validation refuses before any HIP call
// (the device pointers are never dereferenced).  A sanitizer finding aborts
// the program; an unexpected status makes it exit 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <limits>
#include <random>
#include <vector>

#include "../../include/moe.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    fprintf(stderr, "FAIL line %d: %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

std::vector<uint8_t> random_bytes(size_t n, uint32_t seed) {
  std::mt19937 g(seed);
  std::vector<uint8_t> v(n);
  for (auto& b : v) b = static_cast<uint8_t>(g());
  return v;
}

// Fake device addresses: never dereferenced, every call using them is refused.
uint16_t* const kFakeX = reinterpret_cast<uint16_t*>(uintptr_t{0x7f0000000000});
float* const kFakeF = reinterpret_cast<float*>(uintptr_t{0x7f0000100000});
int32_t* const kFakeI = reinterpret_cast<int32_t*>(uintptr_t{0x7f0000200000});
void* const kFakeWs = reinterpret_cast<void*>(uintptr_t{0x7f0000300000});
void* const kFakeMis = reinterpret_cast<void*>(uintptr_t{0x7f0000300008});

void check_pack_round_trips() {
  for (int shape = 0; shape < 2; ++shape) {
    const int32_t H = shape ? 1024 : 512, I = 512, n = 2;
    const uint64_t eb = moe_expert_bytes(H, I);
    EXPECT(eb == 3ull * H * I * 17 / 32);
    auto src = random_bytes(eb * n, 1 + shape);
    std::vector<uint8_t> dev(src.size()), back(src.size());
    EXPECT(moe_pack_mxfp4(src.data(), src.size(), n, H, I, dev.data(), dev.size()) == MOE_OK);
    EXPECT(moe_unpack_mxfp4(dev.data(), dev.size(), n, H, I, back.data(), back.size()) == MOE_OK);
    EXPECT(back == src);
    EXPECT(dev != src);
    // refusals: short buffers, bad shapes, overlap, NULL
    EXPECT(moe_pack_mxfp4(src.data(), src.size() - 1, n, H, I, dev.data(), dev.size()) == MOE_EINVAL);
    EXPECT(moe_pack_mxfp4(src.data(), src.size(), n, H, I, dev.data(), dev.size() - 1) == MOE_EINVAL);
    EXPECT(moe_pack_mxfp4(src.data(), src.size(), n, H + 1, I, dev.data(), dev.size()) == MOE_ESHAPE);
    EXPECT(moe_pack_mxfp4(src.data(), src.size(), 0, H, I, dev.data(), dev.size()) == MOE_EINVAL);
    EXPECT(moe_pack_mxfp4(src.data(), src.size(), n, H, I, src.data() + 16, src.size()) == MOE_EINVAL);
    EXPECT(moe_pack_mxfp4(nullptr, src.size(), n, H, I, dev.data(), dev.size()) == MOE_EINVAL);
  }
  {
    const int32_t H = 512, I = 1536;
    const uint64_t eb = moe_expert_bytes_mxfp8(H, I);
    EXPECT(eb == 3ull * H * I * 33 / 32);
    auto src = random_bytes(eb, 7);
    std::vector<uint8_t> dev(src.size()), back(src.size());
    EXPECT(moe_pack_mxfp8(src.data(), src.size(), H, I, dev.data(), dev.size()) == MOE_OK);
    EXPECT(moe_unpack_mxfp8(dev.data(), dev.size(), H, I, back.data(), back.size()) == MOE_OK);
    EXPECT(back == src);
    EXPECT(moe_pack_mxfp8(src.data(), src.size() - 1, H, I, dev.data(), dev.size()) == MOE_EINVAL);
    EXPECT(moe_pack_mxfp8(src.data(), src.size(), H, I + 1, dev.data(), dev.size()) == MOE_ESHAPE);
  }
  {
    const int32_t H = 1024, I = 512, n = 3;
    const uint64_t eb = moe_expert_bytes_affine2(H, I);
    EXPECT(eb == static_cast<uint64_t>(H) * I);
    auto src = random_bytes(eb * n, 9);
    std::vector<uint8_t> dev(src.size()), back(src.size());
    EXPECT(moe_pack_affine2(src.data(), src.size(), n, H, I, dev.data(), dev.size()) == MOE_OK);
    EXPECT(moe_unpack_affine2(dev.data(), dev.size(), n, H, I, back.data(), back.size()) == MOE_OK);
    EXPECT(back == src);
    EXPECT(moe_pack_affine2(src.data(), src.size(), n, H, I, src.data() + 8, src.size()) == MOE_EINVAL);
  }
  // sizes: unsupported shapes give 0, including ones whose byte count would
  // not fit 64 bits; the largest supported shape is exact
  EXPECT(moe_expert_bytes(0, 512) == 0 && moe_expert_bytes(512, -512) == 0 && moe_expert_bytes(4000, 512) == 0);
  const int32_t big = std::numeric_limits<int32_t>::max() / 512 * 512;
  EXPECT(moe_expert_bytes(big, big) == 0 && moe_expert_bytes_mxfp8(big, 512) == 0);
  EXPECT(moe_expert_bytes_affine2(MOE_MAX_DIM + 512, 512) == 0);
  EXPECT(moe_expert_bytes(MOE_MAX_DIM, MOE_MAX_DIM) == 3ull * MOE_MAX_DIM * MOE_MAX_DIM * 17 / 32);
  EXPECT(moe_route_workspace_size(64, MOE_MAX_DIM + 512, 256) == 0);
}

void check_descriptor_and_sizes() {
  moe_experts d;
  EXPECT(moe_experts_init(nullptr, kFakeWs, 256, 4096, 2048) == MOE_EINVAL);
  EXPECT(moe_experts_init(&d, nullptr, 256, 4096, 2048) == MOE_EINVAL);
  EXPECT(moe_experts_init(&d, kFakeWs, 0, 4096, 2048) == MOE_ESHAPE);
  EXPECT(moe_experts_init(&d, kFakeWs, 256, 4000, 2048) == MOE_ESHAPE);
  EXPECT(moe_experts_init(&d, kFakeWs, 256, 4096, 2048) == MOE_OK);
  EXPECT(d.expert_bytes == 13369344ull && d.layout == MOE_LAYOUT_GFX950_TILED_V1 && d.flags == 0);
  // workspace queries at the largest and beyond the largest token count
  EXPECT(moe_route_workspace_size(MOE_MAX_TOKENS, 4096, 256) > 0);
  EXPECT(moe_route_workspace_size(MOE_MAX_TOKENS + 1, 4096, 256) == 0);
  EXPECT(moe_dispatch_workspace_size(MOE_MAX_TOKENS, 1023, 8) > 0);
  EXPECT(moe_dispatch_workspace_size(-1, 256, 6) == 0);
  EXPECT(moe_ffn_workspace_size(MOE_MAX_TOKENS, &d, 8) > 0);
  EXPECT(moe_ffn_workspace_size(MOE_MAX_TOKENS + 1, &d, 6) == 0);
  moe_experts bad = d;
  bad.layout = MOE_LAYOUT_CANONICAL_MXFP4;
  EXPECT(moe_ffn_workspace_size(64, &bad, 6) == 0);
  for (int s = -1; s < 9; ++s) EXPECT(moe_status_str(s) != nullptr);
}

void check_call_refusals() {
  const size_t rws = moe_route_workspace_size(64, 4096, 256);
  // moe_route
  EXPECT(moe_route(kFakeX, 0, 4096, kFakeF, nullptr, nullptr, nullptr, 0, 256, 6, 1.5f, kFakeI, kFakeF, kFakeWs, rws,
                   nullptr) == MOE_OK);
  EXPECT(moe_route(kFakeX, -1, 4096, kFakeF, nullptr, nullptr, nullptr, 0, 256, 6, 1.5f, kFakeI, kFakeF, kFakeWs, rws,
                   nullptr) == MOE_EINVAL);
  EXPECT(moe_route(kFakeX, 64, 4096, kFakeF, nullptr, nullptr, nullptr, 0, 256, 9, 1.5f, kFakeI, kFakeF, kFakeWs, rws,
                   nullptr) == MOE_ESHAPE);
  EXPECT(moe_route(kFakeX, 64, 4000, kFakeF, nullptr, nullptr, nullptr, 0, 256, 6, 1.5f, kFakeI, kFakeF, kFakeWs, rws,
                   nullptr) == MOE_ESHAPE);
  EXPECT(moe_route(kFakeX, 64, 4096, kFakeF, nullptr, nullptr, nullptr, 0, 256, 6,
                   std::numeric_limits<float>::quiet_NaN(), kFakeI, kFakeF, kFakeWs, rws, nullptr) == MOE_EINVAL);
  EXPECT(moe_route(kFakeX, 64, 4096, kFakeF, nullptr, nullptr, nullptr, 0, 256, 6, 1.5f, kFakeI, kFakeF, kFakeMis, rws,
                   nullptr) == MOE_EALIGN);
  EXPECT(moe_route(kFakeX, 64, 4096, kFakeF, nullptr, nullptr, nullptr, 0, 256, 6, 1.5f, kFakeI, kFakeF, kFakeWs,
                   rws - 1, nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_route(nullptr, 64, 4096, nullptr, nullptr, kFakeI, kFakeI, 0, 256, 6, 1.5f, kFakeI, kFakeF, nullptr, 0,
                   nullptr) == MOE_EINVAL);
  // moe_dispatch and its allocation-free variant
  const size_t dws = moe_dispatch_workspace_size(64, 256, 6);
  EXPECT(moe_dispatch(kFakeI, 64, 256, 6, kFakeI, kFakeI, kFakeI, kFakeWs, dws - 1, nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_dispatch(kFakeI, 64, 1024, 6, kFakeI, kFakeI, kFakeI, kFakeWs, dws, nullptr) == MOE_ESHAPE);
  EXPECT(moe_dispatch(nullptr, 64, 256, 6, kFakeI, kFakeI, kFakeI, kFakeWs, dws, nullptr) == MOE_EINVAL);
  EXPECT(moe_dispatch(kFakeI, 64, 256, 6, kFakeI, kFakeI, kFakeI, kFakeMis, dws, nullptr) == MOE_EALIGN);
  EXPECT(moe_dispatch_noalloc(kFakeI, 200000, 256, 6, kFakeI, kFakeI, kFakeI, nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_dispatch_noalloc(kFakeI, MOE_MAX_TOKENS + 1, 256, 6, kFakeI, kFakeI, kFakeI, nullptr) == MOE_ESHAPE);
  EXPECT(moe_dispatch_noalloc(kFakeI, 64, 256, 6, nullptr, kFakeI, kFakeI, nullptr) == MOE_EINVAL);
  // moe_expert_ffn / moe_expert_ffn_phase
  moe_experts d;
  moe_experts_init(&d, kFakeWs, 256, 4096, 2048);
  const size_t fws = moe_ffn_workspace_size(64, &d, 6);
  uint16_t* out = reinterpret_cast<uint16_t*>(kFakeWs);
  EXPECT(moe_expert_ffn(kFakeX, 64, &d, 6, kFakeI, kFakeI, 10.f, out, kFakeWs, fws - 1, nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_expert_ffn(kFakeX, 64, &d, 6, kFakeI, kFakeI, 0.f, out, kFakeWs, fws, nullptr) == MOE_EINVAL);
  EXPECT(moe_expert_ffn(kFakeX, 64, nullptr, 6, kFakeI, kFakeI, 10.f, out, kFakeWs, fws, nullptr) == MOE_EINVAL);
  EXPECT(moe_expert_ffn_phase(kFakeX, 64, &d, 6, kFakeI, kFakeI, 10.f, out, kFakeWs, fws, 3, nullptr) == MOE_EINVAL);
  EXPECT(moe_expert_ffn(kFakeX, 64, &d, 6, kFakeI, kFakeI, 10.f, reinterpret_cast<uint16_t*>(kFakeMis), kFakeWs, fws,
                        nullptr) == MOE_EALIGN);
  moe_experts flags = d;
  flags.flags = MOE_FFN_SPLIT_FP8 | MOE_SHARED_MXFP8;
  EXPECT(moe_expert_ffn(kFakeX, 64, &flags, 6, kFakeI, kFakeI, 10.f, out, kFakeWs, fws, nullptr) == MOE_EINVAL);
  flags.flags = 8;
  EXPECT(moe_expert_ffn(kFakeX, 64, &flags, 6, kFakeI, kFakeI, 10.f, out, kFakeWs, fws, nullptr) == MOE_EINVAL);
  moe_experts wrong = d;
  wrong.abi_version = MOE_ABI_VERSION + 1;
  EXPECT(moe_expert_ffn(kFakeX, 64, &wrong, 6, kFakeI, kFakeI, 10.f, out, kFakeWs, fws, nullptr) == MOE_ELAYOUT);
  // moe_combine
  EXPECT(moe_combine(out, kFakeI, kFakeF, 64, 4096, 9, kFakeX, nullptr) == MOE_ESHAPE);
  EXPECT(moe_combine(out, kFakeI, kFakeF, 64, 4100, 6, kFakeX, nullptr) == MOE_ESHAPE);
  EXPECT(moe_combine(nullptr, kFakeI, kFakeF, 64, 4096, 6, kFakeX, nullptr) == MOE_EINVAL);
  EXPECT(moe_combine(out, kFakeI, kFakeF, 64, 4096, 6, reinterpret_cast<uint16_t*>(kFakeMis), nullptr) ==
         MOE_EALIGN);
}

}  // namespace

int main() {
  check_pack_round_trips();
  check_descriptor_and_sizes();
  check_call_refusals();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
