// Drives every entry point of include/moda.h through its host-side
// validation, built with AddressSanitizer and UndefinedBehaviorSanitizer
// against host stand-ins of the kernel launchers (launch_stubs.cpp), so no
// GPU is needed.  For each entry point:
//   - a valid call returns MODA_OK and reaches its launcher;
//   - NULL shape, each required pointer NULL, each pointer misaligned, each
//     size argument one byte short, and a set of invalid shapes are rejected
//     with a non-OK status, a non-empty moda_last_error() and no launch.
// Exit status 0 when every expectation holds; the sanitizers abort on any
// memory or undefined-behaviour error in the validation code.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <functional>
#include <string>
#include <vector>

#include "../../include/moda.h"

extern int g_stub_launches;

namespace {

int g_fail = 0;

void expect(bool c, const std::string &what) {
  if (!c) {
    std::fprintf(stderr, "FAIL: %s\n", what.c_str());
    ++g_fail;
  }
}

// Fake device addresses: distinct, 256-byte aligned, never dereferenced.
void *dev(int i) { return (void *)(uintptr_t)(0x100000u + 0x1000u * (unsigned)i); }
void *misaligned(void *p) { return (void *)((uintptr_t)p + 2); }

struct Call {
  const char *name;
  int nptr;                      // pointer arguments, in order
  std::vector<int> nullable;     // indices of pointers that may be NULL
  int nsize;                     // size arguments, in order
  // runs the call with these pointers and sizes
  std::function<moda_status(const moda_shape *, void **, size_t *)> run;
  std::function<void(const moda_shape *, size_t *)> sizes;  // exact sizes for a valid call
  bool ignores_L = false;        // the entry point documents that it ignores s->L
};

void check_call(const Call &c, const moda_shape &good) {
  std::vector<void *> p(c.nptr);
  std::vector<size_t> sz(c.nsize > 0 ? c.nsize : 1);
  auto reset = [&]() {
    for (int i = 0; i < c.nptr; ++i) p[i] = dev(i);
    if (c.nsize) c.sizes(&good, sz.data());
  };
  auto rejected = [&](const moda_shape *s, const std::string &why) {
    const int before = g_stub_launches;
    const moda_status st = c.run(s, p.data(), sz.data());
    expect(st != MODA_OK, std::string(c.name) + " accepted " + why);
    expect(g_stub_launches == before, std::string(c.name) + " launched on " + why);
    expect(std::strlen(moda_last_error()) > 0, std::string(c.name) + " gave no detail on " + why);
    expect(std::strlen(moda_status_string(st)) > 0, "status text");
  };

  reset();
  {
    const int before = g_stub_launches;
    const moda_status st = c.run(&good, p.data(), sz.data());
    expect(st == MODA_OK, std::string(c.name) + " rejected a valid call: " + moda_last_error());
    expect(g_stub_launches > before, std::string(c.name) + " valid call reached no launcher");
    expect(std::strlen(moda_last_error()) == 0, std::string(c.name) + " left an error after success");
  }
  reset();
  rejected(nullptr, "a NULL shape");
  for (int i = 0; i < c.nptr; ++i) {
    bool may_be_null = false;
    for (int j : c.nullable) may_be_null |= (j == i);
    reset();
    p[i] = nullptr;
    if (!may_be_null) rejected(&good, "NULL pointer " + std::to_string(i));
    reset();
    p[i] = misaligned(dev(i));
    rejected(&good, "misaligned pointer " + std::to_string(i));
  }
  for (int i = 0; i < c.nsize; ++i) {
    reset();
    if (sz[i] == 0) continue;
    sz[i] -= 1;
    rejected(&good, "size " + std::to_string(i) + " one byte short");
  }
  std::vector<std::pair<moda_shape, std::string>> bad;
  moda_shape s = good;
  s.B = 0; bad.push_back({s, "B = 0"}); s = good;
  s.T = 0; bad.push_back({s, "T = 0"}); s = good;
  s.Hkv = good.Hq + 1; bad.push_back({s, "Hq not a multiple of Hkv"}); s = good;
  s.d = 48; bad.push_back({s, "d = 48"}); s = good;
  s.dtype = (moda_dtype)7; bad.push_back({s, "an unknown dtype"}); s = good;
  if (!c.ignores_L) {
    s.L = -1;
    bad.push_back({s, "L = -1"});
    s = good;
  }
  s.B = (int64_t)1 << 40; s.T = (int64_t)1 << 22; bad.push_back({s, "an overflowing size"}); s = good;
  s.Hq = -4; bad.push_back({s, "Hq < 0"}); s = good;
  for (auto &b : bad) {
    reset();
    rejected(&b.first, b.second);
  }
}

}  // namespace

int main() {
  const moda_shape bf = {2, 8, 2, 300, 5, 128, MODA_BF16};
  const moda_shape f32 = {1, 4, 2, 70, 3, 64, MODA_F32};

  std::vector<Call> calls = {
      {"moda_pack_depth_cache", 3, {}, 1,
       [](const moda_shape *s, void **p, size_t *z) {
         return moda_pack_depth_cache(s, p[0], p[1], p[2], z[0], nullptr);
       },
       [](const moda_shape *s, size_t *z) { z[0] = moda_depth_cache_bytes(s); }},
      {"moda_fwd", 6, {5}, 1,
       [](const moda_shape *s, void **p, size_t *z) {
         return moda_fwd(s, p[0], p[1], p[2], p[3], z[0], p[4], (float *)p[5], nullptr);
       },
       [](const moda_shape *s, size_t *z) { z[0] = moda_depth_cache_bytes(s); }},
      {"moda_causal_fwd", 5, {4}, 0,
       [](const moda_shape *s, void **p, size_t *) {
         return moda_causal_fwd(s, p[0], p[1], p[2], p[3], (float *)p[4], nullptr);
       },
       nullptr, true},
      {"moda_depth_fwd", 4, {3}, 1,
       [](const moda_shape *s, void **p, size_t *z) {
         return moda_depth_fwd(s, p[0], p[1], z[0], p[2], (float *)p[3], nullptr);
       },
       [](const moda_shape *s, size_t *z) { z[0] = moda_depth_cache_bytes(s); }},
      {"moda_append_depth", 3, {}, 1,
       [](const moda_shape *s, void **p, size_t *z) {
         return moda_append_depth(s, 1, 2, p[0], p[1], p[2], z[0], nullptr);
       },
       [](const moda_shape *s, size_t *z) { z[0] = moda_depth_cache_bytes(s); }},
  };
  for (const auto &c : calls) {
    check_call(c, bf);
    check_call(c, f32);
  }

  // MFMA-only entry points (bf16, d = 128)
  std::vector<Call> mfma = {
      {"moda_fwd_natural", 7, {6}, 0,
       [](const moda_shape *s, void **p, size_t *) {
         return moda_fwd_natural(s, p[0], p[1], p[2], p[3], p[4], p[5], (float *)p[6], nullptr);
       },
       nullptr},
      {"moda_fwd_layers", 7, {6}, 0,
       [](const moda_shape *s, void **p, size_t *) {
         return moda_fwd_layers(s, p[0], p[1], p[2], p[3], p[4], p[5], (float *)p[6], nullptr);
       },
       nullptr},
      {"moda_fwd_masked_scan", 7, {6}, 0,
       [](const moda_shape *s, void **p, size_t *) {
         return moda_fwd_masked_scan(s, p[0], p[1], p[2], p[3], p[4], p[5], (float *)p[6],
                                     nullptr);
       },
       nullptr},
      {"moda_fwd_strided", 7, {6}, 0,
       [](const moda_shape *s, void **p, size_t *) {
         const int64_t L = s ? s->L : 0, TL = s ? s->T * s->L : 0;
         return moda_fwd_strided(s, p[0], p[1], p[2], p[3], p[4], TL, L, 1, p[5], (float *)p[6],
                                 nullptr);
       },
       nullptr},
      {"moda_bwd", 15, {}, 1,
       [](const moda_shape *s, void **p, size_t *z) {
         return moda_bwd(s, p[0], p[1], p[2], p[3], p[4], p[5], z[0], p[6], (const float *)p[7],
                         p[8], p[9], p[10], p[11], p[12], p[13], (float *)p[14], nullptr);
       },
       [](const moda_shape *s, size_t *z) { z[0] = moda_depth_cache_bytes(s); }},
      {"moda_decode", 8, {5}, 1,
       [](const moda_shape *s, void **p, size_t *z) {
         return moda_decode(s, p[0], p[1], p[2], p[3], p[4], p[6], (float *)p[5], p[7], z[0],
                            nullptr);
       },
       [](const moda_shape *s, size_t *z) { z[0] = moda_decode_workspace_bytes(s); }},
      {"moda_decode_varlen", 9, {6}, 1,
       [](const moda_shape *s, void **p, size_t *z) {
         return moda_decode_varlen(s, (const int32_t *)p[0], p[1], p[2], p[3], p[4], p[5], p[7],
                                   (float *)p[6], p[8], z[0], nullptr);
       },
       [](const moda_shape *s, size_t *z) { z[0] = moda_decode_workspace_bytes(s); }},
      {"moda_decode_noalloc", 8, {0, 6}, 0,
       [](const moda_shape *s, void **p, size_t *) {
         return moda_decode_noalloc(s, (const int32_t *)p[0], p[1], p[2], p[3], p[4], p[5], p[7],
                                    (float *)p[6], nullptr);
       },
       nullptr},
  };
  for (const auto &c : mfma) check_call(c, bf);
  {
    // a shape whose partial states outgrow the static scratch is refused before any launch
    const moda_shape big = {4096, 128, 4, 64, 0, 128, MODA_BF16};
    expect(moda_decode_workspace_bytes(&big) > ((size_t)8 << 20), "big decode shape");
    const int before = g_stub_launches;
    const moda_status st = moda_decode_noalloc(&big, nullptr, dev(1), dev(2), dev(3), nullptr,
                                               nullptr, dev(4), nullptr, nullptr);
    expect(st == MODA_ERR_UNSUPPORTED && g_stub_launches == before,
           "moda_decode_noalloc refuses a shape beyond its scratch");
  }

  // moda_bwd's unused slot 15 and the workspace variant: a valid split call
  {
    const moda_shape small = {1, 16, 4, 4096, 8, 128, MODA_BF16};
    const size_t ws = moda_bwd_workspace_bytes(&small);
    expect(ws > 0, "the small-grid backward asks for a split workspace");
    std::vector<void *> p(17);
    for (int i = 0; i < 17; ++i) p[i] = dev(i);
    const int before = g_stub_launches;
    moda_status st = moda_bwd_ws(&small, p[0], p[1], p[2], p[3], p[4], p[5],
                                 moda_depth_cache_bytes(&small), p[6], (const float *)p[7], p[8],
                                 p[9], p[10], p[11], p[12], p[13], (float *)p[14], p[15], ws,
                                 nullptr);
    expect(st == MODA_OK && g_stub_launches > before, "moda_bwd_ws valid call");
    st = moda_bwd_ws(&small, p[0], p[1], p[2], p[3], p[4], p[5], moda_depth_cache_bytes(&small),
                     p[6], (const float *)p[7], p[8], p[9], p[10], p[11], p[12], p[13],
                     (float *)p[14], p[15], ws - 1, nullptr);
    expect(st != MODA_OK, "moda_bwd_ws accepted a short workspace");
  }

  // host-only queries never fail on bad input
  expect(moda_depth_cache_bytes(nullptr) == 0, "cache bytes of NULL");
  expect(std::strcmp(moda_fwd_variant(nullptr), "") == 0, "variant of NULL");
  expect(moda_decode_workspace_bytes(nullptr) == 0, "decode workspace of NULL");
  expect(moda_bwd_workspace_bytes(nullptr) == 0, "bwd workspace of NULL");
  for (int st = -1; st < 6; ++st) expect(moda_status_string((moda_status)st) != nullptr, "status");
  expect(std::strncmp(moda_fwd_variant(&f32), "mfma_f32_d", 10) == 0, "f32 variant");
  moda_shape wide = f32;  // G above 128: the VALU kernel
  wide.Hq = 256 * wide.Hkv;
  expect(std::strcmp(moda_fwd_variant(&wide), "generic") == 0, "f32 variant, G = 256");

  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi driver: all expectations hold (%d launches reached)\n", g_stub_launches);
  return 0;
}
