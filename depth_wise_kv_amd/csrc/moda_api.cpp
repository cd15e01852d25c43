// C ABI of libmoda (declared in include/moda.h): host-side validation,
// kernel selection and launch.  No device memory is allocated here.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/moda.h"
#include "moda_internal.h"
#include "moda_small.h"

namespace {

thread_local std::string g_last_error;

moda_status fail(moda_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

moda_status ok() {
  g_last_error.clear();
  return MODA_OK;
}

// MODA_LOG=1 (any value but "0") makes every call that enqueues work print one
// line to stderr when it returns: the entry point, the shape, the kernel the
// shape selects, and "ok" or the error.  The calls' own error texts are what
// moda_last_error() returns.
bool log_enabled() {
  static const bool on = [] {
    const char *e = std::getenv("MODA_LOG");
    return e && *e && std::strcmp(e, "0") != 0;
  }();
  return on;
}

struct CallLog {
  const char *name;
  const moda_shape *s;
  CallLog(const char *n, const moda_shape *sh) : name(n), s(sh) { g_last_error.clear(); }
  ~CallLog();
};

constexpr int64_t kMaxElems = (int64_t)1 << 62;

// a * b * ... without overflow past kMaxElems; returns -1 on overflow
int64_t checked_prod(std::initializer_list<int64_t> xs) {
  int64_t acc = 1;
  for (int64_t x : xs) {
    if (x < 0) return -1;
    if (x != 0 && acc > kMaxElems / x) return -1;
    acc *= x;
  }
  return acc;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

moda_status check_shape_impl(const moda_shape *s) {
  if (!s) return fail(MODA_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 1 || s->Hq < 1 || s->Hkv < 1 || s->T < 1)
    return fail(MODA_ERR_INVALID_ARG, "B, Hq, Hkv and T must be >= 1");
  if (s->L < 0) return fail(MODA_ERR_INVALID_ARG, "L must be >= 0");
  if (s->L > ((int64_t)1 << 30)) return fail(MODA_ERR_UNSUPPORTED, "L above 2^30");
  if (s->Hq % s->Hkv != 0) return fail(MODA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (s->dtype != MODA_F32 && s->dtype != MODA_BF16)
    return fail(MODA_ERR_INVALID_ARG, "dtype must be MODA_F32 or MODA_BF16");
  if (s->d != 32 && s->d != 64 && s->d != 128)
    return fail(MODA_ERR_UNSUPPORTED, "head dim d must be 32, 64 or 128");
  if (checked_prod({s->B, s->Hq, s->T, s->d}) < 0 ||
      checked_prod({s->B, s->Hkv, s->T, s->L, s->d}) < 0 ||
      checked_prod({s->B, s->Hkv, s->T, s->L, s->d, 4}) < 0)
    return fail(MODA_ERR_INVALID_ARG, "tensor size overflows");
  if (s->dtype == MODA_BF16 && s->d == moda::kMfmaD && s->T > ((int64_t)1 << 23))
    return fail(MODA_ERR_UNSUPPORTED, "bf16 with d = 128 supports T up to 2^23");
  if (s->dtype == MODA_BF16 && s->d == moda::kMfmaD && s->Hq / s->Hkv > moda::kMfmaRows)
    return fail(MODA_ERR_UNSUPPORTED, "bf16 with d = 128 supports G = Hq / Hkv up to 256");
  return MODA_OK;
}

// The MFMA path (and its packed depth layout) serves every bf16 shape with
// d == 128; the layout does not depend on G, so a cache can be packed
// without knowing the query head count.
bool use_mfma(const moda_shape *s) { return s->dtype == MODA_BF16 && s->d == moda::kMfmaD; }

// The matrix-core kernel for the other head dims and fp32 (moda_fwd_small.hip)
// serves the rest up to G = 128; the one-wave-per-row VALU kernel only G above.
bool use_small(const moda_shape *s) {
  return !use_mfma(s) && moda::small_supported(s->dtype == MODA_BF16, s->d, s->Hq / s->Hkv);
}

hipError_t launch_fwd_other(const moda_shape *s, const moda::FwdArgs &a, hipStream_t stream) {
  const bool bf16 = s->dtype == MODA_BF16;
  return use_small(s) ? moda::launch_fwd_small(a, bf16, stream)
                      : moda::launch_fwd_generic(a, bf16, stream);
}

// Blocks of the packed cache per (b, kv head): one per (group of 8 tokens,
// group of 4 entries).
int64_t depth_blocks(const moda_shape *s) {
  return (s->T + moda::kGroupTokens - 1) / moda::kGroupTokens *
         ((s->L + moda::kGroupEntries - 1) / moda::kGroupEntries);
}

size_t cache_bytes(const moda_shape *s) {
  if (s->L == 0) return 0;
  if (use_mfma(s)) return (size_t)(s->B * s->Hkv * depth_blocks(s) * moda::kPackedBlockBytes);
  const int64_t es = s->dtype == MODA_BF16 ? 2 : 4;
  return (size_t)(2 * s->B * s->Hkv * s->T * s->L * s->d * es);
}

moda_status grid_fits(const moda_shape *s) {
  int64_t grid;
  if (use_mfma(s)) {
    const int64_t G = s->Hq / s->Hkv, tq = moda::kMfmaRows / G;
    grid = (s->T + tq - 1) / tq * s->B * s->Hkv;
    if (s->L > 0 && depth_blocks(s) > 0x7FFFFFFFll)
      return fail(MODA_ERR_UNSUPPORTED, "depth cache too long for the pack grid");
    if (s->B * s->Hkv > 65535) return fail(MODA_ERR_UNSUPPORTED, "B * Hkv above 65535");
  } else if (use_small(s)) {
    grid = moda::small_grid(s->B, s->Hkv, s->T, s->Hq / s->Hkv);
  } else {
    grid = s->B * s->Hq * s->T;
  }
  if (grid > 0x7FFFFFFFll) return fail(MODA_ERR_UNSUPPORTED, "problem too large for one launch");
  return MODA_OK;
}

// Forward workgroup size: 8 waves (256 rows) when there are many tiles; 4
// waves (128 rows, two workgroups per CU) when the 256-row grid would fill
// the 256 CUs at most twice over.  Then the causal tiles' unequal lengths
// leave CUs idle at the end, and a second, smaller workgroup per CU fills
// them (18-25% less time at T = 4096, B = 1; no change at 1024 tiles).  When
// even the 128-row grid fills the chip's 512 four-wave slots at most once, the
// heaviest tile alone sets the time; the key-split form runs it on two waves
// per SIMD (8 waves on 128 rows) and takes 2-10% less time there, but more
// wherever a CU would run workgroups one after another.
int fwd_waves(const moda_shape *s) {
  const int64_t G = s->Hq / s->Hkv, tq = moda::kMfmaRows / G;
  const int64_t tiles = (s->T + tq - 1) / tq * s->B * s->Hkv;  // of 256 rows
  const bool rows128 = G <= moda::kMfmaRows / 2;
  // tiles of 128 rows (G <= 128): twice the grid of 256-row tiles at most
  const int64_t tq2 = rows128 ? moda::kMfmaRows / 2 / G : 1;
  const int64_t tiles2 = (s->T + tq2 - 1) / tq2 * s->B * s->Hkv;
  // a forced choice (for tests and timing) is taken when its grid fits one launch
  const char *env = std::getenv("MODA_FWD_VARIANT");
  if (env && std::strcmp(env, "w8") == 0) return 8;
  if (env && rows128 && tiles2 <= 0x7FFFFFFFll) {
    if (std::strcmp(env, "w4") == 0) return 4;
    if (std::strcmp(env, "ks") == 0) return moda::kFwdKeySplit;
  }
  if (rows128 && tiles2 <= 512) return moda::kFwdKeySplit;
  return (rows128 && tiles <= 512) ? 4 : 8;
}

moda_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(MODA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

moda::FwdArgs make_fwd_args(const moda_shape *s, const void *q, const void *k, const void *v,
                            const void *packed, void *out, float *lse, bool has_depth,
                            bool has_seq = true) {
  moda::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.packed = packed;
  a.out = out;
  a.lse = lse;
  a.B = s->B;
  a.Hq = s->Hq;
  a.Hkv = s->Hkv;
  a.T = s->T;
  a.L = has_depth ? s->L : 0;
  a.d = s->d;
  a.nblk = depth_blocks(s);
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)s->d));
  a.has_depth = has_depth && s->L > 0;
  a.has_seq = has_seq;
  return a;
}

moda_status check_packed(const moda_shape *s, const void *packed, size_t packed_bytes) {
  if (!packed) return fail(MODA_ERR_INVALID_ARG, "packed must be non-NULL when L > 0");
  if (!aligned16(packed)) return fail(MODA_ERR_INVALID_ARG, "packed must be 16-byte aligned");
  const size_t need = cache_bytes(s);
  if (packed_bytes < need)
    return fail(MODA_ERR_INVALID_ARG, "packed buffer too small: need " + std::to_string(need) +
                                          " bytes, got " + std::to_string(packed_bytes));
  return MODA_OK;
}

moda_status check_qkvo(const void *q, const void *k, const void *v, const void *out,
                       const float *lse) {
  if (!q || !k || !v || !out) return fail(MODA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (lse && !aligned16(lse)))
    return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  return MODA_OK;
}

// Decode split: per (b, kv head) the cache's and the depth entries' 32-entry
// blocks form one list, cut into nsplit even parts, one workgroup each.  The
// parts fill the chip once (one 8-wave workgroup per compute unit, 256 units)
// while every wave still gets a block.  Where the blocks, not the chip, limit
// that split to half the units or fewer (short caches, few heads), parts of 4
// waves double the count: more units share the stream, and a part waits for
// its slowest of 4 waves, not 8, before the waves merge.
constexpr int64_t kDecodeUnits = 256;

struct DecodePlan {
  int64_t nsplit;
  int waves;
};

DecodePlan decode_plan(const moda_shape *s) {
  const int64_t BH = s->B * s->Hkv;
  const int64_t nb = (s->T + 31) / 32 + (s->L + 31) / 32;
  auto splits = [&](int64_t waves) {
    int64_t n = kDecodeUnits * (8 / waves) / BH;
    if (n > nb / waves) n = nb / waves;
    return n < 1 ? (int64_t)1 : n;
  };
  const int64_t n8 = splits(8);
  if (BH * n8 <= kDecodeUnits / 2) {
    const int64_t n4 = splits(4);
    if (n4 > n8) return {n4, 4};
  }
  return {n8, 8};
}

moda_status check_decode_shape(const moda_shape *s) {
  moda_status st = check_shape_impl(s);
  if (st != MODA_OK) return st;
  if (!use_mfma(s)) return fail(MODA_ERR_UNSUPPORTED, "moda_decode supports bf16 with d = 128");
  if (s->Hq / s->Hkv > 32) return fail(MODA_ERR_UNSUPPORTED, "moda_decode supports G up to 32");
  if (s->L >= ((int64_t)1 << 23)) return fail(MODA_ERR_UNSUPPORTED, "moda_decode supports L below 2^23");
  if (s->B * s->Hkv > 65535) return fail(MODA_ERR_UNSUPPORTED, "B * Hkv above 65535");
  return MODA_OK;
}

size_t decode_ws_bytes(const moda_shape *s) {
  return (size_t)(s->B * s->Hq * decode_plan(s).nsplit * moda::kDecodeRecord * 4);
}

// shape and tensor arguments of a decode call (everything but the workspace)
moda_status decode_check_args(const moda_shape *s, const void *q, const void *k_cache,
                              const void *v_cache, const void *k_depth, const void *v_depth,
                              const void *out, const float *lse) {
  moda_status st = check_decode_shape(s);
  if (st != MODA_OK) return st;
  st = check_qkvo(q, k_cache, v_cache, out, lse);
  if (st != MODA_OK) return st;
  if (s->L > 0) {
    if (!k_depth || !v_depth)
      return fail(MODA_ERR_INVALID_ARG, "k_depth and v_depth must be non-NULL when L > 0");
    if (!aligned16(k_depth) || !aligned16(v_depth))
      return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  } else if (k_depth || v_depth) {
    return fail(MODA_ERR_INVALID_ARG, "depth inputs must be NULL when L == 0");
  }
  return MODA_OK;
}

moda_status decode_impl(const moda_shape *s, const int32_t *lens, const void *q,
                        const void *k_cache, const void *v_cache, const void *k_depth,
                        const void *v_depth, void *out, float *lse, void *workspace,
                        size_t workspace_bytes, void *hip_stream) {
  moda_status st = decode_check_args(s, q, k_cache, v_cache, k_depth, v_depth, out, lse);
  if (st != MODA_OK) return st;
  if (!workspace || !aligned16(workspace))
    return fail(MODA_ERR_INVALID_ARG, "workspace must be non-NULL and 16-byte aligned");
  const size_t need = decode_ws_bytes(s);
  if (workspace_bytes < need)
    return fail(MODA_ERR_INVALID_ARG, "workspace too small: need " + std::to_string(need) +
                                          " bytes, got " + std::to_string(workspace_bytes));
  moda::DecArgs a{};
  a.q = q;
  a.lens = lens;
  a.k = k_cache;
  a.v = v_cache;
  a.kd = k_depth;
  a.vd = v_depth;
  a.out = out;
  a.lse = lse;
  a.ws = (float *)workspace;
  a.B = s->B;
  a.Hq = s->Hq;
  a.Hkv = s->Hkv;
  a.T = s->T;
  a.L = s->L;
  const DecodePlan plan = decode_plan(s);
  a.nsplit = plan.nsplit;
  a.waves = plan.waves;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)s->d));
  return hip_status(moda::launch_decode(a, (hipStream_t)hip_stream), "decode launch");
}

}  // namespace

namespace {
CallLog::~CallLog() {
  if (!log_enabled()) return;
  // the variant lookup validates the shape again, which sets or clears the
  // thread's last error: keep the call's own
  const std::string err = g_last_error;
  const char *result = err.empty() ? "ok" : err.c_str();
  if (!s) {
    std::fprintf(stderr, "moda: %s (no shape): %s\n", name, result);
    return;
  }
  const std::string variant = moda_fwd_variant(s);
  g_last_error = err;
  std::fprintf(stderr, "moda: %s B=%lld Hq=%lld Hkv=%lld T=%lld L=%lld d=%lld %s [%s]: %s\n",
               name, (long long)s->B, (long long)s->Hq, (long long)s->Hkv, (long long)s->T,
               (long long)s->L, (long long)s->d, s->dtype == MODA_BF16 ? "bf16" : "f32",
               variant.c_str(), result);
}
}  // namespace

extern "C" {

moda_status moda_check_shape(const moda_shape *s) {
  moda_status st = check_shape_impl(s);
  if (st != MODA_OK) return st;
  st = grid_fits(s);
  if (st != MODA_OK) return st;
  return ok();
}

size_t moda_depth_cache_bytes(const moda_shape *s) {
  if (check_shape_impl(s) != MODA_OK) return 0;
  return cache_bytes(s);
}

const char *moda_fwd_variant(const moda_shape *s) {
  if (check_shape_impl(s) != MODA_OK) return "";
  if (use_small(s)) {
    static const char *const names[2][3] = {{"mfma_f32_d32", "mfma_f32_d64", "mfma_f32_d128"},
                                            {"mfma_bf16_d32", "mfma_bf16_d64", ""}};
    return names[s->dtype == MODA_BF16][s->d == 32 ? 0 : s->d == 64 ? 1 : 2];
  }
  if (!use_mfma(s)) return "generic";
  const int w = fwd_waves(s);
  return w == 4 ? "mfma_bf16_d128_w4" : w == 8 ? "mfma_bf16_d128_w8" : "mfma_bf16_d128_ks";
}

moda_status moda_pack_depth_cache(const moda_shape *s, const void *k_depth, const void *v_depth,
                                  void *packed, size_t packed_bytes, void *hip_stream) {
  CallLog log_("moda_pack_depth_cache", s);
  moda_status st = moda_check_shape(s);
  if (st != MODA_OK) return st;
  if (s->L < 1) return fail(MODA_ERR_INVALID_ARG, "moda_pack_depth_cache needs L >= 1");
  if (!k_depth || !v_depth || !packed)
    return fail(MODA_ERR_INVALID_ARG, "k_depth, v_depth and packed must be non-NULL");
  if (!aligned16(k_depth) || !aligned16(v_depth) || !aligned16(packed))
    return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const size_t need = cache_bytes(s);
  if (packed_bytes < need)
    return fail(MODA_ERR_INVALID_ARG, "packed buffer too small: need " + std::to_string(need) +
                                          " bytes, got " + std::to_string(packed_bytes));
  moda::PackArgs a{k_depth, v_depth, packed, s->B, s->Hkv, s->T, s->L, s->d, depth_blocks(s)};
  hipStream_t stream = (hipStream_t)hip_stream;
  if (use_mfma(s)) return hip_status(moda::launch_pack_mfma(a, stream), "pack launch");
  return hip_status(moda::launch_pack_generic(a, s->dtype == MODA_BF16, stream), "pack launch");
}

moda_status moda_append_depth(const moda_shape *s, int64_t first, int64_t n, const void *k_new,
                              const void *v_new, void *packed, size_t packed_bytes,
                              void *hip_stream) {
  CallLog log_("moda_append_depth", s);
  moda_status st = moda_check_shape(s);
  if (st != MODA_OK) return st;
  if (s->L < 1) return fail(MODA_ERR_INVALID_ARG, "moda_append_depth needs L >= 1");
  if (n < 1 || first < 0 || first > s->L - n)
    return fail(MODA_ERR_INVALID_ARG, "entries [first, first + n) must lie in [0, L) with n >= 1");
  if (!k_new || !v_new || !packed)
    return fail(MODA_ERR_INVALID_ARG, "k_new, v_new and packed must be non-NULL");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(packed))
    return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const size_t need = cache_bytes(s);
  if (packed_bytes < need)
    return fail(MODA_ERR_INVALID_ARG, "packed buffer too small: need " + std::to_string(need) +
                                          " bytes, got " + std::to_string(packed_bytes));
  const int64_t es = s->dtype == MODA_BF16 ? 2 : 4;
  if (use_mfma(s) ? n > 65535 : (s->T * n * (s->d * es / 16) + 255) / 256 > 0x7FFFFFFFll)
    return fail(MODA_ERR_UNSUPPORTED, use_mfma(s) ? "moda_append_depth writes at most 65535 "
                                                    "entries per call"
                                                  : "problem too large for one launch");
  moda::AppendArgs a{k_new, v_new, packed, s->B, s->Hkv, s->T, s->L, depth_blocks(s), first, n};
  return hip_status(moda::launch_append(a, use_mfma(s), (int)(s->d * es), (hipStream_t)hip_stream),
                    "append launch");
}

moda_status moda_fwd(const moda_shape *s, const void *q, const void *k, const void *v,
                     const void *packed, size_t packed_bytes, void *out, float *lse,
                     void *hip_stream) {
  CallLog log_("moda_fwd", s);
  moda_status st = moda_check_shape(s);
  if (st != MODA_OK) return st;
  st = check_qkvo(q, k, v, out, lse);
  if (st != MODA_OK) return st;
  if (s->L > 0) {
    st = check_packed(s, packed, packed_bytes);
    if (st != MODA_OK) return st;
  } else if (packed || packed_bytes) {
    return fail(MODA_ERR_INVALID_ARG, "packed must be NULL with size 0 when L == 0");
  }
  moda::FwdArgs a = make_fwd_args(s, q, k, v, packed, out, lse, true);
  hipStream_t stream = (hipStream_t)hip_stream;
  if (use_mfma(s))
    return hip_status(moda::launch_fwd_mfma(a, (int)(s->Hq / s->Hkv), fwd_waves(s), stream), "fwd launch");
  return hip_status(launch_fwd_other(s, a, stream), "fwd launch");
}

moda_status moda_causal_fwd(const moda_shape *s, const void *q, const void *k, const void *v,
                            void *out, float *lse, void *hip_stream) {
  CallLog log_("moda_causal_fwd", s);
  if (!s) return fail(MODA_ERR_INVALID_ARG, "shape is NULL");
  moda_shape s0 = *s;
  s0.L = 0;
  moda_status st = moda_check_shape(&s0);
  if (st != MODA_OK) return st;
  st = check_qkvo(q, k, v, out, lse);
  if (st != MODA_OK) return st;
  moda::FwdArgs a = make_fwd_args(&s0, q, k, v, nullptr, out, lse, false);
  hipStream_t stream = (hipStream_t)hip_stream;
  if (use_mfma(&s0))
    return hip_status(moda::launch_fwd_mfma(a, (int)(s0.Hq / s0.Hkv), fwd_waves(&s0), stream), "causal launch");
  return hip_status(launch_fwd_other(&s0, a, stream), "causal launch");
}

moda_status moda_depth_fwd(const moda_shape *s, const void *q, const void *packed,
                           size_t packed_bytes, void *out, float *lse, void *hip_stream) {
  CallLog log_("moda_depth_fwd", s);
  moda_status st = moda_check_shape(s);
  if (st != MODA_OK) return st;
  if (s->L < 1) return fail(MODA_ERR_INVALID_ARG, "moda_depth_fwd needs L >= 1");
  if (!q || !out) return fail(MODA_ERR_INVALID_ARG, "q and out must be non-NULL");
  if (!aligned16(q) || !aligned16(out) || (lse && !aligned16(lse)))
    return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  st = check_packed(s, packed, packed_bytes);
  if (st != MODA_OK) return st;
  moda::FwdArgs a = make_fwd_args(s, q, nullptr, nullptr, packed, out, lse, true, false);
  hipStream_t stream = (hipStream_t)hip_stream;
  if (use_mfma(s))
    return hip_status(moda::launch_fwd_mfma(a, (int)(s->Hq / s->Hkv), fwd_waves(s), stream), "depth launch");
  return hip_status(launch_fwd_other(s, a, stream), "depth launch");
}

namespace {

// dK/dV split of the backward: when 128-key workgroups would not fill the chip
// twice over, each key tile's query range goes to S parts (S <= 8, and at
// least 4 query tiles per part of the heaviest key tile).
int64_t bwd_splits(const moda_shape *s) {
  const int64_t G = s->Hq / s->Hkv;
  const int64_t base = (s->T + 127) / 128 * s->B * s->Hkv;
  if (base >= 512) return 1;
  int64_t S = (512 + base - 1) / base;
  if (S > 8) S = 8;
  const int64_t heaviest = (s->T + 64 / G - 1) / (64 / G);  // query tiles of key tile 0
  if (S > heaviest / 4) S = heaviest / 4;
  return S < 1 ? 1 : S;
}

size_t bwd_ws_bytes(const moda_shape *s) {
  const int64_t S = bwd_splits(s);
  return S > 1 ? (size_t)(2 * S * s->B * s->Hkv * s->T * s->d * 4) : 0;
}

moda_status bwd_check(const moda_shape *s) {
  moda_status st = moda_check_shape(s);
  if (st != MODA_OK) return st;
  if (!use_mfma(s)) return fail(MODA_ERR_UNSUPPORTED, "moda_bwd supports bf16 with d = 128");
  if (s->Hq / s->Hkv > 64) return fail(MODA_ERR_UNSUPPORTED, "moda_bwd supports G up to 64");
  if (s->Hq / s->Hkv * s->T >= ((int64_t)1 << 23))
    return fail(MODA_ERR_UNSUPPORTED, "moda_bwd supports G * T below 2^23");
  if (s->L > 0) {
    if (s->Hq / s->Hkv > 32)
      return fail(MODA_ERR_UNSUPPORTED, "moda_bwd with depth entries supports G up to 32");
    if (s->T * s->L >= ((int64_t)1 << 23))
      return fail(MODA_ERR_UNSUPPORTED, "moda_bwd supports T * L below 2^23");
  }
  return MODA_OK;
}

moda_status bwd_impl(const moda_shape *s, const void *q, const void *k, const void *v,
                     const void *k_depth, const void *v_depth, const void *packed,
                     size_t packed_bytes, const void *out, const float *lse, const void *dout,
                     void *dq, void *dk, void *dv, void *dk_depth, void *dv_depth, float *delta,
                     int64_t nsplit, void *workspace, void *hip_stream) {
  moda_status st = bwd_check(s);
  if (st != MODA_OK) return st;
  if (s->L > 0) {
    if (!k_depth || !v_depth || !dk_depth || !dv_depth)
      return fail(MODA_ERR_INVALID_ARG, "depth inputs and gradients must be non-NULL when L > 0");
    if (!aligned16(k_depth) || !aligned16(v_depth) || !aligned16(dk_depth) || !aligned16(dv_depth))
      return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    st = check_packed(s, packed, packed_bytes);
    if (st != MODA_OK) return st;
  }
  st = check_qkvo(q, k, v, out, lse);
  if (st != MODA_OK) return st;
  if (!lse || !dout || !dq || !dk || !dv || !delta)
    return fail(MODA_ERR_INVALID_ARG, "lse, dout, dq, dk, dv and delta must be non-NULL");
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(delta))
    return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (s->L == 0 && (k_depth || v_depth || packed || packed_bytes || dk_depth || dv_depth))
    return fail(MODA_ERR_INVALID_ARG, "depth arguments must be NULL when L == 0");
  moda::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.packed = packed;
  a.kd = k_depth;
  a.vd = v_depth;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dkd = dk_depth;
  a.dvd = dv_depth;
  a.B = s->B;
  a.Hq = s->Hq;
  a.Hkv = s->Hkv;
  a.T = s->T;
  a.L = s->L;
  a.d = s->d;
  a.nblk = depth_blocks(s);
  a.scale = (float)(1.0 / std::sqrt((double)s->d));
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)s->d));
  a.nsplit = nsplit;
  a.kv_ws = (float *)workspace;
  return hip_status(moda::launch_bwd(a, (hipStream_t)hip_stream), "bwd launch");
}

}  // namespace

moda_status moda_bwd(const moda_shape *s, const void *q, const void *k, const void *v,
                     const void *k_depth, const void *v_depth, const void *packed,
                     size_t packed_bytes, const void *out, const float *lse, const void *dout,
                     void *dq, void *dk, void *dv, void *dk_depth, void *dv_depth, float *delta,
                     void *hip_stream) {
  CallLog log_("moda_bwd", s);
  return bwd_impl(s, q, k, v, k_depth, v_depth, packed, packed_bytes, out, lse, dout, dq, dk, dv,
                  dk_depth, dv_depth, delta, 1, nullptr, hip_stream);
}

size_t moda_bwd_workspace_bytes(const moda_shape *s) {
  if (!s || bwd_check(s) != MODA_OK) return 0;
  return bwd_ws_bytes(s);
}

moda_status moda_bwd_ws(const moda_shape *s, const void *q, const void *k, const void *v,
                        const void *k_depth, const void *v_depth, const void *packed,
                        size_t packed_bytes, const void *out, const float *lse, const void *dout,
                        void *dq, void *dk, void *dv, void *dk_depth, void *dv_depth,
                        float *delta, void *workspace, size_t workspace_bytes,
                        void *hip_stream) {
  CallLog log_("moda_bwd_ws", s);
  moda_status st = bwd_check(s);
  if (st != MODA_OK) return st;
  const size_t need = bwd_ws_bytes(s);
  if (workspace_bytes < need)
    return fail(MODA_ERR_INVALID_ARG, "workspace too small: need " + std::to_string(need) +
                                          " bytes, got " + std::to_string(workspace_bytes));
  if (need && (!workspace || !aligned16(workspace)))
    return fail(MODA_ERR_INVALID_ARG, "workspace must be a 16-byte aligned device pointer");
  return bwd_impl(s, q, k, v, k_depth, v_depth, packed, packed_bytes, out, lse, dout, dq, dk, dv,
                  dk_depth, dv_depth, delta, need ? bwd_splits(s) : 1, workspace, hip_stream);
}

moda_status moda_fwd_natural(const moda_shape *s, const void *q, const void *k, const void *v,
                             const void *k_depth, const void *v_depth, void *out, float *lse,
                             void *hip_stream) {
  CallLog log_("moda_fwd_natural", s);
  moda_status st = moda_check_shape(s);
  if (st != MODA_OK) return st;
  if (!use_mfma(s))
    return fail(MODA_ERR_UNSUPPORTED, "moda_fwd_natural supports bf16 with d = 128");
  st = check_qkvo(q, k, v, out, lse);
  if (st != MODA_OK) return st;
  if (s->L == 0) {
    if (k_depth || v_depth)
      return fail(MODA_ERR_INVALID_ARG, "depth inputs must be NULL when L == 0");
    return moda_fwd(s, q, k, v, nullptr, 0, out, lse, hip_stream);
  }
  if (!k_depth || !v_depth)
    return fail(MODA_ERR_INVALID_ARG, "k_depth and v_depth must be non-NULL when L > 0");
  if (!aligned16(k_depth) || !aligned16(v_depth))
    return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (s->T * s->L >= ((int64_t)1 << 23))
    return fail(MODA_ERR_UNSUPPORTED, "moda_fwd_natural supports T * L below 2^23");
  moda::FwdArgs a = make_fwd_args(s, q, k, v, nullptr, out, lse, true);
  a.kd_nat = k_depth;
  a.vd_nat = v_depth;
  return hip_status(moda::launch_fwd_mfma(a, (int)(s->Hq / s->Hkv), fwd_waves(s), (hipStream_t)hip_stream),
                    "fwd launch");
}

size_t moda_decode_workspace_bytes(const moda_shape *s) {
  if (check_decode_shape(s) != MODA_OK) return 0;
  return decode_ws_bytes(s);
}

moda_status moda_decode(const moda_shape *s, const void *q, const void *k_cache,
                        const void *v_cache, const void *k_depth, const void *v_depth, void *out,
                        float *lse, void *workspace, size_t workspace_bytes, void *hip_stream) {
  CallLog log_("moda_decode", s);
  return decode_impl(s, nullptr, q, k_cache, v_cache, k_depth, v_depth, out, lse, workspace,
                     workspace_bytes, hip_stream);
}

moda_status moda_decode_noalloc(const moda_shape *s, const int32_t *cache_lens, const void *q,
                                const void *k_cache, const void *v_cache, const void *k_depth,
                                const void *v_depth, void *out, float *lse, void *hip_stream) {
  CallLog log_("moda_decode_noalloc", s);
  moda_status st = decode_check_args(s, q, k_cache, v_cache, k_depth, v_depth, out, lse);
  if (st != MODA_OK) return st;
  if (cache_lens && ((uintptr_t)cache_lens & 3u) != 0)
    return fail(MODA_ERR_INVALID_ARG, "cache_lens must be 4-byte aligned");
  const size_t need = decode_ws_bytes(s);
  if (need > moda::kDecodeScratchBytes)
    return fail(MODA_ERR_UNSUPPORTED,
                "moda_decode_noalloc: the shape needs " + std::to_string(need) +
                    " bytes of partial states; the static scratch holds " +
                    std::to_string(moda::kDecodeScratchBytes) + " (use moda_decode)");
  void *ws = nullptr;
  const hipError_t e = moda::decode_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "decode scratch lookup");
  return decode_impl(s, cache_lens, q, k_cache, v_cache, k_depth, v_depth, out, lse, ws,
                     moda::kDecodeScratchBytes, hip_stream);
}

moda_status moda_decode_varlen(const moda_shape *s, const int32_t *cache_lens, const void *q,
                               const void *k_cache, const void *v_cache, const void *k_depth,
                               const void *v_depth, void *out, float *lse, void *workspace,
                               size_t workspace_bytes, void *hip_stream) {
  CallLog log_("moda_decode_varlen", s);
  if (!cache_lens) return fail(MODA_ERR_INVALID_ARG, "cache_lens must be non-NULL");
  if (((uintptr_t)cache_lens & 3u) != 0)
    return fail(MODA_ERR_INVALID_ARG, "cache_lens must be 4-byte aligned");
  return decode_impl(s, cache_lens, q, k_cache, v_cache, k_depth, v_depth, out, lse, workspace,
                     workspace_bytes, hip_stream);
}

moda_status moda_fwd_strided(const moda_shape *s, const void *q, const void *k, const void *v,
                             const void *k_depth, const void *v_depth, int64_t stride_bh,
                             int64_t stride_t, int64_t stride_i, void *out, float *lse,
                             void *hip_stream) {
  CallLog log_("moda_fwd_strided", s);
  moda_status st = moda_check_shape(s);
  if (st != MODA_OK) return st;
  if (!use_mfma(s))
    return fail(MODA_ERR_UNSUPPORTED, "the strided depth forward supports bf16 with d = 128");
  st = check_qkvo(q, k, v, out, lse);
  if (st != MODA_OK) return st;
  if (s->L == 0) {
    if (k_depth || v_depth)
      return fail(MODA_ERR_INVALID_ARG, "depth inputs must be NULL when L == 0");
    return moda_fwd(s, q, k, v, nullptr, 0, out, lse, hip_stream);
  }
  if (!k_depth || !v_depth)
    return fail(MODA_ERR_INVALID_ARG, "depth inputs must be non-NULL when L > 0");
  if (!aligned16(k_depth) || !aligned16(v_depth))
    return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (stride_bh < 0 || stride_t < 0 || stride_i < 0)
    return fail(MODA_ERR_INVALID_ARG, "depth strides must be >= 0");
  if (s->T * s->L >= ((int64_t)1 << 23))
    return fail(MODA_ERR_UNSUPPORTED, "the strided depth forward supports T * L below 2^23");
  // the largest row index must stay addressable
  const int64_t last = checked_prod({s->B * s->Hkv - 1, stride_bh});
  const int64_t last_t = checked_prod({s->T - 1, stride_t});
  const int64_t last_i = checked_prod({s->L - 1, stride_i});
  if (last < 0 || last_t < 0 || last_i < 0 || last + last_t + last_i >= ((int64_t)1 << 54))
    return fail(MODA_ERR_INVALID_ARG, "depth strides address rows beyond 2^54");
  moda::FwdArgs a = make_fwd_args(s, q, k, v, nullptr, out, lse, true);
  a.kd_nat = k_depth;
  a.vd_nat = v_depth;
  a.depth_layers = true;
  a.inv_L = 1.0f / (float)s->L;
  a.ds_bh = stride_bh;
  a.ds_t = stride_t;
  a.ds_i = stride_i;
  return hip_status(moda::launch_fwd_mfma(a, (int)(s->Hq / s->Hkv), fwd_waves(s), (hipStream_t)hip_stream),
                    "fwd launch");
}

moda_status moda_fwd_layers(const moda_shape *s, const void *q, const void *k, const void *v,
                            const void *k_layers, const void *v_layers, void *out, float *lse,
                            void *hip_stream) {
  CallLog log_("moda_fwd_layers", s);
  const moda_status st = moda_check_shape(s);
  if (st != MODA_OK) return st;
  // [L, B, Hkv, T, d]: row (b, g, t, i) at (i * B * Hkv + b * Hkv + g) * T + t
  return moda_fwd_strided(s, q, k, v, k_layers, v_layers, s->T, 1, s->B * s->Hkv * s->T, out,
                          lse, hip_stream);
}

moda_status moda_fwd_masked_scan(const moda_shape *s, const void *q, const void *k,
                                 const void *v, const void *k_depth, const void *v_depth,
                                 void *out, float *lse, void *hip_stream) {
  CallLog log_("moda_fwd_masked_scan", s);
  moda_status st = moda_check_shape(s);
  if (st != MODA_OK) return st;
  if (!use_mfma(s) || s->L < 1)
    return fail(MODA_ERR_UNSUPPORTED, "moda_fwd_masked_scan supports bf16 with d = 128, L >= 1");
  st = check_qkvo(q, k, v, out, lse);
  if (st != MODA_OK) return st;
  if (!k_depth || !v_depth)
    return fail(MODA_ERR_INVALID_ARG, "k_depth and v_depth must be non-NULL");
  if (!aligned16(k_depth) || !aligned16(v_depth))
    return fail(MODA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (s->T * s->L >= ((int64_t)1 << 23))
    return fail(MODA_ERR_UNSUPPORTED, "moda_fwd_masked_scan supports T * L below 2^23");
  moda::FwdArgs a = make_fwd_args(s, q, k, v, nullptr, out, lse, true);
  a.kd_nat = k_depth;
  a.vd_nat = v_depth;
  a.depth_scan = true;
  return hip_status(moda::launch_fwd_mfma(a, (int)(s->Hq / s->Hkv), fwd_waves(s), (hipStream_t)hip_stream),
                    "fwd launch");
}

const char *moda_status_string(moda_status st) {
  switch (st) {
    case MODA_OK: return "MODA_OK";
    case MODA_ERR_INVALID_ARG: return "MODA_ERR_INVALID_ARG";
    case MODA_ERR_UNSUPPORTED: return "MODA_ERR_UNSUPPORTED";
    case MODA_ERR_HIP: return "MODA_ERR_HIP";
  }
  return "MODA_ERR_UNKNOWN";
}

const char *moda_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
