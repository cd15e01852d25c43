// Internal interface of the matrix-core forward for the shapes outside the
// bf16, d = 128 kernel (moda_fwd_small.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "moda_internal.h"

namespace moda {

constexpr int kSmallWaves = 4;                // waves per workgroup
constexpr int kSmallRows = 32 * kSmallWaves;  // query rows (token x head pairs) per workgroup

// bf16 with d in {32, 64}, fp32 with d in {32, 64, 128}; G = Hq / Hkv <= 128.
inline bool small_supported(bool bf16, int64_t d, int64_t G) {
  if (G < 1 || G > kSmallRows) return false;
  return bf16 ? (d == 32 || d == 64) : (d == 32 || d == 64 || d == 128);
}
// workgroups of one launch: one per (b, kv head, tile of floor(128 / G) tokens)
inline int64_t small_grid(int64_t B, int64_t Hkv, int64_t T, int64_t G) {
  const int64_t TQ = kSmallRows / G;
  return (T + TQ - 1) / TQ * B * Hkv;
}
// Forward over the generic packed layout (Kd then Vd, each [B,Hkv,T,L,d]):
// sequence and depth (has_seq, has_depth), causal only, or depth only.
hipError_t launch_fwd_small(const FwdArgs &a, bool bf16, hipStream_t s);

}  // namespace moda
