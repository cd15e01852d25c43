// Internal interface between the C-ABI layer (moda_api.cpp) and the HIP
// kernels (moda_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace moda {

// Geometry of the MFMA path (bf16, head dim 128).
constexpr int kMfmaD = 128;         // head dimension
constexpr int kMfmaRows = 256;      // query rows (token x head pairs) per 8-wave workgroup
constexpr int kDepthBlock = 32;     // depth entries per packed block
constexpr int64_t kPackedBlockBytes = 2 * kDepthBlock * kMfmaD * 2;  // K part + V part
// a packed block holds kGroupTokens consecutive tokens x kGroupEntries entries
constexpr int kGroupTokens = 8;
constexpr int kGroupEntries = 4;

struct FwdArgs {
  const void *q, *k, *v, *packed;
  const void *kd_nat, *vd_nat;  // depth K, V read row by row: natural or layer-major layout
  void *out;
  float *lse;
  int64_t B, Hq, Hkv, T, L, d;
  int64_t nblk;   // packed depth blocks per (b, kv head) (MFMA path)
  float scale_log2;  // log2(e) / sqrt(d)
  bool has_depth;  // the token's depth entries join the softmax
  bool has_seq;    // the causal sequence keys join the softmax
  bool depth_layers;  // kd_nat, vd_nat rows are strided (ds_*) (else [B,Hkv,T,L,d])
  bool depth_scan;    // natural layout, scanned from entry 0 under the own-token mask
  float inv_L;        // 1 / L (strided row lookup)
  int64_t ds_bh, ds_t, ds_i;  // strided depth rows: (b, g, t, i) at bh*ds_bh + t*ds_t + i*ds_i
};

// Kernel modes: causal attention, MoDA (sequence + depth), depth attention alone.
constexpr int kModeCausal = 0;
constexpr int kModeModa = 1;
constexpr int kModeDepth = 2;
constexpr int kModeModaNatural = 3;  // MoDA reading depth K, V in their natural layout
constexpr int kModeModaLayers = 4;   // MoDA reading depth K, V rows at given strides
constexpr int kModeModaScan = 5;     // natural layout, every earlier token's entries scanned

struct BwdArgs {
  const void *q, *k, *v, *packed, *kd, *vd, *out, *dout;
  const float *lse;
  float *delta;  // [B,Hq,T] scratch: <dO, O> per query row
  void *dq, *dk, *dv, *dkd, *dvd;
  int64_t B, Hq, Hkv, T, L, d;
  int64_t nblk;      // packed depth blocks per (b, kv head)
  float scale_log2;  // log2(e) / sqrt(d)
  float scale;       // 1 / sqrt(d)
  // dK/dV split: each key tile's query range in nsplit parts; with nsplit > 1
  // the parts leave fp32 partial sums in kv_ws [2][nsplit][B*Hkv][T][d]
  // (dV, then unscaled dK), which a reduction kernel adds up
  int64_t nsplit;
  float *kv_ws;
};

// Decode step: one query row per (b, head) over a KV cache of T entries and
// the new token's L depth entries.  Per (b, kv head) the cache's 32-entry
// blocks and then the depth entries' blocks form one list, split evenly into
// nsplit workgroup parts.  Each part leaves one record per query row in ws:
// O (unnormalised, kMfmaD floats), reference max (log2 units), weight sum.
constexpr int kDecodeRecord = kMfmaD + 4;  // floats per record (2 of padding)

struct DecArgs {
  const void *q, *k, *v, *kd, *vd;  // q [B,Hq,d]; k, v [B,Hkv,T,d]; kd, vd [B,Hkv,L,d]
  const int32_t *lens;              // [B] cache entries per sequence (<= T), or null: all T
  void *out;                        // [B,Hq,d]
  float *lse;                       // [B,Hq] or null
  float *ws;                        // [B*Hq, nsplit, kDecodeRecord]
  int64_t B, Hq, Hkv, T, L;
  int64_t nsplit;
  int waves;         // waves per part workgroup: 4 or 8
  float scale_log2;  // log2(e) / sqrt(d)
};

struct PackArgs {
  const void *kd, *vd;
  void *packed;
  int64_t B, Hkv, T, L, d;
  int64_t nblk;
};

// Depth-stream write: entries [first, first + n) of every token, from
// knew, vnew [B,Hkv,T,n,d], into a packed cache of L entries per token.
struct AppendArgs {
  const void *knew, *vnew;
  void *packed;
  int64_t B, Hkv, T, L;
  int64_t nblk;  // packed depth blocks per (b, kv head) (MFMA layout)
  int64_t first, n;
};

// MFMA path: dtype bf16, d == 128.
// waves = 8 (256 rows per workgroup) or 4 (128 rows), G <= 32 * waves; or
// kFwdKeySplit: 8 waves on 128 rows, pairs of waves splitting each key tile
// (causal and packed MoDA modes; the other modes run the 4-wave kernel), G <= 128.
constexpr int kFwdKeySplit = 9;
hipError_t launch_fwd_mfma(const FwdArgs &a, int G, int waves, hipStream_t s);
hipError_t launch_pack_mfma(const PackArgs &a, hipStream_t s);

// Backward, bf16, d == 128, G <= 64: delta, dQ, then dK/dV.
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s);

// Decode step, bf16, d == 128, G <= 32: partial states, then their merge.
hipError_t launch_decode(const DecArgs &a, hipStream_t s);

// The allocation-free decode's device scratch: kDecodeScratchBytes bytes per
// GPU, at the address decode_scratch returns for the current device.
constexpr size_t kDecodeScratchBytes = (size_t)8 << 20;
hipError_t decode_scratch(void **ptr);

// Depth-stream write into the MFMA block layout (mfma) or the generic one
// (rows of row_bytes bytes).
hipError_t launch_append(const AppendArgs &a, bool mfma, int row_bytes, hipStream_t s);

// Generic path: fp32 or bf16, d in {32, 64, 128}, any G.
hipError_t launch_fwd_generic(const FwdArgs &a, bool bf16, hipStream_t s);
hipError_t launch_pack_generic(const PackArgs &a, bool bf16, hipStream_t s);

}  // namespace moda
