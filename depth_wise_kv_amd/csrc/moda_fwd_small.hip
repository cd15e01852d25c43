// MoDA forward on the matrix cores for the shapes outside the bf16, d = 128
// kernel: bf16 with d in {32, 64}, and fp32 with d in {32, 64, 128}.
//
// The operation is the one of moda_kernels.hip (hyper.ai, section "混合深度注意力
// (MoDA)": one softmax per query row over its causal sequence keys and its own
// token's L depth entries, G query heads per KV head).  The depth entries come
// from the generic packed layout: Kd then Vd, each [B, Hkv, T, L, d].
//
// Structure (per workgroup: 4 waves, 128 query rows = floor(128 / G) tokens
// x G heads, rows folded as in the d = 128 kernel, heaviest causal tile first):
//   * keys are visited in tiles of 64, computed as two halves of 32: the
//     sequence keys 0 .. last token of the tile, then the flat depth entries of
//     the tile's tokens; every tile is staged in LDS once and read by all four
//     waves;
//   * scores are computed transposed, S^T = K Q^T, so that a lane owns one
//     query row (lanes l and l ^ 32 share it): row max and row sum are in-lane
//     work plus one exchange;
//   * the K rows feed the MFMA A operand in a permuted order chosen so that
//     the score registers a lane ends up holding are exactly the keys it must
//     supply as the B operand of O^T += V^T P^T: P needs no shuffle;
//   * bf16 uses v_mfma_f32_32x32x16_bf16 (P rounded to bf16 as the operand),
//     fp32 uses v_mfma_f32_32x32x2_f32 (fp32 operands throughout).
// ---------------------------------------------------------------------------
#include "moda_device.h"
#include "moda_small.h"

namespace moda {
namespace {

constexpr int kSmallKeys = 64;  // keys (or depth entries) per tile: two 32-key halves

template <typename E>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int kBytes = 4;
  static constexpr bool kBf16 = false;
};
template <>
struct Elt<uint16_t> {
  static constexpr int kBytes = 2;
  static constexpr bool kBf16 = true;
};

// LDS geometry of one tile.
//   bf16: K rows of 2D bytes padded to 2D + 16 (16-byte fragment reads from 16
//         different rows fall in distinct banks); V stored transposed, rows of
//         64 keys (128 bytes) padded to 144, read as 8 consecutive keys of one dim.
//   fp32: K rows of D floats padded to D + 1 (32 lanes read one float from 32
//         rows: distinct banks); V row-major, lanes read consecutive dims.
template <typename E, int D>
struct SmallTile {
  static constexpr int kEs = Elt<E>::kBytes;
  static constexpr int kKStride = Elt<E>::kBf16 ? 2 * D + 16 : 4 * (D + 1);
  static constexpr int kVStride = Elt<E>::kBf16 ? 2 * kSmallKeys + 16 : 4 * D;
  static constexpr int kKBytes = kSmallKeys * kKStride;
  static constexpr int kVBytes = Elt<E>::kBf16 ? D * kVStride : kSmallKeys * kVStride;
  static constexpr int kChunksPerRow = D * kEs / 16;
  static constexpr int kChunks = kSmallKeys * kChunksPerRow;  // per tensor and tile
  static constexpr int kChunksPerThread = (kChunks + 64 * kSmallWaves - 1) / (64 * kSmallWaves);
};

// Key held by A-operand row m of the score MFMA, and key of output register i
// in lane half h (see the file comment).  32x32 MFMA outputs: register i of
// lane (n, h) is row 8 (i / 4) + 4 h + i % 4 of the 32 x 32 result.
template <bool BF16>
__device__ __forceinline__ int key_of_arow(int m) {
  const int j = m >> 3, hh = (m >> 2) & 1, r = m & 3;
  return BF16 ? 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + r : 2 * (4 * j + r) + hh;
}
template <bool BF16>
__device__ __forceinline__ int key_of_reg(int i, int h) {
  return BF16 ? 16 * (i >> 3) + 8 * h + (i & 7) : 2 * i + h;
}

template <typename E, int D, bool SEQ, bool DEPTH>
__global__ __launch_bounds__(64 * kSmallWaves) void moda_fwd_small(FwdArgs p) {
  using Tile = SmallTile<E, D>;
  constexpr bool BF16 = Elt<E>::kBf16;
  constexpr int NB = D / 32;  // 32-dim output blocks
  __shared__ __attribute__((aligned(16))) char k_lds[Tile::kKBytes];
  __shared__ __attribute__((aligned(16))) char v_lds[Tile::kVBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, h = lane >> 5;

  const int64_t T = p.T, L = DEPTH ? p.L : 0;
  const int G = (int)(p.Hq / p.Hkv);
  const int TQ = kSmallRows / G;  // tokens per tile
  const int64_t BH = p.B * p.Hkv;
  const int64_t ntiles = (T + TQ - 1) / TQ;
  const int64_t x = blockIdx.x;
  const int64_t tile = ntiles - 1 - x / BH;  // heaviest causal tiles first
  const int64_t bh = x % BH;
  const int64_t b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int64_t t0 = tile * TQ;
  const int64_t t_end = t0 + TQ < T ? t0 + TQ : T;  // one past the tile's last token

  // this lane's query row (row r = token-in-tile * G + head-in-group)
  const int r = wave * 32 + ln;
  const bool row_used = r < TQ * G;
  const int64_t tok = row_used ? t0 + r / G : T;
  const int64_t head = hkv * G + (row_used ? r % G : 0);
  const bool row_ok = tok < T;
  // the wave's token range (wave-uniform): [w_lo, w_hi], empty if w_lo > w_hi
  const int r_last = wave * 32 + 31 < TQ * G - 1 ? wave * 32 + 31 : TQ * G - 1;
  const int64_t w_lo = t0 + (wave * 32) / G;
  const int64_t w_hi = (t0 + r_last / G < t_end - 1) ? t0 + r_last / G : t_end - 1;

  // Q as the B operand: bf16 lane (n, h) holds dims 16 ks + 8 h .. + 7 of row n;
  // fp32 lane (n, h) holds dim 2 s + h of row n.
  constexpr int NQ = BF16 ? D / 16 : D / 2;
  typedef typename std::conditional<BF16, bf16x8, float>::type QOp;
  QOp qop[NQ];
  {
    const E *qrow = (const E *)p.q + ((b * p.Hq + head) * T + (row_ok ? tok : 0)) * D;
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      if constexpr (BF16) {
        const u32x4 u = row_ok ? *(const u32x4 *)(qrow + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
        qop[s] = __builtin_bit_cast(bf16x8, u);
      } else {
        qop[s] = row_ok ? qrow[2 * s + h] : 0.f;
      }
    }
  }

  floatx16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[nb][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;  // running max (log2 units, scaled) and lane-half sum
  const float sc = p.scale_log2;
  const int arow_key = key_of_arow<BF16>(ln);

  // ---- staging: one tile of 32 rows of K and V (rows >= row_end read as zeros)
  u32x4 kst[Tile::kChunksPerThread], vst[Tile::kChunksPerThread];
  auto prefetch = [&](const E *ksrc, const E *vsrc, int64_t row0, int64_t row_end) {
#pragma unroll
    for (int c = 0; c < Tile::kChunksPerThread; ++c) {
      const int ch = tid + c * 64 * kSmallWaves;
      const int row = ch / Tile::kChunksPerRow, cc = ch % Tile::kChunksPerRow;
      const bool ok = ch < Tile::kChunks && row0 + row < row_end;
      const int64_t off = (row0 + row) * D * Tile::kEs + cc * 16;
      kst[c] = ok ? *(const u32x4 *)((const char *)ksrc + off) : u32x4{0, 0, 0, 0};
      vst[c] = ok ? *(const u32x4 *)((const char *)vsrc + off) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int c = 0; c < Tile::kChunksPerThread; ++c) {
      const int ch = tid + c * 64 * kSmallWaves;
      if (ch >= Tile::kChunks) continue;
      const int row = ch / Tile::kChunksPerRow, cc = ch % Tile::kChunksPerRow;
      if constexpr (BF16) {
        *(u32x4 *)(k_lds + row * Tile::kKStride + cc * 16) = kst[c];
        // V transposed: element e of the chunk is dim 8 cc + e of key `row`
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *(uint16_t *)(v_lds + (8 * cc + e) * Tile::kVStride + row * 2) =
              (uint16_t)(vst[c][e >> 1] >> (16 * (e & 1)));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *(uint32_t *)(k_lds + row * Tile::kKStride + (4 * cc + e) * 4) = kst[c][e];
        *(u32x4 *)(v_lds + row * Tile::kVStride + cc * 16) = vst[c];
      }
    }
  };

  // ---- one 32-key half kh of the tile for this wave: scores, mask, online
  // softmax, P V.  keep(k) says whether tile key k (0..63) joins this row.
  auto compute = [&](int kh, auto keep) {
    floatx16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    const int krow = 32 * kh + arow_key;
    if constexpr (BF16) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = *(const bf16x8 *)(k_lds + krow * Tile::kKStride + (16 * ks + 8 * h) * 2);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], s, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks) {
        const float a = *(const float *)(k_lds + krow * Tile::kKStride + (2 * ks + h) * 4);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qop[ks], s, 0, 0, 0);
      }
    }
    float xs[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xs[i] = keep(32 * kh + key_of_reg<BF16>(i, h)) ? s[i] * sc : -INFINITY;
      tmax = fmaxf(tmax, xs[i]);
    }
    tmax = pair_max(tmax);
    const float m_new = fmaxf(m, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no key yet: all weights 0
    const float alpha = fast_exp2(m - m_use);              // 0 while m is -inf
    m = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xs[i] = fast_exp2(xs[i] - m_use);
      psum += xs[i];
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] *= alpha;
    if constexpr (BF16) {
      // P^T as the B operand: key step kk takes registers 8 kk .. 8 kk + 7
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pu;
#pragma unroll
        for (int e = 0; e < 4; ++e) pu[e] = cvt_bf16x2(xs[8 * kk + 2 * e], xs[8 * kk + 2 * e + 1]);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pu);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 a = *(const bf16x8 *)(v_lds + (32 * nb + ln) * Tile::kVStride +
                                             (32 * kh + 16 * kk + 8 * h) * 2);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[nb], 0, 0, 0);
        }
      }
    } else {
      // key step ks (keys 2 ks, 2 ks + 1 of the half) takes register ks
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float a = *(const float *)(v_lds + (32 * kh + 2 * ks + h) * Tile::kVStride +
                                           (32 * nb + ln) * 4);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, xs[ks], acc[nb], 0, 0, 0);
        }
      }
    }
  };

  // ---- a pass over rows [lo, hi) of (ksrc, vsrc) in tiles of 64; every wave
  // takes part in the staging and the barriers, and computes the 32-key halves
  // that touch its rows (has_work(first key of the half)).
  auto pass = [&](const E *ksrc, const E *vsrc, int64_t lo, int64_t hi, auto has_work,
                  auto keep_at) {
    const int64_t nt = (hi - lo + kSmallKeys - 1) / kSmallKeys;
    if (nt <= 0) return;
    prefetch(ksrc, vsrc, lo, hi);
    for (int64_t j = 0; j < nt; ++j) {
      const int64_t k0 = lo + j * kSmallKeys;
      __syncthreads();  // the previous tile's LDS reads are done
      store();
      __syncthreads();
      if (j + 1 < nt) prefetch(ksrc, vsrc, k0 + kSmallKeys, hi);
      // the second half only where it holds keys of the pass
      if (has_work(k0)) compute(0, [&](int k) { return keep_at(k0 + k); });
      if (k0 + 32 < hi && has_work(k0 + 32)) compute(1, [&](int k) { return keep_at(k0 + k); });
    }
  };

  if constexpr (SEQ) {
    const E *kseq = (const E *)p.k + bh * T * D;
    const E *vseq = (const E *)p.v + bh * T * D;
    // keys 0 .. t_end - 1; a wave works on a tile while it starts at or before
    // its last token; key k is kept iff k <= the row's token
    pass(kseq, vseq, 0, t_end, [&](int64_t k0) { return w_lo <= w_hi && k0 <= w_hi; },
         [&](int64_t key) { return key <= tok; });
  }
  if constexpr (DEPTH) {
    if (L > 0) {
      const int64_t half = p.B * p.Hkv * T * L * D;  // elements of Kd
      const E *kdep = (const E *)p.packed + bh * T * L * D;
      const E *vdep = (const E *)p.packed + half + bh * T * L * D;
      // flat entries e = token * L + i of the tile's tokens; entry e joins the
      // row iff it is one of the row's own token's L entries
      pass(kdep, vdep, t0 * L, t_end * L,
           [&](int64_t e0) {
             return w_lo <= w_hi && e0 < (w_hi + 1) * L && e0 + 32 > w_lo * L;
           },
           [&](int64_t e) { return (uint64_t)(e - tok * L) < (uint64_t)L; });
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l)
  const float ltot = pair_sum(lsum);
  if (row_ok) {
    const float inv = 1.f / ltot;
    E *orow = (E *)p.out + ((b * p.Hq + head) * T + tok) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dim = 32 * nb + 8 * j + 4 * h;  // registers 4 j .. 4 j + 3
        if constexpr (BF16) {
          u32x2 w;
          w[0] = cvt_bf16x2(acc[nb][4 * j] * inv, acc[nb][4 * j + 1] * inv);
          w[1] = cvt_bf16x2(acc[nb][4 * j + 2] * inv, acc[nb][4 * j + 3] * inv);
          *(u32x2 *)(orow + dim) = w;
        } else {
          float4 w = {acc[nb][4 * j] * inv, acc[nb][4 * j + 1] * inv, acc[nb][4 * j + 2] * inv,
                      acc[nb][4 * j + 3] * inv};
          *(float4 *)(orow + dim) = w;
        }
      }
    if (p.lse && h == 0)
      p.lse[(b * p.Hq + head) * T + tok] = (m + __log2f(ltot)) * 0.69314718055994531f;
  }
}

template <typename E, int D>
hipError_t launch_small_d(const FwdArgs &a, hipStream_t s) {
  const int64_t G = a.Hq / a.Hkv, TQ = kSmallRows / G;
  const int64_t grid = (a.T + TQ - 1) / TQ * a.B * a.Hkv;
  const dim3 g((uint32_t)grid), blk(64 * kSmallWaves);
  if (!a.has_seq)
    hipLaunchKernelGGL((moda_fwd_small<E, D, false, true>), g, blk, 0, s, a);
  else if (a.has_depth && a.L > 0)
    hipLaunchKernelGGL((moda_fwd_small<E, D, true, true>), g, blk, 0, s, a);
  else
    hipLaunchKernelGGL((moda_fwd_small<E, D, true, false>), g, blk, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_small(const FwdArgs &a, bool bf16, hipStream_t s) {
  const int64_t G = a.Hq / a.Hkv;
  if (!small_supported(bf16, a.d, G)) return hipErrorInvalidValue;
  if (bf16) {
    if (a.d == 32) return launch_small_d<uint16_t, 32>(a, s);
    return launch_small_d<uint16_t, 64>(a, s);
  }
  if (a.d == 32) return launch_small_d<float, 32>(a, s);
  if (a.d == 64) return launch_small_d<float, 64>(a, s);
  return launch_small_d<float, 128>(a, s);
}

}  // namespace moda
