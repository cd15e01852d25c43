// Device helpers shared by the forward (moda_kernels.hip) and backward
// (moda_bwd.hip) kernels: vector types, bf16 conversion, lane-pair
// reductions and LDS transpose reads for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_internal.h"

namespace moda {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float floatx16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return float_to_bf16_bits(lo) | (float_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short shortx4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));

__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// max / sum of x over the lane pair (l, l ^ 32) that shares one query row
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ shortx4 lds_read_tr(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4 *)(const_cast<char *>(p)));
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Per-lane LDS addressing for a 64-row tile of 256-byte rows.
//   rowfrag(buf, i): A or B operand holding row 32*(i & 1) + lane%32, dims
//                    64*(lane/32) + 8*(i >> 1) .. +7 (row-swizzled tile)
//   colfrag(buf, i): A operand of a transposed product, i = 4*nb + kk: dims
//                    32*nb + lane%32, the 8 rows of k-step kk that pair with
//                    the register order of an MFMA result (column-swizzled)
struct TileFrags {
  int k_row, k_x;
  int vaddr[4];
  __device__ explicit TileFrags(int lane) {
    const int li = lane & 31, lh = lane >> 5;
    k_row = li * 256 + 16 * ((8 * lh) ^ (li & 8));
    k_x = li & 7;
    const int lg = lane >> 4, lq = lane & 15;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      vaddr[nb] = (4 * (lg >> 1) + (lq >> 2)) * 256 +
                  16 * (4 * (nb ^ (lq >> 2)) + 2 * (lg & 1) + ((lq & 3) >> 1)) + 8 * (lq & 1);
  }
  __device__ bf16x8 rowfrag(const char *b, int i) const {
    return *(const bf16x8 *)(b + k_row + 16 * ((i >> 1) ^ k_x) + (i & 1) * 32 * 256);
  }
  __device__ bf16x8 colfrag(const char *b, int i) const {
    const char *vp = b + vaddr[i >> 2] + 16 * (i & 3) * 256;
    const shortx4 lo = lds_read_tr(vp);
    const shortx4 hi = lds_read_tr(vp + 8 * 256);
    return __builtin_bit_cast(
        bf16x8, (u32x4){__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                        __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
  }
};

// 16-byte chunk that LDS slot `slot` of tile row `row` holds
__device__ __forceinline__ int row_swz(int row, int slot) { return slot ^ (row & 15); }
__device__ __forceinline__ int col_swz(int row, int slot) { return slot ^ (4 * (row & 3)); }


// Packed depth blocks (bf16, d = 128): 32 rows = 8 consecutive tokens (a token
// group) x 4 consecutive entries (an entry group).  Block row r is the MFMA row
// of the K half and the k index of the V half; it holds token tok_of_row(r) of
// the group and entry ent_of_row(r) of the entry group.  With this order the
// 8 consecutive k values of a V-half chunk (rows 16kk + 8(j/4) + 4h + j%4,
// j = 0..7) are one entry of the group's 8 tokens, token j at element j, and an
// entry written alone fills whole chunks.
__host__ __device__ constexpr int tok_of_row(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }
__host__ __device__ constexpr int ent_of_row(int r) { return ((r >> 4) << 1) | ((r >> 2) & 1); }

struct MfmaState {
  float m;          // reference max of scaled logits (log2 units)
  float lsum;       // this lane's partial sum of 2^(x - m)
  floatx16 acc[4];  // O^T accumulator: 4 blocks of 32 head-dim rows
};

// Weights 2^(s * scale_log2 - m) of NB score blocks as bf16 B operands,
// pb[2*i + {0,1}] for block i, and their sum (this lane's share of the row).
template <int NB>
__device__ __forceinline__ float tile_weights(const floatx16 *s, float scale_log2, float neg_m,
                                              bf16x8 *pb) {
  float sum = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    u32x4 w[2];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(fmaf(s[b][r], scale_log2, neg_m));
      const float p1 = fast_exp2(fmaf(s[b][r + 1], scale_log2, neg_m));
      sum += p0 + p1;
      w[r >> 3][(r & 7) >> 1] = cvt_bf16x2(p0, p1);
    }
    pb[2 * b] = __builtin_bit_cast(bf16x8, w[0]);
    pb[2 * b + 1] = __builtin_bit_cast(bf16x8, w[1]);
  }
  return sum;
}

// A row's weights in one tile may sum to at most this much before the row
// moves its reference max; every weight stays <= 2^12.
constexpr float TILE_SUM_LIMIT = 4096.0f;

// Online-softmax update for NB score blocks of 32 entries each (already
// masked with -inf): turn scores into weights against the row's reference
// max and return them as bf16 B operands, pb[2*i + {0,1}] for block i.
// The weights are first taken against the current reference.  A row with no
// reference yet, or whose weights in this tile sum past TILE_SUM_LIMIT, moves
// its reference to the tile's max, rescales its state and takes its weights
// again.  The branch is wave-wide, but each row decides from its own scores and
// a row that does not move recomputes exactly the same weights, so a row's
// result never depends on the other rows of the wave.
template <int NB>
__device__ __forceinline__ void softmax_update(MfmaState &st, const floatx16 *s, float scale_log2,
                                               bf16x8 *pb) {
  const bool fresh = st.m == -INFINITY;
  float sum = tile_weights<NB>(s, scale_log2, fresh ? 0.f : -st.m, pb);
  const bool need = fresh || !(pair_sum(sum) <= TILE_SUM_LIMIT);
  if (__builtin_amdgcn_ballot_w64(need)) {
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
    const float mt = pair_max(mx) * scale_log2;
    const float m_new = need ? fmaxf(mt, st.m) : st.m;
    const float alpha = m_new == st.m ? 1.0f : fast_exp2(st.m - m_new);
    st.m = m_new;
    st.lsum *= alpha;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[nb][r] *= alpha;
    // a row that has seen no unmasked entry yet keeps m = -inf and weight 0
    sum = tile_weights<NB>(s, scale_log2, st.m == -INFINITY ? 0.f : -st.m, pb);
  }
  st.lsum += sum;
}

// Online-softmax update that moves the reference max to every tile's max
// (for the HBM-bound depth loop, whose VALU has room for the reduction).  A
// new running maximum then gets weight exactly 1, so bf16 rounding of the
// weights never touches the entry that dominates a row.
template <int NB>
__device__ __forceinline__ void softmax_update_eager(MfmaState &st, const floatx16 *s,
                                                     float scale_log2, bf16x8 *pb) {
  float mx = s[0][0];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
  const float m_new = fmaxf(pair_max(mx) * scale_log2, st.m);
  if (__builtin_amdgcn_ballot_w64(m_new != st.m)) {
    const float alpha = m_new == st.m ? 1.0f : fast_exp2(st.m - m_new);  // 0 from -inf
    st.lsum *= alpha;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[nb][r] *= alpha;
  }
  st.m = m_new;
  // a row that has seen no unmasked entry yet keeps m = -inf and weight 0
  st.lsum += tile_weights<NB>(s, scale_log2, m_new == -INFINITY ? 0.f : -m_new, pb);
}

// softmax_update_eager<1> for a block in which a row holds at most two
// entries: its scores sa and sb (-inf where absent) sit in registers pos and
// pos + 8 of its 16, and the other 14 are masked (pos < 0: none).  The result
// is bit for bit that of softmax_update_eager<1> on the masked block (the same
// reference max, weights, sum and bf16 operands, zeros elsewhere), without the
// 14 exponentials of zero weights.
__device__ __forceinline__ void softmax_update_pair(MfmaState &st, float sa, float sb, int pos,
                                                    float scale_log2, bf16x8 *pb) {
  const float m_new = fmaxf(pair_max(fmaxf(sa, sb)) * scale_log2, st.m);
  if (__builtin_amdgcn_ballot_w64(m_new != st.m)) {
    const float alpha = m_new == st.m ? 1.0f : fast_exp2(st.m - m_new);  // 0 from -inf
    st.lsum *= alpha;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[nb][r] *= alpha;
  }
  st.m = m_new;
  // a row that has seen no unmasked entry yet keeps m = -inf and weight 0
  const float neg_m = m_new == -INFINITY ? 0.f : -m_new;
  const float wa = fast_exp2(fmaf(sa, scale_log2, neg_m));
  const float wb = fast_exp2(fmaf(sb, scale_log2, neg_m));
  st.lsum += wa + wb;
  // register pos of each 8-register half: half (pos & 1) of 32-bit word pos / 2
  const int sh = 16 * (pos & 1);
  const uint32_t ba = cvt_bf16x2(wa, 0.f) << sh, bb = cvt_bf16x2(wb, 0.f) << sh;
  u32x4 w0, w1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool here = (pos >> 1) == q;
    w0[q] = here ? ba : 0u;
    w1[q] = here ? bb : 0u;
  }
  pb[0] = __builtin_bit_cast(bf16x8, w0);
  pb[1] = __builtin_bit_cast(bf16x8, w1);
}

}  // namespace moda
