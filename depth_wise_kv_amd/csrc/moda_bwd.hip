// HIP kernels of the MoDA backward for gfx950 (MI355X): bf16, head dim 128.
//
// Given dO, the loss gradient with respect to the MoDA output O, and the
// forward's per-row log-sum-exp, the gradients follow from the chain rule
// through the one softmax over sequence and depth entries (hyper.ai page on
// arXiv 2603.15619, section "Mixture-of-Depths Attention (MoDA)"):
//   p_n = exp(s <q, key_n> - lse)           (the forward's weights)
//   D   = <dO, O>                            per query row
//   ds_n = p_n (<dO, value_n> - D)
//   dQ  = s sum_n ds_n key_n;  dKey_n += s ds_n q;  dValue_n += p_n dO
// with s = 1/sqrt(d).  Sums over query rows run over every row that reads
// the entry: the G query heads of the KV group, and for a sequence key j
// every token t >= j.
//
// Kernels:
//   moda_bwd_delta  D for every query row.
//   moda_bwd_dq     dQ over the sequence keys.  A workgroup owns 256 query
//                   rows (the forward's tiling: 256/G tokens x the G heads of
//                   one KV group) and walks the key tiles up to the diagonal.
//                   Per tile: S^T = K Q^T, P^T, dP^T = V dO^T, dS^T,
//                   dQ^T += K^T dS^T, all on v_mfma_f32_32x32x16_bf16 with a
//                   lane owning a row.
//   moda_bwd_dkdv   dK, dV.  A workgroup owns 128 sequence keys (4 groups of
//                   32, a lane per key) and walks the query tiles of 64 rows
//                   (64/G tokens x G heads) from its first key to the end.
//                   Each group has two waves on one SIMD: one computes
//                   S = Q K^T and P and accumulates dV^T += dO^T P; the other
//                   computes dP = dO V^T, takes P through LDS after a
//                   mid-tile barrier, and accumulates dK^T += Q^T dS.
//   moda_bwd_ddepth dKd, dVd, and the depth entries' part of dQ (added to
//                   the sequence part dq wrote): each span of whole tokens
//                   has a wave per entry orientation and a wave per row
//                   orientation reading the same depth blocks.
// The key and query tiles go from global memory straight into LDS, once each,
// in a layout (UniFrags) that serves both operand reads without bank
// conflicts: row reads (operands that hold 8 dims of one row) and transpose
// reads (4 rows of one dim).  The depth-gradient kernel hands K rows over in
// the "column-swizzled" layout (chunk c of row r in slot c ^ 4 (r % 4)), which
// only transpose reads use.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moda_device.h"
#include "moda_internal.h"

namespace moda {
namespace {

constexpr int BD = kMfmaD;                 // 128
constexpr int BTILE = 64 * BD * 2;         // 16 KiB: 64 rows of 256 B
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, char *lds, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds,
                                           16, voff, soff, 0, 0);
}

// Row r of a 256-B-row bf16 matrix into the B (or A) operand layout used for
// Q in the forward: lane half h holds dims 64h .. 64h+63, 8 per k-step.
__device__ __forceinline__ void load_row_operand(const __bf16 *row, bool ok, int lh,
                                                 bf16x8 (&dst)[8]) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const u32x4 u = ok ? *(const u32x4 *)(row + 64 * lh + 8 * ks) : u32x4{0, 0, 0, 0};
    dst[ks] = __builtin_bit_cast(bf16x8, u);
  }
}

// Store an MFMA accumulator of a 128-dim row (column lane%32, registers over
// dims 32*nb + 8*(r/4) + 4*(lane/32) + r%4) as bf16, scaled.
__device__ __forceinline__ void store_row(__bf16 *row, const floatx16 (&acc)[4], float scale,
                                          int lh) {
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 o;
      o[0] = cvt_bf16x2(acc[nb][4 * g + 0] * scale, acc[nb][4 * g + 1] * scale);
      o[1] = cvt_bf16x2(acc[nb][4 * g + 2] * scale, acc[nb][4 * g + 3] * scale);
      *(u32x2 *)(row + 32 * nb + 8 * g + 4 * lh) = o;
    }
}

// One copy of a 64-row tile that serves both kinds of operand read without
// bank conflicts: chunk c of row r sits in slot c ^ sigma(r), with sigma
// swapping the two 2-bit fields of r % 16.  The 16 lanes of a row-operand read
// (16 consecutive rows, one chunk) see 16 distinct slots, and the 16 lanes of
// a transpose read (rows 4h .. 4h+3 of a 16-row step, chunks 4nb + 2g + b)
// see 8 distinct slots, two 8-byte halves each.
__device__ __forceinline__ int uni_sigma(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ int uni_swz(int row, int slot) { return slot ^ uni_sigma(row); }

// Per-lane addressing of that layout, with the operands of TileFrags:
//   rowfrag(buf, i): row 32*(i & 1) + lane%32, dims 64*(lane/32) + 8*(i >> 1) .. +7
//   colfrag(buf, i): i = 4*nb + kk: dims 32*nb + lane%32, the 8 rows of
//                    k-step kk in the register order of an MFMA result
struct UniFrags {
  int k_row, k_x;
  int lo[4], hi[4];
  __device__ explicit UniFrags(int lane) {
    const int li = lane & 31, lh = lane >> 5;
    const int sg = uni_sigma(li);  // rows li and li + 32 share it
    k_row = li * 256 + 16 * ((8 * lh) ^ (sg & 8));
    k_x = sg & 7;
    // transpose reads: lane (lg, lq) reads row 4*(lg/2) + lq/4 (and 8 below
    // it), 8-byte half lq%2 of chunk 4nb + 2(lg%2) + (lq%4)/2
    const int lg = lane >> 4, lq = lane & 15;
    const int r0 = 4 * (lg >> 1) + (lq >> 2);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int c = 4 * nb + 2 * (lg & 1) + ((lq & 3) >> 1);
      lo[nb] = r0 * 256 + 16 * uni_swz(r0, c) + 8 * (lq & 1);
      hi[nb] = (r0 + 8) * 256 + 16 * uni_swz(r0 + 8, c) + 8 * (lq & 1);
    }
  }
  __device__ bf16x8 rowfrag(const char *b, int i) const {
    return *(const bf16x8 *)(b + k_row + 16 * ((i >> 1) ^ k_x) + (i & 1) * 32 * 256);
  }
  __device__ bf16x8 colfrag(const char *b, int i) const {
    const shortx4 l = lds_read_tr(b + lo[i >> 2] + 16 * (i & 3) * 256);
    const shortx4 h = lds_read_tr(b + hi[i >> 2] + 16 * (i & 3) * 256);
    return __builtin_bit_cast(
        bf16x8, (u32x4){__builtin_bit_cast(u32x2, l)[0], __builtin_bit_cast(u32x2, l)[1],
                        __builtin_bit_cast(u32x2, h)[0], __builtin_bit_cast(u32x2, h)[1]});
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// D = <dO, O> per query row (fp32), one thread per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moda_bwd_delta(BwdArgs p) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= p.B * p.Hq * p.T) return;
  const u32x4 *o = (const u32x4 *)((const __bf16 *)p.out + r * BD);
  const u32x4 *g = (const u32x4 *)((const __bf16 *)p.dout + r * BD);
  float acc = 0.f;
#pragma unroll 4
  for (int c = 0; c < BD / 8; ++c) {
    const u32x4 a = o[c], b = g[c];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16_bits_to_float(a[w] & 0xFFFFu), bf16_bits_to_float(b[w] & 0xFFFFu), acc);
      acc = fmaf(bf16_bits_to_float(a[w] >> 16), bf16_bits_to_float(b[w] >> 16), acc);
    }
  }
  p.delta[r] = acc;
}

// ---------------------------------------------------------------------------
// dQ: 8 waves x 32 query rows, key tiles of 64.
// ---------------------------------------------------------------------------
constexpr int DQ_WAVES = 8;
constexpr int DQ_ROWS = 32 * DQ_WAVES;  // 256

__global__ __launch_bounds__(64 * DQ_WAVES, 1) void moda_bwd_dq(BwdArgs p) {
  const int G = (int)(p.Hq / p.Hkv);
  const int TQ = DQ_ROWS / G;
  // K and V tiles of each parity, one copy each in the layout UniFrags reads
  // both ways (K is read both ways, V by rows)
  __shared__ __attribute__((aligned(1024))) char a_k0[BTILE];
  __shared__ __attribute__((aligned(1024))) char a_k1[BTILE];
  __shared__ __attribute__((aligned(1024))) char a_v0[BTILE];
  __shared__ __attribute__((aligned(1024))) char a_v1[BTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, lh = lane >> 5;
  const UniFrags fr(lane);

  const int64_t T = p.T;
  const int64_t BH = p.B * p.Hkv;
  const int64_t ntiles = (T + TQ - 1) / TQ;
  const int64_t x = blockIdx.x;
  const int64_t tile = ntiles - 1 - x / BH;  // heaviest causal tiles first
  const int64_t bh = x % BH;
  const int64_t b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int64_t t0 = tile * TQ;

  const int r = wave * 32 + li;
  const bool row_used = r < TQ * G;
  const int64_t tok = row_used ? t0 + r / G : T;
  const int64_t head = hkv * G + (row_used ? r % G : 0);
  const bool row_ok = tok < T;
  const int64_t qrow = (b * p.Hq + head) * T + (row_ok ? tok : 0);

  bf16x8 qb[8], gb[8];
  load_row_operand((const __bf16 *)p.q + qrow * BD, row_ok, lh, qb);
  load_row_operand((const __bf16 *)p.dout + qrow * BD, row_ok, lh, gb);
  const float c = p.scale_log2;
  // S^T starts at -lse2/c, dP^T at -D: then P = exp2(c * S^T) and dS = P dP^T
  const float init_s = row_ok ? -(p.lse[qrow] * LOG2E) / c : -INFINITY;
  const float init_dp = row_ok ? -p.delta[qrow] : 0.f;

  floatx16 dq[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) dq[nb][rr] = 0.f;

  const int64_t tok_end = (t0 + TQ < T) ? t0 + TQ : T;
  const int n_kt = (int)((tok_end + 63) / 64);
  const int64_t wave_tok_lo = t0 + (wave * 32) / G;

  // Tile loads: this wave fills tile rows 8*wave .. +7 of K and of V, 2
  // instructions of 4 rows each per tile.  Rows at or past T read as zeros
  // (descriptor range).
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const char *)p.k + bh * T * (BD * 2)), (short)0, (int)(T * (BD * 2)), 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const char *)p.v + bh * T * (BD * 2)), (short)0, (int)(T * (BD * 2)), 0x00020000);
  uint32_t off_u[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * wave + 4 * i + (lane >> 4);
    off_u[i] = (uint32_t)(row * 256 + 16 * uni_swz(row, lane & 15));
  }
  // load q = 0..3 of tile kt: K, then V
  auto dma_one = [&](int qi, int kt, char *kn, char *vn) {
    const uint32_t soff = (uint32_t)kt * BTILE;
    const int i = qi & 1;
    char *dst = (qi < 2 ? kn : vn) + (8 * wave + 4 * i) * 256;
    dma16(qi < 2 ? k_rsrc : v_rsrc, dst, off_u[i], soff);
  };
  // causal mask of key half kb2 of tile kt: register rr holds key
  // 64*kt + 32*kb2 + 8*(rr/4) + 4*lh + rr%4
  auto mask_half = [&](floatx16 &s, int kt, int kb2) {
    const int lim = (int)max((int64_t)-8, min((int64_t)64, tok - (int64_t)kt * 64 - 4 * lh));
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      if (32 * kb2 + 8 * (rr >> 2) + (rr & 3) > lim) s[rr] = -INFINITY;
  };

  for (int o = tid * 16; o < BTILE; o += 64 * DQ_WAVES * 16) {
    *(u32x4 *)(a_k0 + o) = u32x4{0, 0, 0, 0};
    *(u32x4 *)(a_k1 + o) = u32x4{0, 0, 0, 0};
    *(u32x4 *)(a_v0 + o) = u32x4{0, 0, 0, 0};
    *(u32x4 *)(a_v1 + o) = u32x4{0, 0, 0, 0};
  }
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) dma_one(qi, 0, a_k0, a_v0);
  wait_vmem();
  __syncthreads();

  auto body = [&](int j, auto parity, bool masked) {
    constexpr int P = decltype(parity)::value;
    const char *const kn_rd = P ? a_k1 : a_k0;
    const char *const kt_rd = kn_rd;
    const char *const vn_rd = P ? a_v1 : a_v0;
    char *const kn_wr = P ? a_k0 : a_k1;
    char *const vn_wr = P ? a_v0 : a_v1;
    // The tile is taken as two halves of 32 keys (kb2), which keeps one
    // half's scores, dP and dS in registers at a time.  The loads of tile
    // j+1 are spread between the first half's MFMAs.
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      // S^T = K Q^T (from -lse2/c) and dP^T = V dO^T (from -D) for keys
      // 32*kb2 .. +31: two independent MFMA chains, interleaved
      floatx16 s, dp;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        s[rr] = init_s;
        dp[rr] = init_dp;
      }
      {
        bf16x8 a[4], av[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a[i] = fr.rowfrag(kn_rd, 2 * i + kb2);
          av[i] = fr.rowfrag(vn_rd, 2 * i + kb2);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks & 3], qb[ks], s, 0, 0, 0);
          if (ks + 2 < 8) a[(ks + 2) & 3] = fr.rowfrag(kn_rd, 2 * (ks + 2) + kb2);
          if (kb2 == 0 && ks < 4) dma_one(ks, j + 1, kn_wr, vn_wr);
          __builtin_amdgcn_sched_barrier(0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks & 3], gb[ks], dp, 0, 0, 0);
          if (ks + 2 < 8) av[(ks + 2) & 3] = fr.rowfrag(vn_rd, 2 * (ks + 2) + kb2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (masked) mask_half(s, j, kb2);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s[rr] = fast_exp2(c * s[rr]);
      // dS^T = P^T (dP^T - D) as bf16 B operands of k-steps 2*kb2, 2*kb2 + 1
      bf16x8 dsb[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = 8 * kk + 2 * q;
          w[q] = cvt_bf16x2(s[rr] * dp[rr], s[rr + 1] * dp[rr + 1]);
        }
        dsb[kk] = __builtin_bit_cast(bf16x8, w);
      }
      // dQ^T += K^T dS^T over these 32 keys
      {
        bf16x8 a[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) a[i] = fr.colfrag(kt_rd, 4 * (i & 3) + 2 * kb2 + (i >> 2));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int nb = i & 3, kk = i >> 2;
          dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % 3], dsb[kk], dq[nb], 0, 0, 0);
          if (i + 3 < 8)
            a[i % 3] = fr.colfrag(kt_rd, 4 * ((i + 3) & 3) + 2 * kb2 + ((i + 3) >> 2));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  const int n_nm = (int)min((int64_t)n_kt, (wave_tok_lo + 1) / 64);
  int j = 0;
  for (; j + 1 < n_nm; j += 2) {
    body(j, I0{}, false);
    body(j + 1, I1{}, false);
  }
  for (; j < n_kt; ++j) {
    if (j & 1) body(j, I1{}, j >= n_nm);
    else body(j, I0{}, j >= n_nm);
  }

  if (row_ok) store_row((__bf16 *)p.dq + qrow * BD, dq, p.scale, lh);
}

// ---------------------------------------------------------------------------
// dK, dV: 4 key groups x 32 sequence keys; query tiles of 64 rows.  Each key
// group has two waves on one SIMD: one computes S and P and accumulates dV,
// the other computes dP, takes P from the first through LDS, and accumulates
// dK.
// ---------------------------------------------------------------------------
constexpr int KV_GROUPS = 4;             // key groups of 32 per workgroup
constexpr int KV_WAVES = 2 * KV_GROUPS;  // a dV wave and a dK wave per group
constexpr int KV_KEYS = 32 * KV_GROUPS;
constexpr int QROWS = 64;
constexpr int KV_ROWS = QROWS / KV_WAVES;  // query tile rows each wave loads
constexpr int KV_DMA = KV_ROWS / 4;        // 4-row load instructions per copy

// SPLIT: the query range of each key tile is cut into p.nsplit parts, one per
// workgroup, that leave fp32 partial sums (moda_bwd_kv_reduce adds them up);
// without it, one part that stores the bf16 gradients itself.
template <bool SPLIT>
__global__ __launch_bounds__(64 * KV_WAVES, 1) void moda_bwd_dkdv(BwdArgs p) {
  const int G = (int)(p.Hq / p.Hkv);
  const int TQr = QROWS / G;  // tokens per query tile (G <= 64)
  // Q and dO tiles of each parity, one copy each in the layout UniFrags reads
  // both ways.  Distinct objects, so that the compiler sees that loads in
  // flight into one parity's buffers never alias the other parity's being
  // read; the compiler lays out equally aligned LDS objects in name order,
  // which puts these (named to sort first) in the low 64 KiB, where every
  // read reaches its address through the 16-bit offset field.
  __shared__ __attribute__((aligned(1024))) char a_g0[BTILE];
  __shared__ __attribute__((aligned(1024))) char a_g1[BTILE];
  __shared__ __attribute__((aligned(1024))) char a_q0[BTILE];
  __shared__ __attribute__((aligned(1024))) char a_q1[BTILE];
  __shared__ __attribute__((aligned(16))) float lse_s[2][QROWS];  // -lse * log2(e)
  __shared__ __attribute__((aligned(16))) float del_s[2][QROWS];  // -D
  // P of the tile in fp32, in the dV wave's register order: [group][block][4 rows][lane]
  __shared__ __attribute__((aligned(16))) float4 p_x[KV_GROUPS][2][4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, lh = lane >> 5;
  const UniFrags fr(lane);
  // waves kg and kg + 4 share a SIMD and the key group kg: the first
  // accumulates dV (from S and P), the second dK (from S, dP and dS)
  const int kg = wave % KV_GROUPS;
  const bool dk_wave = wave >= KV_GROUPS;

  const int64_t T = p.T;
  const int64_t BH = p.B * p.Hkv;
  const int64_t S = SPLIT ? p.nsplit : 1;
  const int64_t x = blockIdx.x;
  const int64_t ktile = x / (BH * S);  // key tile 0 (the heaviest) first
  const int64_t bh = (x % (BH * S)) / S;
  const int64_t part = x % S;
  const int64_t b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int64_t k0 = ktile * KV_KEYS;

  // this lane's key (the column of every product) and its K row (dV wave) or
  // V row (dK wave) as B operands
  const int64_t key = k0 + 32 * kg + li;
  const bool key_ok = key < T;
  const int64_t krow = bh * T + (key_ok ? key : 0);
  bf16x8 kvb[8];
  load_row_operand((const __bf16 *)(dk_wave ? p.v : p.k) + krow * BD, key_ok, lh, kvb);

  floatx16 acc[4];  // dV^T or dK^T of the 32 keys
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) acc[nb][rr] = 0.f;

  const float c = p.scale_log2;
  // query tiles: tokens from k0 (the first that sees a key of this workgroup);
  // this workgroup takes part `part` of S even chunks of them
  const int64_t n_all = (T - k0 + TQr - 1) / TQr;
  const int64_t chunk = (n_all + S - 1) / S;
  const int64_t qt_lo = part * chunk;
  const int64_t n_qt = qt_lo + chunk < n_all ? qt_lo + chunk : n_all;  // one past the last

  // Tile loads.  Tile row r holds token t0 + r / G of head hkv*G + r % G; this
  // wave loads rows KV_ROWS*wave .. +KV_ROWS-1 of Q and of dO in instructions
  // of 4 rows.  Rows past the tile's tokens point outside the descriptor range
  // and read as zeros.
  const int64_t grp = b * p.Hq + hkv * G;  // first query head row block of the group
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const char *)p.q + grp * T * (BD * 2)), (short)0, (int)(G * T * (BD * 2)),
      0x00020000);
  const __amdgpu_buffer_rsrc_t g_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const char *)p.dout + grp * T * (BD * 2)), (short)0, (int)(G * T * (BD * 2)),
      0x00020000);
  uint32_t off_u[KV_DMA];
#pragma unroll
  for (int i = 0; i < KV_DMA; ++i) {
    const int row = KV_ROWS * wave + 4 * i + (lane >> 4);
    const bool used = row < TQr * G;
    const uint32_t base = (uint32_t)(((row % G) * T + row / G) * 256);
    off_u[i] = used ? base + 16 * uni_swz(row, lane & 15) : 0x80000000u;
  }
  auto dma_tile = [&](int64_t qt, char *qn, char *gn) {
    const uint32_t soff = (uint32_t)((k0 + qt * TQr) * 256);
#pragma unroll
    for (int i = 0; i < KV_DMA; ++i) {
      const int lrow = (KV_ROWS * wave + 4 * i) * 256;
      dma16(q_rsrc, qn + lrow, off_u[i], soff);
      dma16(g_rsrc, gn + lrow, off_u[i], soff);
    }
  };
  // lse and D of tile row `lane`, loaded by every wave without a branch (rows
  // outside the problem read row 0 and are replaced when stored).  Nothing
  // uses them until the tile's loads have landed: a use right after the load
  // would make the wave wait for the tile loads issued before it.
  struct RowStats {
    float l, dl;
    bool ok;
  };
  auto row_stats = [&](int64_t qt) {
    const int row = lane;
    const int64_t tk = k0 + qt * TQr + row / G;
    const bool ok = qt >= 0 && row < TQr * G && tk < T;
    const int64_t qr = ok ? (grp + row % G) * T + tk : 0;
    return RowStats{p.lse[qr], p.delta[qr], ok};
  };
  // -lse * log2(e) and -D; rows outside the problem get weight 0
  auto store_stats = [&](int buf, const RowStats &r) {
    lse_s[buf][lane] = r.ok ? -LOG2E * r.l : -INFINITY;
    del_s[buf][lane] = r.ok ? -r.dl : 0.f;
  };

  for (int o = tid * 16; o < BTILE; o += 64 * KV_WAVES * 16) {
    *(u32x4 *)(a_q0 + o) = u32x4{0, 0, 0, 0};
    *(u32x4 *)(a_q1 + o) = u32x4{0, 0, 0, 0};
    *(u32x4 *)(a_g0 + o) = u32x4{0, 0, 0, 0};
    *(u32x4 *)(a_g1 + o) = u32x4{0, 0, 0, 0};
  }
  __syncthreads();
  if (qt_lo < n_qt) {
    dma_tile(n_qt - 1, a_q0, a_g0);
    const RowStats r0 = row_stats(n_qt - 1);
    if (wave == 0) store_stats(0, r0);
  }
  wait_vmem();
  __syncthreads();

  // Query tiles are walked from the last one down: the workgroups of a dispatch
  // round then read the same query tiles at about the same time, as the forward's
  // workgroups read the same key tiles, and find them in L2.
  // Query tile qt in buffers of parity P; loads of tile qt-1 are issued first.
  auto body = [&](int64_t qt, auto parity, auto is_dk) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    constexpr bool DK = decltype(is_dk)::value;
    const char *const qn = P ? a_q1 : a_q0;
    const char *const gn = P ? a_g1 : a_g0;
    const bool more = qt > qt_lo;
    if (more) dma_tile(qt - 1, P ? a_q0 : a_q1, P ? a_g0 : a_g1);
    const RowStats rn = row_stats(qt - 1);
    const int64_t tq0 = k0 + qt * TQr;  // first token of the tile
    // the tile needs the causal mask unless its first token is at or past
    // this group's last key
    const bool masked = tq0 < k0 + 32 * kg + 31;
    // tile row r is token tq0 + r / G: it precedes this lane's key exactly
    // when r < (key - tq0) * G
    const int lim = (int)min(max(key - tq0, (int64_t)-1), (int64_t)QROWS) * G - 4 * lh;
    // register rr of 32-row block sb holds tile row 32*sb + 8*(rr/4) + 4*lh + rr%4.
    // Phase 1: S = Q K^T and P (dV wave, P also to LDS), dP = dO V^T (dK wave)
    floatx16 x[2];
    bf16x8 wb[2][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) x[sb][rr] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        x[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.rowfrag(DK ? gn : qn, 2 * ks + sb),
                                                        kvb[ks], x[sb], 0, 0, 0);
    }
    if constexpr (DK) {
      // dP - D, ahead of the barrier
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 d4 = *(const float4 *)&del_s[P][32 * sb + 8 * g + 4 * lh];
          x[sb][4 * g + 0] += d4.x;
          x[sb][4 * g + 1] += d4.y;
          x[sb][4 * g + 2] += d4.z;
          x[sb][4 * g + 3] += d4.w;
        }
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if (masked) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (32 * sb + 8 * (rr >> 2) + (rr & 3) < lim) x[sb][rr] = -INFINITY;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 l4 = *(const float4 *)&lse_s[P][32 * sb + 8 * g + 4 * lh];
          x[sb][4 * g + 0] = fast_exp2(fmaf(c, x[sb][4 * g + 0], l4.x));
          x[sb][4 * g + 1] = fast_exp2(fmaf(c, x[sb][4 * g + 1], l4.y));
          x[sb][4 * g + 2] = fast_exp2(fmaf(c, x[sb][4 * g + 2], l4.z));
          x[sb][4 * g + 3] = fast_exp2(fmaf(c, x[sb][4 * g + 3], l4.w));
          p_x[kg][sb][g][lane] = float4{x[sb][4 * g], x[sb][4 * g + 1], x[sb][4 * g + 2],
                                        x[sb][4 * g + 3]};
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 u;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            u[q] = cvt_bf16x2(x[sb][8 * kk + 2 * q], x[sb][8 * kk + 2 * q + 1]);
          wb[sb][kk] = __builtin_bit_cast(bf16x8, u);
        }
      }
    }
    __syncthreads();
    // Phase 2: dV^T += dO^T P (dV wave); dS = P (dP - D), dK^T += Q^T dS (dK wave)
    if constexpr (DK) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const floatx16 &d = x[sb];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const float4 p0 = p_x[kg][sb][2 * kk][lane], p1 = p_x[kg][sb][2 * kk + 1][lane];
          const int rr = 8 * kk;
          u32x4 u;
          u[0] = cvt_bf16x2(p0.x * d[rr + 0], p0.y * d[rr + 1]);
          u[1] = cvt_bf16x2(p0.z * d[rr + 2], p0.w * d[rr + 3]);
          u[2] = cvt_bf16x2(p1.x * d[rr + 4], p1.y * d[rr + 5]);
          u[3] = cvt_bf16x2(p1.z * d[rr + 6], p1.w * d[rr + 7]);
          wb[sb][kk] = __builtin_bit_cast(bf16x8, u);
        }
      }
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              fr.colfrag(DK ? qn : gn, 4 * nb + 2 * sb + kk), wb[sb][kk], acc[nb], 0, 0, 0);
    wait_vmem();
    if (more && wave == 0) store_stats(P ^ 1, rn);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto run = [&](auto is_dk) __attribute__((always_inline)) {
    int64_t qt = n_qt - 1;
    for (; qt - 1 >= qt_lo; qt -= 2) {
      body(qt, I0{}, is_dk);
      body(qt - 1, I1{}, is_dk);
    }
    if (qt >= qt_lo) body(qt, I0{}, is_dk);
  };
  if (dk_wave)
    run(std::true_type{});
  else
    run(std::false_type{});

  if (!key_ok) return;
  if constexpr (!SPLIT) {
    store_row((__bf16 *)(dk_wave ? p.dk : p.dv) + (bh * T + key) * BD, acc,
              dk_wave ? p.scale : 1.0f, lh);
    return;
  }
  // this part's fp32 partial sums (zero if it had no query tile)
  float *const ws =
      p.kv_ws + (((dk_wave ? S : 0) + part) * BH * T + bh * T + key) * (int64_t)BD;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(float4 *)(ws + 32 * nb + 8 * g + 4 * lh) =
          float4{acc[nb][4 * g], acc[nb][4 * g + 1], acc[nb][4 * g + 2], acc[nb][4 * g + 3]};
}

// Sum of the S parts' partial dV and dK (fp32) into the bf16 gradients; one
// thread per 8 dims of a key.
__global__ __launch_bounds__(256) void moda_bwd_kv_reduce(BwdArgs p) {
  const int64_t BHT = p.B * p.Hkv * p.T;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (which * BHT + row) * 16 + c
  if (i >= 2 * BHT * (BD / 8)) return;
  const int64_t which = i / (BHT * (BD / 8));
  const int64_t rc = i % (BHT * (BD / 8));
  const int64_t S = p.nsplit;
  const float *src = p.kv_ws + which * S * BHT * BD + rc * 8;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t sp = 0; sp < S; ++sp) {
    const float4 lo = *(const float4 *)(src + sp * BHT * BD);
    const float4 hi = *(const float4 *)(src + sp * BHT * BD + 4);
    a[0] += lo.x; a[1] += lo.y; a[2] += lo.z; a[3] += lo.w;
    a[4] += hi.x; a[5] += hi.y; a[6] += hi.z; a[7] += hi.w;
  }
  const float sc = which ? p.scale : 1.0f;
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = cvt_bf16x2(a[2 * q] * sc, a[2 * q + 1] * sc);
  *(u32x4 *)((__bf16 *)(which ? p.dk : p.dv) + rc * 8) = o;
}

// ---------------------------------------------------------------------------
// Depth gradients: dKd, dVd and the depth entries' part of dQ.  A workgroup
// covers DD_SPANS spans of TW = floor(32/G) whole tokens (their G query rows
// each, 32 rows at most), with two waves per span on one SIMD:
//   the entry wave (a lane per entry of a 32-entry block) reads the block
//     (natural Kd and Vd rows) once and computes S_d = Q Kd^T, P_d,
//     dP_d = dO Vd^T and dS_d; it passes the block's K rows and dS_d to the
//     row wave through LDS, then forms dVd^T = dO^T P_d and dKd^T = Q^T dS_d,
//     with Q^T and dO^T read transposed from the span's rows stored once in
//     LDS; the next block's loads are in flight meanwhile;
//   the row wave (a lane per query row) accumulates dQ^T += Kd^T dS_d^T from
//     the two hand-over buffers and at the end adds the sum to dQ, which holds
//     the sequence part.
// Two workgroup barriers per block order the hand-over.  Every row that reads
// an entry is in the entry's span, so no atomics are needed.
// ---------------------------------------------------------------------------
constexpr int DD_SPANS = 4;
constexpr int DD_WAVES = 2 * DD_SPANS;

__global__ __launch_bounds__(64 * DD_WAVES, 1) void moda_bwd_ddepth(BwdArgs p) {
  const int G = (int)(p.Hq / p.Hkv);
  const int TW = 32 / G;            // tokens per span (G <= 32)
  const int TWG = TW * DD_SPANS;    // tokens per workgroup
  __shared__ __attribute__((aligned(1024))) char q_s[DD_SPANS][32 * 256];
  __shared__ __attribute__((aligned(1024))) char g_s[DD_SPANS][32 * 256];
  __shared__ __attribute__((aligned(1024))) char k_s[DD_SPANS][32 * 256];
  __shared__ __attribute__((aligned(1024))) char o_s[DD_SPANS][32 * 256];  // output staging
  __shared__ __attribute__((aligned(1024))) char x_s[DD_SPANS][32 * 64];   // dS_d^T, bf16
  __shared__ __attribute__((aligned(16))) float lse_s[DD_SPANS][32];  // -lse * log2(e)
  __shared__ __attribute__((aligned(16))) float del_s[DD_SPANS][32];  // -D

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves s and s + DD_SPANS share a SIMD and span s
  const int span = wave % DD_SPANS;
  const bool row_wave = wave >= DD_SPANS;
  const int li = lane & 31, lh = lane >> 5;
  const TileFrags fr(lane);

  const int64_t T = p.T, L = p.L, TL = p.T * p.L;
  const int64_t BH = p.B * p.Hkv;
  const int64_t x = blockIdx.x;
  const int64_t bh = x % BH;
  const int64_t b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int64_t wg_lo = (x / BH) * TWG;
  // blocks holding entries of the span starting at token lo (0 past the end)
  auto span_blocks = [&](int64_t lo) -> int64_t {
    if (lo >= T) return 0;
    const int64_t hi = lo + TW < T ? lo + TW : T;
    return (hi * L + kDepthBlock - 1) / kDepthBlock - lo * L / kDepthBlock;
  };
  // every wave walks the workgroup's longest span so that all meet at each barrier
  int64_t n_iter = 0;
  for (int s = 0; s < DD_SPANS; ++s) {
    const int64_t n = span_blocks(wg_lo + (int64_t)s * TW);
    n_iter = n > n_iter ? n : n_iter;
  }
  const int64_t wt_lo = wg_lo + (int64_t)span * TW;  // the span's first token
  const int64_t wt_hi = wt_lo + TW < T ? wt_lo + TW : T;
  const int64_t e_lo = wt_lo * L, e_hi = wt_hi * L;  // entries of the span's tokens
  const int64_t blk_lo = e_lo / kDepthBlock;
  const int64_t blk_hi = blk_lo + span_blocks(wt_lo);

  // this lane's row: the entry wave's copy into LDS, the row wave's dQ row
  const int r = li;
  const bool row_used = r < TW * G;
  const int64_t tok = wt_lo + r / G;
  const bool row_ok = row_used && tok < T;
  const int64_t head = hkv * G + (row_used ? r % G : 0);
  const int64_t qrow = (b * p.Hq + head) * T + (row_ok ? tok : 0);
  if (!row_wave) {
    bf16x8 qb[8], gb[8];
    load_row_operand((const __bf16 *)p.q + qrow * BD, row_ok, lh, qb);
    load_row_operand((const __bf16 *)p.dout + qrow * BD, row_ok, lh, gb);
    // rows outside the problem get weight 0
    const float l_row = row_ok ? -LOG2E * p.lse[qrow] : -INFINITY;
    const float d_row = row_ok ? -p.delta[qrow] : 0.f;
    char *const qs = q_s[span];
    char *const gs = g_s[span];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int off = r * 256 + 16 * col_swz(r, 8 * lh + ks);
      *(bf16x8 *)(qs + off) = qb[ks];
      *(bf16x8 *)(gs + off) = gb[ks];
    }
    if (lh == 0) {
      lse_s[span][r] = l_row;
      del_s[span][r] = d_row;
    }
  }

  const float c = p.scale_log2;
  char *const ks_ = k_s[span];
  char *const xs = x_s[span];
  // the row wave's B operand: dS_d^T read transposed from x_s (rows of 64
  // bytes, no swizzle), the same lane pattern as TileFrags::colfrag
  const int lg = lane >> 4, lq = lane & 15;
  const int xaddr = (4 * (lg >> 1) + (lq >> 2)) * 64 + 16 * (2 * (lg & 1) + ((lq & 3) >> 1)) +
                    8 * (lq & 1);

  // Per block: the entry wave (a lane per entry) computes S_d = Q Kd^T,
  // dP_d = dO Vd^T, P_d and dS_d, hands the K rows and dS_d to the row wave
  // through LDS, then forms dVd and dKd; the row wave (a lane per query row)
  // accumulates dQ^T += Kd^T dS_d^T.  The depth block is read from memory once.
  // Both kinds of wave pass the same barriers, n_iter times each: one before
  // the hand-over buffers are rewritten, one after they are filled.
  if (!row_wave) {
    // Every load and store of the loop is a buffer instruction over the
    // block's own range, so none is skipped: entries past the stream and
    // blocks past the span read zeros, and rows the span does not own are
    // dropped.  The loads of the next block then stay counted ahead of this
    // block's stores, and the wait for them never waits for the stores.
    const char *const knat = (const char *)p.kd + bh * TL * (BD * 2);
    const char *const vnat = (const char *)p.vd + bh * TL * (BD * 2);
    // 32 consecutive entries of the natural [B,Hkv,T,L,d] depth K and V: lane l
    // takes row l % 32, dims 64*(l/32) + 8*ks .. +7 of each (MFMA operand order)
    auto load_block = [&](int64_t blk, u32x4(&kd)[8], u32x4(&vr)[8])
                          __attribute__((always_inline)) {
      const bool in = blk < blk_hi;
      const int64_t left = TL - blk * kDepthBlock;
      const int vrows = !in ? 0 : left < kDepthBlock ? (int)left : kDepthBlock;
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(knat + blk * kDepthBlock * (BD * 2)), (short)0, vrows * (BD * 2), 0x00020000);
      const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(vnat + blk * kDepthBlock * (BD * 2)), (short)0, vrows * (BD * 2), 0x00020000);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        kd[ks] = __builtin_amdgcn_raw_buffer_load_b128(kr, li * 256 + 128 * lh + 16 * ks, 0, 0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        vr[ks] = __builtin_amdgcn_raw_buffer_load_b128(vrs, li * 256 + 128 * lh + 16 * ks, 0, 0);
    };
    // S_d = Q Kd^T and dP_d = dO Vd^T (rows x entries), then P_d and
    // dS_d = P_d (dP_d - D) as bf16 B operands
    auto scores = [&](int64_t blk, const u32x4(&kd)[8], const u32x4(&vr)[8], bf16x8(&pb)[2],
                      bf16x8(&dsb)[2]) __attribute__((always_inline)) {
      const int64_t e = blk * kDepthBlock + li;  // this lane's entry
      floatx16 sd, dpd;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sd[rr] = dpd[rr] = 0.f;
      // the row operands come from their LDS copies (registers are kept for
      // the next block's loads); the opaque offset keeps them in the loop
      int roff = r * 256;
      asm volatile("" : "+v"(roff));
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = roff + 16 * col_swz(r, 8 * lh + ks);
        sd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(q_s[span] + off),
                                                     __builtin_bit_cast(bf16x8, kd[ks]), sd, 0, 0,
                                                     0);
        dpd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(g_s[span] + off),
                                                      __builtin_bit_cast(bf16x8, vr[ks]), dpd, 0,
                                                      0, 0);
      }
      // register rr holds row 8*(rr/4) + 4*lh + rr%4: keep it iff the row is
      // one of the G rows of the entry's token, i.e. row - etok*G in [0, G)
      const int etok = (int)(e / L - wt_lo);
      const int base = 4 * lh - etok * G;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        if ((unsigned)(8 * (rr >> 2) + (rr & 3) + base) >= (unsigned)G) sd[rr] = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const float4 la = *(const float4 *)&lse_s[span][8 * (2 * kk) + 4 * lh];
        const float4 lb = *(const float4 *)&lse_s[span][8 * (2 * kk + 1) + 4 * lh];
        const float4 da = *(const float4 *)&del_s[span][8 * (2 * kk) + 4 * lh];
        const float4 db = *(const float4 *)&del_s[span][8 * (2 * kk + 1) + 4 * lh];
        const float lr[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
        const float dr[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
        u32x4 w, wd;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = 8 * kk + 2 * q;
          const float p0 = fast_exp2(fmaf(c, sd[rr], lr[2 * q]));
          const float p1 = fast_exp2(fmaf(c, sd[rr + 1], lr[2 * q + 1]));
          w[q] = cvt_bf16x2(p0, p1);
          wd[q] = cvt_bf16x2(p0 * (dpd[rr] + dr[2 * q]), p1 * (dpd[rr + 1] + dr[2 * q + 1]));
        }
        pb[kk] = __builtin_bit_cast(bf16x8, w);
        dsb[kk] = __builtin_bit_cast(bf16x8, wd);
      }
    };

    u32x4 kd[8], vr[8];
    bf16x8 pb[2], dsb[2];
    load_block(blk_lo, kd, vr);
    __syncthreads();  // the span's rows and statistics are in LDS
    scores(blk_lo, kd, vr, pb, dsb);
    for (int64_t it = 0; it < n_iter; ++it) {
      const int64_t blk = blk_lo + it;
      __syncthreads();  // the row waves are done with the previous block's K rows and dS_d
      // K rows column-swizzled; dS_d^T as [entry][row]: dsb[kk] holds rows
      // 16kk + 4lh + 0..3 and 16kk + 8 + 4lh + 0..3 of entry li
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        *(u32x4 *)(ks_ + li * 256 + 16 * col_swz(li, 8 * lh + ks)) = kd[ks];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 w = __builtin_bit_cast(u32x4, dsb[kk]);
        *(u32x2 *)(xs + li * 64 + 32 * kk + 8 * lh) = u32x2{w[0], w[1]};
        *(u32x2 *)(xs + li * 64 + 32 * kk + 16 + 8 * lh) = u32x2{w[2], w[3]};
      }
      // the next block's loads land while this one's gradients are formed
      load_block(blk + 1, kd, vr);
      __syncthreads();  // K rows and dS_d of this block are in LDS
      // dVd^T = dO^T P_d, then dKd^T = Q^T dS_d (the span's 32 rows as two
      // k-steps), one accumulator set at a time.  Each goes to LDS as the
      // block's 32 rows (chunk c of row r in slot c ^ (r % 16)) and from there
      // to memory four whole rows per instruction, rows the span owns only.
      const char *const qs = q_s[span];
      const char *const gs = g_s[span];
      char *const os = o_s[span];
      const int64_t b0 = blk * kDepthBlock;
      const int lo_r = e_lo > b0 ? (int)(e_lo - b0) : 0;
      const int hi_r = e_hi - b0 < kDepthBlock ? (int)(e_hi - b0) : kDepthBlock;
      const int nrec = hi_r > 0 ? hi_r * (BD * 2) : 0;
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        floatx16 acc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) acc[nb][rr] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                fr.colfrag(which ? qs : gs, 4 * nb + kk), which ? dsb[kk] : pb[kk], acc[nb], 0,
                0, 0);
        const float sc = which ? p.scale : 1.0f;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2 o;
            o[0] = cvt_bf16x2(acc[nb][4 * g + 0] * sc, acc[nb][4 * g + 1] * sc);
            o[1] = cvt_bf16x2(acc[nb][4 * g + 2] * sc, acc[nb][4 * g + 3] * sc);
            *(u32x2 *)(os + li * 256 + 16 * ((4 * nb + g) ^ (li & 15)) + 8 * lh) = o;
          }
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const __bf16 *)(which ? p.dkd : p.dvd) + (bh * TL + b0) * BD), (short)0,
            nrec, 0x00020000);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int rr = 4 * i + (lane >> 4), cc = lane & 15;
          const u32x4 v = *(const u32x4 *)(os + rr * 256 + 16 * (cc ^ (rr & 15)));
          const int voff = rr >= lo_r ? rr * (BD * 2) + 16 * cc : (int)0x80000000;
          __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, voff, 0, 0);
        }
      }
      // the next block's scores (past the span: unused)
      scores(blk + 1, kd, vr, pb, dsb);
    }
    return;
  }

  // row wave
  floatx16 dq[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) dq[nb][rr] = 0.f;
  __syncthreads();
  for (int64_t it = 0; it < n_iter; ++it) {
    __syncthreads();
    __syncthreads();
    if (blk_lo + it >= blk_hi) continue;
    // dQ^T += Kd^T dS_d^T over the block's 32 entries (two k-steps)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const char *const vp = xs + xaddr + kk * 16 * 64;
      const shortx4 lo = lds_read_tr(vp);
      const shortx4 hi = lds_read_tr(vp + 8 * 64);
      const bf16x8 xb = __builtin_bit_cast(
          bf16x8, (u32x4){__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.colfrag(ks_, 4 * nb + kk), xb,
                                                         dq[nb], 0, 0, 0);
    }
  }
  // dQ (the sequence part, as written) += s * the depth part
  if (row_ok) {
    __bf16 *const row = (__bf16 *)p.dq + qrow * BD;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 *const pp = (u32x2 *)(row + 32 * nb + 8 * g + 4 * lh);
        const u32x2 o = *pp;
        u32x2 n;
        n[0] = cvt_bf16x2(bf16_bits_to_float(o[0] & 0xFFFFu) + dq[nb][4 * g + 0] * p.scale,
                          bf16_bits_to_float(o[0] >> 16) + dq[nb][4 * g + 1] * p.scale);
        n[1] = cvt_bf16x2(bf16_bits_to_float(o[1] & 0xFFFFu) + dq[nb][4 * g + 2] * p.scale,
                          bf16_bits_to_float(o[1] >> 16) + dq[nb][4 * g + 3] * p.scale);
        *pp = n;
      }
  }
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
  const int64_t G = a.Hq / a.Hkv;
  const int64_t rows = a.B * a.Hq * a.T;
  hipLaunchKernelGGL(moda_bwd_delta, dim3((uint32_t)((rows + 255) / 256)), dim3(256), 0, s, a);
  const int64_t tq = DQ_ROWS / G;
  const int64_t dq_grid = (a.T + tq - 1) / tq * a.B * a.Hkv;
  hipLaunchKernelGGL(moda_bwd_dq, dim3((uint32_t)dq_grid), dim3(64 * DQ_WAVES), 0, s, a);
  const int64_t kv_grid = (a.T + KV_KEYS - 1) / KV_KEYS * a.B * a.Hkv * a.nsplit;
  if (a.nsplit > 1)
    hipLaunchKernelGGL(moda_bwd_dkdv<true>, dim3((uint32_t)kv_grid), dim3(64 * KV_WAVES), 0, s, a);
  else
    hipLaunchKernelGGL(moda_bwd_dkdv<false>, dim3((uint32_t)kv_grid), dim3(64 * KV_WAVES), 0, s,
                       a);
  if (a.nsplit > 1) {
    const int64_t n = 2 * a.B * a.Hkv * a.T * (BD / 8);
    hipLaunchKernelGGL(moda_bwd_kv_reduce, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  if (a.L > 0) {
    // after dq: it adds the depth entries' part to dQ
    const int64_t twg = (32 / G) * DD_SPANS;
    const int64_t dd_grid = (a.T + twg - 1) / twg * a.B * a.Hkv;
    hipLaunchKernelGGL(moda_bwd_ddepth, dim3((uint32_t)dd_grid), dim3(64 * DD_WAVES), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moda
