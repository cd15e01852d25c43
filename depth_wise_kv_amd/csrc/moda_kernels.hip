// HIP kernels of the MoDA forward for gfx950 (MI355X).
//
// What is computed (hyper.ai page on arXiv 2603.15619, section
// "Mixture-of-Depths Attention (MoDA)"): each query row (b, h, t) takes one
// softmax, scaled by 1/sqrt(d), over the causal sequence keys 0..t of KV head
// h / G and over its own token's L depth keys, and returns the weighted sum
// of the matching values.  Sequence and depth logits update one online-softmax
// state; the output is normalised once at the end (section
// "Hardware-efficient implementation").
//
// Kernels:
//   moda_fwd_mfma   bf16, d = 128.  A workgroup owns 256 query rows (128 on
//                   grids too small to fill the chip) made of rows/G tokens x
//                   the G heads of one KV group, so one K/V tile in LDS and
//                   one depth span serve all G heads (the group-aware indexing
//                   of the same section).  QK^T and PV run on
//                   v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//   moda_pack_mfma  repacks [B,Hkv,T,L,d] depth K/V into blocks of 8 tokens x
//                   4 entries laid out in MFMA operand order, K half then V
//                   half, so each wave streams its depth span with fully
//                   contiguous loads.
//   moda_fwd_generic / moda_copy_generic: one wave per query row on the VALU,
//                   for fp32 or bf16 with d in {32, 64} when G is above 128
//                   (below that, moda_fwd_small.hip's matrix-core kernel), and
//                   the copy that fills their depth layout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moda_device.h"
#include "moda_internal.h"


namespace moda {

__device__ __forceinline__ float wave_swap32(float x) {
  // value held by lane (l ^ 32)
  return __shfl_xor(x, 32, 64);
}

// ---------------------------------------------------------------------------
// MFMA path geometry.
//
// 32x32x16 bf16 MFMA operand/result layout used below (lane l, h = l / 32):
//   A operand: row (l % 32), 8 consecutive k values of lane half h
//   B operand: column (l % 32), the same 8 k values as A
//   result   : column (l % 32), register r holds row 8*(r/4) + 4*h + r%4
// Only the pairing of k between A and B matters for a contraction, so each
// operand load below picks whichever k order makes its own load contiguous.
//
// Scores are computed transposed, S^T = K * Q^T, so a lane owns one query row
// (column l % 32) and holds that row's scores in registers: row max and row
// sum are in-lane work plus one exchange with lane l ^ 32.
// ---------------------------------------------------------------------------
constexpr int D = kMfmaD;             // 128
constexpr int NKEY = 64;              // keys per sequence tile
constexpr int BLK_HALF = kDepthBlock * D * 2;  // bytes of the K (or V) half of a packed block

// Optional cycle tracing of the fused kernel's phases (off unless the build
// defines MODA_TRACE_ENABLED; then moda_trace_buf receives per-phase cycle
// sums, summed over waves, from the shader clock).
#ifdef MODA_TRACE_ENABLED
__device__ unsigned long long moda_trace_buf[16];
#define MODA_TRACE_DECL                          \
  long long tr_last = __builtin_amdgcn_s_memtime(); \
  long long tr_acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#define MODA_TRACE(i)                                   \
  do {                                                  \
    const long long tr_now = __builtin_amdgcn_s_memtime(); \
    tr_acc[i] += tr_now - tr_last;                      \
    tr_last = tr_now;                                   \
  } while (0)
#define MODA_TRACE_FLUSH                                                            \
  do {                                                                              \
    if ((threadIdx.x & 63) == 0)                                                    \
      for (int i_ = 0; i_ < 8; ++i_) atomicAdd(&moda_trace_buf[i_], (unsigned long long)tr_acc[i_]); \
  } while (0)
#else
#define MODA_TRACE_DECL
#define MODA_TRACE(i) \
  do {                \
  } while (0)
#define MODA_TRACE_FLUSH \
  do {                   \
  } while (0)
#endif

// ---------------------------------------------------------------------------
// Fused forward, MFMA path.
//
// A workgroup has 8 waves and owns 256 query rows (32 per wave): two waves on
// every SIMD, and each K/V tile brought into LDS serves 256 rows.  (Small
// grids use 4-wave workgroups of 128 rows instead, two per CU.)  K and V tiles of 64
// keys go straight from global memory into LDS (buffer_load_dwordx4 ... lds), no
// registers in between, into XOR-swizzled 16 KiB buffers:
//   K: 16-byte chunk c of key row r sits in slot c ^ (r % 16)    (ds_read_b128
//      of 16 consecutive rows at one chunk hits 16 distinct slots)
//   V: chunk c of key row r sits in slot c ^ 4*(r % 4)           (each 16-lane
//      group of a transpose read touches 4 rows x 2 chunks, 8 distinct slots)
// Iteration j of the key loop computes S(j) = K(j) Q^T, turns it into weights,
// adds V(j)^T P(j)^T to the accumulator, and meanwhile loads tile j+1 (this
// wave's eighth of it) into the other K and V buffers, whose last readers
// finished before the barrier that ended iteration j-1.  The two waves that
// share a SIMD overlap one's softmax with the other's MFMAs.  The four buffers
// are distinct LDS objects and the loop is unrolled by buffer parity, so the
// compiler can see that the loads in flight never alias the buffers read.
// ---------------------------------------------------------------------------
constexpr int TILE_BYTES = NKEY * D * 2;  // 16 KiB: one K or V tile

// Order of the 16 PV MFMAs: fragment f = 4*nb + kk feeds accumulator nb with
// key step kk.  Going round-robin over the four accumulators keeps
// consecutive MFMAs independent.
__device__ __forceinline__ constexpr int pv_order(int i) { return 4 * (i & 3) + (i >> 2); }


// NW waves of 32 query rows each: 8 (one workgroup per CU, two waves per
// SIMD) or 4 (two workgroups per CU, for grids too small to fill the chip
// several times over with 256-row tiles).  With ROWS = 128 and NW = 8 (the
// key-split form, causal and packed MoDA modes only) the waves pair up:
// waves 2i and 2i+1 own the same 32 rows, one the first 32 keys of every
// 64-key tile and one the last 32 (and alternate depth blocks), and merge
// their softmax states at the end.  A 128-row tile then runs on two waves per
// SIMD, as the 8-wave kernel does, instead of one.
template <int MODE, int NW, int ROWS>
__global__ __launch_bounds__(64 * NW, 8 / NW) void moda_fwd_mfma(FwdArgs p) {
  constexpr int NWAVE = NW;                  // waves per workgroup
  constexpr int MR = ROWS;                   // query rows per workgroup
  constexpr bool KS = ROWS < 32 * NW;        // key-split pairs of waves
  static_assert(!KS || (NW == 8 && ROWS == 128 && (MODE == kModeCausal || MODE == kModeModa)),
                "the key-split form has 8 waves, 128 rows, causal or packed MoDA mode");
  constexpr int NKB = KS ? 1 : 2;            // 32-key blocks of each tile a wave takes
  constexpr int DMA_ROWS = NKEY / NWAVE;     // tile rows each wave loads
  constexpr int DMA_INSTR = DMA_ROWS / 4;    // 1 KiB (4-row) load instructions per wave per tile
  static_assert(DMA_INSTR >= 1 && 16 % (2 * DMA_INSTR) == 0, "tile loads must divide the MFMAs");
  constexpr bool HAS_DEPTH = MODE != kModeCausal;  // depth entries are read
  constexpr bool HAS_SEQ = MODE != kModeDepth;     // sequence keys are read
  // depth K, V read row by row (not from the packed cache): natural or layer-major layout
  constexpr bool NATURAL =
      MODE == kModeModaNatural || MODE == kModeModaLayers || MODE == kModeModaScan;
  constexpr bool LAYERS = MODE == kModeModaLayers;  // strided depth rows
  constexpr bool SCAN = MODE == kModeModaScan;  // depth scanned from the first token's entries
  // A tile holds TQ = floor(MR / G) tokens x G heads; rows past TQ * G idle.
  const int G = (int)(p.Hq / p.Hkv);
  const int TQ = MR / G;
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, lh = lane >> 5;
  const int rw = KS ? wave >> 1 : wave;  // this wave's 32-row block
  const int kh = KS ? wave & 1 : 0;      // its 32-key half of each tile (key split)

  const int64_t T = p.T;
  const int64_t BH = p.B * p.Hkv;
  const int64_t ntiles = (T + TQ - 1) / TQ;
  // Heaviest causal tiles first: blocks 0..BH-1 take the last tile of each head.
  const int64_t x = blockIdx.x;
  const int64_t tile = ntiles - 1 - x / BH;
  const int64_t bh = x % BH;
  const int64_t b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int64_t t0 = tile * TQ;

  // This lane's query row: row r = token-in-tile * G + head-in-group.
  const int r = rw * 32 + li;
  const bool row_used = r < TQ * G;
  const int64_t tok = row_used ? t0 + r / G : T;  // idle rows sit past the end
  const int64_t head = hkv * G + (row_used ? r % G : 0);
  const bool row_ok = tok < T;

  // Q row as the B operand of S^T = K Q^T: lane half h holds dims 64h..64h+63,
  // 8 per k-step.
  bf16x8 qb[8];
  {
    const __bf16 *qrow = (const __bf16 *)p.q + ((b * p.Hq + head) * T + (row_ok ? tok : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 u = row_ok ? *(const u32x4 *)(qrow + 64 * lh + 8 * ks) : u32x4{0, 0, 0, 0};
      qb[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  MfmaState st;
  st.m = -INFINITY;
  st.lsum = 0.f;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) st.acc[nb][rr] = 0.f;
  const float sc = p.scale_log2;

  // ---------------- depth part: this wave's tokens' contiguous depth span.
  // Odd workgroups stream their depth span before the key loop, even ones
  // after it, so that at any time part of the chip streams depth blocks from
  // HBM while the rest runs the matrix-core-bound key loop.
  // Depth blocks [blk_lo, blk_hi) read in the natural [B,Hkv,T,L,d] layout
  // (the natural-layout mode): a block's 32 Kd rows load straight into MFMA
  // operand registers (16 bytes of one row per lane), and its 32 Vd rows go
  // into this wave's 8 KiB of the tile buffers, column-swizzled, to be read
  // transposed as the A operand of O^T += Vd^T P^T.
  // In the strided mode (row (b, g, token, entry) of the depth K and V at
  // (b*Hkv + g) * s_bh + token * s_t + entry * s_i: e.g. layer-major
  // [Lcap, B, Hkv, T, d], where entry i of every token is the K or V layer i
  // wrote, or [B, Hkv, T, Lcap, d] with room for more entries) the same flat
  // (token, entry) blocks are gathered row by row with 64-bit addresses.
  auto depth_natural = [&](int64_t blk_lo, int64_t blk_hi, int64_t my_lo) {
    if constexpr (NATURAL) {
      const int64_t L = p.L, TL = T * L;
      const __bf16 *knat = (const __bf16 *)p.kd_nat + (LAYERS ? 0 : bh * TL * D);
      const __amdgpu_buffer_rsrc_t vd_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void *)((const char *)p.vd_nat + bh * TL * (D * 2)), (short)0, (int)(TL * (D * 2)),
          0x00020000);
      char *const slot = (wave < 2 ? k_lds0 : wave < 4 ? k_lds1 : wave < 6 ? v_lds0 : v_lds1) +
                         (wave & 1) * (TILE_BYTES / 2);
      const TileFrags fr(lane);
      // row of flat entry e (= token * L + entry, e < T * L < 2^23) in the strided
      // depth tensors: bh * s_bh + token * s_t + entry * s_i (rows of d elements)
      auto layer_row = [&](int64_t e) -> int64_t {
        const uint32_t eu = (uint32_t)e, Lu = (uint32_t)L;
        uint32_t t = (uint32_t)((float)eu * p.inv_L);  // floor(e / L), or one off
        if (t * Lu > eu) --t;
        else if ((t + 1) * Lu <= eu) ++t;
        return bh * p.ds_bh + (int64_t)t * p.ds_t + (int64_t)(eu - t * Lu) * p.ds_i;
      };
      auto load_k = [&](int64_t blk, u32x4 (&kd)[8]) {
        const int64_t e = blk * kDepthBlock + li;
        const __bf16 *src = knat + (LAYERS ? layer_row(e < TL ? e : 0) : e) * D + 64 * lh;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          kd[ks] = e < TL ? *(const u32x4 *)(src + 8 * ks) : u32x4{0, 0, 0, 0};
      };
      // this wave's Vd rows of block blk into its slot, column-swizzled; a row past
      // T * L reads zeros (natural) or repeats the last row (layer-major): its weight is 0
      auto load_v = [&](int64_t blk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 4 * i + (lane >> 4);
          const int chunk = 16 * ((lane & 15) ^ (4 * (row & 3)));
          __attribute__((address_space(3))) void *dst =
              (__attribute__((address_space(3))) void *)(slot + 4 * i * 256);
          if constexpr (LAYERS) {
            const int64_t e = blk * kDepthBlock + row;
            const char *src =
                (const char *)p.vd_nat + layer_row(e < TL ? e : TL - 1) * (D * 2) + chunk;
            __builtin_amdgcn_global_load_lds((const void *)src, dst, 16, 0, 0);
          } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vd_rsrc, dst, 16,
                                                     (uint32_t)(row * 256 + chunk),
                                                     (uint32_t)(blk * kDepthBlock * 256), 0, 0);
          }
        }
      };
      u32x4 kd[8];
      load_k(blk_lo, kd);
      for (int64_t blk = blk_lo; blk < blk_hi; ++blk) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slot's last reads are done
        load_v(blk);
        floatx16 sd[1];
        floatx16 sd2[2] = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          sd2[ks & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, kd[ks]), qb[ks], sd2[ks & 1], 0, 0, 0);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sd[0][rr] = sd2[0][rr] + sd2[1][rr];
        const bool more = blk + 1 < blk_hi;
        if (more) load_k(blk + 1, kd);
        const int64_t rel64 = blk * kDepthBlock + 4 * lh - my_lo;
        const int rel = (int)(rel64 < -64 ? -64 : (rel64 > L ? L : rel64));
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if ((unsigned)(8 * (rr >> 2) + (rr & 3) + rel) >= (unsigned)L) sd[0][rr] = -INFINITY;
        bf16x8 pb[2];
        softmax_update<1>(st, sd, p.scale_log2, pb);
        // the Vd rows have landed (the next block's Kd loads may still be in flight)
        if (more) __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
        else wait_vmem();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            st.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.colfrag(slot, 4 * nb + kk),
                                                                 pb[kk], st.acc[nb], 0, 0, 0);
      }
    }
  };
  auto depth_part = [&]() {
    if constexpr (HAS_DEPTH) {
      const int64_t L = p.L;
      const int64_t wt_lo = t0 + (rw * 32) / G;
      int64_t wt_hi = t0 + (rw * 32 + 31) / G + 1;  // one past the wave's last token
      if (wt_hi > t0 + TQ) wt_hi = t0 + TQ;
      if (wt_hi > T) wt_hi = T;
      if (L > 0 && wt_lo < wt_hi) {
        // the masked-scan mode (the Flash-compatible layout: depth entries as one causal
        // key range, each row masked to its own token's entries) starts at entry 0
        const int64_t blk_lo = SCAN ? 0 : (wt_lo * L) / kDepthBlock;
        const int64_t blk_hi = (wt_hi * L + kDepthBlock - 1) / kDepthBlock;
        const int64_t my_lo = tok * L;  // this row's entries: [my_lo, my_lo + L)
        if constexpr (NATURAL) {
          depth_natural(blk_lo, blk_hi, my_lo);
          return;
        }
        // packed cache: the blocks of the token groups that hold this wave's
        // tokens, all entry groups of each (a contiguous run of blocks)
        const int64_t ne = (L + kGroupEntries - 1) / kGroupEntries;
        const int64_t pblk_lo = (wt_lo / kGroupTokens) * ne;
        const int64_t pblk_hi = ((wt_hi - 1) / kGroupTokens + 1) * ne;
        const char *pk = (const char *)p.packed + bh * p.nblk * kPackedBlockBytes + lane * 16;
        // a key-split pair of waves takes alternate blocks
        constexpr int KSTEP = KS ? 2 : 1;
        const int64_t pblk_first = pblk_lo + kh;
        u32x4 kd[8], vd[8];
        if (pblk_first < pblk_hi) {
#pragma unroll
          for (int ks = 0; ks < 8; ++ks)
            kd[ks] = *(const u32x4 *)(pk + pblk_first * kPackedBlockBytes + ks * 1024);
        }
        // token group, entry group of blk
        int64_t tg = wt_lo / kGroupTokens + (kh < ne ? 0 : 1), eg = kh < ne ? kh : kh - ne;
        for (int64_t blk = pblk_first; blk < pblk_hi; blk += KSTEP) {
          const char *kp = pk + blk * kPackedBlockBytes;
#pragma unroll
          for (int j = 0; j < 8; ++j) vd[j] = *(const u32x4 *)(kp + BLK_HALF + j * 1024);
          floatx16 sd[1];
          // two independent MFMA chains over the even and odd k-steps
          floatx16 sd2[2] = {};
#pragma unroll
          for (int ks = 0; ks < 8; ++ks)
            sd2[ks & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, kd[ks]), qb[ks], sd2[ks & 1], 0, 0, 0);
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) sd[0][rr] = sd2[0][rr] + sd2[1][rr];
          if (blk + KSTEP < pblk_hi) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
              kd[ks] = *(const u32x4 *)(kp + KSTEP * kPackedBlockBytes + ks * 1024);
          }
          // register rr holds block row 8*(rr/4) + 4*lh + rr%4: token rr%8 of
          // the group and entry 4*eg + 2*(rr/8) + lh.  Of a row's 16 scores only
          // registers tpos and tpos + 8 (its own token tpos; entries ebase and
          // ebase + 2) can count, and each only for an entry below L; a row of
          // another group, or an idle row, keeps none.
          const int64_t tpos64 = tok - kGroupTokens * tg;
          const int tpos = (int)(tpos64 < 0 || tpos64 >= kGroupTokens ? -1 : tpos64);
          const int64_t ebase = kGroupEntries * eg + lh;
          float sa = sd[0][0], sb = sd[0][8];
#pragma unroll
          for (int r = 1; r < kGroupTokens; ++r) {
            sa = tpos == r ? sd[0][r] : sa;
            sb = tpos == r ? sd[0][r + 8] : sb;
          }
          sa = tpos >= 0 && ebase < L ? sa : -INFINITY;
          sb = tpos >= 0 && ebase + 2 < L ? sb : -INFINITY;
          eg += KSTEP;
          while (eg >= ne) {
            eg -= ne;
            ++tg;
          }
          // a row's L entries span ceil(L/4) blocks: take each block's max, so
          // that a dominant entry in a later block still gets weight 1 exactly
          bf16x8 pb[2];
          softmax_update_pair(st, sa, sb, tpos, p.scale_log2, pb);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              st.acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, vd[nb * 2 + kk]), pb[kk], st.acc[nb], 0, 0, 0);
        }
      }
    }
  };
  const bool depth_first = HAS_DEPTH && (!HAS_SEQ || (blockIdx.x & 1));
  MODA_TRACE_DECL
  if (depth_first) {
    depth_part();
    // the natural-layout depth loop used the tile buffers as per-wave slots
    if constexpr (NATURAL && HAS_SEQ) __syncthreads();
  }

  if constexpr (HAS_SEQ) {
    // ---------------- sequence part
    const int64_t tok_end = (t0 + TQ < T) ? t0 + TQ : T;
    const int n_kt = (int)((tok_end + NKEY - 1) / NKEY);
    const int64_t wave_tok_lo = t0 + (rw * 32) / G;

    // direct loads: instruction i of this wave fills tile rows 16*wave + 4i .. +3.
    // Buffer descriptors cover one (b, kv head) of K and of V; the tile offset
    // goes in the scalar offset, the lane's row/chunk in the vector offset.
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)p.k + bh * T * (D * 2)), (short)0, (int)(T * (D * 2)), 0x00020000);
    const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)p.v + bh * T * (D * 2)), (short)0, (int)(T * (D * 2)), 0x00020000);
    const int dma_row = DMA_ROWS * wave + (lane >> 4);  // + 4i
    uint32_t dk_off[DMA_INSTR], dv_off[DMA_INSTR];
#pragma unroll
    for (int i = 0; i < DMA_INSTR; ++i) {
      const int row = dma_row + 4 * i;
      dk_off[i] = (uint32_t)(row * 256 + 16 * ((lane & 15) ^ (row & 15)));
      dv_off[i] = (uint32_t)(row * 256 + 16 * ((lane & 15) ^ (4 * (row & 3))));
    }
    auto dma = [&](__amdgpu_buffer_rsrc_t rsrc, char *lds, uint32_t voff, uint32_t soff) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds,
                                               16, voff, soff, 0, 0);
    };
    // instruction q of this wave's 2*DMA_INSTR loads of tile kt: q < DMA_INSTR
    // loads K rows, the rest V rows.  Rows at or past T fall outside the descriptor's range and read as
    // zeros, which every mask removes.
    auto dma_one = [&](int q, int kt, char *k_dst, char *v_dst) {
      const uint32_t soff = (uint32_t)kt * TILE_BYTES;
      const int i = q % DMA_INSTR;
      if (q < DMA_INSTR) dma(k_rsrc, k_dst + wave * DMA_ROWS * 256 + i * 1024, dk_off[i], soff);
      else dma(v_rsrc, v_dst + wave * DMA_ROWS * 256 + i * 1024, dv_off[i], soff);
    };
    // MFMA operand reads.  K: row 32*kb2 + li, chunk 8*lh + ks, in slot
    // (8*lh + ks) ^ (li % 16) = (8*lh ^ (li & 8)) + (ks ^ (li & 7)).
    const int k_row = li * 256 + 16 * ((8 * lh) ^ (li & 8));
    const int k_x = li & 7;
    // V (transpose reads): lane group lg = lane/16 and lq = lane%16 read key row
    // 16*kk + 8*hi + 4*(lg/2) + lq/4, dims 32*nb + 16*(lg%2) + 4*(lq%4) .. +3.
    const int lg = lane >> 4, lq = lane & 15;
    int vaddr[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      vaddr[nb] = (4 * (lg >> 1) + (lq >> 2)) * 256 +
                  16 * (4 * (nb ^ (lq >> 2)) + 2 * (lg & 1) + ((lq & 3) >> 1)) + 8 * (lq & 1);

    auto kfrag = [&](const char *kb, int i) {  // i = 2*ks + kb2
      return *(const bf16x8 *)(kb + k_row + 16 * ((i >> 1) ^ k_x) + (i & 1) * 32 * 256);
    };
    auto vfrag = [&](const char *vb, int i) {  // i = 4*nb + kk
      const char *vp = vb + vaddr[i >> 2] + 16 * (i & 3) * 256;
      const shortx4 lo = lds_read_tr(vp);
      const shortx4 hi = lds_read_tr(vp + 8 * 256);
      return __builtin_bit_cast(
          bf16x8, (u32x4){__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
    };
    auto mask = [&](floatx16 (&s)[NKB], int kt) {
      // key offset within the tile of register rr of block kb2: 32*kb2 + 8*(rr/4) + 4*lh + rr%4
      const int lim = (int)max((int64_t)-8, min((int64_t)64, tok - (int64_t)kt * NKEY - 4 * lh));
#pragma unroll
      for (int b2 = 0; b2 < NKB; ++b2)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (32 * (b2 + kh) + 8 * (rr >> 2) + (rr & 3) > lim) s[b2][rr] = -INFINITY;
    };

    // start from zeroed buffers: loads of rows past T may leave LDS untouched
    for (int o = tid * 16; o < TILE_BYTES; o += 64 * NWAVE * 16) {
      *(u32x4 *)(k_lds0 + o) = u32x4{0, 0, 0, 0};
      *(u32x4 *)(k_lds1 + o) = u32x4{0, 0, 0, 0};
      *(u32x4 *)(v_lds0 + o) = u32x4{0, 0, 0, 0};
      *(u32x4 *)(v_lds1 + o) = u32x4{0, 0, 0, 0};
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2 * DMA_INSTR; ++q) dma_one(q, 0, k_lds0, v_lds0);
    wait_vmem();
    __syncthreads();
    MODA_TRACE(0);  // prologue

    // iteration j with buffer parity P = j % 2: loads tile j+1 into the other
    // buffers (last read in iteration j-1), computes tile j
    auto body = [&](int j, auto parity, auto masked) {
      constexpr int P = decltype(parity)::value;
      const char *const k_rd = P ? k_lds1 : k_lds0;
      const char *const v_rd = P ? v_lds1 : v_lds0;
      char *const k_wr = P ? k_lds0 : k_lds1;
      char *const v_wr = P ? v_lds0 : v_lds1;
      MODA_TRACE(1);  // (loads are issued inside the QK^T sequence)
      // S^T = K Q^T: the two 32-key chains alternate, K fragments are read four
      // MFMAs ahead and the eight loads of tile j+1 are spread between the
      // MFMAs; sched_barrier fences keep this order.
      // (key split: this wave's 32-key block kh only, 8 MFMAs)
      constexpr int NQK = 8 * NKB;
      // fragment i = 2*ks + kb2 of kfrag for MFMA number n
      auto qk_frag = [&](int n) { return KS ? 2 * n + kh : n; };
      floatx16 s[NKB];
      {
        bf16x8 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = kfrag(k_rd, qk_frag(i));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
          const int ks = KS ? i : i >> 1, kb2 = KS ? 0 : i & 1;
          const floatx16 c = ks == 0 ? (floatx16){} : s[kb2];
          s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i & 3], qb[ks], c, 0, 0, 0);
          if (i + 4 < NQK) a[i & 3] = kfrag(k_rd, qk_frag(i + 4));
          if (i % (NQK / (2 * DMA_INSTR)) == 0) dma_one(i / (NQK / (2 * DMA_INSTR)), j + 1, k_wr, v_wr);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      MODA_TRACE(2);  // QK^T
      if constexpr (decltype(masked)::value) mask(s, j);
      bf16x8 pb[2 * NKB];
      softmax_update<NKB>(st, s, sc, pb);
      MODA_TRACE(3);  // mask + softmax
      // O^T += V^T P^T: V fragments (two transpose reads each) three MFMAs ahead
      // (key split: the two 16-key steps 2kh, 2kh+1 of this wave's block, 8 MFMAs)
      {
        constexpr int NPV = 8 * NKB;
        auto pv_frag = [&](int n) {  // vfrag index 4*nb + kk of MFMA number n
          const int f = pv_order(n);
          return KS ? 4 * (f >> 2) + 2 * kh + (f & 3) : f;
        };
        bf16x8 a[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) a[i] = vfrag(v_rd, pv_frag(i));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          const int f = pv_order(i);
          st.acc[f >> 2] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % 3], pb[f & 3], st.acc[f >> 2], 0, 0, 0);
          if (i + 3 < NPV) a[i % 3] = vfrag(v_rd, pv_frag(i + 3));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      MODA_TRACE(4);  // PV
      wait_vmem();
      MODA_TRACE(5);  // wait for this wave's loads
      __syncthreads();
      MODA_TRACE(6);  // barrier
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // key tiles [0, n_nm) lie entirely at or before this wave's first token
    const int n_nm = (int)min((int64_t)n_kt, (wave_tok_lo + 1) / NKEY);
    int j = 0;
    for (; j + 1 < n_nm; j += 2) {
      body(j, I0{}, std::false_type{});
      body(j + 1, I1{}, std::false_type{});
    }
    for (; j < n_kt; ++j) {
      const bool mk = j >= n_nm;
      if (j & 1) {
        if (mk) body(j, I1{}, std::true_type{});
        else body(j, I1{}, std::false_type{});
      } else {
        if (mk) body(j, I0{}, std::true_type{});
        else body(j, I0{}, std::false_type{});
      }
    }
  }

  if (!depth_first) depth_part();
  MODA_TRACE(7);  // depth part
  MODA_TRACE_FLUSH;
  if constexpr (KS) {
    // Merge each pair's two states: wave 2i+1 leaves (m, l, O^T) in LDS (the
    // tile buffers, free after the key loop's last barrier; 16 KiB per pair,
    // register-major so that a lane's reads and writes are consecutive across
    // lanes), wave 2i rescales both to the larger reference and adds them.
    __shared__ float ml_s[4][2][64];
    float *const xs = (float *)(rw == 0 ? k_lds0 : rw == 1 ? k_lds1 : rw == 2 ? v_lds0 : v_lds1);
    __syncthreads();
    if (kh == 1) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) xs[(16 * nb + rr) * 64 + lane] = st.acc[nb][rr];
      ml_s[rw][0][lane] = st.m;
      ml_s[rw][1][lane] = st.lsum;
    }
    __syncthreads();
    if (kh == 0) {
      const float m1 = ml_s[rw][0][lane], l1 = ml_s[rw][1][lane];
      const float mm = fmaxf(st.m, m1);
      // a half that saw no entry of the row has m = -inf and weight 0
      const float a0 = st.m == -INFINITY ? 0.f : fast_exp2(st.m - mm);
      const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
      st.m = mm;
      st.lsum = st.lsum * a0 + l1 * a1;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          st.acc[nb][rr] = st.acc[nb][rr] * a0 + xs[(16 * nb + rr) * 64 + lane] * a1;
    }
  }
  // ---------------- epilogue: the single normalisation
  const float ltot = pair_sum(st.lsum);
  if (row_ok && kh == 0) {
    const float inv = 1.0f / ltot;
    __bf16 *orow = (__bf16 *)p.out + ((b * p.Hq + head) * T + tok) * D;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 o;
        o[0] = cvt_bf16x2(st.acc[nb][4 * g + 0] * inv, st.acc[nb][4 * g + 1] * inv);
        o[1] = cvt_bf16x2(st.acc[nb][4 * g + 2] * inv, st.acc[nb][4 * g + 3] * inv);
        *(u32x2 *)(orow + 32 * nb + 8 * g + 4 * lh) = o;
      }
    if (p.lse && lh == 0)
      p.lse[(b * p.Hq + head) * T + tok] = (st.m + __log2f(ltot)) * 0.69314718055994531f;
  }
}

// Depth repack into MFMA operand order.  One workgroup per block of one
// (b, kv head): 8 tokens x 4 entries, block tg * ceil(L/4) + eg holding tokens
// 8tg .. 8tg+7 and entries 4eg .. 4eg+3, block row r = (token tok_of_row(r),
// entry ent_of_row(r)):
//   K half: 8 k-steps x 64 lanes x 16 B; lane l of k-step ks holds row
//           l % 32, dims 64*(l/32) + 8*ks .. +7   (the A operand of S^T = K Q^T)
//   V half: 4 dim blocks x 2 k-steps x 64 lanes x 16 B; lane l of (nb, kk)
//           holds dim 32*nb + l%32 of rows 16kk + 8*(j/4) + 4*(l/32) + j%4,
//           j = 0..7, i.e. of entry 4eg + 2kk + l/32 of tokens 0..7 of the
//           group (the A operand of O^T += V^T P^T)
// Rows of tokens past T or entries past L are zero.
constexpr int PK_ROW = D * 2 + 16;  // LDS row stride (bytes) while repacking

__global__ __launch_bounds__(256) void moda_pack_mfma(PackArgs p) {
  __shared__ __attribute__((aligned(16))) char ks_lds[kDepthBlock * PK_ROW];
  __shared__ __attribute__((aligned(16))) char vs_lds[kDepthBlock * PK_ROW];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t blk = blockIdx.x;
  const int64_t TL = p.T * p.L;
  const int64_t ne = (p.L + kGroupEntries - 1) / kGroupEntries;  // entry groups per token
  const int64_t tg = blk / ne, eg = blk - tg * ne;              // token group, entry group
  const __bf16 *kd = (const __bf16 *)p.kd + bh * TL * D;
  const __bf16 *vd = (const __bf16 *)p.vd + bh * TL * D;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;  // 512 chunks of 16 B per half
    const int row = c >> 4, ch = c & 15;
    const int64_t t = kGroupTokens * tg + tok_of_row(row);
    const int64_t e = kGroupEntries * eg + ent_of_row(row);
    u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (t < p.T && e < p.L) {  // padding rows (past T, or past L) stay zero
      kv = *(const u32x4 *)(kd + (t * p.L + e) * D + ch * 8);
      vv = *(const u32x4 *)(vd + (t * p.L + e) * D + ch * 8);
    }
    *(u32x4 *)(ks_lds + row * PK_ROW + ch * 16) = kv;
    *(u32x4 *)(vs_lds + row * PK_ROW + ch * 16) = vv;
  }
  __syncthreads();
  char *dst = (char *)p.packed + (bh * p.nblk + blk) * kPackedBlockBytes;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int o = tid + 256 * i;  // output chunk
    const int ks = o >> 6, l = o & 63;
    const u32x4 kv = *(const u32x4 *)(ks_lds + (l & 31) * PK_ROW + (64 * (l >> 5) + 8 * ks) * 2);
    *(u32x4 *)(dst + o * 16) = kv;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int o = tid + 256 * i;
    const int nbkk = o >> 6, l = o & 63;
    const int nb = nbkk >> 1, kk = nbkk & 1;
    const int n = 32 * nb + (l & 31), hh = l >> 5;
    uint32_t h16[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ent = 16 * kk + 8 * (j >> 2) + 4 * hh + (j & 3);
      h16[j] = *(const uint16_t *)(vs_lds + ent * PK_ROW + n * 2);
    }
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = h16[2 * j] | (h16[2 * j + 1] << 16);
    *(u32x4 *)(dst + BLK_HALF + o * 16) = w;
  }
}

// ---------------------------------------------------------------------------
// Generic VALU path (fp32, or bf16 with d in {32, 64}, with G above 128).
// One wave per query row.  Each lane keeps its own online-softmax state over
// a strided subset of the row's entries; the 64 states are merged at the end.
// Depth is read from the generic packed layout: [Kd natural | Vd natural].
// ---------------------------------------------------------------------------
template <typename E>
__device__ __forceinline__ float load_elem(const E *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}
template <typename E>
__device__ __forceinline__ void store_elem(E *p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float *p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t *p, int64_t i, float v) {
  p[i] = (uint16_t)float_to_bf16_bits(v);
}

template <typename E, int DG, bool HAS_DEPTH, bool HAS_SEQ>
__global__ __launch_bounds__(64) void moda_fwd_generic(FwdArgs p) {
  __shared__ float qs[DG];
  __shared__ float red[64][DG + 1];
  __shared__ float lred[64];
  __shared__ float mred[64];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;  // (b, h, t) flattened
  const int64_t T = p.T;
  const int64_t t = row % T, h = (row / T) % p.Hq, b = row / (T * p.Hq);
  const int64_t G = p.Hq / p.Hkv;
  const int64_t bh = b * p.Hkv + h / G;
  const E *q = (const E *)p.q + row * DG;
  const E *k = (const E *)p.k + bh * T * DG;
  const E *v = (const E *)p.v + bh * T * DG;
  for (int n = lane; n < DG; n += 64) qs[n] = load_elem(q, n);
  __syncthreads();

  float m = -INFINITY, l = 0.f, o[DG];
#pragma unroll
  for (int n = 0; n < DG; ++n) o[n] = 0.f;

  auto visit = [&](const E *kr, const E *vr) {
    float s = 0.f;
#pragma unroll
    for (int n = 0; n < DG; ++n) s = fmaf(qs[n], load_elem(kr, n), s);
    const float xv = s * p.scale_log2;
    if (xv > m) {
      const float a = fast_exp2(m - xv);
      l *= a;
#pragma unroll
      for (int n = 0; n < DG; ++n) o[n] *= a;
      m = xv;
    }
    const float pw = fast_exp2(xv - m);
    l += pw;
#pragma unroll
    for (int n = 0; n < DG; ++n) o[n] = fmaf(pw, load_elem(vr, n), o[n]);
  };

  if (HAS_SEQ)
    for (int64_t j = lane; j <= t; j += 64) visit(k + j * DG, v + j * DG);
  if (HAS_DEPTH && p.L > 0) {
    const int64_t L = p.L;
    const int64_t half = p.B * p.Hkv * T * L * DG;  // elements of Kd
    const E *kd = (const E *)p.packed + (bh * T + t) * L * DG;
    const E *vd = (const E *)p.packed + half + (bh * T + t) * L * DG;
    for (int64_t i = lane; i < L; i += 64) visit(kd + i * DG, vd + i * DG);
  }

  // merge the 64 lane states
  mred[lane] = m;
  __syncthreads();
  float mall = -INFINITY;
  for (int i = 0; i < 64; ++i) mall = fmaxf(mall, mred[i]);
  const float sc = (m == -INFINITY) ? 0.f : fast_exp2(m - mall);
  lred[lane] = l * sc;
#pragma unroll
  for (int n = 0; n < DG; ++n) red[lane][n] = o[n] * sc;
  __syncthreads();
  float lall = 0.f;
  for (int i = 0; i < 64; ++i) lall += lred[i];
  E *out = (E *)p.out + row * DG;
  for (int n = lane; n < DG; n += 64) {
    float acc = 0.f;
    for (int i = 0; i < 64; ++i) acc += red[i][n];
    store_elem(out, n, acc / lall);
  }
  if (p.lse && lane == 0) p.lse[row] = (mall + log2f(lall)) * 0.69314718055994531f;
}

// Generic packed layout = Kd then Vd, both in their natural layout.
__global__ __launch_bounds__(256) void moda_copy_generic(const u32x4 *kd, const u32x4 *vd,
                                                         u32x4 *dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    dst[i] = kd[i];
    dst[n16 + i] = vd[i];
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int NW>
static hipError_t launch_fwd_nw(const FwdArgs &a, int G, hipStream_t s) {
  if (G < 1 || G > 32 * NW) return hipErrorInvalidValue;
  const int64_t TQ = 32 * NW / G;
  const int64_t ntiles = (a.T + TQ - 1) / TQ;
  const dim3 grid((uint32_t)(ntiles * a.B * a.Hkv)), block(64 * NW);
  constexpr int R = 32 * NW;
  if (a.kd_nat && a.depth_layers)
    hipLaunchKernelGGL((moda_fwd_mfma<kModeModaLayers, NW, R>), grid, block, 0, s, a);
  else if (a.kd_nat && a.depth_scan)
    hipLaunchKernelGGL((moda_fwd_mfma<kModeModaScan, NW, R>), grid, block, 0, s, a);
  else if (a.kd_nat)
    hipLaunchKernelGGL((moda_fwd_mfma<kModeModaNatural, NW, R>), grid, block, 0, s, a);
  else if (!a.has_seq)
    hipLaunchKernelGGL((moda_fwd_mfma<kModeDepth, NW, R>), grid, block, 0, s, a);
  else if (a.has_depth)
    hipLaunchKernelGGL((moda_fwd_mfma<kModeModa, NW, R>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((moda_fwd_mfma<kModeCausal, NW, R>), grid, block, 0, s, a);
  return hipGetLastError();
}

// The key-split form: 8 waves on 128-row tiles (causal and packed MoDA modes;
// the other modes take the 4-wave kernel on the same tiles).
static hipError_t launch_fwd_ks(const FwdArgs &a, int G, hipStream_t s) {
  if (a.kd_nat || !a.has_seq) return launch_fwd_nw<4>(a, G, s);
  if (G < 1 || G > 128) return hipErrorInvalidValue;
  const int64_t TQ = 128 / G;
  const int64_t ntiles = (a.T + TQ - 1) / TQ;
  const dim3 grid((uint32_t)(ntiles * a.B * a.Hkv)), block(64 * 8);
  if (a.has_depth)
    hipLaunchKernelGGL((moda_fwd_mfma<kModeModa, 8, 128>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((moda_fwd_mfma<kModeCausal, 8, 128>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(const FwdArgs &a, int G, int waves, hipStream_t s) {
  if (waves == 4) return launch_fwd_nw<4>(a, G, s);
  if (waves == 8) return launch_fwd_nw<8>(a, G, s);
  if (waves == kFwdKeySplit) return launch_fwd_ks(a, G, s);
  return hipErrorInvalidValue;
}

hipError_t launch_pack_mfma(const PackArgs &a, hipStream_t s) {
  dim3 grid((uint32_t)a.nblk, (uint32_t)(a.B * a.Hkv));
  hipLaunchKernelGGL(moda_pack_mfma, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename E, int DG>
static hipError_t launch_generic_d(const FwdArgs &a, hipStream_t s) {
  const int64_t rows = a.B * a.Hq * a.T;
  if (!a.has_seq)
    hipLaunchKernelGGL((moda_fwd_generic<E, DG, true, false>), dim3((uint32_t)rows), dim3(64), 0,
                       s, a);
  else if (a.has_depth)
    hipLaunchKernelGGL((moda_fwd_generic<E, DG, true, true>), dim3((uint32_t)rows), dim3(64), 0,
                       s, a);
  else
    hipLaunchKernelGGL((moda_fwd_generic<E, DG, false, true>), dim3((uint32_t)rows), dim3(64), 0,
                       s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_generic(const FwdArgs &a, bool bf16, hipStream_t s) {
  if (bf16) {
    switch (a.d) {
      case 32: return launch_generic_d<uint16_t, 32>(a, s);
      case 64: return launch_generic_d<uint16_t, 64>(a, s);
      case 128: return launch_generic_d<uint16_t, 128>(a, s);
    }
  } else {
    switch (a.d) {
      case 32: return launch_generic_d<float, 32>(a, s);
      case 64: return launch_generic_d<float, 64>(a, s);
      case 128: return launch_generic_d<float, 128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pack_generic(const PackArgs &a, bool bf16, hipStream_t s) {
  const int64_t bytes = a.B * a.Hkv * a.T * a.L * a.d * (bf16 ? 2 : 4);
  const int64_t n16 = bytes / 16;  // d * es is a multiple of 16 for every supported d
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(moda_copy_generic, dim3((uint32_t)blocks), dim3(256), 0, s,
                     (const u32x4 *)a.kd, (const u32x4 *)a.vd, (u32x4 *)a.packed, n16);
  return hipGetLastError();
}

}  // namespace moda
