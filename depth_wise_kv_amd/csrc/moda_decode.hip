// HIP kernels of the MoDA decode step for gfx950 (MI355X): bf16, head dim 128.
//
// One new token per sequence: its G query heads per KV head attend, under
// one softmax scaled by 1/sqrt(d), over the whole KV cache (every cached key
// is at or before the new token) and over the new token's own L depth
// entries (hyper.ai page on arXiv 2603.15619, section "Mixture-of-Depths
// Attention (MoDA)").  This is the last query row of the forward.
//
// The cache is read once, split over many workgroups for bandwidth:
//   moda_decode_part   a workgroup takes one part of one (b, kv head)'s
//                      entries (the cache's, then the depth entries, as one
//                      list of 32-entry blocks split into nsplit even parts).
//                      Each of its W waves (8; 4 where 8-wave parts would
//                      leave half the chip or more idle) walks every W-th
//                      block of the part; the waves then merge their softmax
//                      states through LDS and the workgroup leaves one partial
//                      state (unnormalised O, reference max, weight sum) per
//                      row.
//   moda_decode_merge  merges the partial states of each query row (one wave
//                      per 8 of them, up to 16) and normalises once.  With one part per (b, kv head) (large
//                      batches, short caches) the part kernel normalises and
//                      writes the result itself and the merge is not launched.
// Per block: K rows straight into MFMA operand registers (16 bytes of a row
// per lane, the next block's already in flight), V rows into the wave's
// 8 KiB of LDS, column-swizzled, read transposed; S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with a lane owning a query row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "moda_device.h"
#include "moda_internal.h"

namespace moda {

constexpr int DEC_D = kMfmaD;  // 128
constexpr int MERGE_WAVES = 16;
constexpr int MERGE_UNROLL = 8;

template <int DEC_WAVES>
__global__ __launch_bounds__(64 * DEC_WAVES) void moda_decode_part(DecArgs p) {
  __shared__ __attribute__((aligned(1024))) char slots[DEC_WAVES][32 * 256];
  __shared__ float m_s[DEC_WAVES][32], l_s[DEC_WAVES][32];
  const int G = (int)(p.Hq / p.Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, lh = lane >> 5;
  const TileFrags fr(lane);

  const int64_t BH = p.B * p.Hkv;
  const int64_t bh = blockIdx.x % BH;
  const int64_t part = blockIdx.x / BH;
  const int64_t b = bh / p.Hkv, hkv = bh % p.Hkv;

  // this lane's query row: head hkv*G + li (lanes past G compute on zeros)
  const bool row_ok = li < G;
  const int64_t qrow = b * p.Hq + hkv * G + (row_ok ? li : 0);
  bf16x8 qb[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const u32x4 u = row_ok ? *(const u32x4 *)((const __bf16 *)p.q + qrow * DEC_D + 64 * lh + 8 * ks)
                           : u32x4{0, 0, 0, 0};
    qb[ks] = __builtin_bit_cast(bf16x8, u);
  }

  // The (b, kv head)'s entries as one list of 32-entry blocks: the cache's
  // nbc blocks, then the depth entries' blocks.  This part takes blocks
  // [j_lo, j_hi) of it; wave w takes every DEC_WAVES-th of those from j_lo + w.
  const int64_t nbc = (p.T + 31) / 32;
  // entries of this sequence's cache (the first n_c of its T slots)
  int64_t n_c = p.T;
  if (p.lens) {
    const int64_t len = p.lens[b];
    n_c = len < 0 ? 0 : (len > p.T ? p.T : len);
  }
  const int64_t jc_end = (n_c + 31) / 32;  // cache blocks [jc_end, nbc) hold no entry
  const int64_t nb = nbc + (p.L + 31) / 32;
  const int64_t j_lo = part * nb / p.nsplit, j_hi = (part + 1) * nb / p.nsplit;
  const __bf16 *kc = (const __bf16 *)p.k + bh * p.T * DEC_D;
  const __bf16 *kdp = (const __bf16 *)p.kd + bh * p.L * DEC_D;
  // (the V descriptor ends at the sequence's last entry: the rest of its slots
  // may hold anything, and a masked row must still read as finite zeros)
  const __amdgpu_buffer_rsrc_t vc_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const char *)p.v + bh * p.T * (DEC_D * 2)), (short)0, (int)(n_c * (DEC_D * 2)),
      0x00020000);
  const __amdgpu_buffer_rsrc_t vd_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const char *)p.vd + bh * p.L * (DEC_D * 2)), (short)0, (int)(p.L * (DEC_D * 2)),
      0x00020000);
  char *const slot = slots[wave];

  MfmaState st;
  st.m = -INFINITY;
  st.lsum = 0.f;
#pragma unroll
  for (int nb4 = 0; nb4 < 4; ++nb4)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) st.acc[nb4][rr] = 0.f;

  // K rows of block j as MFMA A operands: entry 32*j' + li of its source, dims
  // 64*lh + 8*ks.  A row past the source's last entry reads that entry instead
  // (its scores are masked below); the loads carry no per-lane condition, which
  // would put branches around them and make the compiler wait for them early.
  auto load_k = [&](int64_t j, u32x4 (&kd)[8]) {
    const bool dep = j >= nbc;
    const int64_t e = (dep ? j - nbc : j) * 32 + li;
    const int64_t n = dep ? p.L : n_c;  // >= 1 for every block visited
    const __bf16 *src = (dep ? kdp : kc) + (e < n ? e : n - 1) * DEC_D + 64 * lh;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kd[ks] = *(const u32x4 *)(src + 8 * ks);
  };
  // this wave's blocks: every DEC_WAVES-th from j_lo + wave, stepping over the
  // empty cache blocks, so that every block visited has an entry in lane 0
  auto skip_empty = [&](int64_t j) -> int64_t {
    return (j >= jc_end && j < nbc) ? j + (nbc - j + DEC_WAVES - 1) / DEC_WAVES * DEC_WAVES : j;
  };
  u32x4 kd[8];
  // One block: its V rows into the slot, S^T on the K rows in kd, then (but
  // for the wave's last block) the next block's K rows into kd, the softmax,
  // the PV products.  The V loads go out before the next K loads (loads
  // complete in order), so the PV products wait for V alone; the last block is
  // a separate copy without the K request, since behind a branch the compiler
  // would wait for those loads too before the V reads.
  auto block_step = [&](int64_t j, int64_t jn, auto prefetch) {
    const bool dep = j >= nbc;
    const int64_t e0 = (dep ? j - nbc : j) * 32;
    const int64_t n = dep ? p.L : n_c;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slot's last reads are done
    // V rows e0 .. e0+31 into the slot, column-swizzled (rows past the source read as zeros)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + (lane >> 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          dep ? vd_rsrc : vc_rsrc, (__attribute__((address_space(3))) void *)(slot + 4 * i * 256),
          16, (uint32_t)(row * 256 + 16 * ((lane & 15) ^ (4 * (row & 3)))), (uint32_t)(e0 * 256),
          0, 0);
    }
    // every V load is issued before the first MFMA waits for its K operands
    __builtin_amdgcn_sched_barrier(0);
    floatx16 sd[1];
    floatx16 sd2[2] = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      sd2[ks & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kd[ks]),
                                                            qb[ks], sd2[ks & 1], 0, 0, 0);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sd[0][rr] = sd2[0][rr] + sd2[1][rr];
    if constexpr (decltype(prefetch)::value) load_k(jn, kd);
    // register rr holds entry e0 + 8*(rr/4) + 4*lh + rr%4: entries past the source drop out
    const int64_t lim64 = n - e0 - 4 * lh;
    const int lim = (int)(lim64 > 64 ? 64 : lim64);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      if (8 * (rr >> 2) + (rr & 3) >= lim) sd[0][rr] = -INFINITY;
    bf16x8 pb[2];
    softmax_update<1>(st, sd, p.scale_log2, pb);
    // the V rows have landed (the next block's K loads may still be in flight)
    if constexpr (decltype(prefetch)::value) __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
    else wait_vmem();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int nb4 = 0; nb4 < 4; ++nb4)
        st.acc[nb4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.colfrag(slot, 4 * nb4 + kk),
                                                              pb[kk], st.acc[nb4], 0, 0, 0);
  };
  int64_t j = skip_empty(j_lo + wave);
  if (j < j_hi) {
    load_k(j, kd);
    for (int64_t jn = skip_empty(j + DEC_WAVES); jn < j_hi; j = jn, jn = skip_empty(j + DEC_WAVES))
      block_step(j, jn, std::true_type{});
    block_step(j, j, std::false_type{});
  }

  // Merge the 8 waves' states: a common reference max per row, then the
  // rescaled accumulators summed pairwise through LDS (the V slots, now free).
  if (lh == 0) m_s[wave][li] = st.m;
  __syncthreads();
  float m_row = m_s[0][li];
#pragma unroll
  for (int w = 1; w < DEC_WAVES; ++w) m_row = fmaxf(m_row, m_s[w][li]);
  const float alpha = st.m == -INFINITY ? 0.f : fast_exp2(st.m - m_row);
  const float l_wave = pair_sum(st.lsum) * alpha;
  if (lh == 0) l_s[wave][li] = l_wave;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) st.acc[nb][rr] *= alpha;
  // Only the lanes of the G real rows carry data; they move their 64
  // accumulators as 16 float4s per step (16 KiB regions, a lane's float4 i at
  // 64*i + lane, so a wave's store covers 1 KiB of consecutive banks).
  float4 *const red = (float4 *)&slots[0][0];
#pragma unroll
  for (int step = DEC_WAVES / 2; step >= 1; step >>= 1) {
    if (wave >= step && wave < 2 * step && row_ok) {
      float4 *r = red + (wave - step) * 1024 + lane;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        r[64 * i] = make_float4(st.acc[i >> 2][4 * (i & 3)], st.acc[i >> 2][4 * (i & 3) + 1],
                                st.acc[i >> 2][4 * (i & 3) + 2], st.acc[i >> 2][4 * (i & 3) + 3]);
    }
    __syncthreads();
    if (wave < step && row_ok) {
      const float4 *r = red + wave * 1024 + lane;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 x = r[64 * i];
        st.acc[i >> 2][4 * (i & 3)] += x.x;
        st.acc[i >> 2][4 * (i & 3) + 1] += x.y;
        st.acc[i >> 2][4 * (i & 3) + 2] += x.z;
        st.acc[i >> 2][4 * (i & 3) + 3] += x.w;
      }
    }
    __syncthreads();
  }

  // wave 0 writes the workgroup's state of each row: O (unnormalised), max, sum
  if (wave == 0 && row_ok) {
    float l_row = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) l_row += l_s[w][li];
    if (p.nsplit == 1) {
      // the only part: normalise once and write O and LSE here, exactly as the
      // merge would from this one state (no merge launch follows)
      const float inv = m_row == -INFINITY ? 0.f : 1.0f / l_row;
      __bf16 *const o = (__bf16 *)p.out + qrow * DEC_D;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 w;
          w[0] = cvt_bf16x2(st.acc[nb][4 * q4] * inv, st.acc[nb][4 * q4 + 1] * inv);
          w[1] = cvt_bf16x2(st.acc[nb][4 * q4 + 2] * inv, st.acc[nb][4 * q4 + 3] * inv);
          *(u32x2 *)(o + 32 * nb + 8 * q4 + 4 * lh) = w;
        }
      if (p.lse && lh == 0)
        p.lse[qrow] = m_row == -INFINITY ? -INFINITY : (m_row + __log2f(l_row)) * 0.69314718055994531f;
      return;
    }
    float *rec = p.ws + (qrow * p.nsplit + part) * kDecodeRecord;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(float4 *)(rec + 32 * nb + 8 * q4 + 4 * lh) =
            make_float4(st.acc[nb][4 * q4], st.acc[nb][4 * q4 + 1], st.acc[nb][4 * q4 + 2],
                        st.acc[nb][4 * q4 + 3]);
    if (lh == 0) {
      rec[DEC_D] = m_row;
      rec[DEC_D + 1] = l_row;
    }
  }
}

// One workgroup per query row, of NW waves (one per MERGE_UNROLL records, a
// power of two up to MERGE_WAVES): each wave folds every NW-th partial state
// into a running (max, sum, O), its loads in flight together; the NW wave
// states merge in LDS, one normalisation.  NW depends on nsplit alone, so the
// order of the sums is fixed by the shape.
template <int NW>
__global__ __launch_bounds__(64 * NW) void moda_decode_merge(DecArgs p) {
  __shared__ float o_s[NW][DEC_D];
  __shared__ float m_s[NW], l_s[NW];
  const int64_t row = blockIdx.x;  // b * Hq + head
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int nw = NW;
  const int64_t n = p.nsplit;
  const float *rec = p.ws + row * n * kDecodeRecord;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int64_t base = wave; base < n; base += (int64_t)nw * MERGE_UNROLL) {
    float mi[MERGE_UNROLL], li[MERGE_UNROLL];
    float2 oi[MERGE_UNROLL];
#pragma unroll
    for (int u = 0; u < MERGE_UNROLL; ++u) {
      const int64_t idx = base + (int64_t)nw * u;
      const float *r = rec + (idx < n ? idx : 0) * kDecodeRecord;
      mi[u] = idx < n ? r[DEC_D] : -INFINITY;
      li[u] = r[DEC_D + 1];
      oi[u] = *(const float2 *)(r + 2 * lane);
    }
#pragma unroll
    for (int u = 0; u < MERGE_UNROLL; ++u) {
      if (mi[u] == -INFINITY) continue;  // past the end, or a state with no entry
      const float m_new = fmaxf(m, mi[u]);
      const float a = m == -INFINITY ? 0.f : fast_exp2(m - m_new);
      const float c = fast_exp2(mi[u] - m_new);
      l = l * a + li[u] * c;
      o0 = o0 * a + oi[u].x * c;
      o1 = o1 * a + oi[u].y * c;
      m = m_new;
    }
  }
  if (lane == 0) {
    m_s[wave] = m;
    l_s[wave] = l;
  }
  o_s[wave][2 * lane] = o0;
  o_s[wave][2 * lane + 1] = o1;
  __syncthreads();
  if (wave != 0) return;
  float M = m_s[0];
#pragma unroll
  for (int w = 1; w < nw; ++w) M = fmaxf(M, m_s[w]);
  float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
  for (int w = 0; w < nw; ++w) {
    if (m_s[w] == -INFINITY) continue;
    const float c = fast_exp2(m_s[w] - M);
    L += l_s[w] * c;
    O0 += o_s[w][2 * lane] * c;
    O1 += o_s[w][2 * lane + 1] * c;
  }
  // a row with no entry (empty cache and L = 0) gets O = 0 and LSE = -inf
  const float inv = M == -INFINITY ? 0.f : 1.0f / L;
  *(uint32_t *)((__bf16 *)p.out + row * DEC_D + 2 * lane) = cvt_bf16x2(O0 * inv, O1 * inv);
  if (p.lse && lane == 0)
    p.lse[row] = M == -INFINITY ? -INFINITY : (M + __log2f(L)) * 0.69314718055994531f;
}

// Device scratch of the allocation-free decode (moda_decode_noalloc): its
// per-part partial states live here instead of in a caller workspace.  Every
// GPU the library runs on holds one copy for the life of the process; all
// moda_decode_noalloc calls on a GPU share it, so calls that overlap in time on
// one GPU race.  The decode writes every record before reading it, so nothing
// in it needs clearing between calls.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

// Device address of `scratch` on the current device.  Host code may not use
// the array's name as a device address (it is a host-side stand-in), so the
// address is looked up once per device, with that device current, and kept.
hipError_t decode_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecArgs &a, hipStream_t s) {
  const int64_t BH = a.B * a.Hkv;
  if (a.waves == 4)
    hipLaunchKernelGGL(moda_decode_part<4>, dim3((uint32_t)(BH * a.nsplit)), dim3(64 * 4), 0, s, a);
  else
    hipLaunchKernelGGL(moda_decode_part<8>, dim3((uint32_t)(BH * a.nsplit)), dim3(64 * 8), 0, s, a);
  // with one part per (b, kv head) the part kernel writes the result itself
  if (a.nsplit > 1) {
    // one merge wave per MERGE_UNROLL records, a power of two up to MERGE_WAVES
    int nw = 1;
    while (nw < MERGE_WAVES && (int64_t)nw * MERGE_UNROLL < a.nsplit) nw *= 2;
    const dim3 grid((uint32_t)(a.B * a.Hq));
    switch (nw) {
      case 1: hipLaunchKernelGGL(moda_decode_merge<1>, grid, dim3(64), 0, s, a); break;
      case 2: hipLaunchKernelGGL(moda_decode_merge<2>, grid, dim3(128), 0, s, a); break;
      case 4: hipLaunchKernelGGL(moda_decode_merge<4>, grid, dim3(256), 0, s, a); break;
      case 8: hipLaunchKernelGGL(moda_decode_merge<8>, grid, dim3(512), 0, s, a); break;
      default: hipLaunchKernelGGL(moda_decode_merge<16>, grid, dim3(1024), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace moda
