// HIP kernels of the depth-stream write step for gfx950 (MI355X): a layer's
// K and V for every token join the token's depth stream as entries
// [first, first + n) (hyper.ai page on arXiv 2603.15619, section "Depth
// stream mechanism": each layer appends what it wrote to the stream the later
// layers read; FFN layers add a light KV projection, so a layer may write
// two entries).  The cache is written in place, in the layout the forward
// reads, instead of repacking the whole stream after every layer.
//
//   moda_append_mfma     bf16, d = 128: the packed block layout of the repack
//                        (blocks of 8 tokens x 4 entries; K half in MFMA
//                        A-operand order, V half with each 16-byte chunk
//                        holding one entry's dim for the group's 8 tokens).
//                        One workgroup per (kv head, token group, entry pair
//                        touched), writing the pair's new entries in turn:
//                        the 8 tokens' new K rows go into the K half as 16-byte
//                        chunks in 64-byte runs (two entries fill a 128-byte
//                        line), and their V rows, regrouped through LDS by dim,
//                        fill whole V chunks, four contiguous 512-byte runs.
//   moda_append_generic  the generic layout (natural Kd, then natural Vd):
//                        one thread per 16 bytes, a strided copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_device.h"
#include "moda_internal.h"

namespace moda {

constexpr int AP_D = kMfmaD;                     // 128
constexpr int AP_HALF = kDepthBlock * AP_D * 2;  // bytes of a block's K half

__global__ __launch_bounds__(256) void moda_append_mfma(AppendArgs p) {
  // grid: x = token group, y = kv head (b * Hkv + g), z = the entry pairs
  // (2k, 2k + 1) that [first, first + n) touches, in order.  A workgroup writes
  // the new entries of its pair, one after the other: the two share the K
  // half's 128-byte lines (64 bytes each), which then fill in one L2 instead
  // of leaving two L2s as two partial writes.
  __shared__ __attribute__((aligned(16))) uint16_t v_s[kGroupTokens][AP_D + 8];
  const int tid = threadIdx.x;
  const int64_t tg = blockIdx.x, bh = blockIdx.y;
  const int64_t pr = p.first / 2 + blockIdx.z;  // the pair: entries 2pr, 2pr + 1
  const int64_t e_lo = 2 * pr > p.first ? 2 * pr : p.first;
  const int64_t e_end = p.first + p.n, e_hi = 2 * pr + 2 < e_end ? 2 * pr + 2 : e_end;
  const int64_t eg = pr / 2;  // its entry group
  const int64_t ne = (p.L + kGroupEntries - 1) / kGroupEntries;
  char *const blk = (char *)p.packed + (bh * p.nblk + tg * ne + eg) * kPackedBlockBytes;
  // thread (token j = tid / 16 % 8, 16-byte column c16 = tid % 16); threads 128..255
  // handle V, 0..127 K.  Tokens past T keep the cache's zero padding.
  const int j = (tid >> 4) & 7, c16 = tid & 15;
  const int64_t t = kGroupTokens * tg + j;
  const bool valid = t < p.T;
  for (int64_t e = e_lo; e < e_hi; ++e) {
    const int64_t el = e - p.first;  // the entry's index among the new ones
    const int eo = (int)(e - kGroupEntries * eg);  // entry within the entry group
    const int kk = eo >> 1, h = eo & 1;            // block rows 16kk + 8a + 4h + b hold it
    const int64_t src = ((bh * p.T + (valid ? t : 0)) * p.n + el) * AP_D + 8 * c16;
    if (tid < 128) {
      // K row of token j: dims 8*c16 .. +7 go to k-step c16 % 8, lane r + 32 * (c16 / 8)
      // of block row r = 16kk + 8(j/4) + 4h + j%4
      if (valid) {
        const u32x4 kv = *(const u32x4 *)((const __bf16 *)p.knew + src);
        const int r = 16 * kk + 8 * (j >> 2) + 4 * h + (j & 3);
        *(u32x4 *)(blk + ((c16 & 7) * 64 + r + 32 * (c16 >> 3)) * 16) = kv;
      }
    } else {
      const u32x4 vv = valid ? *(const u32x4 *)((const __bf16 *)p.vnew + src) : u32x4{0, 0, 0, 0};
      *(u32x4 *)&v_s[j][8 * c16] = vv;
    }
    __syncthreads();
    if (tid >= 128) {
      // V chunk (nb, kk, lane 32h + dl): dim 32nb + dl of the 8 tokens, token j at element j
      const int u = tid - 128, nb = u >> 5, dl = u & 31, dim = 32 * nb + dl;
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = (uint32_t)v_s[2 * q][dim] | ((uint32_t)v_s[2 * q + 1][dim] << 16);
      // tokens past T: their elements are zero (the loads above read zeros for them)
      *(u32x4 *)(blk + AP_HALF + ((2 * nb + kk) * 64 + 32 * h + dl) * 16) = w;
    }
    __syncthreads();  // v_s is refilled for the next entry
  }
}

__global__ __launch_bounds__(256) void moda_append_generic(AppendArgs p, int row16) {
  const int64_t bh = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // ((t * n) + el) * row16 + c
  if (idx >= p.T * p.n * row16) return;
  const int64_t c = idx % row16, te = idx / row16;
  const int64_t t = te / p.n, el = te % p.n;
  const u32x4 *kn = (const u32x4 *)p.knew + (bh * p.T * p.n + te) * row16 + c;
  const u32x4 *vn = (const u32x4 *)p.vnew + (bh * p.T * p.n + te) * row16 + c;
  const int64_t dst_row = (bh * p.T + t) * p.L + p.first + el;  // row of Kd (and of Vd)
  u32x4 *const dst = (u32x4 *)p.packed;
  const int64_t half16 = p.B * p.Hkv * p.T * p.L * row16;  // 16-byte chunks of Kd
  dst[dst_row * row16 + c] = *kn;
  dst[half16 + dst_row * row16 + c] = *vn;
}

hipError_t launch_append(const AppendArgs &a, bool mfma, int row_bytes, hipStream_t s) {
  if (mfma) {
    // the entry pairs (2k, 2k + 1) that [first, first + n) touches
    const int64_t pairs = (a.first + a.n - 1) / 2 - a.first / 2 + 1;
    const dim3 grid((uint32_t)((a.T + kGroupTokens - 1) / kGroupTokens), (uint32_t)(a.B * a.Hkv),
                    (uint32_t)pairs);
    hipLaunchKernelGGL(moda_append_mfma, grid, dim3(256), 0, s, a);
  } else {
    const int row16 = row_bytes / 16;
    const int64_t per_bh = a.T * a.n * row16;
    const dim3 grid((uint32_t)((per_bh + 255) / 256), (uint32_t)(a.B * a.Hkv));
    hipLaunchKernelGGL(moda_append_generic, grid, dim3(256), 0, s, a, row16);
  }
  return hipGetLastError();
}

}  // namespace moda
