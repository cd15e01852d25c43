// HIP kernels of the depth-stream write step for gfx950 (MI355X): a layer's
// K and V for every token join the token's depth stream as entries
// [first, first + n) (hyper.ai page on arXiv 2603.15619, section "Depth
// stream mechanism": each layer appends what it wrote to the stream the later
// layers read; FFN layers add a light KV projection, so a layer may write
// two entries).  The cache is written in place, in the layout the forward
// reads, instead of repacking the whole stream after every layer.
//
//   moda_append_mfma     bf16, d = 128: the 32-entry block layout of the
//                        repack (K half in MFMA A-operand order, V half with
//                        each 16-byte chunk holding 8 entries of one dim).
//                        One thread per 16 bytes (8 dims) of two consecutive
//                        new entries of a token: their K chunks land whole,
//                        their V values land in 8 chunks that other entries
//                        share, as 4-byte stores when the two sit side by side
//                        in each chunk (the first at an even position in its
//                        block), else as 2-byte stores.
//   moda_append_generic  the generic layout (natural Kd, then natural Vd):
//                        one thread per 16 bytes, a strided copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_device.h"
#include "moda_internal.h"

namespace moda {

constexpr int AP_D = kMfmaD;                                       // 128
constexpr int AP_HALF = kDepthBlock * AP_D * 2;                    // bytes of a block's K half

// dims 8*c16 .. 8*c16+7 of the K row of entry e of a block: k-step c16 % 8,
// lane e + 32 * (c16 / 8) of the block's K half
__device__ __forceinline__ void append_k(char *blk_base, int e, int c16, const u32x4 &kv) {
  *(u32x4 *)(blk_base + ((c16 & 7) * 64 + e + 32 * (c16 >> 3)) * 16) = kv;
}

// address of element j of the V chunk that holds dims 8*c16 .. of entry e
// (dim c = 8*c16 + q sits in chunk (nb = c/32, kk = e/16, lane c%32 + 32*hh) at
// element j, where e % 16 = 8*(j/4) + 4*hh + j%4; consecutive q are 16 bytes apart)
__device__ __forceinline__ char *v_elem(char *blk_base, int e, int c16) {
  const int kk = e >> 4, r = e & 15;
  const int hh = (r & 7) >> 2, j = 4 * (r >> 3) + (r & 3);
  return blk_base + AP_HALF + (((c16 >> 2) * 2 + kk) * 64 + 8 * (c16 & 3) + 32 * hh) * 16 + 2 * j;
}

__global__ __launch_bounds__(256) void moda_append_mfma(AppendArgs p) {
  // one thread per (token, pair of new entries, 16 bytes of a row): entries
  // 2*pr and 2*pr + 1 of the n (the second may not exist)
  const int64_t bh = blockIdx.y;
  const int64_t npair = (p.n + 1) / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // ((t * npair) + pr) * 16 + c16
  if (idx >= p.T * npair * 16) return;
  const int c16 = (int)(idx & 15);
  const int64_t tp = idx >> 4;
  const int64_t t = tp / npair, el = 2 * (tp % npair);
  const bool two = el + 1 < p.n;
  const int64_t src = ((bh * p.T + t) * p.n + el) * AP_D + 8 * c16;
  const u32x4 k0 = *(const u32x4 *)((const __bf16 *)p.knew + src);
  const u32x4 v0 = *(const u32x4 *)((const __bf16 *)p.vnew + src);
  u32x4 k1 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
  if (two) {
    k1 = *(const u32x4 *)((const __bf16 *)p.knew + src + AP_D);
    v1 = *(const u32x4 *)((const __bf16 *)p.vnew + src + AP_D);
  }
  char *const base = (char *)p.packed + bh * p.nblk * kPackedBlockBytes;
  const int64_t f0 = t * p.L + p.first + el;  // flat (token, entry) position of the first
  const int e0 = (int)(f0 & (kDepthBlock - 1));
  char *const blk0 = base + (f0 >> 5) * kPackedBlockBytes;
  append_k(blk0, e0, c16, k0);
  char *const v0p = v_elem(blk0, e0, c16);
  if (two && (e0 & 1) == 0) {
    // the two entries sit side by side in every V chunk: 4-byte stores
    append_k(blk0, e0 + 1, c16, k1);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t lo = (v0[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
      const uint32_t hi = (v1[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
      *(uint32_t *)(v0p + 16 * q) = lo | (hi << 16);
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *(uint16_t *)(v0p + 16 * q) = (uint16_t)(v0[q >> 1] >> (16 * (q & 1)));
  if (two) {
    const int64_t f1 = f0 + 1;
    const int e1 = (int)(f1 & (kDepthBlock - 1));
    char *const blk1 = base + (f1 >> 5) * kPackedBlockBytes;
    append_k(blk1, e1, c16, k1);
    char *const v1p = v_elem(blk1, e1, c16);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *(uint16_t *)(v1p + 16 * q) = (uint16_t)(v1[q >> 1] >> (16 * (q & 1)));
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
  const int row16 = mfma ? 16 : row_bytes / 16;
  const int64_t per_bh = mfma ? a.T * ((a.n + 1) / 2) * 16 : a.T * a.n * row16;
  const dim3 grid((uint32_t)((per_bh + 255) / 256), (uint32_t)(a.B * a.Hkv));
  if (mfma)
    hipLaunchKernelGGL(moda_append_mfma, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(moda_append_generic, grid, dim3(256), 0, s, a, row16);
  return hipGetLastError();
}

}  // namespace moda
