// Device helpers shared by the forward (moda_kernels.hip) and backward
// (moda_bwd.hip) kernels: vector types, bf16 conversion, lane-pair
// reductions and LDS transpose reads for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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


}  // namespace moda
