// Matrix-core (MFMA) building blocks for the chunked GDN kernels on gfx950.
//
// All products are 16x16 output tiles.  Layout facts used throughout (wave64):
//   D (fp32 accumulator, 4 values per lane): lane l holds D[4*(l/16) + q][l%16], q = 0..3.
//   16-bit operands of v_mfma_f32_16x16x32_{bf16,f16}: lane l holds 8 values
//     A[l%16][slot 8*(l/16) + j] and B[slot 8*(l/16) + j][l%16], j = 0..7.
//   fp32 operands of v_mfma_f32_16x16x4_f32: lane l holds A[l%16][l/16], B[l/16][l%16].
//
// The contraction index can be permuted freely as long as A and B agree.  We
// pick, for a 32-wide block of the contraction index made of two 16-row tiles
// (lo, hi), the slot order
//     slot 8g + j  <->  index  (j < 4 ? lo*16 + 4g + j : hi*16 + 4g + (j - 4)),
// so that the B operand of a product can be taken straight from two fp32
// accumulator tiles of an earlier product (lane l already holds rows 4g..4g+3 of
// column l%16 in each), and the A operand is read as two 4-element runs from a
// row-major matrix.  For fp32 the same 32-block is eight K=4 steps, step (t, q)
// using accumulator element q of tile t and A[i][16t + 4g + q].
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  static __device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<_Float16> {
  static __device__ __forceinline__ f32x4 mma(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> { using type = bf16x8; using half = bf16x4; };
template <> struct Vec8<_Float16> { using type = f16x8; using half = f16x4; };

// 4 consecutive 16-bit elements (8 bytes, 8-byte aligned) from LDS or global.
template <typename T>
__device__ __forceinline__ typename Vec8<T>::half ld4(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::half*>(p);
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type cat(typename Vec8<T>::half lo, typename Vec8<T>::half hi) {
  typename Vec8<T>::type r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::half cvt4(const f32x4& x) {
  typename Vec8<T>::half r;
  r[0] = Elem<T>::from_f(x[0]); r[1] = Elem<T>::from_f(x[1]);
  r[2] = Elem<T>::from_f(x[2]); r[3] = Elem<T>::from_f(x[3]);
  return r;
}

// acc += A_blk * B_blk over one 32-wide contraction block.
//   a_lo / a_hi: this lane's A row at contraction offsets (lo tile) 16*lo + 4g and
//                (hi tile) 16*hi + 4g; 4 consecutive elements each.
//   b_lo / b_hi: accumulator tiles holding B rows of the lo / hi tile.
//   has_hi:      false when the hi tile does not exist (treated as zero).
template <typename T>
__device__ __forceinline__ void kblock_acc(f32x4& acc, const T* a_lo, const T* a_hi, const f32x4& b_lo,
                                           const f32x4& b_hi, bool has_hi) {
  if constexpr (sizeof(T) == 4) {
    const f32x4 al = *reinterpret_cast<const f32x4*>(a_lo);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(al[q], b_lo[q], acc, 0, 0, 0);
    if (has_hi) {
      const f32x4 ah = *reinterpret_cast<const f32x4*>(a_hi);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ah[q], b_hi[q], acc, 0, 0, 0);
    }
  } else {
    typename Vec8<T>::half zl = {}, al = ld4<T>(a_lo);
    typename Vec8<T>::half ah = has_hi ? ld4<T>(a_hi) : zl;
    typename Vec8<T>::half bh = has_hi ? cvt4<T>(b_hi) : zl;
    acc = Mfma<T>::mma(cat<T>(al, ah), cat<T>(cvt4<T>(b_lo), bh), acc);
  }
}

// acc += A_blk * B_blk where both operands are rows of row-major matrices
// (B given as the rows of B^T, i.e. the product A * Bmat^T).
template <typename T>
__device__ __forceinline__ void kblock_rows(f32x4& acc, const T* a_lo, const T* a_hi, const T* b_lo,
                                            const T* b_hi, bool has_hi) {
  if constexpr (sizeof(T) == 4) {
    const f32x4 al = *reinterpret_cast<const f32x4*>(a_lo);
    const f32x4 bl = *reinterpret_cast<const f32x4*>(b_lo);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(al[q], bl[q], acc, 0, 0, 0);
    if (has_hi) {
      const f32x4 ah = *reinterpret_cast<const f32x4*>(a_hi);
      const f32x4 bh = *reinterpret_cast<const f32x4*>(b_hi);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ah[q], bh[q], acc, 0, 0, 0);
    }
  } else {
    typename Vec8<T>::half z = {};
    typename Vec8<T>::half al = ld4<T>(a_lo), bl = ld4<T>(b_lo);
    typename Vec8<T>::half ah = has_hi ? ld4<T>(a_hi) : z;
    typename Vec8<T>::half bh = has_hi ? ld4<T>(b_hi) : z;
    acc = Mfma<T>::mma(cat<T>(al, ah), cat<T>(bl, bh), acc);
  }
}

}  // namespace gdn
