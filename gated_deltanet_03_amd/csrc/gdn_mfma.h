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
// column l%16 in each), and an A operand is two 4-element runs of a row-major
// matrix.  For fp32 the same 32-block is eight K=4 steps, step (t, q) using
// accumulator element q of tile t and A[i][16t + 4g + q].
//
// A "fragment" is one lane's 8 operand values for one 16 x 32 block.  The
// fragment-native storage of a block is 64 lanes x 8 consecutive elements, so a
// whole block is read or written with one 16-byte (32-byte for fp32) access per
// lane, conflict-free in LDS and fully coalesced in global memory.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T> struct Frag;
template <> struct Frag<__bf16> { bf16x8 v; };
template <> struct Frag<_Float16> { f16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

template <typename T> struct Half4;
template <> struct Half4<__bf16> { using type = bf16x4; };
template <> struct Half4<_Float16> { using type = f16x4; };

template <typename T>
__device__ __forceinline__ typename Half4<T>::type cvt4(const f32x4& x) {
  typename Half4<T>::type r;
  r[0] = Elem<T>::from_f(x[0]); r[1] = Elem<T>::from_f(x[1]);
  r[2] = Elem<T>::from_f(x[2]); r[3] = Elem<T>::from_f(x[3]);
  return r;
}

// Fragment from two accumulator tiles (the B operand of the next product).
template <typename T>
__device__ __forceinline__ Frag<T> make_frag(const f32x4& lo, const f32x4& hi) {
  Frag<T> f;
  if constexpr (sizeof(T) == 4) {
    f.lo = lo;
    f.hi = hi;
  } else {
    const auto a = cvt4<T>(lo), b = cvt4<T>(hi);
    f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
    f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
  }
  return f;
}

// Fragment from two 4-element runs of a row-major matrix (A operand).
template <typename T>
__device__ __forceinline__ Frag<T> load_frag_rows(const T* lo, const T* hi) {
  Frag<T> f;
  if constexpr (sizeof(T) == 4) {
    f.lo = *reinterpret_cast<const f32x4*>(lo);
    f.hi = *reinterpret_cast<const f32x4*>(hi);
  } else {
    const auto a = *reinterpret_cast<const typename Half4<T>::type*>(lo);
    const auto b = *reinterpret_cast<const typename Half4<T>::type*>(hi);
    f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
    f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
  }
  return f;
}

// Fragment stored natively: 8 consecutive elements for this lane.
template <typename T>
__device__ __forceinline__ Frag<T> load_frag_native(const T* p) {
  Frag<T> f;
  if constexpr (sizeof(T) == 4) {
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  } else {
    f.v = *reinterpret_cast<const decltype(f.v)*>(p);
  }
  return f;
}

template <typename T>
__device__ __forceinline__ void store_frag_native(T* p, const Frag<T>& f) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(p) = f.lo;
    *reinterpret_cast<f32x4*>(p + 4) = f.hi;
  } else {
    *reinterpret_cast<decltype(f.v)*>(const_cast<T*>(p)) = f.v;
  }
}

// acc += A_blk * B_blk over one 32-wide contraction block.
template <typename T>
__device__ __forceinline__ void mma(f32x4& acc, const Frag<T>& a, const Frag<T>& b) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[q], b.lo[q], acc, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[q], b.hi[q], acc, 0, 0, 0);
  } else if constexpr (__is_same(T, __bf16)) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
  }
}

// acc += A_blk * B_blk where only the lo tile of the block exists (the hi half
// of both operands is zero): used for 16-wide contractions.
template <typename T>
__device__ __forceinline__ void mma_lo(f32x4& acc, const Frag<T>& a, const Frag<T>& b) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[q], b.lo[q], acc, 0, 0, 0);
  } else {
    mma<T>(acc, a, b);
  }
}

template <typename T>
__device__ __forceinline__ Frag<T> zero_frag() {
  Frag<T> f;
  if constexpr (sizeof(T) == 4) {
    f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
    f.hi = f.lo;
  } else {
    f.v = decltype(f.v){};
  }
  return f;
}

// One 16-byte read of 8 consecutive elements as a fragment.
template <typename T>
__device__ __forceinline__ Frag<T> load_frag_8(const T* p) {
  return load_frag_native<T>(p);
}


}  // namespace gdn
