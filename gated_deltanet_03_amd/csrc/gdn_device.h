// Device-side helpers shared by the GDN kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Element traits: storage type of q, k, v, o and of 16-bit MFMA operands.
// ---------------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};
template <> struct Elem<_Float16> {
  static __device__ __forceinline__ float to_f(_Float16 x) { return (float)x; }
  static __device__ __forceinline__ _Float16 from_f(float x) { return (_Float16)x; }
};
template <> struct Elem<__bf16> {
  static __device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
  static __device__ __forceinline__ __bf16 from_f(float x) { return (__bf16)x; }  // RNE (v_cvt_pk_bf16_f32)
};

// Load N consecutive elements (N * sizeof(T) bytes, naturally aligned to the
// largest power of two dividing that size, at most 16) and widen to fp32.
template <typename T, int N>
__device__ __forceinline__ void load_row_f32(const T* __restrict__ p, float* out) {
  constexpr int BYTES = N * (int)sizeof(T);
  if constexpr (BYTES % 16 == 0) {
    constexpr int V = BYTES / 16;
    constexpr int PER = 16 / (int)sizeof(T);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      uint4 raw = *reinterpret_cast<const uint4*>(p + i * PER);
      const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int j = 0; j < PER; ++j) out[i * PER + j] = Elem<T>::to_f(e[j]);
    }
  } else if constexpr (BYTES % 8 == 0) {
    constexpr int V = BYTES / 8;
    constexpr int PER = 8 / (int)sizeof(T);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      uint2 raw = *reinterpret_cast<const uint2*>(p + i * PER);
      const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int j = 0; j < PER; ++j) out[i * PER + j] = Elem<T>::to_f(e[j]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = Elem<T>::to_f(p[i]);
  }
}

// Store 4 fp32 values as 4 consecutive elements of T (rounded RNE for 16-bit T).
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  } else {
    union { T e[4]; uint2 u; } pk;
    pk.e[0] = Elem<T>::from_f(a);
    pk.e[1] = Elem<T>::from_f(b);
    pk.e[2] = Elem<T>::from_f(c);
    pk.e[3] = Elem<T>::from_f(d);
    *reinterpret_cast<uint2*>(p) = pk.u;
  }
}

// Workgroup barrier for LDS traffic only.  __syncthreads() carries a
// workgroup-scope fence that also drains this wave's outstanding global loads
// and stores (vmcnt); that would wait for register prefetches of the next chunk
// and for output stores at every barrier.  Here only LDS operations (lgkmcnt)
// are completed before the s_barrier; the clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// [a, b) clamped to [0, total], so malformed offsets stay in bounds.
__device__ __forceinline__ void clamp_range(int a, int b, int32_t total, int& t0, int& t1) {
  a = a < 0 ? 0 : (a > total ? total : a);
  b = b < a ? a : (b > total ? total : b);
  t0 = a;
  t1 = b;
}

// Token range of sequence s: dense rows of T tokens when cu == nullptr, else
// [cu[s], cu[s+1]) clamped to [0, total] so malformed offsets stay in bounds.
__device__ __forceinline__ void seq_range(const int32_t* __restrict__ cu, int32_t T, int32_t total,
                                          int s, int& t0, int& t1) {
  if (cu == nullptr) {
    t0 = s * T;
    t1 = t0 + T;
  } else {
    clamp_range(cu[s], cu[s + 1], total, t0, t1);
  }
}

}  // namespace gdn
