// Recurrent (token-by-token) GDN step with compact state-update capture, the
// replay of captured updates, and the plain fill / copy kernels used for the
// inactive-capture zero fill and for state snapshots.
//
// Method: the gated delta rule, alpha = exp(g), delta = beta (v - alpha S^T k),
// S <- alpha S + k delta^T, o = scale S^T q (post-update state).  Capture and
// replay follow [onnxruntime PR 32767, "[WebGPU EP] adds state update capacity
// support for GatedDeltaNet", section "Changes"]: a clamped per-row prefix of
// (decay, shared key, delta) factors whose replay is S = decay*S + outer(key, delta).
//
// Design (memory-bound; no matrix cores): one wave64 owns a [dk x DVS] column
// slice of one (row, value head) state.  Columns of S never interact (only the
// dk-reductions S^T k and S^T q couple rows), so slices are independent.
// Lane layout: lane = rg * CG + cg; cg picks 4 adjacent columns (one 16-byte
// float4), rg picks RPL = dk / RG adjacent rows.  A wave's load of one row
// index covers RG rows x DVS*4 contiguous bytes, fully using every 64/128-byte
// segment.  The dk-reductions are a per-lane partial sum over RPL rows plus a
// butterfly over the RG row groups.  The state is read once and written once
// per call; token inputs for step t+1 are fetched while step t computes.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <typename T, int DK, int DVS>
struct DecodeGeom {
  static constexpr int CG = DVS / 4;   // column groups (float4) per wave
  static constexpr int RG = 64 / CG;   // row groups per wave
  static constexpr int RPL = DK / RG;  // rows per lane
  static_assert(RPL >= 1 && RG * RPL == DK, "unsupported dk / slice width");
};

template <typename T, int RPL>
struct TokenIn {
  float k[RPL];
  float q[RPL];
  float v[4];
  float g, beta;
};

template <typename T, int DK, int DVS>
__global__ __launch_bounds__(64) void recurrent_step_kernel(DecodeArgs p) {
  using Gm = DecodeGeom<T, DK, DVS>;
  constexpr int CG = Gm::CG, RPL = Gm::RPL;
  const int lane = threadIdx.x;
  const int cg = lane % CG, rg = lane / CG;
  const int slice = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = p.Hv / p.Hq;
  const int hk = h / G;
  const int dv = p.dv;
  const int col = slice * DVS + cg * 4;
  const int row0 = rg * RPL;

  int t0, t1;
  seq_range(p.cu, p.T, p.total, b, t0, t1);

  const T* __restrict__ qp = static_cast<const T*>(p.q);
  const T* __restrict__ kp = static_cast<const T*>(p.k);
  const T* __restrict__ vp = static_cast<const T*>(p.v);
  T* __restrict__ op = static_cast<T*>(p.o);

  auto load_tok = [&](int t, TokenIn<T, RPL>& in) {
    const size_t qk = ((size_t)t * p.Hq + hk) * DK + row0;
    load_row_f32<T, RPL>(kp + qk, in.k);
    load_row_f32<T, RPL>(qp + qk, in.q);
    load_row_f32<T, 4>(vp + ((size_t)t * p.Hv + h) * dv + col, in.v);
    in.g = p.g[(size_t)t * p.Hv + h];
    in.beta = p.beta[(size_t)t * p.Hv + h];
  };

  TokenIn<T, RPL> nxt;
  if (t0 < t1) load_tok(t0, nxt);

  // State slice: rows row0..row0+RPL-1, columns col..col+3.
  float4 S[RPL];
  if (p.s0 != nullptr) {
    const float* s0 = p.s0 + (int64_t)b * p.s0_stride + (size_t)h * DK * dv;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      S[r] = *reinterpret_cast<const float4*>(s0 + (size_t)(row0 + r) * dv + col);
  } else {
#pragma unroll
    for (int r = 0; r < RPL; ++r) S[r] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  int ncap = 0;
  if (p.cap > 0 && p.active) {
    int c = p.counts[b];
    int lim = p.cap < (t1 - t0) ? p.cap : (t1 - t0);
    ncap = c < 0 ? 0 : (c > lim ? lim : c);
  }
  const size_t R = (size_t)p.Hv + (size_t)p.Hq * DK + (size_t)p.Hv * dv;
  const bool write_key = (h % G == 0) && slice == 0 && cg == 0;

  for (int t = t0; t < t1; ++t) {
    TokenIn<T, RPL> in = nxt;
    if (t + 1 < t1) load_tok(t + 1, nxt);
    const float a = expf(in.g);

    // Partial dk-reductions over this lane's rows: u = S^T k, w = S^T q, kq = k.q
    float u0 = 0.f, u1 = 0.f, u2 = 0.f, u3 = 0.f;
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f, kq = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const float kr = in.k[r], qr = in.q[r];
      u0 = fmaf(S[r].x, kr, u0); u1 = fmaf(S[r].y, kr, u1);
      u2 = fmaf(S[r].z, kr, u2); u3 = fmaf(S[r].w, kr, u3);
      w0 = fmaf(S[r].x, qr, w0); w1 = fmaf(S[r].y, qr, w1);
      w2 = fmaf(S[r].z, qr, w2); w3 = fmaf(S[r].w, qr, w3);
      kq = fmaf(kr, qr, kq);
    }
#pragma unroll
    for (int m = CG; m < 64; m <<= 1) {
      u0 += __shfl_xor(u0, m); u1 += __shfl_xor(u1, m);
      u2 += __shfl_xor(u2, m); u3 += __shfl_xor(u3, m);
      w0 += __shfl_xor(w0, m); w1 += __shfl_xor(w1, m);
      w2 += __shfl_xor(w2, m); w3 += __shfl_xor(w3, m);
      kq += __shfl_xor(kq, m);
    }
    // delta = beta (v - alpha S^T k); o = scale (alpha S^T q + delta (k.q)) = scale S_t^T q
    const float d0 = in.beta * (in.v[0] - a * u0);
    const float d1 = in.beta * (in.v[1] - a * u1);
    const float d2 = in.beta * (in.v[2] - a * u2);
    const float d3 = in.beta * (in.v[3] - a * u3);
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const float kr = in.k[r];
      S[r].x = fmaf(kr, d0, a * S[r].x);
      S[r].y = fmaf(kr, d1, a * S[r].y);
      S[r].z = fmaf(kr, d2, a * S[r].z);
      S[r].w = fmaf(kr, d3, a * S[r].w);
    }
    if (rg == 0) {
      store4<T>(op + ((size_t)t * p.Hv + h) * dv + col,
                p.scale * fmaf(d0, kq, a * w0), p.scale * fmaf(d1, kq, a * w1),
                p.scale * fmaf(d2, kq, a * w2), p.scale * fmaf(d3, kq, a * w3));
    }
    const int tt = t - t0;
    if (tt < ncap) {
      float* rec = p.su + ((size_t)b * p.cap + tt) * R;
      if (slice == 0 && lane == 0) rec[h] = a;
      if (write_key) {
        float* kd = rec + p.Hv + (size_t)hk * DK + row0;
#pragma unroll
        for (int r = 0; r < RPL; ++r) kd[r] = in.k[r];
      }
      if (rg == 0) {
        float* dd = rec + p.Hv + (size_t)p.Hq * DK + (size_t)h * dv + col;
        dd[0] = d0; dd[1] = d1; dd[2] = d2; dd[3] = d3;
      }
    }
  }

  if (p.s_out != nullptr) {
    float* so = p.s_out + ((size_t)b * p.Hv + h) * DK * dv;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      *reinterpret_cast<float4*>(so + (size_t)(row0 + r) * dv + col) = S[r];
  }
}

template <int DK, int DVS>
__global__ __launch_bounds__(64) void replay_kernel(ReplayArgs p) {
  using Gm = DecodeGeom<float, DK, DVS>;
  constexpr int CG = Gm::CG, RPL = Gm::RPL;
  const int lane = threadIdx.x;
  const int cg = lane % CG, rg = lane / CG;
  const int slice = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (p.Hv / p.Hq);
  const int dv = p.dv;
  const int col = slice * DVS + cg * 4;
  const int row0 = rg * RPL;

  int m = p.counts[b];
  m = m < 0 ? 0 : (m > p.cap ? p.cap : m);
  if (m == 0) return;

  float* st = p.state + ((size_t)b * p.Hv + h) * DK * dv;
  float4 S[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) S[r] = *reinterpret_cast<const float4*>(st + (size_t)(row0 + r) * dv + col);

  const size_t R = (size_t)p.Hv + (size_t)p.Hq * DK + (size_t)p.Hv * dv;
  for (int c = 0; c < m; ++c) {
    const float* rec = p.su + ((size_t)b * p.cap + c) * R;
    const float a = rec[h];
    const float* kr = rec + p.Hv + (size_t)hk * DK + row0;
    const float* dd = rec + p.Hv + (size_t)p.Hq * DK + (size_t)h * dv + col;
    const float d0 = dd[0], d1 = dd[1], d2 = dd[2], d3 = dd[3];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const float k = kr[r];
      // same operation order as the recurrent step: fma(k, delta, alpha * S)
      S[r].x = fmaf(k, d0, a * S[r].x);
      S[r].y = fmaf(k, d1, a * S[r].y);
      S[r].z = fmaf(k, d2, a * S[r].z);
      S[r].w = fmaf(k, d3, a * S[r].w);
    }
  }
#pragma unroll
  for (int r = 0; r < RPL; ++r) *reinterpret_cast<float4*>(st + (size_t)(row0 + r) * dv + col) = S[r];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, size_t n) {
  const size_t n4 = n / 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t j = i; j < n4; j += stride) reinterpret_cast<float4*>(p)[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (size_t j = n4 * 4 + i; j < n; j += stride) p[j] = 0.f;
}

__global__ __launch_bounds__(256) void copy_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                   size_t n) {
  const size_t n4 = n / 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t j = i; j < n4; j += stride)
    reinterpret_cast<float4*>(dst)[j] = reinterpret_cast<const float4*>(src)[j];
  for (size_t j = n4 * 4 + i; j < n; j += stride) dst[j] = src[j];
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <typename T, int DK>
static hipError_t launch_rec_dk(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  prof_begin(K_RECURRENT, s);
  if (a.dv >= 32) {
    dim3 grid(a.dv / 32, a.Hv, a.B);
    hipLaunchKernelGGL((recurrent_step_kernel<T, DK, 32>), grid, dim3(64), 0, s, a);
  } else {
    dim3 grid(a.dv / 16, a.Hv, a.B);
    hipLaunchKernelGGL((recurrent_step_kernel<T, DK, 16>), grid, dim3(64), 0, s, a);
  }
  prof_end(K_RECURRENT, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_rec_t(const DecodeArgs& a, hipStream_t s) {
  switch (a.dk) {
    case 16: return launch_rec_dk<T, 16>(a, s);
    case 32: return launch_rec_dk<T, 32>(a, s);
    case 64: return launch_rec_dk<T, 64>(a, s);
    case 128: return launch_rec_dk<T, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_recurrent(DType dt, const DecodeArgs& a, hipStream_t s) {
  switch (dt) {
    case DType::F32: return launch_rec_t<float>(a, s);
    case DType::F16: return launch_rec_t<_Float16>(a, s);
    case DType::BF16: return launch_rec_t<__bf16>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int DK>
static hipError_t launch_replay_dk(const ReplayArgs& a, hipStream_t s) {
  if (a.B == 0 || a.cap == 0) return hipSuccess;
  prof_begin(K_REPLAY, s);
  if (a.dv >= 32) {
    hipLaunchKernelGGL((replay_kernel<DK, 32>), dim3(a.dv / 32, a.Hv, a.B), dim3(64), 0, s, a);
  } else {
    hipLaunchKernelGGL((replay_kernel<DK, 16>), dim3(a.dv / 16, a.Hv, a.B), dim3(64), 0, s, a);
  }
  prof_end(K_REPLAY, s);
  return hipGetLastError();
}

hipError_t launch_replay(const ReplayArgs& a, hipStream_t s) {
  switch (a.dk) {
    case 16: return launch_replay_dk<16>(a, s);
    case 32: return launch_replay_dk<32>(a, s);
    case 64: return launch_replay_dk<64>(a, s);
    case 128: return launch_replay_dk<128>(a, s);
  }
  return hipErrorInvalidValue;
}

static unsigned stream_grid(size_t n) {
  size_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  return (unsigned)blocks;
}

hipError_t launch_zero_fill(float* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  prof_begin(K_ZERO_FILL, s);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(stream_grid(n)), dim3(256), 0, s, p, n);
  prof_end(K_ZERO_FILL, s);
  return hipGetLastError();
}

hipError_t launch_copy(const float* src, float* dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  prof_begin(K_COPY, s);
  hipLaunchKernelGGL(copy_kernel, dim3(stream_grid(n)), dim3(256), 0, s, src, dst, n);
  prof_end(K_COPY, s);
  return hipGetLastError();
}

}  // namespace gdn
