// Recurrent (token-by-token) GDN step with compact state-update capture (and,
// when capture is inactive, the zero fill of the capture buffer), the replay
// of captured updates, and the plain copy kernel used for state snapshots.
//
// Method: the gated delta rule, alpha = exp(g), delta = beta (v - alpha S^T k),
// S <- alpha S + k delta^T, o = scale S^T q (post-update state).  Capture and
// replay follow [onnxruntime PR 32767, "[WebGPU EP] adds state update capacity
// support for GatedDeltaNet", section "Changes"]: a clamped per-row prefix of
// (decay, shared key, delta) factors whose replay is S = decay*S + outer(key, delta).
//
// Design (memory- and VALU-bound; no matrix cores): one wave64 owns a
// [dk x 16] column slice of one (row, value head) state.  Columns of S never
// interact (only the dk-reductions S^T k and S^T q couple rows), so slices are
// independent.  Lane layout: lane = rg * 4 + cg; cg picks 4 adjacent columns
// (one 16-byte float4), rg picks RPL = dk / 16 adjacent rows.  The
// dk-reductions are a per-lane partial sum over RPL rows plus a butterfly over
// the 16 row groups done entirely on the VALU: two DPP row rotations (lanes
// +-4, +-8 inside a row of 16) and the permlane16 / permlane32 swaps, the
// column sums of S^T k and S^T q in pairs (sum_rowgroups4).
// Token inputs are prefetched NPF tokens ahead as raw 16-byte words.  A
// workgroup of the recurrent step holds WPG waves, the adjacent column slices
// of one (row, head) state (up to 4 of its dv / 16 slices), so the two
// 64-byte halves of every 128-byte state line are requested from one CU at
// about the same time (34-token decode: 12.8 us instead of 13.9 us per call).
// The replay, which needs no dk-reduction, uses 32-column slices split over
// two waves by rows instead (whole 128-byte lines per instruction).  Each
// row's wave-uniform values (token range, capture count, gates, per-token g
// and beta) come through scalar loads.  Workgroups of one state get ids that
// agree mod 8, so they run on one XCD.  The state is read once and written
// once per call.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int DVS = 16;   // columns per wave

// State reads are ordinary loads: a replay right after a step reads the same
// pre-step state and finds it in the caches.  State writes are not read again
// by this call and are streamed out with non-temporal stores.
__device__ __forceinline__ float4 load_state4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void store_state4(float* p, const float4& v) {
  __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}
constexpr int NPF = 4;    // token prefetch depth

// sum over the 16 lanes sharing lane % 4
__device__ __forceinline__ float sum_rowgroups(float x) {
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x128, 0xf, 0xf, false);   // row_ror:8
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x124, 0xf, 0xf, false);   // row_ror:4
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);                   // + lane ^ 16
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);                // + lane ^ 32
}

// In-place lane swaps of two registers.  permlane32: lanes 32..63 of x trade
// with lanes 0..31 of y, so afterwards x = (x_lo, y_lo) and y = (x_hi, y_hi).
// permlane16: the odd 16-lane rows of x trade with the even rows of y, so
// x = (x_r0, y_r0, x_r2, y_r2) and y = (x_r1, y_r1, x_r3, y_r3).
__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// Sums over the 16 row groups (lane bits 2..5) of four per-column partials
// c0..c3, left bitwise identical in every lane.  The two permlane levels reduce
// pairs at one swap and one add per pair (a lane half keeps one member of each
// pair), which leaves the four sums in the four 16-lane rows (c0, c2, c1, c3);
// the DPP levels finish each row, and two levels of swaps with copies gather
// the four back into every lane.  About 19 instructions instead of 32.
__device__ __forceinline__ void sum_rowgroups4(float& c0, float& c1, float& c2, float& c3) {
  swap32(c0, c1);
  swap32(c2, c3);
  float a = c0 + c1, b = c2 + c3;      // a: c0 in lanes 0..31, c1 in 32..63; b: c2, c3
  swap16(a, b);
  float x = a + b;                     // rows: c0, c2, c1, c3
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x128, 0xf, 0xf, false);   // row_ror:8
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x124, 0xf, 0xf, false);   // row_ror:4
  float lo = x, hi = x;
  swap32(lo, hi);                      // lo: rows (c0, c2, c0, c2); hi: (c1, c3, c1, c3)
  float lo2 = lo, hi2 = hi;
  swap16(lo, lo2);                     // lo: c0 everywhere, lo2: c2
  swap16(hi, hi2);                     // hi: c1, hi2: c3
  c0 = lo;
  c1 = hi;
  c2 = lo2;
  c3 = hi2;
}

// N consecutive elements of T kept as raw 32-bit words until use.
template <typename T, int N>
struct Raw {
  static constexpr int BYTES = N * (int)sizeof(T);
  static constexpr int W = BYTES >= 4 ? BYTES / 4 : 1;
  uint32_t w[W];
  __device__ __forceinline__ void load(const T* __restrict__ p) {
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
      for (int i = 0; i < BYTES / 16; ++i) {
        const uint4 u = reinterpret_cast<const uint4*>(p)[i];
        w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
      }
    } else if constexpr (BYTES == 8) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      w[0] = u.x; w[1] = u.y;
    } else if constexpr (BYTES == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      static_assert(BYTES == 2, "unsupported row width");
      w[0] = *reinterpret_cast<const uint16_t*>(p);
    }
  }
  __device__ __forceinline__ float get(int i) const {
    if constexpr (sizeof(T) == 4) {
      return __uint_as_float(w[i]);
    } else {
      const uint16_t bits = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
      return Elem<T>::to_f(__builtin_bit_cast(T, bits));
    }
  }
};

template <typename T, int RPL>
struct TokenIn {
  Raw<T, RPL> k, q;
  Raw<T, 4> v;
  float g, beta;
};

// Workgroup id and wave -> (row, value head, column slice, row part):
// workgroups of NWR * SPG waves, SPG adjacent column slices of one (row, head)
// state, each slice served by NWR waves that split its dk rows.  The
// workgroups of one state get ids congruent mod 8 (one XCD).  False for
// padding workgroups.
template <int NWR, int SPG>
__device__ __forceinline__ bool slice_of(int Hv, int nsl, int B, int& b, int& h, int& slice, int& wr) {
  const int ngr = nsl / SPG;
  const int xcd = (int)(blockIdx.x & 7), rnd = (int)(blockIdx.x >> 3);
  const int grp = (rnd / ngr) * 8 + xcd;
  if (grp >= B * Hv) return false;
  const int wi = (int)(threadIdx.x >> 6);
  slice = (rnd % ngr) * SPG + wi / NWR;
  wr = wi % NWR;
  b = grp / Hv;
  h = grp % Hv;
  return true;
}

__device__ const int32_t kZeroWords[4] = {0, 0, 0, 0};
__device__ const float kZeroFloats[4] = {0.f, 0.f, 0.f, 0.f};

// Read-only wave-uniform value through the constant address space, so it is
// fetched with a scalar load (counted apart from the vector loads in flight).
template <typename X>
__device__ __forceinline__ X load_uniform(const X* ptr) {
  return *(const __attribute__((address_space(4))) X*)ptr;
}

__device__ __forceinline__ void zero_fill_records(const DecodeArgs& p, int dk) {
  const size_t n = (size_t)p.B * p.cap * ((size_t)p.Hv + (size_t)p.Hq * dk + (size_t)p.Hv * p.dv);
  const size_t n4 = n / 4, stride = (size_t)gridDim.x * blockDim.x;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t j = i; j < n4; j += stride) reinterpret_cast<float4*>(p.su)[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (size_t j = n4 * 4 + i; j < n; j += stride) p.su[j] = 0.f;
}

template <typename T, int DK, int WPG>
__global__ __launch_bounds__(64 * WPG) void recurrent_step_kernel(DecodeArgs p) {
  constexpr int RPL = DK / 16;
  const int lane = threadIdx.x & 63;
  const int cg = lane & 3, rg = lane >> 2;
  // inactive capture: every thread of the grid zero-fills its share of the
  // whole state_update buffer [B, cap, R] (16-byte aligned) after its step,
  // which writes no records; placed after every load of the kernel so that
  // the compiler may fetch the row's wave-uniform values with scalar loads
  const bool fill = p.cap > 0 && !p.active;
  int b, h, slice, wr;
  if (!slice_of<1, WPG>(p.Hv, p.dv / DVS, p.B, b, h, slice, wr)) {
    if (fill) zero_fill_records(p, DK);
    return;
  }
  b = __builtin_amdgcn_readfirstlane(b);
  h = __builtin_amdgcn_readfirstlane(h);
  slice = __builtin_amdgcn_readfirstlane(slice);
  const int G = p.Hv / p.Hq;
  const int hk = h / G;
  const int dv = p.dv;
  const int col = slice * DVS + cg * 4;
  const int row0 = rg * RPL;

  // The row's wave-uniform data: scalar loads issued before the state loads,
  // unconditionally (absent arrays read zeros), so that nothing waits for them
  // before the state is requested.
  const bool capture = p.cap > 0 && p.active;
  const bool gate = p.pro.A_log != nullptr;   // g = -exp(A_log) softplus(g_in + dt_bias)
  const int cu0 = load_uniform(p.cu != nullptr ? p.cu + b : kZeroWords);
  const int cu1 = load_uniform(p.cu != nullptr ? p.cu + b + 1 : kZeroWords);
  const int cnt = load_uniform(capture ? p.counts + b : kZeroWords);
  const float alog = load_uniform(gate ? p.pro.A_log + h : kZeroFloats);
  const float dtb = load_uniform(gate && p.pro.dt_bias != nullptr ? p.pro.dt_bias + h : kZeroFloats);

  // State slice: rows row0..row0+RPL-1, columns col..col+3.
  float4 S[RPL];
  if (p.s0 != nullptr) {
    const float* s0 = p.s0 + (int64_t)b * p.s0_stride + (size_t)h * DK * dv;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      S[r] = load_state4(s0 + (size_t)(row0 + r) * dv + col);
  } else {
#pragma unroll
    for (int r = 0; r < RPL; ++r) S[r] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  int t0, t1;
  if (p.cu == nullptr) {
    t0 = b * p.T;
    t1 = t0 + p.T;
  } else {
    clamp_range(cu0, cu1, p.total, t0, t1);
  }

  const T* __restrict__ qp = static_cast<const T*>(p.q);
  const T* __restrict__ kp = static_cast<const T*>(p.k);
  const T* __restrict__ vp = static_cast<const T*>(p.v);
  T* __restrict__ op = static_cast<T*>(p.o);

  const float negA = gate ? -expf(alog) : 0.f;

  auto load_tok = [&](int t, TokenIn<T, RPL>& in) {
    const size_t qk = ((size_t)t * p.Hq + hk) * DK + row0;
    in.k.load(kp + qk);
    in.q.load(qp + qk);
    in.v.load(vp + ((size_t)t * p.Hv + h) * dv + col);
    in.g = load_uniform(p.g + (size_t)t * p.Hv + h);
    in.beta = load_uniform(p.beta + (size_t)t * p.Hv + h);
  };

  TokenIn<T, RPL> ring[NPF];
#pragma unroll
  for (int u = 0; u < NPF; ++u)
    if (t0 + u < t1) load_tok(t0 + u, ring[u]);

  int ncap = 0;
  if (capture) {
    const int lim = p.cap < (t1 - t0) ? p.cap : (t1 - t0);
    ncap = cnt < 0 ? 0 : (cnt > lim ? lim : cnt);
  }
  const size_t R = (size_t)p.Hv + (size_t)p.Hq * DK + (size_t)p.Hv * dv;
  const bool write_key = (h % G == 0) && slice == 0 && cg == 0;
  // 16-byte record stores: the buffer is 16-byte aligned, Hv and R are
  // multiples of 4, and a lane's key rows come in fours
  const bool vec_rec = RPL % 4 == 0 && (reinterpret_cast<uintptr_t>(p.su) & 15) == 0 && p.Hv % 4 == 0 && R % 4 == 0;
  for (int tb = t0; tb < t1; tb += NPF) {
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      const int t = tb + u;
      if (t >= t1) break;
      const TokenIn<T, RPL> in = ring[u];
      if (t + NPF < t1) load_tok(t + NPF, ring[u]);
      float gt = in.g, bt = in.beta;
      if (gate) {
        const float x = gt + dtb;
        gt = negA * (x > 20.f ? x : log1pf(expf(x)));   // softplus
      }
      if (p.pro.beta_logit) bt = 1.f / (1.f + expf(-bt));
      const float a = expf(gt);
      float kr[RPL];
#pragma unroll
      for (int r = 0; r < RPL; ++r) kr[r] = in.k.get(r);

      // Partial dk-reductions over this lane's rows: u = S^T k, w = S^T q, kq = k.q
      float u0 = 0.f, u1 = 0.f, u2 = 0.f, u3 = 0.f;
      float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f, kq = 0.f;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const float qr = in.q.get(r);
        u0 = fmaf(S[r].x, kr[r], u0); u1 = fmaf(S[r].y, kr[r], u1);
        u2 = fmaf(S[r].z, kr[r], u2); u3 = fmaf(S[r].w, kr[r], u3);
        w0 = fmaf(S[r].x, qr, w0); w1 = fmaf(S[r].y, qr, w1);
        w2 = fmaf(S[r].z, qr, w2); w3 = fmaf(S[r].w, qr, w3);
        kq = fmaf(kr[r], qr, kq);
      }
      // l2norm prologue: squared norms reduced together with the products above;
      // the unit vectors enter through their factors rk, rq
      float sk = 0.f, sq = 0.f;
      if (p.pro.l2norm) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
          const float qr = in.q.get(r);
          sk = fmaf(kr[r], kr[r], sk);
          sq = fmaf(qr, qr, sq);
        }
        sk = sum_rowgroups(sk);
        sq = sum_rowgroups(sq);
      }
      sum_rowgroups4(u0, u1, u2, u3);
      sum_rowgroups4(w0, w1, w2, w3);
      kq = sum_rowgroups(kq);
      float rk = 1.f;
      if (p.pro.l2norm) {
        rk = rsqrtf(sk + p.pro.eps);
        const float rq = rsqrtf(sq + p.pro.eps);
        w0 *= rq; w1 *= rq; w2 *= rq; w3 *= rq; kq *= rk * rq;
      }
      // delta = beta (v - alpha S^T k); o = scale (alpha S^T q + delta (k.q)) = scale S_t^T q
      const float d0 = bt * (in.v.get(0) - a * (rk * u0));
      const float d1 = bt * (in.v.get(1) - a * (rk * u1));
      const float d2 = bt * (in.v.get(2) - a * (rk * u2));
      const float d3 = bt * (in.v.get(3) - a * (rk * u3));
      // S = alpha S + (rk k) delta^T
      const float e0 = rk * d0, e1 = rk * d1, e2 = rk * d2, e3 = rk * d3;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        S[r].x = fmaf(kr[r], e0, a * S[r].x);
        S[r].y = fmaf(kr[r], e1, a * S[r].y);
        S[r].z = fmaf(kr[r], e2, a * S[r].z);
        S[r].w = fmaf(kr[r], e3, a * S[r].w);
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
        float* kd = rec + p.Hv + (size_t)hk * DK + row0;
        float* dd = rec + p.Hv + (size_t)p.Hq * DK + (size_t)h * dv + col;
        if (vec_rec) {   // every field this lane writes starts on a 16-byte boundary
          if (write_key) {
#pragma unroll
            for (int r = 0; r < RPL; r += 4)
              *reinterpret_cast<float4*>(kd + r) =
                  make_float4(rk * kr[r], rk * kr[r + 1], rk * kr[r + 2], rk * kr[r + 3]);
          }
          if (rg == 0) *reinterpret_cast<float4*>(dd) = make_float4(d0, d1, d2, d3);
        } else {         // records are only 4-byte aligned in general (R need not be a multiple of 4)
          if (write_key) {
#pragma unroll
            for (int r = 0; r < RPL; ++r) kd[r] = rk * kr[r];
          }
          if (rg == 0) {
            dd[0] = d0; dd[1] = d1; dd[2] = d2; dd[3] = d3;
          }
        }
      }
    }
  }

  if (p.s_out != nullptr) {
    float* so = p.s_out + ((size_t)b * p.Hv + h) * DK * dv;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      store_state4(so + (size_t)(row0 + r) * dv + col, S[r]);
  }
  if (fill) zero_fill_records(p, DK);
}

// Replay of captured records.  Records are fetched in batches (all of a
// batch's loads issued before its first record is applied) since each
// application is only two VALU operations per state element.  Geometry: column
// slices of CW columns, each split over NWR waves by dk rows (no reduction
// couples rows here); lane = rg * (CW / 4) + cg, cg a float4 of columns, rg a
// group of RPL adjacent rows.  With CW = 32 every wave load or store
// instruction moves whole 128-byte state lines.  VEC: every record field this
// lane reads starts on a 16-byte boundary (the record buffer is 16-byte aligned
// and Hv and R are multiples of 4), so keys and deltas are read as float4.
#ifndef REPLAY_SPG
#define REPLAY_SPG 2
#endif
constexpr int RB = 4;   // records per full batch; a tail of 2 and 1 follows

template <int DK, bool VEC, int CW, int NWR, int SPG>
__global__ __launch_bounds__(64 * NWR * SPG) void replay_kernel(ReplayArgs p) {
  constexpr int CPL = CW / 4, RG = 64 / CPL, RPL = DK / (NWR * RG);
  static_assert(RPL >= 1, "more row groups than rows");
  static_assert(!VEC || RPL % 4 == 0, "vector key reads need 4 rows per lane");
  const int lane = threadIdx.x & 63;
  const int cg = lane % CPL, rg = lane / CPL;
  int b, h, slice, wr;
  if (!slice_of<NWR, SPG>(p.Hv, p.dv / CW, p.B, b, h, slice, wr)) return;
  const int hk = h / (p.Hv / p.Hq);
  const int dv = p.dv;
  const int col = slice * CW + cg * 4;
  const int row0 = wr * (DK / NWR) + rg * RPL;
  int m = p.counts[b];
  m = m < 0 ? 0 : (m > p.cap ? p.cap : m);
  if (m == 0) return;

  float* st = p.state + ((size_t)b * p.Hv + h) * DK * dv;
  float4 S[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) S[r] = load_state4(st + (size_t)(row0 + r) * dv + col);

  const size_t R = (size_t)p.Hv + (size_t)p.Hq * DK + (size_t)p.Hv * dv;
  const float* base = p.su + (size_t)b * p.cap * R;
  // N records from c0 on: every load issued, then every application, with no
  // condition in between (so the loads stay hoisted and in flight together)
  auto batch = [&](auto nrec, int c0) {
    constexpr int N = decltype(nrec)::value;
    float a[N];
    float kk[N][RPL];
    float4 d[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float* rec = base + (size_t)(c0 + j) * R;
      a[j] = rec[h];
      const float* kr = rec + p.Hv + (size_t)hk * DK + row0;
      const float* dd = rec + p.Hv + (size_t)p.Hq * DK + (size_t)h * dv + col;
      if constexpr (VEC) {
#pragma unroll
        for (int r = 0; r < RPL; r += 4) {
          const float4 k4 = *reinterpret_cast<const float4*>(kr + r);
          kk[j][r] = k4.x; kk[j][r + 1] = k4.y; kk[j][r + 2] = k4.z; kk[j][r + 3] = k4.w;
        }
        d[j] = *reinterpret_cast<const float4*>(dd);
      } else {   // 4-byte aligned only
#pragma unroll
        for (int r = 0; r < RPL; ++r) kk[j][r] = kr[r];
        d[j] = make_float4(dd[0], dd[1], dd[2], dd[3]);
      }
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const float k = kk[j][r];
        // same operation order as the recurrent step: fma(k, delta, alpha * S)
        S[r].x = fmaf(k, d[j].x, a[j] * S[r].x);
        S[r].y = fmaf(k, d[j].y, a[j] * S[r].y);
        S[r].z = fmaf(k, d[j].z, a[j] * S[r].z);
        S[r].w = fmaf(k, d[j].w, a[j] * S[r].w);
      }
    }
  };
  int c = 0;
  for (; c + RB <= m; c += RB) batch(std::integral_constant<int, RB>{}, c);
  if (m - c >= 2) {
    batch(std::integral_constant<int, 2>{}, c);
    c += 2;
  }
  if (m - c >= 1) batch(std::integral_constant<int, 1>{}, c);
#pragma unroll
  for (int r = 0; r < RPL; ++r) store_state4(st + (size_t)(row0 + r) * dv + col, S[r]);
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
// Padded 1-D grid for the XCD-aware slice order: 8 * (dv / cw / spg) *
// ceil(B*Hv / 8) workgroups, each of spg column slices of cw columns.
static unsigned slice_grid(int B, int Hv, int dv, int cw, int spg) {
  const long long groups = (long long)B * Hv;
  return (unsigned)(8LL * (dv / cw / spg) * ((groups + 7) / 8));
}

// Waves per workgroup of the recurrent step: the state's slices in groups of
// up to 4.
static int slices_per_group(int dv) { return dv / DVS >= 4 ? 4 : dv / DVS; }

template <typename T, int DK, int WPG>
static hipError_t launch_rec_w(const DecodeArgs& a, hipStream_t s) {
  prof_begin(K_RECURRENT, s);
  hipLaunchKernelGGL((recurrent_step_kernel<T, DK, WPG>), dim3(slice_grid(a.B, a.Hv, a.dv, DVS, WPG)),
                     dim3(64 * WPG), 0, s, a);
  prof_end(K_RECURRENT, s);
  return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_rec_dk(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  switch (slices_per_group(a.dv)) {
    case 1: return launch_rec_w<T, DK, 1>(a, s);
    case 2: return launch_rec_w<T, DK, 2>(a, s);
    default: return launch_rec_w<T, DK, 4>(a, s);
  }
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

template <int DK, bool VEC, int CW, int NWR, int SPG>
static hipError_t launch_replay_w(const ReplayArgs& a, hipStream_t s) {
  prof_begin(K_REPLAY, s);
  hipLaunchKernelGGL((replay_kernel<DK, VEC, CW, NWR, SPG>), dim3(slice_grid(a.B, a.Hv, a.dv, CW, SPG)),
                     dim3(64 * NWR * SPG), 0, s, a);
  prof_end(K_REPLAY, s);
  return hipGetLastError();
}

// 32-column slices over two waves each (whole 128-byte lines per instruction);
// dv = 16 keeps one wave per 16-column slice.
template <int DK, bool VEC>
static hipError_t launch_replay_v(const ReplayArgs& a, hipStream_t s) {
  if (a.dv % 32 == 0) {
    if (REPLAY_SPG >= 2 && a.dv >= 64) return launch_replay_w<DK, VEC, 32, 2, REPLAY_SPG>(a, s);
    return launch_replay_w<DK, VEC, 32, 2, 1>(a, s);
  }
  return launch_replay_w<DK, VEC, 16, 1, 1>(a, s);
}

template <int DK>
static hipError_t launch_replay_dk(const ReplayArgs& a, hipStream_t s) {
  if (a.B == 0 || a.cap == 0) return hipSuccess;
  const size_t R = (size_t)a.Hv + (size_t)a.Hq * DK + (size_t)a.Hv * a.dv;
  const bool vec = (reinterpret_cast<uintptr_t>(a.su) & 15) == 0 && a.Hv % 4 == 0 && R % 4 == 0;
  if constexpr (DK >= 64) {
    if (vec) return launch_replay_v<DK, true>(a, s);
  }
  return launch_replay_v<DK, false>(a, s);
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

hipError_t launch_copy(const float* src, float* dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  prof_begin(K_COPY, s);
  hipLaunchKernelGGL(copy_kernel, dim3(stream_grid(n)), dim3(256), 0, s, src, dst, n);
  prof_end(K_COPY, s);
  return hipGetLastError();
}

}  // namespace gdn
