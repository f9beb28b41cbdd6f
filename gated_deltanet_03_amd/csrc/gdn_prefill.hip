// Chunked GDN prefill on gfx950: two or three launches on the caller's stream.
//
//  1. chunk_plan_kernel   per-sequence chunk offsets (exclusive scan of
//                         ceil(len_s / C)) into the workspace header; only for
//                         more than 64 sequences (below that every wave of
//                         kernels 2 and 3 scans the lengths itself).
//  2. chunk_prep_kernel   fully parallel over (chunk, key head): everything that
//                         does not depend on the carried state.
//  3. chunk_state_kernel  parallel over (sequence, value head, column slice),
//                         sequential over the chunks of the sequence: the state
//                         contractions, with S kept in fp32 accumulators.
//
// The chunked form of the gated delta rule (sources: [executorch issue 23097,
// "Enable the native Kev example on NVIDIA GPUs ...", "Work to cover"]: chunked
// prefill with explicit initial/final state and FP32 recurrence; the replay
// identity of [onnxruntime PR 32767, "Changes"] fixes decay/key/delta).  For a
// chunk of C tokens starting from state S0, with G_i the in-chunk cumulative
// sum of g and gamma_i = exp(G_i):
//
//   L_ij  = beta_i exp(G_i - G_j) k_i.k_j        (j < i)
//   A'    = (I + L)^-1 diag(beta)                UT transform (kernel 2)
//   MP_ij = exp(G_i - G_j) q_i.k_j               (j <= i)     (kernel 2)
//   Delta = A' (V - diag(gamma) K S0)                          (kernel 3)
//   O     = scale (diag(gamma) Q S0 + MP Delta)                (kernel 3)
//   S_end = gamma_last S0 + K^T diag(exp(G_last - G)) Delta    (kernel 3)
//
// Only exp(G_i - G_j) with j <= i, exp(G_i) and exp(G_last - G_j) are ever
// formed, all <= 1 for non-positive g, so nothing overflows in 16-bit operands.
// Kernel 3 never forms the W = A diag(beta gamma) K of the WY form: it applies
// A' to the state-dependent right-hand side, so its chain per chunk is
// K*S -> A'*X -> K^T*Delta, all on MFMA with fp32 accumulation.
//
// A' and MP are written in fragment-native order (gdn_mfma.h), lower-triangular
// 16x32 blocks only: block (r, kb) with kb <= r/2, i.e. 6 blocks per matrix.
#include <atomic>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {

constexpr int NTRI = 6;   // lower-triangular 16x32 blocks of a 64x64 matrix
constexpr int FRAG = 512; // elements per fragment-native block (64 lanes x 8)

__device__ __forceinline__ int tri_idx(int r, int kb) { return r < 2 ? r : 2 * r - 2 + kb; }
__device__ __forceinline__ void tri_rc(int f, int& r, int& kb) {
  if (f < 2) { r = f; kb = 0; } else { r = (f + 2) >> 1; kb = f & 1; }
}

// ---------------------------------------------------------------------------
// 1. plan
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_plan_kernel(PrefillArgs p) {
  __shared__ int scan[256];
  __shared__ int carry_s;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < p.B; base += 256) {
    const int s = base + threadIdx.x;
    int n = 0;
    if (s < p.B) {
      int t0, t1;
      seq_range(p.cu, p.T, p.total, s, t0, t1);
      n = (t1 - t0 + p.chunk - 1) / p.chunk;
    }
    scan[threadIdx.x] = n;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int v = (int)threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    const int carry = carry_s;
    if (s < p.B) {
      long long excl = (long long)carry + scan[threadIdx.x] - n;
      p.chunk_offsets[s] = (int)(excl < p.max_chunks ? excl : p.max_chunks);
    }
    __syncthreads();
    if (threadIdx.x == 255) {
      long long c = (long long)carry + scan[255];
      carry_s = (int)(c < p.max_chunks ? c : p.max_chunks);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) p.chunk_offsets[p.B] = carry_s;
  __syncthreads();   // the offsets written above are visible to the whole workgroup
  // per-chunk (first token, length), one thread per chunk: the sequence of
  // chunk c is the last s with offsets[s] <= c; entries past the last chunk
  // get length 0
  const int nch = carry_s;
  for (int c = threadIdx.x; c < p.max_chunks; c += 256) {
    int a = 0, n = 0;
    if (c < nch) {
      int lo = 0, hi = p.B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.chunk_offsets[mid] <= c) lo = mid; else hi = mid - 1;
      }
      int t0, t1;
      seq_range(p.cu, p.T, p.total, lo, t0, t1);
      a = t0 + (c - p.chunk_offsets[lo]) * p.chunk;
      n = min(p.chunk, t1 - a);
    }
    p.chunk_info[2 * c] = a;
    p.chunk_info[2 * c + 1] = n;
  }
}

// The same plan for at most 64 sequences, computed by one wave at the start of
// the prep and state kernels (which then need no plan launch): lane s < B gets
// the saturated exclusive chunk offset of sequence s, every lane the saturated
// chunk total.  Offsets, totals and the chunk -> (first token, length) map are
// those chunk_plan_kernel writes.
constexpr int kWavePlanMaxSeqs = 64;

template <int C>
__device__ __forceinline__ void wave_plan(const PrefillArgs& p, int lane, int& excl, int& total) {
  int n = 0;
  if (lane < p.B) {
    int t0, t1;
    seq_range(p.cu, p.T, p.total, lane, t0, t1);
    n = (t1 - t0 + C - 1) / C;
  }
  int x = n;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  excl = min(x - n, p.max_chunks);
  total = min(__shfl(x, 63), p.max_chunks);
}

// First token and length of global chunk gc from a wave plan (length 0 past the
// last chunk): its sequence is the last s with offset <= gc.
template <int C>
__device__ __forceinline__ int2 wave_plan_chunk(const PrefillArgs& p, int lane, int excl, int total, int gc) {
  if (gc >= total) return make_int2(0, 0);
  const unsigned long long m = __ballot(lane < p.B && excl <= gc);
  const int s = 63 - __clzll((long long)m);
  const int off = __shfl(excl, s);
  int t0, t1;
  seq_range(p.cu, p.T, p.total, s, t0, t1);
  const int a = t0 + (gc - off) * C;
  return make_int2(a, min(C, t1 - a));
}

template <typename T>
struct Block {  // views of one (chunk, value head) workspace block
  T* A;        // NTRI fragment-native blocks of A'
  T* MP;       // NTRI fragment-native blocks of MP
  float* gk;   // [64] gamma_i * rk_i
  float* tk;   // [64] exp(G_last - G_i) * rk_i
  float* gq;   // [64] gamma_i * rq_i
  float* gl;   // [64] gamma_last (every entry)
  __device__ Block(void* base, size_t gc, int Hv, int h) {
    char* b = static_cast<char*>(base) + (gc * Hv + h) * (2 * NTRI * FRAG * sizeof(T) + 1024);
    A = reinterpret_cast<T*>(b);
    MP = A + NTRI * FRAG;
    gk = reinterpret_cast<float*>(MP + NTRI * FRAG);
    tk = gk + 64;
    gq = gk + 128;
    gl = gk + 192;
  }
};

// Input prologue helpers (fp32).  softplus(x) = log(1 + e^x), returned as x
// itself above 20 where the two agree to fp32 precision.
__device__ __forceinline__ float softplus_f(float x) { return x > 20.f ? x : log1pf(expf(x)); }
__device__ __forceinline__ float gate_log_decay(const Prologue& pr, int h, float a) {
  const float dtb = pr.dt_bias != nullptr ? pr.dt_bias[h] : 0.f;
  return -expf(pr.A_log[h]) * softplus_f(a + dtb);
}
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// Sum of squares of the 8 values of a fragment (16-bit) or of its two fp32 halves.
template <typename T>
__device__ __forceinline__ float frag_sumsq(const Frag<T>& f) {
  float s = 0.f;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s = fmaf(f.lo[j], f.lo[j], fmaf(f.hi[j], f.hi[j], s));
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = Elem<T>::to_f(f.v[j]);
      s = fmaf(x, x, s);
    }
  }
  return s;
}

// ---------------------------------------------------------------------------
// 2. chunk prep: one wave per (chunk, value head), 1-D grid.
//
//    K and Q fragments are read straight from global memory (8 consecutive dk
//    entries = one 16-byte load per lane) and the Gram products K K^T and K Q^T
//    run on MFMA with fp32 accumulation.  MP fragments come straight out of the
//    K Q^T accumulators: lane (g, n) of tile (c, r) of K Q^T holds
//    P[16r + n][16c + 4g + q], which is the A fragment of block (r, c) of Q K^T.
//
//    UT inverse X = (I + L)^-1 by 16 x 16 blocks, all in fp32:
//      * diagonal blocks X_jj = (I + L_jj)^-1: back-substitution on the VALU,
//        lane (b, r) computing row r of block b (the only LDS traffic);
//      * off-diagonal blocks from X N = I, N = I + L:
//          X_ij = -(sum_{k=j+1..i} X_ik L_kj) X_jj,
//        carried transposed, Z_ij = X_ij^T = -Z_jj sum_k L_kj^T Z_ik, on fp32
//        MFMA with every operand already in accumulator layout (an accumulator
//        tile E is the A operand of E^T and the B operand of E).
//    Lane (g, n) of Z_ij holds X[16i + n][16j + 4g + q], so A' = X diag(beta)
//    is written in fragment order straight from the Z tiles.
//    Rows past a sequence's end see zero keys, queries and beta, so their L and
//    MP entries vanish and their rows/columns of A' are exactly zero.
// ---------------------------------------------------------------------------
constexpr int DS = 20;   // row stride (floats) of the 16 x 16 diagonal blocks in LDS

// Fragment of K or Q row `row` (a pointer to its first element), 32-wide dk
// block kb, in the contiguous slot order of the state kernel (slots 8g..8g+7 =
// dk 32kb + 8g .. +7); dk = 16 puts dk 4g..4g+3 in the lo half, zero in the hi.
// Loads are unconditional (callers clamp the row into the chunk) so a wave's
// loads issue back to back; rows past the chunk end are zeroed afterwards.
template <typename T, int DK>
__device__ __forceinline__ Frag<T> gload_frag(const T* __restrict__ row, int kb, int g4) {
  Frag<T> f = zero_frag<T>();
  if constexpr (DK >= 32) {
    f = load_frag_native<T>(row + 32 * kb + 8 * g4);
  } else {
    if constexpr (sizeof(T) == 4) {
      f.lo = *reinterpret_cast<const f32x4*>(row + 4 * g4);
    } else {
      const auto a = *reinterpret_cast<const typename Half4<T>::type*>(row + 4 * g4);
      f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
    }
  }
  return f;
}

// Zero a fragment without branching (rows past the chunk end).
template <typename T>
__device__ __forceinline__ Frag<T> keep_if(const Frag<T>& f, bool keep) {
  Frag<T> r;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) { r.lo[j] = keep ? f.lo[j] : 0.f; r.hi[j] = keep ? f.hi[j] : 0.f; }
  } else {
    const auto u = __builtin_bit_cast(uint4, f.v);
    const uint4 z = keep ? u : make_uint4(0, 0, 0, 0);
    r.v = __builtin_bit_cast(decltype(r.v), z);
  }
  return r;
}

template <typename T, int DK>
__device__ __forceinline__ void gram_mma(f32x4& acc, const Frag<T>& a, const Frag<T>& b) {
  if constexpr (DK >= 32) mma<T>(acc, a, b); else mma_lo<T>(acc, a, b);
}

// acc += E^T F for 16 x 16 fp32 tiles E, F given in accumulator layout (lane
// (g, n) holds row 4g + q, column n): contraction index 4g + s in step s.
__device__ __forceinline__ void mma_tn(f32x4& acc, const f32x4& e, const f32x4& f) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(e[s], f[s], acc, 0, 0, 0);
}

// exp2 on the transcendental unit (1 ulp; results below 2^-126 flush to zero,
// which only drops terms already below fp32 resolution of the sums they enter).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T, int DK, int C, int HPW>
__global__ __launch_bounds__(64, (sizeof(T) == 4 && DK == 128) ? 1 : ((HPW == 1 && DK == 128 && C == 64) ? 2 : 3)) void chunk_prep_kernel(PrefillArgs p) {
  constexpr int nrt = C / 16;
  constexpr int NKB = DK >= 32 ? DK / 32 : 1;
  constexpr float LOG2E = 1.4426950408889634f;
  __shared__ __align__(16) float Ld[4 * 16 * DS];        // diagonal blocks of L, one head at a time
  __shared__ __align__(16) float Xd[4 * 16 * DS];        // their inverses, row-major
  // log2 cumulative decay G_i log2(e) with the log2 inverse norms folded in:
  // rows of L (+ log2 rk_i), columns of L and MP (- log2 rk_j), rows of MP
  // (+ log2 rq_i); all three are G log2(e) without the l2norm prologue
  __shared__ __align__(16) float GR[HPW][64];
  __shared__ __align__(16) float GC[HPW][64];
  __shared__ __align__(16) float GQ[HPW][64];
  __shared__ __align__(16) float Bs[HPW][64];            // beta
  __shared__ __align__(16) float Rk[64], Rq[64];         // inverse norms of k_i, q_i

  // One item = (chunk, HPW value heads that share a key head).  XCD-aware
  // order: workgroup w runs on XCD w % 8; each XCD gets a contiguous run of
  // items so neighbouring key heads' rows share an L2.
  const int npairs = p.Hv / HPW;
  const int nitems = p.max_chunks * npairs;
  const int per = (nitems + 7) >> 3;
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= nitems) return;
  const int gc = item / npairs, h0 = (item % npairs) * HPW;
  const int lane = threadIdx.x;
  int2 info;
  if (p.B <= kWavePlanMaxSeqs) {
    int excl, total;
    wave_plan<C>(p, lane, excl, total);
    info = wave_plan_chunk<C>(p, lane, excl, total, gc);
  } else {
    info = reinterpret_cast<const int2*>(p.chunk_info)[gc];
  }
  const int t0 = __builtin_amdgcn_readfirstlane(info.x), len = __builtin_amdgcn_readfirstlane(info.y);
  if (len <= 0) return;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int hk = h0 / (p.Hv / p.Hq);

  // ---- K and Q fragments of every row tile (one batch of loads) ------------
  const T* kp = static_cast<const T*>(p.k);
  const T* qp = static_cast<const T*>(p.q);
  auto row_off = [&](int r) { return ((size_t)(t0 + min(r, len - 1)) * p.Hq + hk) * DK; };
  Frag<T> kf[nrt][NKB], qa[nrt][NKB];
#pragma unroll
  for (int r = 0; r < nrt; ++r)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      kf[r][kb] = gload_frag<T, DK>(kp + row_off(16 * r + i16), kb, g4);
      qa[r][kb] = gload_frag<T, DK>(qp + row_off(16 * r + i16), kb, g4);
    }

  // ---- l2norm prologue: inverse norms of the chunk's k and q rows (1 for
  //      rows past the chunk end), shared by the key head's value heads -------
  float rk = 1.f, rq = 1.f;
  if (p.pro.l2norm) {
    Rk[lane] = 1.f;
    Rq[lane] = 1.f;
#pragma unroll
    for (int r = 0; r < nrt; ++r) {
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sk += frag_sumsq<T>(kf[r][kb]);
        sq += frag_sumsq<T>(qa[r][kb]);
      }
      // the four lanes holding parts of row 16r + i16 are i16 + 16 g
      sk += __shfl_xor(sk, 16);
      sk += __shfl_xor(sk, 32);
      sq += __shfl_xor(sq, 16);
      sq += __shfl_xor(sq, 32);
      const int row = 16 * r + i16;
      if (g4 == 0 && row < len) {
        Rk[row] = 1.f / sqrtf(sk + p.pro.eps);
        Rq[row] = 1.f / sqrtf(sq + p.pro.eps);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    rk = Rk[lane];
    rq = Rq[lane];
  }
  const float lk = p.pro.l2norm ? log2f(rk) : 0.f, lq = p.pro.l2norm ? log2f(rq) : 0.f;

  // ---- per head: gates, log2 cumulative decay, beta and the block factors ---
#pragma unroll
  for (int v = 0; v < HPW; ++v) {
    const int h = h0 + v;
    const size_t gi = (size_t)(t0 + min(lane, len - 1)) * p.Hv + h;
    float gv = lane < len ? p.g[gi] : 0.f;
    float bv = lane < len ? p.beta[gi] : 0.f;
    if (p.pro.A_log != nullptr && lane < len) gv = gate_log_decay(p.pro, h, gv);
    if (p.pro.beta_logit && lane < len) bv = sigmoid_f(bv);
    float x = gv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    const float glast = __shfl(x, C - 1);
    GR[v][lane] = x * LOG2E + lk;
    GC[v][lane] = x * LOG2E - lk;
    GQ[v][lane] = x * LOG2E + lq;
    Bs[v][lane] = bv;
    Block<T> blk(p.chunk_data, (size_t)gc, p.Hv, h);
    const float gam = expf(x);
    blk.gk[lane] = gam * rk;
    blk.tk[lane] = expf(glast - x) * rk;
    blk.gq[lane] = gam * rq;
    blk.gl[lane] = expf(glast);
  }
#pragma unroll
  for (int r = 0; r < nrt; ++r)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      kf[r][kb] = keep_if<T>(kf[r][kb], 16 * r + i16 < len);
      qa[r][kb] = keep_if<T>(qa[r][kb], 16 * r + i16 < len);
    }

  // ---- MP = exp(G_i - G_j) (Q K^T)_ij, j <= i, for every head from one
  //      Gram tile: lane (g, n) of K_c Q_r^T holds P[16r + n][16c + 4g + q] ----
#pragma unroll
  for (int r = 0; r < nrt; ++r) {
    f32x4 kq[nrt];
#pragma unroll
    for (int c = 0; c <= r; ++c) {
      kq[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) gram_mma<T, DK>(kq[c], kf[c][kb], qa[r][kb]);
    }
    const int i = 16 * r + i16;
#pragma unroll
    for (int v = 0; v < HPW; ++v) {
      const float gi = GQ[v][i];
      f32x4 mp[nrt];
#pragma unroll
      for (int c = 0; c <= r; ++c) {
        const f32x4 gj = *reinterpret_cast<const f32x4*>(&GC[v][16 * c + 4 * g4]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = 16 * c + 4 * g4 + q;
          mp[c][q] = j <= i ? fast_exp2(gi - gj[q]) * kq[c][q] : 0.f;
        }
      }
      Block<T> blk(p.chunk_data, (size_t)gc, p.Hv, h0 + v);
#pragma unroll
      for (int kb = 0; kb <= r / 2; ++kb) {
        const f32x4 hi = 2 * kb + 1 <= r ? mp[2 * kb + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
        store_frag_native<T>(blk.MP + (tri_idx(r, kb) * 64 + lane) * 8, make_frag<T>(mp[2 * kb], hi));
      }
    }
  }
#pragma unroll
  for (int v = 0; v < HPW; ++v) {
    Block<T> blk(p.chunk_data, (size_t)gc, p.Hv, h0 + v);
#pragma unroll
    for (int f = 0; f < NTRI; ++f) {
      int r, kb;
      tri_rc(f, r, kb);
      if (r >= nrt) store_frag_native<T>(blk.MP + (f * 64 + lane) * 8, zero_frag<T>());
    }
  }

  // ---- L_ij = beta_i exp(G_i - G_j) (K K^T)_ij, j < i, for every head:
  //      off-diagonal tiles stay in registers; the diagonal K K^T tiles are kept
  //      and scaled into LDS per head just before that head's inverse (one LDS
  //      buffer for all heads keeps the wave's LDS small enough for three waves
  //      per SIMD) ---------------------------------------------------------------
  f32x4 Lt[HPW][nrt][nrt];   // [v][r][c], c < r used
  f32x4 kkd[nrt];            // diagonal tiles of K K^T
#pragma unroll
  for (int r = 0; r < nrt; ++r) {
#pragma unroll
    for (int c = 0; c <= r; ++c) {
      f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) gram_mma<T, DK>(kk, kf[r][kb], kf[c][kb]);
      if (c == r) {
        kkd[r] = kk;
        continue;
      }
#pragma unroll
      for (int v = 0; v < HPW; ++v) {
        const f32x4 gi = *reinterpret_cast<const f32x4*>(&GR[v][16 * r + 4 * g4]);
        const f32x4 bi = *reinterpret_cast<const f32x4*>(&Bs[v][16 * r + 4 * g4]);
        const float gj = GC[v][16 * c + i16];
        f32x4 l;
#pragma unroll
        for (int q = 0; q < 4; ++q) l[q] = bi[q] * fast_exp2(gi[q] - gj) * kk[q];
        Lt[v][r][c] = l;
      }
    }
  }

#pragma unroll
  for (int v = 0; v < HPW; ++v) {
    // ---- this head's diagonal blocks of L into LDS (strictly lower part) ------
#pragma unroll
    for (int r = 0; r < nrt; ++r) {
      const f32x4 gi = *reinterpret_cast<const f32x4*>(&GR[v][16 * r + 4 * g4]);
      const f32x4 bi = *reinterpret_cast<const f32x4*>(&Bs[v][16 * r + 4 * g4]);
      const float gj = GC[v][16 * r + i16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool below = i16 < 4 * g4 + q;
        Ld[(r * 16 + 4 * g4 + q) * DS + i16] = below ? bi[q] * fast_exp2(gi[q] - gj) * kkd[r][q] : 0.f;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): every lane's entries are in LDS
    __builtin_amdgcn_wave_barrier();
    // ---- diagonal blocks: lane (b, r) computes row r of (I + L_bb)^-1 by
    //      back-substitution, X (I + L) = I, over k = 15 .. 1 -----------------
    {
      const int b = lane >> 4, r = lane & 15;
      const float* Lb = Ld + b * 16 * DS;
      float x[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = (j == r) ? 1.f : 0.f;
#pragma unroll
      for (int k = 15; k >= 1; --k) {
        const float xk = x[k];
#pragma unroll
        for (int j4 = 0; j4 < k; j4 += 4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lb + k * DS + j4);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (j4 + u < k) x[j4 + u] = fmaf(-l4[u], xk, x[j4 + u]);
        }
      }
      // the previous head's reads of Xd are complete (LDS is in order per wave)
      float* xr = Xd + (b * 16 + r) * DS;
#pragma unroll
      for (int j = 0; j < 16; j += 4) *reinterpret_cast<f32x4*>(xr + j) = f32x4{x[j], x[j + 1], x[j + 2], x[j + 3]};
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the whole wave's rows are in LDS
    __builtin_amdgcn_wave_barrier();

    // ---- off-diagonal blocks row by row: Z[i][j] = X_ij^T = -Z_jj sum_k
    //      L_kj^T Z[i][k]; a finished row goes straight out as A' fragments ---
    f32x4 Xa[nrt], Zd[nrt];   // X_jj in accumulator layout; Z_jj
#pragma unroll
    for (int j = 0; j < nrt; ++j) {
      const float* xb = Xd + j * 16 * DS;
#pragma unroll
      for (int q = 0; q < 4; ++q) Xa[j][q] = xb[(4 * g4 + q) * DS + i16];
      Zd[j] = *reinterpret_cast<const f32x4*>(xb + i16 * DS + 4 * g4);
    }
    Block<T> blk(p.chunk_data, (size_t)gc, p.Hv, h0 + v);
#pragma unroll
    for (int i = 0; i < nrt; ++i) {
      f32x4 Z[nrt];
      Z[i] = Zd[i];
#pragma unroll
      for (int j = i - 1; j >= 0; --j) {
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = j + 1; k <= i; ++k) mma_tn(P, Lt[v][k][j], Z[k]);
        f32x4 zij = {0.f, 0.f, 0.f, 0.f};
        mma_tn(zij, Xa[j], P);
        Z[j] = -zij;
      }
      // A' = X diag(beta): lane (g, n) of Z[j] holds X[16i + n][16j + 4g + q]
#pragma unroll
      for (int kb = 0; kb <= i / 2; ++kb) {
        const int c0 = 2 * kb, c1 = 2 * kb + 1;
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(&Bs[v][16 * c0 + 4 * g4]);
        const f32x4 lo = Z[c0] * b0;
        f32x4 hi = {0.f, 0.f, 0.f, 0.f};
        if (c1 <= i) {
          const f32x4 b1 = *reinterpret_cast<const f32x4*>(&Bs[v][16 * c1 + 4 * g4]);
          hi = Z[c1] * b1;
        }
        store_frag_native<T>(blk.A + (tri_idx(i, kb) * 64 + lane) * 8, make_frag<T>(lo, hi));
      }
    }
#pragma unroll
    for (int f = 0; f < NTRI; ++f) {
      int r, kb;
      tri_rc(f, r, kb);
      if (r >= nrt) store_frag_native<T>(blk.A + (f * 64 + lane) * 8, zero_frag<T>());
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // this head's Xd reads are done before the next head writes it
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// 3. state pass: one workgroup per (sequence, value head, slice of 16*NG columns),
//    2*NG compute waves (NG = 1, 2 or 4 column groups of 16) plus NDW load-issuing
//    waves.
//
//    Each 16-column group of the slice is served by two waves: a chain wave
//    (waves 0..NG-1) owning the fp32 state of those columns and
//    running the sequential part, K*S -> X -> A'*X -> S update; and an output
//    wave (waves NG..2NG-1) running everything off that path: Q*S, the K^T fragments,
//    MP*Delta and the o stores.  The state crosses over as bf16/f16 fragments
//    (written by the chain wave after each update), Delta goes the other way.
//
//    Chunk inputs are staged with direct global->LDS loads (one wave
//    instruction writes 64 lanes x 16 bytes contiguously at a wave-uniform LDS
//    address), double-buffered so chunk c+1 streams in while chunk c computes;
//    with dedicated load-issuing waves and room for a third stage, chunks c+1
//    and c+2 are both in flight, so a load has two chunk steps to land.
//    Row-major tiles are XOR-swizzled per 16-byte piece (piece p of row r lives
//    at piece p ^ (r mod pieces-per-row)) so fragment reads of 16 consecutive
//    rows hit distinct banks.  Rows past a sequence's end are loaded from its
//    last row instead of being zeroed: A' and MP carry exact zeros in those rows
//    and columns, so the finite stand-in values never reach an output.
//
//    Per chunk: barrier TOP (chunk c landed; buffers of chunk c-1 free),
//    chain: KS, X, Delta -> exchange; output: QS, K^T -> LDS; barrier MID;
//    chain: S update, next state fragments -> exchange; output: O, stores.
// ---------------------------------------------------------------------------
// One wave instruction: every lane copies 16 bytes from its src to
// lds + 16 * lane (lds must be wave-uniform).
__device__ __forceinline__ void dma16(const void* src, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// The state is carried with its dk rows permuted inside each 32-row block:
// state row 32kb + 16h + 4g + j holds dk index 32kb + 8g + 4h + j.  A lane's 8
// contraction slots of a K or Q fragment (rows 4g..4g+3 of the lo and hi tile of
// the block, the order an accumulator hands them over) then map to 8
// consecutive dk entries: one 16-byte read.  K * S is unchanged because K's
// columns are read through the same permutation.  A 16-row block (dk = 16)
// keeps the identity order.
template <int DK>
__device__ __forceinline__ int perm_dk(int r) {
  if constexpr (DK < 32) {
    return r;
  } else {
    const int kb = r >> 5, h = (r >> 4) & 1, g = (r >> 2) & 3, j = r & 3;
    return 32 * kb + 8 * g + 4 * h + j;
  }
}

// Row-dependent XOR swizzle of the 16-byte pieces of a K/Q tile row: piece p of
// row r is stored at slot p ^ kq_swz(r).  Any bijection of r mod 16 keeps the
// fragment reads (16 consecutive rows, one piece each) on distinct banks; for
// 16-piece rows read by transpose reads (TR) the two 2-bit halves of r are swapped so that the transpose
// reads of K^T fragments (4 rows x 4 pieces per 16 lanes) also hit 16
// distinct pieces.
template <int PPR, bool TR>
__device__ __forceinline__ int kq_swz(int r) {
  if constexpr (TR && PPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return r % PPR;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte chunks addressed by lanes
// 4j + i / 4, j = 0..3 (its element j).
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// LDS plan of the state kernel.  TR: K^T comes from transpose reads, so no K^T
// region.  DED: dedicated load-issuing waves, which keep chunk inputs three
// stages deep when they fit (two chunks in flight while one is computed), else
// two; chain-issued loads use at most two.
template <typename T, int DK, int NG, bool TR, bool DED>
struct StateSmem {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int SW = 16 * NG;                // columns per workgroup (NG groups of 16)
  static constexpr int PER = 16 / ES;               // elements per 16-byte piece
  static constexpr int PPR = DK / PER;              // pieces per K/Q row
  static constexpr int ROWB = DK * ES;              // bytes per K/Q row
  static constexpr int NST = DK / 16;               // state row tiles
  static constexpr int NSB = (NST + 1) / 2;         // state fragments (32-row blocks)
  static constexpr int NKT = 2 * NST;               // K^T fragments (dk tile, token block)
  static constexpr int FB = FRAG * ES;              // bytes per fragment block
  static constexpr int KB = 64 * ROWB;              // K (or Q) tile bytes
  static constexpr int VB = 64 * SW * ES;           // V tile bytes (up to SW columns)
  static constexpr int AB = 2 * NTRI * FB;          // A' and MP fragments
  static constexpr int STAGE = 2 * KB + VB + AB + 1024;
  static constexpr int KTB = TR ? 0 : NKT * FB;     // K^T fragments
  static constexpr int SXB = NG * NSB * FB;         // state fragments, one set per column group
  static constexpr int DXB = NG * 2 * FB;           // Delta fragments, one set per column group
  static constexpr int FIXED = KTB + SXB + DXB;
  static constexpr int NBUF = (DED && 3 * STAGE + FIXED <= 160 * 1024) ? 3 : (2 * STAGE + FIXED <= 160 * 1024 ? 2 : 1);
  static constexpr size_t total = (size_t)NBUF * STAGE + FIXED;
  // byte offsets inside one stage buffer
  static constexpr int OK_ = 0, OQ = KB, OV = 2 * KB, OA = 2 * KB + VB, OG = 2 * KB + VB + AB;
};

template <typename T, int DK, int C, int NG, int NDW, bool EMIT>
__global__ __launch_bounds__(64 * (2 * NG + NDW)) void chunk_state_kernel(PrefillArgs p) {
  // K^T fragments by transpose reads of the K tile (16-bit, dk = 128, both
  // 16-token tiles of each 32-token block present); else built by the output
  // waves with permutation products
  constexpr bool TRK = sizeof(T) == 2 && DK == 128 && C >= 32;
  // three stages need dedicated loaders; the state-emitting variant keeps two
  // (the third costs it a register spill)
  using SM = StateSmem<T, DK, NG, TRK, (NDW > 0 && !EMIT)>;
  constexpr int SW = SM::SW;
  constexpr int nrt = C / 16;
  constexpr int NST = SM::NST, NSB = SM::NSB, PER = SM::PER, PPR = SM::PPR, ES = SM::ES;
  constexpr int RPI_K = 64 / PPR;         // K rows per DMA instruction
  constexpr int NA = SM::AB / 1024;       // 1 KB pieces of the A' and MP region
  // 16-bit inputs with dedicated loaders: the chain fetches A' into its
  // registers and only MP is staged (fp32 A' fragments are too wide for the
  // chain's registers; where the chain waves issue the loads themselves the
  // staged form measured faster).  The state-emitting variant stages A' too:
  // its chain waves store every chunk's state, and a wait for register-held A'
  // would also wait for those stores.
  constexpr bool AREG = ES == 2 && NDW > 0 && !EMIT;
  constexpr int NA0 = AREG ? NA / 2 : 0;  // first staged piece of the A'/MP region
  extern __shared__ __align__(16) unsigned char smem_raw[];
  unsigned char* fixed = smem_raw + SM::NBUF * SM::STAGE;
  T* KT = reinterpret_cast<T*>(fixed);
  T* SX = reinterpret_cast<T*>(fixed + SM::KTB);
  T* DX = reinterpret_cast<T*>(fixed + SM::KTB + SM::SXB);

  // XCD-aware order: workgroup w runs on XCD w % 8.  The workgroups reading the
  // same keys and queries -- every column slice of every value head of one
  // (sequence, key head) group -- are given ids that agree mod 8, so they share
  // one L2; groups are still dispatched in sequence order.
  const int G = p.Hv / p.Hq, nsl = (p.dv + SW - 1) / SW, GS = nsl * G;
  const int xcd = (int)(blockIdx.x & 7), rnd = (int)(blockIdx.x >> 3);
  const int grp = (rnd / GS) * 8 + xcd, mem = rnd % GS;
  if (grp >= p.Hq * p.B) return;
  const int s = grp / p.Hq, slice = mem % nsl, h = (grp % p.Hq) * G + mem / nsl;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const bool chain = wave < NG;
  // NDW > 0: waves 2NG.. only issue the chunk loads (they stall on the load
  // address unit, which would otherwise stall the chain); NDW = 0: the chain
  // waves issue them
  const bool dmaw = NDW > 0 && wave >= 2 * NG;
  const bool issuer = NDW > 0 ? dmaw : chain;
  const int wq = wave & (NG - 1);                               // column group (load slot for loaders)
  // the chain waves carry the sequential dependence: let them win instruction
  // arbitration against any wave that shares their SIMD
  if (chain) __builtin_amdgcn_s_setprio(2);
  const int ncols = min(SW, p.dv - SW * slice);
  const int col0 = SW * slice + 16 * wq;
  const bool active = 16 * wq < ncols;    // slices narrower than SW columns idle some groups
  const int i16 = lane & 15, g4 = lane >> 4;
  const int hk = h / (p.Hv / p.Hq);
  const int dv = p.dv;
  const int pprv = ncols / PER;           // pieces per V row (power of two)
  const int rowbv = ncols * ES;           // bytes per V row
  const int rpiv = 64 / pprv;             // V rows per DMA instruction

  int st0, st1;
  seq_range(p.cu, p.T, p.total, s, st0, st1);
  int cbeg, nch;
  if (p.B <= kWavePlanMaxSeqs) {
    int excl, total;
    wave_plan<C>(p, lane, excl, total);
    // wave-uniform by construction; readfirstlane keeps them in scalar registers
    cbeg = __builtin_amdgcn_readfirstlane(__shfl(excl, s));
    nch = __builtin_amdgcn_readfirstlane((s + 1 < p.B ? __shfl(excl, s + 1) : total)) - cbeg;
  } else {
    cbeg = p.chunk_offsets[s];
    nch = p.chunk_offsets[s + 1] - cbeg;
  }

  const T* kp = static_cast<const T*>(p.k);
  const T* qp = static_cast<const T*>(p.q);
  const T* vp = static_cast<const T*>(p.v);
  T* op = static_cast<T*>(p.o);

  // ---- DMA slots of chain wave wq (compile-time counts, loop-invariant 32-bit
  //      byte offsets from the chunk's wave-uniform base pointers, so each DMA
  //      is one scalar-base + vector-offset load) -------------------------------
  constexpr int KPW = (PPR + NG - 1) / NG, VPW = (SW / PER + NG - 1) / NG, APW = (NA - NA0 + NG - 1) / NG;
  int krow[KPW], vrow[VPW];
  uint32_t kvo[KPW], vvo[VPW];
#pragma unroll
  for (int m = 0; m < KPW; ++m) {
    const int j = wq + NG * m;
    const int r = RPI_K * j + lane / PPR;
    const int pp = (lane % PPR) ^ kq_swz<PPR, TRK>(r);      // logical piece stored at this slot
    krow[m] = r;
    kvo[m] = (uint32_t)(((r * p.Hq + hk) * DK + pp * PER) * ES);
  }
#pragma unroll
  for (int m = 0; m < VPW; ++m) {
    const int j = wq + NG * m;
    const int r = rpiv * j + lane / pprv;
    const int pp = (lane % pprv) ^ (r % pprv);
    vrow[m] = r;
    vvo[m] = (uint32_t)(((r * p.Hv + h) * dv + SW * slice + pp * PER) * ES);
  }
  // Fewest DMA instructions any issuing wave puts in flight per chunk (K, Q and
  // A'/MP slots; V and the factor vector counted as none).  With three stage
  // buffers an issuer waits for chunk c with vmcnt(LB): loads return in issue
  // order, so at most LB outstanding leaves none of chunk c's.
  constexpr int LB = [] {
    int mn = 63;
    for (int w = 0; w < NG; ++w) {
      int n = 0;
      for (int m = 0; m < KPW; ++m) n += (w + NG * m < PPR) ? 2 : 0;
      for (int m = 0; m < APW; ++m) n += (NA0 + w + NG * m < NA) ? 1 : 0;
      mn = n < mn ? n : mn;
    }
    return mn;
  }();
  static_assert(LB >= 0 && LB <= 63, "vmcnt immediate");
  const int kq_row_stride = p.Hq * DK, v_row_stride = p.Hv * dv;
  auto issue = [&](int c, int buf) {
    const int t0 = st0 + c * C;
    const int last = min(C, st1 - t0) - 1;
    unsigned char* sb = smem_raw + buf * SM::STAGE;
    const char* kc = reinterpret_cast<const char*>(kp + (size_t)t0 * kq_row_stride);
    const char* qc = reinterpret_cast<const char*>(qp + (size_t)t0 * kq_row_stride);
    const char* vc = reinterpret_cast<const char*>(vp + (size_t)t0 * v_row_stride);
    Block<T> blk(p.chunk_data, (size_t)(cbeg + c), p.Hv, h);
    if (last == C - 1) {   // full chunk: no row needs clamping
#pragma unroll
      for (int m = 0; m < KPW; ++m) {
        const int j = wq + NG * m;
        if (j < PPR) {
          dma16(kc + kvo[m], sb + SM::OK_ + j * 1024);
          dma16(qc + kvo[m], sb + SM::OQ + j * 1024);
        }
      }
#pragma unroll
      for (int m = 0; m < VPW; ++m) {
        const int j = wq + NG * m;
        if (j < pprv) dma16(vc + vvo[m], sb + SM::OV + j * 1024);
      }
    } else {               // last chunk of a sequence: rows past its end repeat its last row
#pragma unroll
      for (int m = 0; m < KPW; ++m) {
        const int j = wq + NG * m;
        if (j < PPR) {
          const int64_t d = (int64_t)(min(krow[m], last) - krow[m]) * kq_row_stride * ES;
          dma16(kc + kvo[m] + d, sb + SM::OK_ + j * 1024);
          dma16(qc + kvo[m] + d, sb + SM::OQ + j * 1024);
        }
      }
#pragma unroll
      for (int m = 0; m < VPW; ++m) {
        const int j = wq + NG * m;
        if (j < pprv) dma16(vc + vvo[m] + (int64_t)(min(vrow[m], last) - vrow[m]) * v_row_stride * ES,
                            sb + SM::OV + j * 1024);
      }
    }
    const char* ab = reinterpret_cast<const char*>(blk.A);
#pragma unroll
    for (int m = 0; m < APW; ++m) {
      const int j = NA0 + wq + NG * m;
      if (j < NA) dma16(ab + (uint32_t)((j * 64 + lane) * 16), sb + SM::OA + j * 1024);
    }
    if (wq == NG - 1) dma16(reinterpret_cast<const char*>(blk.gk) + 16 * lane, sb + SM::OG);
  };


  // fragment (row r, 32-wide dk block kb) of a swizzled K/Q tile: for dk >= 32
  // the 8 slots of group g are dk 32kb + 8g .. +7 (see perm_dk)
  auto kq_frag = [&](const unsigned char* tile, int r, int kb) {
    if constexpr (DK >= 32) {
      const int piece = (32 * kb + 8 * g4) * ES / 16;
      if constexpr (ES == 2) {
        return load_frag_8<T>(reinterpret_cast<const T*>(tile + r * SM::ROWB + ((piece ^ kq_swz<PPR, TRK>(r)) << 4)));
      } else {
        // fp32: 8 elements span two pieces
        const T* a = reinterpret_cast<const T*>(tile + r * SM::ROWB + ((piece ^ kq_swz<PPR, TRK>(r)) << 4));
        const T* b = reinterpret_cast<const T*>(tile + r * SM::ROWB + (((piece + 1) ^ kq_swz<PPR, TRK>(r)) << 4));
        return load_frag_rows<T>(a, b);
      }
    } else {
      const int b = 4 * g4 * ES;
      const T* a = reinterpret_cast<const T*>(tile + r * SM::ROWB + ((((b >> 4) ^ kq_swz<PPR, TRK>(r))) << 4) + (b & 15));
      Frag<T> f = load_frag_rows<T>(a, a);
      if constexpr (ES == 2) {
#pragma unroll
        for (int j = 4; j < 8; ++j) f.v[j] = 0;
      }
      return f;
    }
  };


  // State tiles (chain waves): tile r holds rows 16r + 4g + q of column col0 + i16.
  f32x4 S[NST];
#pragma unroll
  for (int r = 0; r < NST; ++r) S[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  T* sx_mine = SX + (wq * NSB * 64 + lane) * 8;   // + kb * 64 * 8
  T* dx_mine = DX + (wq * 2 * 64 + lane) * 8;     // + blk * 64 * 8
  if (chain) {
    if (p.s0 != nullptr && active) {
      const float* s0 = p.s0 + (int64_t)s * p.s0_stride + ((size_t)h * DK) * dv + col0 + i16;
#pragma unroll
      for (int r = 0; r < NST; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) S[r][q] = s0[(size_t)perm_dk<DK>(16 * r + 4 * g4 + q) * dv];
    }
  }
  // 16-bit state fragments: B operand of the chain's K*S and, through LDS, of
  // the output wave's Q*S; converted once per chunk after the state update
  Frag<T> Sb[NSB];
  if (chain) {
#pragma unroll
    for (int kb = 0; kb < NSB; ++kb) {
      Sb[kb] = make_frag<T>(S[2 * kb], 2 * kb + 1 < NST ? S[(2 * kb + 1) % NST] : f32x4{0.f, 0.f, 0.f, 0.f});
      store_frag_native<T>(sx_mine + kb * 512, Sb[kb]);
    }
  }
  // an issuing wave's wait for chunk c to land in LDS
  auto wait_chunk = [&](int c) {
    if (SM::NBUF == 3 && c + 1 < nch)
      __builtin_amdgcn_s_waitcnt((LB & 15) | (7 << 4) | (15 << 8) | ((LB >> 4) << 14));   // vmcnt(LB)
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  if (issuer && nch > 0) issue(0, 0);
  if (SM::NBUF == 3 && issuer && nch > 1) issue(1, 1);
  if constexpr (NDW > 0) {
    // Load-issuing waves run a loop of their own with the same workgroup
    // barriers per chunk as the compute waves (TOP, MID, and a third with a
    // single stage buffer), so none of their state is live in the compute
    // waves' loop.  With three stages, chunk c+2 goes into the buffer of chunk
    // c-1, free after TOP.
    if (dmaw) {
      for (int c = 0; c < nch; ++c) {
        wait_chunk(c);
        lds_barrier();   // TOP
        const int cn = c + SM::NBUF - 1;
        if (SM::NBUF >= 2 && cn < nch) issue(cn, SM::NBUF == 3 ? cn % 3 : (c & 1) ^ 1);
        lds_barrier();   // MID
        if constexpr (SM::NBUF == 1) {
          lds_barrier();
          if (c + 1 < nch) issue(c + 1, 0);
        }
      }
      return;
    }
  }

  // B fragment selecting the 16 columns of this group out of a 32-slot V row
  // fragment (slots 8g + j, g < 2, read columns 16 wq + 8g + j): V times it is
  // V in accumulator layout, exactly (products with 1 and 0)
  Frag<T> vsel;
  {
    f32x4 plo, phi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      plo[j] = (g4 < 2 && 8 * g4 + j == i16) ? 1.f : 0.f;
      phi[j] = (g4 < 2 && 8 * g4 + 4 + j == i16) ? 1.f : 0.f;
    }
    vsel = make_frag<T>(plo, phi);
  }
  // V fragment of token row `tok`: columns 16 wq + 8 (g & 1) .. +7 of the slice
  auto v_frag = [&](const unsigned char* Vs, int tok) {
    const int pc = (16 * wq + 8 * (g4 & 1)) * ES / 16;   // first 16-byte piece
    const T* a = reinterpret_cast<const T*>(Vs + tok * rowbv + (((pc) ^ (tok & (pprv - 1))) << 4));
    if constexpr (ES == 2) {
      return load_frag_native<T>(a);
    } else {
      const T* b = reinterpret_cast<const T*>(Vs + tok * rowbv + (((pc + 1) ^ (tok & (pprv - 1))) << 4));
      return load_frag_rows<T>(a, b);
    }
  };
  const size_t ostride = (size_t)p.Hv * dv;
  const size_t olane = (size_t)(4 * g4) * ostride + (size_t)h * dv + col0 + i16;

  // The chunk loop, compiled separately for chain waves (CH) and output waves so
  // that neither role's values are live in the other's loop; both meet at the
  // same barriers.
  auto chunk_loop = [&](auto role) {
    constexpr bool CH = decltype(role)::value;
    // chain: the A' fragments of chunk c+1 are fetched from the workspace into
    // registers while chunk c computes (they are the chain's alone, so they skip
    // the LDS stage)
    Frag<T> a_nx[AREG ? NTRI : 1];
    auto fetch_a = [&](int cc) {
      if constexpr (AREG) {
        const Block<T> blk(p.chunk_data, (size_t)(cbeg + cc), p.Hv, h);
#pragma unroll
        for (int f = 0; f < NTRI; ++f) a_nx[f] = load_frag_native<T>(blk.A + (f * 64 + lane) * 8);
      }
    };
    if (CH && nch > 0) fetch_a(0);
    for (int c = 0; c < nch; ++c) {
      const int buf = SM::NBUF == 3 ? c % 3 : (SM::NBUF == 2 ? (c & 1) : 0);
      const int t0 = st0 + c * C;
      const int len = min(C, st1 - t0);
      // chunk c has landed (the issuing waves wait for their own loads); chunk c-1
      // buffers are free
      if (NDW == 0 && CH) wait_chunk(c);
      lds_barrier();
      const unsigned char* sb = smem_raw + buf * SM::STAGE;
      const unsigned char* Kt = sb + SM::OK_;
      const unsigned char* Qt = sb + SM::OQ;
      const unsigned char* Vs = sb + SM::OV;
      const T* AMP = reinterpret_cast<const T*>(sb + SM::OA);
      const float* GT = reinterpret_cast<const float*>(sb + SM::OG);
      f32x4 QSa[4];
      Frag<T> Tb0, Tb1;
      // K^T fragment (state tile rt, token block kb): for state row 16rt + n,
      // K[32kb + 4g + j][dk(16rt + n)] in slots j < 4 and the same 16 tokens later
      // in slots 4..7.  With transpose reads, lane s of each 16-lane group
      // addresses row 32kb + 4g + s/4 (+16), dk columns 32(rt/2) + 8(s%4) +
      // 4(rt%2) .. +3 of the K tile, whose column block is perm_dk's.
      auto kt_frag = [&](int rt, int kb) {
        if constexpr (TRK) {
          const int piece = 4 * (rt >> 1) + (i16 & 3);
          const int r0 = 32 * kb + 4 * g4 + (i16 >> 2), r1 = r0 + 16;
          const s16x4 a = lds_read_tr16(Kt + r0 * SM::ROWB + ((piece ^ kq_swz<PPR, TRK>(r0)) << 4) + 8 * (rt & 1));
          const s16x4 b = lds_read_tr16(Kt + r1 * SM::ROWB + ((piece ^ kq_swz<PPR, TRK>(r1)) << 4) + 8 * (rt & 1));
          const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
          Frag<T> f;
          f.v = __builtin_bit_cast(decltype(f.v), make_uint4(ua.x, ua.y, ub.x, ub.y));
          return f;
        } else {
          return load_frag_native<T>(KT + ((2 * rt + kb) * 64 + lane) * 8);
        }
      };
      // K^T fragments are read LA ahead of the state-update products that use
      // them; with transpose reads the first LA are issued before MID
      constexpr int NKB2 = nrt > 2 ? 2 : 1, NU = NKB2 * NST, LA = TRK ? 7 : 8;
      Frag<T> kt[NU];
      float gl = 0.f;
      if constexpr (CH) {
        // ---- LDS reads and products in a fixed interleave: at most ~14 reads in
        //      flight (the LDS counter a wait can name stops at 15), K blocks two
        //      ahead of the products that use them, and gamma (A' for fp32) and tail
        //      prefetched behind the last K block ----------------------------------
        constexpr int X1 = NSB >= 2 ? NSB - 2 : 0;   // step that prefetches gamma (and fp32 A')
        Frag<T> ak[NSB][nrt], av[nrt], aa[NTRI];
        if constexpr (AREG) {
#pragma unroll
          for (int f = 0; f < NTRI; ++f) aa[f] = a_nx[f];
          if (c + 1 < nch) fetch_a(c + 1);
        }
        f32x4 gm[4], tl[4];
        auto load_kblock = [&](int kb) {
#pragma unroll
          for (int r = 0; r < nrt; ++r) ak[kb][r] = kq_frag(Kt, 16 * r + i16, kb);
        };
        load_kblock(0);
#pragma unroll
        for (int r = 0; r < nrt; ++r) av[r] = v_frag(Vs, 16 * r + i16);
        if constexpr (NSB > 1) load_kblock(1);
        __builtin_amdgcn_sched_barrier(0);
        if (NDW == 0 && SM::NBUF == 2 && c + 1 < nch) issue(c + 1, buf ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 KSa[4], Va[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) KSa[r] = Va[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb) {
#pragma unroll
          for (int r = 0; r < nrt; ++r) mma<T>(KSa[r], ak[kb][r], Sb[kb]);
          if (kb == 0) {
#pragma unroll
            for (int r = 0; r < nrt; ++r) mma<T>(Va[r], av[r], vsel);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (kb + 2 < NSB) load_kblock(kb + 2);
          if (kb == X1) {
#pragma unroll
            for (int r = 0; r < nrt; ++r) gm[r] = *reinterpret_cast<const f32x4*>(GT + 16 * r + 4 * g4);
            if constexpr (!AREG) {
#pragma unroll
              for (int r = 0; r < nrt; ++r) aa[tri_idx(r, 0)] = load_frag_native<T>(AMP + (tri_idx(r, 0) * 64 + lane) * 8);
#pragma unroll
              for (int r = 2; r < nrt; ++r) aa[tri_idx(r, 1)] = load_frag_native<T>(AMP + (tri_idx(r, 1) * 64 + lane) * 8);
            }
          }
          if (kb == NSB - 1) {
#pragma unroll
            for (int r = 0; r < nrt; ++r) tl[r] = *reinterpret_cast<const f32x4*>(GT + 64 + 16 * r + 4 * g4);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- X = V - gamma * KS ------------------------------------------------
        f32x4 X[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          X[r] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (r < nrt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) X[r][q] = Va[r][q] - gm[r][q] * KSa[r][q];
          }
        }
        const Frag<T> Xb0 = make_frag<T>(X[0], X[1]), Xb1 = make_frag<T>(X[2], X[3]);
        // ---- Delta = A' X --------------------------------------------------------
        f32x4 D[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          D[r] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (r < nrt) mma<T>(D[r], aa[tri_idx(r, 0)], Xb0);
        }
#pragma unroll
        for (int r = 2; r < nrt; ++r) mma<T>(D[r], aa[tri_idx(r, 1)], Xb1);
        if constexpr (TRK) {   // the K tile is complete since TOP: K^T reads overlap Delta's exchange
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < NU && u < LA; ++u) kt[u] = kt_frag(u % NST, u / NST);
          gl = GT[192];
          __builtin_amdgcn_sched_barrier(0);
        }
        store_frag_native<T>(dx_mine, make_frag<T>(D[0], D[1]));
        store_frag_native<T>(dx_mine + 512, make_frag<T>(D[2], D[3]));
        // ---- tail-weighted Delta for the state update ---------------------------
#pragma unroll
        for (int r = 0; r < nrt; ++r)
#pragma unroll
          for (int q = 0; q < 4; ++q) D[r][q] *= tl[r][q];
        Tb0 = make_frag<T>(D[0], D[1]);
        Tb1 = make_frag<T>(D[2], D[3]);
      } else {
        // ---- QS = Q S (state fragments from the chain wave) ----------------------
#pragma unroll
        for (int r = 0; r < 4; ++r) QSa[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        Frag<T> sbf[NSB], aq[NSB][nrt];
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb) {
          sbf[kb] = load_frag_native<T>(sx_mine + kb * 512);
#pragma unroll
          for (int r = 0; r < nrt; ++r) aq[kb][r] = kq_frag(Qt, 16 * r + i16, kb);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < NSB; ++kb)
#pragma unroll
          for (int r = 0; r < nrt; ++r) mma<T>(QSa[r], aq[kb][r], sbf[kb]);
        // ---- K^T fragments: fragment (state tile rt, token block kb) holds, for
        //      state row 16rt + n, K[32kb + 4g + j][dk(16rt + n)] (lo) and the same
        //      16 tokens later (hi): tiles D(2kb, rt), D(2kb+1, rt) of K * P, P the
        //      0/1 matrix picking dk column perm_dk(16rt + n) -------------------------
#pragma unroll
        for (int f0 = 0; f0 < (TRK ? 0 : SM::NKT); f0 += NG) {
          const int f = f0 + wq;
          if (f < SM::NKT) {
            const int rt = f >> 1, kb = f & 1;
            // B fragment of P: slot 8g + j of the 32-block holding this tile
            f32x4 plo, phi;
            if constexpr (DK >= 32) {
              const int tgt = perm_dk<DK>(16 * rt + i16) - 32 * (rt >> 1);   // dk inside the block
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                plo[j] = (8 * g4 + j == tgt) ? 1.f : 0.f;
                phi[j] = (8 * g4 + 4 + j == tgt) ? 1.f : 0.f;
              }
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                plo[j] = (4 * g4 + j == i16) ? 1.f : 0.f;
                phi[j] = 0.f;
              }
            }
            const Frag<T> pf = make_frag<T>(plo, phi);
            f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
            if (2 * kb < nrt) mma<T>(lo, kq_frag(Kt, 32 * kb + i16, rt >> 1), pf);
            if (2 * kb + 1 < nrt) mma<T>(hi, kq_frag(Kt, 32 * kb + 16 + i16, rt >> 1), pf);
            store_frag_native<T>(KT + (f * 64 + lane) * 8, make_frag<T>(lo, hi));
          }
        }
      }
      lds_barrier();   // MID: Delta and K^T fragments are in LDS; state fragments consumed
      if constexpr (CH) {
        // ---- S = gamma_last S + K^T (tail * Delta) ---------------------------------
        if constexpr (!TRK) {   // K^T fragments built by the output waves before MID
#pragma unroll
          for (int u = 0; u < NU && u < LA; ++u) kt[u] = kt_frag(u % NST, u / NST);
          gl = GT[192];
        }
        __builtin_amdgcn_sched_barrier(0);
        // Each tile is scaled by gamma_last right before its first product, and the
        // next chunk's state fragments of a tile pair (kept for the chain's K*S,
        // stored for the output wave) are formed two products after the pair's
        // last one, so VALU work overlaps the matrix products.
        constexpr int U0 = (NKB2 - 1) * NST;   // first product of the last token block
        auto next_sb = [&](int rt) {
          if (rt >= 0 && (rt % 2 == 1 || rt == NST - 1)) {
            const int kb = rt / 2;
            Sb[kb] = make_frag<T>(S[2 * kb], 2 * kb + 1 < NST ? S[(2 * kb + 1) % NST] : f32x4{0.f, 0.f, 0.f, 0.f});
            store_frag_native<T>(sx_mine + kb * 512, Sb[kb]);
          }
        };
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          if (u < NST) {
#pragma unroll
            for (int q = 0; q < 4; ++q) S[u][q] *= gl;
          }
          mma<T>(S[u % NST], kt[u], u / NST == 0 ? Tb0 : Tb1);
          __builtin_amdgcn_sched_barrier(0);
          if (u + LA < NU) kt[u + LA] = kt_frag((u + LA) % NST, (u + LA) / NST);
          if (u - 2 >= U0) next_sb(u - 2 - U0);
          __builtin_amdgcn_sched_barrier(0);
        }
        next_sb(NST - 2);
        next_sb(NST - 1);
        if constexpr (EMIT) {
          // the state after this chunk's last token, in the [dk, dv] state layout:
          // a wave-uniform row base per store plus one per-lane 32-bit offset;
          // non-temporal, so the stream of states does not evict the K/Q tiles
          // the other workgroups of the head still read from L2
          if (active && (int64_t)(cbeg + c) < p.chunk_states_cap) {
            float* cs = p.chunk_states + ((size_t)(cbeg + c) * p.Hv + h) * DK * dv;
            const int lo = (DK < 32 ? 4 * g4 : 8 * g4) * dv + col0 + i16;
#pragma unroll
            for (int r = 0; r < NST; ++r)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int row = perm_dk<DK>(16 * r + q);          // lane group 0's row
                __builtin_nontemporal_store(S[r][q], (cs + (size_t)row * dv) + lo);
              }
          }
        }
      } else {
        // ---- O = scale (gamma QS + MP Delta) -> o -----------------------------------
        const Frag<T> Db0 = load_frag_native<T>(dx_mine), Db1 = load_frag_native<T>(dx_mine + 512);
        f32x4 O[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 gm = *reinterpret_cast<const f32x4*>(GT + 128 + 16 * r + 4 * g4);
#pragma unroll
          for (int q = 0; q < 4; ++q) O[r][q] = gm[q] * QSa[r][q];
          if (r < nrt) mma<T>(O[r], load_frag_native<T>(AMP + ((NTRI + tri_idx(r, 0)) * 64 + lane) * 8), Db0);
        }
#pragma unroll
        for (int r = 2; r < nrt; ++r)
          mma<T>(O[r], load_frag_native<T>(AMP + ((NTRI + tri_idx(r, 1)) * 64 + lane) * 8), Db1);
        if (active) {
          T* oc = op + (size_t)t0 * ostride + olane;
          if (len == C) {
#pragma unroll
            for (int r = 0; r < nrt; ++r)
#pragma unroll
              for (int q = 0; q < 4; ++q) oc[(size_t)(16 * r + q) * ostride] = Elem<T>::from_f(p.scale * O[r][q]);
          } else {
#pragma unroll
            for (int r = 0; r < nrt; ++r)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (16 * r + 4 * g4 + q < len) oc[(size_t)(16 * r + q) * ostride] = Elem<T>::from_f(p.scale * O[r][q]);
          }
        }
      }
      if constexpr (SM::NBUF == 1) {
        // single stage buffer: chunk c+1 may only overwrite it once every wave is
        // done reading chunk c (gamma, tail and MP are read after MID)
        lds_barrier();
        if (NDW == 0 && CH && c + 1 < nch) issue(c + 1, 0);
      }
    }

  };
  if (chain) chunk_loop(std::true_type{});
  else chunk_loop(std::false_type{});

  if (chain && p.s_out != nullptr && active) {
    float* so = p.s_out + ((size_t)s * p.Hv + h) * DK * dv + col0 + i16;
#pragma unroll
    for (int r = 0; r < NST; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) so[(size_t)perm_dk<DK>(16 * r + 4 * g4 + q) * dv] = S[r][q];
  }
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------
// Per-device host caches are atomics: entry points may be called from several
// host threads, each on any device.
constexpr int kMaxDevices = 64;

static int device_cus() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The dynamic-LDS limit of a kernel is a per-device attribute: set it once per
// device on first use.  Setting it is idempotent, so two threads racing on the
// first call of a device both succeed; the flag only skips later calls.
static hipError_t ensure_dynamic_lds(std::atomic<bool>* done, const void* fn, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) done[dev].store(true, std::memory_order_release);
  return e;
}

template <typename T, int DK, int C, int NG, int NDW, bool EMIT>
static hipError_t launch_state(const PrefillArgs& a, hipStream_t st) {
  using SM = StateSmem<T, DK, NG, sizeof(T) == 2 && DK == 128 && C >= 32, (NDW > 0 && !EMIT)>;
  const size_t sm2 = SM::total;
  if (sm2 > 160 * 1024) return hipErrorInvalidValue;
  static std::atomic<bool> attr_set[kMaxDevices];
  const hipError_t ea = ensure_dynamic_lds(attr_set, (const void*)chunk_state_kernel<T, DK, C, NG, NDW, EMIT>, sm2);
  if (ea != hipSuccess) return ea;
  const int nslices = (a.dv + SM::SW - 1) / SM::SW;
  const long long groups = (long long)a.Hq * a.B;
  const long long sblocks = 8LL * nslices * (a.Hv / a.Hq) * ((groups + 7) / 8);
  if (sblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  prof_begin(K_STATE, st);
  hipLaunchKernelGGL((chunk_state_kernel<T, DK, C, NG, NDW, EMIT>), dim3((unsigned)sblocks), dim3(64 * (2 * NG + NDW)),
                     sm2, st, a);
  prof_end(K_STATE, st);
  return hipGetLastError();
}

template <typename T, int DK, int C>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  // up to 64 sequences the prep and state kernels plan for themselves
  hipError_t e = hipSuccess;
  if (a.B > kWavePlanMaxSeqs) {
    prof_begin(K_PLAN, st);
    hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, st, a);
    prof_end(K_PLAN, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.max_chunks > 0) {
    // value heads in pairs when pairs share a key head (Hv / Hq even)
    const bool pairs = ((a.Hv / a.Hq) % 2) == 0;
    const long long items = (long long)a.max_chunks * (pairs ? a.Hv / 2 : a.Hv);
    const long long blocks = 8 * ((items + 7) / 8);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    prof_begin(K_PREP, st);
    if (pairs)
      hipLaunchKernelGGL((chunk_prep_kernel<T, DK, C, 2>), dim3((unsigned)blocks), dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<T, DK, C, 1>), dim3((unsigned)blocks), dim3(64), 0, st, a);
    prof_end(K_PREP, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // Geometry.  While there are at most two (sequence, head, 32-column slice)
  // items per CU the pass is latency bound: 32-column workgroups (2 chain + 2
  // output + 2 load-issuing waves) spread each head over more CUs and keep load
  // issue off the chain.  With at most half a (sequence, head, 16-column slice)
  // item per CU, 16-column workgroups (1 chain + 1 output + 1 load-issuing
  // wave) halve each CU's LDS reads, which shortens the chunk step (fp16
  // 2048-token sequence over 6 value heads: 41.7 us instead of 45.8 us).  Beyond that, 64-column workgroups (4 chain + 4 output
  // waves, the chain issuing the loads), one per CU.  (32-column workgroups of 4
  // waves with a single stage buffer, two per CU, measured 78 us against 45 us
  // on the 16 x 256-token batch: each workgroup then waits for its loads.)
  // The chunk-boundary state stores live in a separate instantiation so that
  // the plain prefill keeps its register allocation.
  const bool emit = a.chunk_states != nullptr;
  // fp32 tiles at dk = 128 fit the LDS only in the 32-column geometry with one
  // stage buffer; 4 waves (the chain waves issuing the loads), so each wave
  // may hold the register budget of a whole SIMD and nothing spills
  constexpr bool only32 = sizeof(T) == 4 && DK == 128;
  if constexpr (only32)
    e = emit ? launch_state<T, DK, C, 2, 0, true>(a, st) : launch_state<T, DK, C, 2, 0, false>(a, st);
  else if ((long long)a.B * a.Hv * ((a.dv + 15) / 16) <= device_cus() / 2)
    e = emit ? launch_state<T, DK, C, 1, 1, true>(a, st)    // 3 waves: chain, output, loader
             : launch_state<T, DK, C, 1, 1, false>(a, st);
  else if ((long long)a.B * a.Hv * ((a.dv + 31) / 32) <= 2LL * device_cus())
    e = emit ? launch_state<T, DK, C, 2, 2, true>(a, st)    // 6 waves: + two load-issuing waves
             : launch_state<T, DK, C, 2, 2, false>(a, st);
  else
    e = emit ? launch_state<T, DK, C, 4, 0, true>(a, st)    // 8 waves: the chain waves issue the loads
             : launch_state<T, DK, C, 4, 0, false>(a, st);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_prefill_c(const PrefillArgs& a, hipStream_t st) {
  switch (a.chunk) {
    case 16: return launch_prefill_t<T, DK, 16>(a, st);
    case 32: return launch_prefill_t<T, DK, 32>(a, st);
    case 64: return launch_prefill_t<T, DK, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_prefill_dt(const PrefillArgs& a, hipStream_t st) {
  switch (a.dk) {
    case 16: return launch_prefill_c<T, 16>(a, st);
    case 32: return launch_prefill_c<T, 32>(a, st);
    case 64: return launch_prefill_c<T, 64>(a, st);
    case 128: return launch_prefill_c<T, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(DType dt, const PrefillArgs& a, hipStream_t st) {
  switch (dt) {
    case DType::F32: return launch_prefill_dt<float>(a, st);
    case DType::F16: return launch_prefill_dt<_Float16>(a, st);
    case DType::BF16: return launch_prefill_dt<__bf16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
