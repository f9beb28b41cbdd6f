// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

// Recurrent step (token-by-token) problem, already validated on the host.
// Optional input prologue applied inside the kernels (identity when zeroed):
//   l2norm:  q_t and k_t (per key head) scaled by (sum x^2 + eps)^(-1/2), in fp32
//   beta_logit: beta = 1 / (1 + exp(-b)) of the beta input
//   A_log != NULL: g = -exp(A_log[h]) * softplus(g_in + dt_bias[h]) (dt_bias NULL = 0)
struct Prologue {
  int32_t l2norm;
  float eps;
  int32_t beta_logit;
  const float* A_log;
  const float* dt_bias;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* s0;       // may be null (zeros)
  int64_t s0_stride;     // elements between sequences' initial states (0 = broadcast)
  float* s_out;          // may be null
  void* o;
  const int32_t* cu;     // null = dense rows
  int32_t B, T, total;   // rows, tokens per row (dense), total packed tokens
  int32_t Hq, Hv, dk, dv;
  float scale;
  int32_t cap;           // capture capacity (0 = no capture)
  const int32_t* counts; // [B] capture counts (device)
  int32_t active;
  float* su;             // [B, cap, R]
  Prologue pro;
};

struct ReplayArgs {
  int32_t B, Hq, Hv, dk, dv, cap;
  const float* su;
  const int32_t* counts;
  float* state;
};

// Chunked prefill problem.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* s0;
  int64_t s0_stride;
  float* s_out;
  void* o;
  const int32_t* cu;
  int32_t B, T, total;   // total = packed tokens
  int32_t Hq, Hv, dk, dv;
  float scale;
  int32_t chunk;         // 16, 32 or 64
  int32_t max_chunks;    // workspace capacity in chunks
  int32_t* chunk_offsets;   // [B+1] inside the workspace
  int32_t* chunk_info;      // [max_chunks][2]: first token, length (0 past the last chunk)
  void* chunk_data;         // per (chunk, value head) blocks inside the workspace
  float* chunk_states;      // NULL, or [chunk_states_cap, Hv, dk, dv]: state after each chunk
  int64_t chunk_states_cap;
  Prologue pro;
};

// Per (chunk, value head) workspace block written by the chunk-prep kernel:
//   A'  6 x 512 elements: lower-triangular 16x32 blocks of the UT inverse times
//       diag(beta), in MFMA fragment order
//   MP  6 x 512 elements: the same blocks of the decay-masked Q K^T
//   gk  [64] fp32 gamma_i * rk_i: exp of the in-chunk cumulative log decay
//            G_i times the key's inverse norm (1 without the l2norm prologue)
//   tk  [64] fp32 exp(G_last - G_i) * rk_i (decay from token i to the chunk end)
//   gq  [64] fp32 gamma_i * rq_i (the query's inverse norm)
//   gl  [64] fp32 gamma_last in entry 0, the rest unused
inline size_t chunk_block_bytes(DType dt) {
  size_t es = dt == DType::F32 ? 4 : 2;
  return 2 * 6 * 512 * es + 64 * 4 * 4;
}

// Opt-in per-kernel event timing (gdn_profile_enable / gdn_profile_collect).
enum KernelId : int {
  K_PLAN = 0, K_PREP, K_STATE, K_RECURRENT, K_REPLAY, K_COPY, kNumKernels
};
void prof_begin(KernelId id, hipStream_t s);
void prof_end(KernelId id, hipStream_t s);

hipError_t launch_recurrent(DType dt, const DecodeArgs& a, hipStream_t s);
hipError_t launch_replay(const ReplayArgs& a, hipStream_t s);
hipError_t launch_copy(const float* src, float* dst, size_t n, hipStream_t s);
hipError_t launch_prefill(DType dt, const PrefillArgs& a, hipStream_t s);

}  // namespace gdn
