/*
 * gdn.h - C ABI of the MI355X (gfx950) Gated DeltaNet engine (libgdn.so).
 *
 * The library implements the data-parallel hot path of a Gated DeltaNet (GDN)
 * layer on one GPU: chunked prefill with explicit initial/final state, the
 * per-token recurrent step with compact state-update capture, replay of the
 * captured updates, and immutable state snapshots.
 *
 * The method (the gated delta rule; value head h reads key/query head
 * h / (Hv/Hq), "inverse-GQA" key sharing):
 *
 *     alpha_t = exp(g_t)
 *     delta_t = beta_t * (v_t - (alpha_t S_{t-1})^T k_t)
 *     S_t     = alpha_t S_{t-1} + k_t delta_t^T          (S is [dk x dv], fp32)
 *     o_t     = scale * S_t^T q_t
 *
 * Sources: [onnxruntime PR 32767, "[WebGPU EP] adds state update capacity
 * support for GatedDeltaNet", sections "Changes", "Test Coverage", "DFlash2
 * Prerequisite"] for capture, the active flag, replay S = decay*S +
 * outer(key, delta) and shared-key heads; [executorch issue 23097, "Enable the
 * native Kev example on NVIDIA GPUs ...", "Work to cover"] for the chunked
 * prefill with explicit initial/final state and FP32 recurrence under 16-bit
 * weights; [executorch issue 23099, "Enable the native Kev example on the
 * WebGPU backend", "Work to cover"] for the prefix snapshot that repeated
 * evaluations must leave unchanged.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - All pointers are DEVICE pointers (hipMalloc'd or torch-allocated on the
 *    current device) unless stated otherwise; the caller owns every buffer.
 *    The library allocates nothing and keeps no pointer after returning.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Buffers must stay alive until the queued work has finished.
 *  - Arguments are validated on the host before anything is enqueued.  A status
 *    other than GDN_OK means nothing was enqueued; gdn_last_error() returns a
 *    thread-local message.  Nothing aborts.
 *  - Layouts are contiguous row-major (last index fastest):
 *        q, k        [T_total, Hq, dk]   dtype = shape.dtype
 *        v, o        [T_total, Hv, dv]   dtype = shape.dtype
 *        g, beta     [T_total, Hv]       fp32 (g = log of the decay alpha)
 *        states      [N, Hv, dk, dv]     fp32 (dv fastest)
 *    T_total = B*T for dense input (B rows of T tokens) or T for packed ragged
 *    input given by cu_seqlens (int32 [N+1], device, 0 = cu[0] <= ... <=
 *    cu[N] = T; empty sequences allowed).  cu_seqlens is not read on the host;
 *    kernels clamp every range to [0, T] and cap the chunk count at the
 *    workspace size, so malformed values give unspecified results, never an
 *    out-of-bounds access.
 *  - Supported sizes: dk, dv in {16, 32, 64, 128}; Hv % Hq == 0; pointers
 *    16-byte aligned; fp32 data for fp32 inputs is computed in fp32, fp16/bf16
 *    inputs use 16-bit matrix-core products with fp32 accumulation and an fp32
 *    state, and o is rounded to the input dtype (round to nearest even).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDN_F32 = 0, GDN_F16 = 1, GDN_BF16 = 2 } gdn_dtype;

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment, aliasing */
  GDN_ERR_UNSUPPORTED = 2, /* valid but outside the compiled set (dk, dv, chunk) */
  GDN_ERR_HIP = 3          /* a HIP launch or runtime call failed */
} gdn_status;

/* Problem description shared by prefill and recurrent step. */
typedef struct {
  int32_t B;     /* dense: rows; ragged: number of sequences N (cu_seqlens has B+1 entries) */
  int32_t T;     /* dense: tokens per row; ragged: total packed tokens */
  int32_t Hq;    /* query/key heads */
  int32_t Hv;    /* value heads, a multiple of Hq */
  int32_t dk;    /* key/query head dim */
  int32_t dv;    /* value head dim */
  float scale;   /* o = scale * S^T q (usually dk^-1/2) */
  int32_t dtype; /* gdn_dtype of q, k, v, o */
} gdn_shape;

/*
 * Optional input prologue, applied inside the kernels of the *_ex entry points
 * [executorch issue 23097, "Work to cover": reusing a GDN prefill means adapting
 * its gate and scaling conventions].  The pages give no formulas; these are the
 * common ones, each switched on separately.  A zeroed struct (or NULL) is the
 * identity: q, k, g and beta are used as given.
 *
 *  qk_l2norm      nonzero: every q_t and k_t (per key head) is replaced by
 *                 x * (sum_i x_i^2 + qk_l2norm_eps)^(-1/2), computed in fp32
 *                 from the input-dtype values.  eps = 0 is allowed; an all-zero
 *                 row then gives non-finite results.
 *  qk_l2norm_eps  finite, >= 0 (read only when qk_l2norm is set).
 *  beta_is_logit  nonzero: beta = 1 / (1 + exp(-b)) of the `beta` input.
 *  gate_A_log     NULL: `g` holds the log decay.  Otherwise fp32 [Hv] on the
 *                 device, and the log decay of value head h is
 *                 -exp(gate_A_log[h]) * softplus(g + gate_dt_bias[h]),
 *                 softplus(x) = log(1 + exp(x)).
 *  gate_dt_bias   fp32 [Hv] on the device, or NULL (zeros); only with gate_A_log.
 * Captured records hold the prologue's results: decay = exp of the gated log
 * decay, key = the normalised fp32 key, delta with the sigmoid beta.
 */
typedef struct {
  int32_t qk_l2norm;
  float qk_l2norm_eps;
  int32_t beta_is_logit;
  const float* gate_A_log;
  const float* gate_dt_bias;
} gdn_prologue;

/* Version of this ABI (bumped on any signature change). */
int32_t gdn_abi_version(void);

/* Bytes of device workspace gdn_prefill_chunked needs for `shape`,
 * `chunk_size` and the input form (`ragged` nonzero when cu_seqlens will be
 * passed, so shape->T is the packed total); 0 if the arguments are invalid.
 * Host only, no HIP call. */
size_t gdn_prefill_workspace_bytes(const gdn_shape* shape, int32_t chunk_size, int32_t ragged);

/*
 * Chunked prefill [executorch issue 23097, "Work to cover": chunked GDN prefill
 * with explicit initial/final state and FP32 recurrence].
 *
 * Computes o for every token and (optionally) the state after each sequence's
 * last token, processing each sequence in chunks of `chunk_size` tokens
 * (16, 32 or 64; chunks restart at each sequence start, the last one may be
 * partial).  The result equals the token-by-token recurrence up to rounding.
 *
 * Precondition on g: every g <= 0 (decay alpha = exp(g) <= 1), the usual case
 * of a forgetting gate.  The chunked form then only forms decay ratios
 * exp(G_i - G_j) with j <= i, exp(G_i) and exp(G_last - G_j) (G = in-chunk
 * cumulative sum of g), all <= 1, which keeps its 16-bit matrix operands in
 * range.  With some g > 0 those factors exceed 1 and can overflow 16-bit
 * operands, so o and final_state are unspecified (the call still completes
 * and accesses only the buffers given).  The precondition is not checked (g is
 * not read on the host); gdn_recurrent_step accepts any finite g.
 *
 *  initial_state   [N, Hv, dk, dv] fp32 or NULL (zeros).  Sequence s reads
 *                  initial_state + s * initial_state_batch_stride (elements);
 *                  stride 0 broadcasts one state to all sequences (snapshot
 *                  reuse).  Never written unless it is also `final_state`.
 *  final_state     [N, Hv, dk, dv] fp32 or NULL (not written).  May equal
 *                  initial_state only with stride Hv*dk*dv (in-place update).
 *  workspace       device scratch of gdn_prefill_workspace_bytes() bytes,
 *                  16-byte aligned; contents on entry are ignored.
 */
gdn_status gdn_prefill_chunked(const gdn_shape* shape, const void* q, const void* k,
                               const void* v, const float* g, const float* beta,
                               const float* initial_state, int64_t initial_state_batch_stride,
                               const int32_t* cu_seqlens, int32_t chunk_size, void* o,
                               float* final_state, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Chunked prefill that also emits the state at every chunk boundary
 * [executorch issue 23097, "Work to cover": GDN chunk boundaries, prefix
 * snapshots retained in device memory and reused; executorch issue 23099,
 * "Work to cover": the reused prefix stays unchanged].  A boundary state is a
 * ready-made snapshot of the prefix that ends there: passing it as
 * `initial_state` of a later call continues the sequence from that point.
 *
 * Same arguments, results and errors as gdn_prefill_chunked, plus
 *  chunk_states           [num_chunks, Hv, dk, dv] fp32, device, 16-byte
 *                         aligned, not NULL.  Sequence s has
 *                         n_s = ceil(L_s / chunk_size) chunks (0 when empty);
 *                         its chunk j has index sum_{s' < s} n_s' + j (dense
 *                         input: s * ceil(T / chunk_size) + j) and receives the
 *                         state after the first min((j+1)*chunk_size, L_s)
 *                         tokens of s, so each sequence's last entry equals its
 *                         final state.  Must not overlap any other buffer.
 *  chunk_states_capacity  entries available (>= 0); chunks with an index at
 *                         or beyond it are not written (size it to
 *                         sum_s n_s to receive them all).
 * Costs one extra fp32 state write per (chunk, value head).
 */
gdn_status gdn_prefill_chunked_states(const gdn_shape* shape, const void* q, const void* k,
                                      const void* v, const float* g, const float* beta,
                                      const float* initial_state, int64_t initial_state_batch_stride,
                                      const int32_t* cu_seqlens, int32_t chunk_size, void* o,
                                      float* final_state, float* chunk_states,
                                      int64_t chunk_states_capacity, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_chunked / gdn_prefill_chunked_states with the input prologue:
 * `prologue` may be NULL (identity) and `chunk_states` may be NULL (no
 * boundary states; chunk_states_capacity is then ignored).  Same layouts,
 * results and errors otherwise.
 */
gdn_status gdn_prefill_chunked_ex(const gdn_shape* shape, const gdn_prologue* prologue, const void* q,
                                  const void* k, const void* v, const float* g, const float* beta,
                                  const float* initial_state, int64_t initial_state_batch_stride,
                                  const int32_t* cu_seqlens, int32_t chunk_size, void* o,
                                  float* final_state, float* chunk_states, int64_t chunk_states_capacity,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The entry point itself allocates nothing:
 * its workspace is a fixed device array of GDN_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held from the first call on that GPU until the process
 * ends.  The caller still passes every input and output.
 *
 * Same arguments (minus workspace), layouts, results and errors as
 * gdn_prefill_chunked, plus GDN_ERR_UNSUPPORTED when the problem needs more
 * workspace than the array holds (gdn_prefill_workspace_bytes() >
 * GDN_NOALLOC_SCRATCH_BYTES; at 16-bit inputs and chunk 64 that is about
 * 10,000 (chunk, value head) pairs, e.g. 20,000 tokens at 32 value heads).
 * The array keeps the last call's contents; every call writes each part of
 * it that it reads, so nothing needs clearing.  All calls on one GPU share
 * the array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and give unspecified results, so order them on one stream.
 * The first call on a device looks up the array's address (no allocation).
 */
#define GDN_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
gdn_status gdn_prefill_chunked_noalloc(const gdn_shape* shape, const void* q, const void* k,
                                       const void* v, const float* g, const float* beta,
                                       const float* initial_state, int64_t initial_state_batch_stride,
                                       const int32_t* cu_seqlens, int32_t chunk_size, void* o,
                                       float* final_state, void* stream);

/*
 * Recurrent step with compact state-update capture [onnxruntime PR 32767,
 * "Changes": state_update_capacity, the required [batch] capture_count input,
 * the packed float32 state_update output, clamped per-row prefix capture,
 * state_update_active = 0 clears the whole output].
 *
 * Runs the recurrence token by token over each row (dense rows of T tokens or
 * ragged rows through cu_seqlens), writing o and (optionally) final_state; the
 * argument rules for initial_state / final_state are those of prefill.
 *
 * Capture (state_update_capacity > 0):
 *  capture_count   int32 [B] device, required.  Row b captures its first
 *                  n_b = min(max(capture_count[b], 0), capacity, L_b) tokens.
 *  state_update    fp32 [B, capacity, R], R = Hv + Hq*dk + Hv*dv, required.
 *                  Record c of row b (token c of the row) is
 *                  [decay: alpha per value head (Hv) | key: fp32 k per key head
 *                  (Hq*dk) | delta: delta per value head (Hv*dv)], so that
 *                  replaying it applies S = decay*S + outer(key, delta).
 *  state_update_active
 *                  nonzero: records c < n_b are written, all other entries are
 *                  left untouched (their content is unspecified);
 *                  0: the whole state_update buffer is zero-filled and no
 *                  record is written (o and final_state are still computed).
 * capacity == 0 disables capture (capture_count, state_update may be NULL);
 * capacity < 0 is GDN_ERR_INVALID_ARG.
 */
gdn_status gdn_recurrent_step(const gdn_shape* shape, const void* q, const void* k,
                              const void* v, const float* g, const float* beta,
                              const float* initial_state, int64_t initial_state_batch_stride,
                              const int32_t* cu_seqlens, void* o, float* final_state,
                              int32_t state_update_capacity, const int32_t* capture_count,
                              int32_t state_update_active, float* state_update, void* stream);

/* gdn_recurrent_step with the input prologue (`prologue` may be NULL). */
gdn_status gdn_recurrent_step_ex(const gdn_shape* shape, const gdn_prologue* prologue, const void* q,
                                 const void* k, const void* v, const float* g, const float* beta,
                                 const float* initial_state, int64_t initial_state_batch_stride,
                                 const int32_t* cu_seqlens, void* o, float* final_state,
                                 int32_t state_update_capacity, const int32_t* capture_count,
                                 int32_t state_update_active, float* state_update, void* stream);

/*
 * Replay of captured state updates [onnxruntime PR 32767, "Changes" and
 * "DFlash2 Prerequisite": compact-state replay after partial acceptance].
 *
 * For each row b and each record c < m_b = min(max(replay_count[b], 0),
 * capacity), in order: S[b,h] = decay_c[h] * S[b,h] + outer(key_c[h/(Hv/Hq)],
 * delta_c[h]).  `state` [B, Hv, dk, dv] fp32 is updated in place (normally the
 * pre-step state); `state_update` is the buffer gdn_recurrent_step filled with
 * the same B, Hq, Hv, dk, dv, capacity and is only read.  The caller keeps
 * m_b <= n_b of the capture (records beyond n_b are unspecified).
 */
gdn_status gdn_replay_state_updates(int32_t B, int32_t Hq, int32_t Hv, int32_t dk, int32_t dv,
                                    int32_t state_update_capacity, const float* state_update,
                                    const int32_t* replay_count, float* state, void* stream);

/*
 * Immutable state snapshot [executorch issue 23099 / 23097, "Work to cover":
 * a prefix snapshot reused across question batches; repeated evaluations must
 * leave the prefix unchanged].
 *
 * Copies num_states * Hv * dk * dv fp32 values from src to dst (bitwise),
 * ordered on `stream`.  src and dst must not overlap.  No entry point ever
 * writes a buffer that is passed to it only as initial_state, so a snapshot
 * used as initial_state stays bit-identical across any number of calls.
 */
gdn_status gdn_state_snapshot(const float* src, float* dst, int64_t num_states, int32_t Hv,
                              int32_t dk, int32_t dv, void* stream);

/*
 * Measurement support (not part of the method).  gdn_profile_enable(1) makes
 * every entry point bracket each kernel it launches with a pair of hipEvents
 * recorded on the launch stream; gdn_profile_collect() waits for all pending
 * events, reports per kernel the number of launches and their summed duration
 * in milliseconds (up to max_kernels entries; names are static strings), and
 * clears the record.  Returns the number of distinct kernels seen.  Disabled by
 * default; costs nothing measurable when disabled.
 */
gdn_status gdn_profile_enable(int32_t on);
int32_t gdn_profile_collect(const char** names, double* total_ms, int32_t* launches, int32_t max_kernels);

/* Static description of a status code. */
const char* gdn_status_string(gdn_status status);

/* Thread-local detail about the last non-OK status returned on this thread. */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
