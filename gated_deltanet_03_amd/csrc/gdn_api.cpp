// C-ABI entry points of libgdn.so: host-side validation, workspace sizing and
// dispatch to the HIP kernels.  Validation runs before any HIP call, so a
// rejected call enqueues nothing (and can be exercised without a GPU).
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

gdn_status hip_fail(hipError_t e, const char* what) {
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

size_t elem_size(int32_t dt) { return dt == GDN_F32 ? 4 : 2; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// [a0, a0+an) and [b0, b0+bn) (bytes) overlap?
bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

// Checks shared by prefill and recurrent step.  Fills total tokens.
gdn_status check_shape(const gdn_shape* sh, const int32_t* cu, int64_t* total_tokens) {
  if (sh == nullptr) return fail(GDN_ERR_INVALID_ARG, "shape is NULL");
  if (sh->B < 0 || sh->T < 0) return fail(GDN_ERR_INVALID_ARG, "B=%d and T=%d must be >= 0", sh->B, sh->T);
  if (sh->Hq <= 0 || sh->Hv <= 0)
    return fail(GDN_ERR_INVALID_ARG, "Hq=%d and Hv=%d must be positive", sh->Hq, sh->Hv);
  if (sh->Hv % sh->Hq != 0)
    return fail(GDN_ERR_INVALID_ARG, "Hv=%d must be a multiple of Hq=%d (shared key heads)", sh->Hv, sh->Hq);
  if (sh->dtype != GDN_F32 && sh->dtype != GDN_F16 && sh->dtype != GDN_BF16)
    return fail(GDN_ERR_INVALID_ARG, "dtype %d is not a gdn_dtype", sh->dtype);
  if (sh->dk <= 0 || sh->dv <= 0) return fail(GDN_ERR_INVALID_ARG, "dk=%d, dv=%d must be positive", sh->dk, sh->dv);
  if (!supported_dim(sh->dk) || !supported_dim(sh->dv))
    return fail(GDN_ERR_UNSUPPORTED, "dk=%d, dv=%d: supported head dims are 16, 32, 64, 128", sh->dk, sh->dv);
  if (sh->B > 65535 || sh->Hv > 65535)
    return fail(GDN_ERR_UNSUPPORTED, "B=%d or Hv=%d exceeds 65535", sh->B, sh->Hv);
  if ((int64_t)sh->B * sh->Hv > (1 << 24))
    return fail(GDN_ERR_UNSUPPORTED, "B*Hv=%lld exceeds 2^24 (row, head) pairs", (long long)sh->B * sh->Hv);
  if (!(sh->scale == sh->scale)) return fail(GDN_ERR_INVALID_ARG, "scale is NaN");
  int64_t total = cu ? (int64_t)sh->T : (int64_t)sh->B * sh->T;
  if (total > (int64_t)0x7fffffff) return fail(GDN_ERR_UNSUPPORTED, "more than 2^31-1 tokens");
  *total_tokens = total;
  return GDN_OK;
}

gdn_status check_tokens(const gdn_shape* sh, int64_t total, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const void* o) {
  if (total == 0) return GDN_OK;
  const void* ptrs[6] = {q, k, v, g, beta, o};
  const char* names[6] = {"q", "k", "v", "g", "beta", "o"};
  for (int i = 0; i < 6; ++i) {
    if (ptrs[i] == nullptr) return fail(GDN_ERR_INVALID_ARG, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(GDN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  size_t es = elem_size(sh->dtype);
  size_t obytes = (size_t)total * sh->Hv * sh->dv * es;
  const void* ins[5] = {q, k, v, g, beta};
  size_t inb[5] = {(size_t)total * sh->Hq * sh->dk * es, (size_t)total * sh->Hq * sh->dk * es, obytes,
                   (size_t)total * sh->Hv * 4, (size_t)total * sh->Hv * 4};
  for (int i = 0; i < 5; ++i)
    if (overlaps(o, obytes, ins[i], inb[i])) return fail(GDN_ERR_INVALID_ARG, "o overlaps %s", names[i]);
  return GDN_OK;
}

gdn_status check_states(const gdn_shape* sh, const float* s0, int64_t stride, const float* s_out) {
  const size_t per = (size_t)sh->Hv * sh->dk * sh->dv;
  if (stride < 0) return fail(GDN_ERR_INVALID_ARG, "initial_state_batch_stride=%lld < 0", (long long)stride);
  if (s0 != nullptr) {
    if (!aligned16(s0)) return fail(GDN_ERR_INVALID_ARG, "initial_state is not 16-byte aligned");
    if (stride % 4 != 0) return fail(GDN_ERR_INVALID_ARG, "initial_state_batch_stride must be a multiple of 4");
  }
  if (s_out != nullptr && !aligned16(s_out)) return fail(GDN_ERR_INVALID_ARG, "final_state is not 16-byte aligned");
  if (s0 != nullptr && s_out != nullptr && sh->B > 0) {
    size_t in_bytes = ((size_t)(sh->B - 1) * (size_t)stride + per) * 4;
    size_t out_bytes = (size_t)sh->B * per * 4;
    if (overlaps(s0, in_bytes, s_out, out_bytes)) {
      if (!(s0 == s_out && (size_t)stride == per))
        return fail(GDN_ERR_INVALID_ARG,
                    "final_state overlaps initial_state; only the exact in-place form "
                    "(same pointer, stride Hv*dk*dv) is allowed");
    }
  }
  return GDN_OK;
}

gdn_status check_prologue(const gdn_prologue* pr, gdn::Prologue* out) {
  *out = gdn::Prologue{};
  if (pr == nullptr) return GDN_OK;
  if (pr->qk_l2norm != 0) {
    if (!(pr->qk_l2norm_eps >= 0.f) || pr->qk_l2norm_eps == INFINITY)
      return fail(GDN_ERR_INVALID_ARG, "qk_l2norm_eps must be finite and >= 0");
    out->l2norm = 1;
    out->eps = pr->qk_l2norm_eps;
  }
  out->beta_logit = pr->beta_is_logit != 0;
  if (pr->gate_dt_bias != nullptr && pr->gate_A_log == nullptr)
    return fail(GDN_ERR_INVALID_ARG, "gate_dt_bias is given without gate_A_log");
  if ((reinterpret_cast<uintptr_t>(pr->gate_A_log) | reinterpret_cast<uintptr_t>(pr->gate_dt_bias)) & 3u)
    return fail(GDN_ERR_INVALID_ARG, "gate_A_log / gate_dt_bias are not 4-byte aligned");
  out->A_log = pr->gate_A_log;
  out->dt_bias = pr->gate_dt_bias;
  return GDN_OK;
}

}  // namespace

extern "C" {

int32_t gdn_abi_version(void) { return 1; }

const char* gdn_status_string(gdn_status st) {
  switch (st) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG: invalid argument";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: size or mode outside the compiled set";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime error";
  }
  return "unknown gdn_status";
}

const char* gdn_last_error(void) { return g_last_error; }

// Workspace: [chunk_offsets: B+1 int32][pad to 16][chunk_info: max_chunks x
// (first token, length) int32 pairs][pad to 256][per (chunk, value head) blocks].
// Upper bound on chunks: every sequence adds at most one partial chunk.
struct WsLayout {
  int64_t max_chunks;
  size_t info_off, head;
};
static WsLayout ws_layout(const gdn_shape* sh, int32_t chunk, int64_t total) {
  WsLayout w;
  w.max_chunks = total / chunk + sh->B + 1;
  w.info_off = align_up((size_t)(sh->B + 1) * 4, 16);
  w.head = align_up(w.info_off + (size_t)w.max_chunks * 8, 256);
  return w;
}

size_t gdn_prefill_workspace_bytes(const gdn_shape* sh, int32_t chunk, int32_t ragged) {
  int64_t total = 0;
  static const int32_t dummy = 0;
  if (check_shape(sh, ragged ? &dummy : nullptr, &total) != GDN_OK) return 0;
  if (chunk != 16 && chunk != 32 && chunk != 64) return 0;
  const WsLayout w = ws_layout(sh, chunk, total);
  return w.head + (size_t)w.max_chunks * sh->Hv * gdn::chunk_block_bytes((gdn::DType)sh->dtype);
}

}  // extern "C"

static gdn_status prefill_impl(const gdn_shape* sh, const gdn_prologue* pro, const void* q, const void* k,
                               const void* v, const float* g, const float* beta, const float* s0,
                               int64_t s0_stride, const int32_t* cu, int32_t chunk, void* o, float* s_out,
                               float* cs, int64_t cs_cap, void* ws, size_t ws_bytes, void* stream,
                               const char* name) {
  int64_t total = 0;
  gdn_status st = check_shape(sh, cu, &total);
  if (st != GDN_OK) return st;
  gdn::Prologue pr;
  if ((st = check_prologue(pro, &pr)) != GDN_OK) return st;
  if (chunk != 16 && chunk != 32 && chunk != 64)
    return fail(GDN_ERR_UNSUPPORTED, "chunk_size=%d: supported chunk sizes are 16, 32, 64", chunk);
  if ((st = check_tokens(sh, total, q, k, v, g, beta, o)) != GDN_OK) return st;
  if ((st = check_states(sh, s0, s0_stride, s_out)) != GDN_OK) return st;
  if (sh->B == 0) return GDN_OK;
  if (cu != nullptr && (reinterpret_cast<uintptr_t>(cu) & 3u))
    return fail(GDN_ERR_INVALID_ARG, "cu_seqlens is not 4-byte aligned");
  size_t need = gdn_prefill_workspace_bytes(sh, chunk, cu != nullptr);
  if (ws == nullptr || ws_bytes < need)
    return fail(GDN_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, need);
  if (!aligned16(ws)) return fail(GDN_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (cs != nullptr) {
    // no sequence set has more chunks than the workspace bound, so entries
    // past it are never written and take no part in the overlap check
    cs_cap = std::min(cs_cap, (int64_t)ws_layout(sh, chunk, total).max_chunks);
    const size_t per = (size_t)sh->Hv * sh->dk * sh->dv * 4;
    const size_t cs_bytes = (size_t)cs_cap * per;
    if (!aligned16(cs)) return fail(GDN_ERR_INVALID_ARG, "chunk_states is not 16-byte aligned");
    const size_t es = elem_size(sh->dtype);
    const size_t tb = (size_t)total;
    const void* bufs[9] = {q, k, v, g, beta, o, s0, s_out, ws};
    const size_t lens[9] = {tb * sh->Hq * sh->dk * es, tb * sh->Hq * sh->dk * es, tb * sh->Hv * sh->dv * es,
                            tb * sh->Hv * 4, tb * sh->Hv * 4, tb * sh->Hv * sh->dv * es,
                            s0 ? ((size_t)(sh->B - 1) * (size_t)s0_stride * 4 + per) : 0,
                            s_out ? (size_t)sh->B * per : 0, ws_bytes};
    const char* names[9] = {"q", "k", "v", "g", "beta", "o", "initial_state", "final_state", "workspace"};
    for (int i = 0; i < 9; ++i)
      if (bufs[i] != nullptr && overlaps(cs, cs_bytes, bufs[i], lens[i]))
        return fail(GDN_ERR_INVALID_ARG, "chunk_states overlaps %s", names[i]);
  }
  if (total == 0 && s_out == nullptr) return GDN_OK;

  gdn::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.s0 = s0; a.s0_stride = s0_stride; a.s_out = s_out; a.o = o; a.cu = cu;
  a.B = sh->B; a.T = sh->T; a.total = (int32_t)total;
  a.Hq = sh->Hq; a.Hv = sh->Hv; a.dk = sh->dk; a.dv = sh->dv; a.scale = sh->scale;
  a.chunk = chunk;
  const WsLayout w = ws_layout(sh, chunk, total);
  if (w.max_chunks * sh->Hv > 0x7fffffffLL - 8)
    return fail(GDN_ERR_UNSUPPORTED, "too many (chunk, head) pairs (%lld)", (long long)w.max_chunks * sh->Hv);
  a.max_chunks = (int32_t)w.max_chunks;
  a.chunk_offsets = static_cast<int32_t*>(ws);
  a.chunk_info = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + w.info_off);
  a.chunk_data = static_cast<char*>(ws) + w.head;
  a.chunk_states = cs;
  a.chunk_states_cap = cs != nullptr ? cs_cap : 0;
  a.pro = pr;
  hipError_t e = gdn::launch_prefill((gdn::DType)sh->dtype, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, name);
  return GDN_OK;
}

extern "C" {

gdn_status gdn_prefill_chunked(const gdn_shape* sh, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const float* s0, int64_t s0_stride,
                               const int32_t* cu, int32_t chunk, void* o, float* s_out, void* ws,
                               size_t ws_bytes, void* stream) {
  return prefill_impl(sh, nullptr, q, k, v, g, beta, s0, s0_stride, cu, chunk, o, s_out, nullptr, 0, ws, ws_bytes,
                      stream, "gdn_prefill_chunked launch");
}

gdn_status gdn_prefill_chunked_states(const gdn_shape* sh, const void* q, const void* k, const void* v,
                                      const float* g, const float* beta, const float* s0, int64_t s0_stride,
                                      const int32_t* cu, int32_t chunk, void* o, float* s_out, float* cs,
                                      int64_t cs_cap, void* ws, size_t ws_bytes, void* stream) {
  if (cs == nullptr) return fail(GDN_ERR_INVALID_ARG, "chunk_states is NULL");
  if (cs_cap < 0) return fail(GDN_ERR_INVALID_ARG, "chunk_states_capacity=%lld < 0", (long long)cs_cap);
  return prefill_impl(sh, nullptr, q, k, v, g, beta, s0, s0_stride, cu, chunk, o, s_out, cs, cs_cap, ws, ws_bytes,
                      stream, "gdn_prefill_chunked_states launch");
}

gdn_status gdn_prefill_chunked_ex(const gdn_shape* sh, const gdn_prologue* pro, const void* q, const void* k,
                                  const void* v, const float* g, const float* beta, const float* s0,
                                  int64_t s0_stride, const int32_t* cu, int32_t chunk, void* o, float* s_out,
                                  float* cs, int64_t cs_cap, void* ws, size_t ws_bytes, void* stream) {
  if (cs != nullptr && cs_cap < 0)
    return fail(GDN_ERR_INVALID_ARG, "chunk_states_capacity=%lld < 0", (long long)cs_cap);
  return prefill_impl(sh, pro, q, k, v, g, beta, s0, s0_stride, cu, chunk, o, s_out, cs, cs_cap, ws, ws_bytes,
                      stream, "gdn_prefill_chunked_ex launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Prefill without a caller workspace: the workspace lives in a fixed device
// array of GDN_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the process
// ends.  Its address on the current device is looked up once per device (the
// first call made with that device current) with hipGetSymbolAddress; host
// code only ever passes that address on, never the array's name.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];

gdn_status scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(GDN_ERR_UNSUPPORTED, "device %d: the allocation-free prefill supports devices 0..%d", dev,
                kScratchDevices - 1);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress(scratch)");
  if (g_scratch_ptr[dev] == nullptr) return fail(GDN_ERR_HIP, "scratch array has no device address");
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}
}  // namespace

extern "C" gdn_status gdn_prefill_chunked_noalloc(const gdn_shape* sh, const void* q, const void* k, const void* v,
                                                  const float* g, const float* beta, const float* s0,
                                                  int64_t s0_stride, const int32_t* cu, int32_t chunk, void* o,
                                                  float* s_out, void* stream) {
  const size_t need = gdn_prefill_workspace_bytes(sh, chunk, cu != nullptr);
  if (need == 0)   // invalid shape or chunk: let the common checks name the problem
    return prefill_impl(sh, nullptr, q, k, v, g, beta, s0, s0_stride, cu, chunk, o, s_out, nullptr, 0, nullptr, 0,
                        stream, "gdn_prefill_chunked_noalloc launch");
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
    return fail(GDN_ERR_UNSUPPORTED,
                "gdn_prefill_chunked_noalloc: this problem needs %zu bytes of workspace, above the fixed %zu-byte "
                "scratch array; use gdn_prefill_chunked with a caller workspace",
                need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  gdn_status st = scratch_on_current_device(&ws);
  if (st != GDN_OK) return st;
  return prefill_impl(sh, nullptr, q, k, v, g, beta, s0, s0_stride, cu, chunk, o, s_out, nullptr, 0, ws,
                      (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream, "gdn_prefill_chunked_noalloc launch");
}

static gdn_status recurrent_impl(const gdn_shape* sh, const gdn_prologue* pro, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta, const float* s0,
                                 int64_t s0_stride, const int32_t* cu, void* o, float* s_out, int32_t cap,
                                 const int32_t* counts, int32_t active, float* su, void* stream, const char* name) {
  int64_t total = 0;
  gdn_status st = check_shape(sh, cu, &total);
  if (st != GDN_OK) return st;
  gdn::Prologue pr;
  if ((st = check_prologue(pro, &pr)) != GDN_OK) return st;
  if ((st = check_tokens(sh, total, q, k, v, g, beta, o)) != GDN_OK) return st;
  if ((st = check_states(sh, s0, s0_stride, s_out)) != GDN_OK) return st;
  if (cap < 0) return fail(GDN_ERR_INVALID_ARG, "state_update_capacity=%d < 0", cap);
  if (cu != nullptr && (reinterpret_cast<uintptr_t>(cu) & 3u))
    return fail(GDN_ERR_INVALID_ARG, "cu_seqlens is not 4-byte aligned");
  const size_t R = (size_t)sh->Hv + (size_t)sh->Hq * sh->dk + (size_t)sh->Hv * sh->dv;
  const size_t su_elems = (size_t)sh->B * (size_t)cap * R;
  if (cap > 0) {
    if (counts == nullptr) return fail(GDN_ERR_INVALID_ARG, "capture_count is required when state_update_capacity > 0");
    if (su == nullptr) return fail(GDN_ERR_INVALID_ARG, "state_update is required when state_update_capacity > 0");
    if (reinterpret_cast<uintptr_t>(counts) & 3u) return fail(GDN_ERR_INVALID_ARG, "capture_count is not 4-byte aligned");
    if (!aligned16(su)) return fail(GDN_ERR_INVALID_ARG, "state_update is not 16-byte aligned");
    if (s_out != nullptr && overlaps(su, su_elems * 4, s_out, (size_t)sh->B * sh->Hv * sh->dk * sh->dv * 4))
      return fail(GDN_ERR_INVALID_ARG, "state_update overlaps final_state");
    if (o != nullptr && overlaps(su, su_elems * 4, o, (size_t)total * sh->Hv * sh->dv * elem_size(sh->dtype)))
      return fail(GDN_ERR_INVALID_ARG, "state_update overlaps o");
  }
  if (sh->B == 0) return GDN_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  // state_update_active = 0: the step kernel itself zero-fills the whole
  // state_update buffer (no separate launch)
  gdn::DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.s0 = s0; a.s0_stride = s0_stride; a.s_out = s_out; a.o = o; a.cu = cu;
  a.B = sh->B; a.T = sh->T; a.total = (int32_t)total;
  a.Hq = sh->Hq; a.Hv = sh->Hv; a.dk = sh->dk; a.dv = sh->dv; a.scale = sh->scale;
  a.cap = cap; a.counts = counts; a.active = active; a.su = su;
  a.pro = pr;
  hipError_t e = gdn::launch_recurrent((gdn::DType)sh->dtype, a, s);
  if (e != hipSuccess) return hip_fail(e, name);
  return GDN_OK;
}

extern "C" {

gdn_status gdn_recurrent_step(const gdn_shape* sh, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* s0, int64_t s0_stride,
                              const int32_t* cu, void* o, float* s_out, int32_t cap, const int32_t* counts,
                              int32_t active, float* su, void* stream) {
  return recurrent_impl(sh, nullptr, q, k, v, g, beta, s0, s0_stride, cu, o, s_out, cap, counts, active, su, stream,
                        "gdn_recurrent_step launch");
}

gdn_status gdn_recurrent_step_ex(const gdn_shape* sh, const gdn_prologue* pro, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta, const float* s0,
                                 int64_t s0_stride, const int32_t* cu, void* o, float* s_out, int32_t cap,
                                 const int32_t* counts, int32_t active, float* su, void* stream) {
  return recurrent_impl(sh, pro, q, k, v, g, beta, s0, s0_stride, cu, o, s_out, cap, counts, active, su, stream,
                        "gdn_recurrent_step_ex launch");
}

gdn_status gdn_replay_state_updates(int32_t B, int32_t Hq, int32_t Hv, int32_t dk, int32_t dv, int32_t cap,
                                    const float* su, const int32_t* counts, float* state, void* stream) {
  if (B < 0 || Hq <= 0 || Hv <= 0) return fail(GDN_ERR_INVALID_ARG, "B=%d, Hq=%d, Hv=%d", B, Hq, Hv);
  if (Hv % Hq != 0) return fail(GDN_ERR_INVALID_ARG, "Hv=%d must be a multiple of Hq=%d", Hv, Hq);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN_ERR_UNSUPPORTED, "dk=%d, dv=%d: supported head dims are 16, 32, 64, 128", dk, dv);
  if (cap < 0) return fail(GDN_ERR_INVALID_ARG, "state_update_capacity=%d < 0", cap);
  if (B > 65535 || Hv > 65535) return fail(GDN_ERR_UNSUPPORTED, "B or Hv exceeds 65535");
  if ((int64_t)B * Hv > (1 << 24)) return fail(GDN_ERR_UNSUPPORTED, "B*Hv exceeds 2^24 (row, head) pairs");
  if (B == 0 || cap == 0) return GDN_OK;
  if (su == nullptr || counts == nullptr || state == nullptr)
    return fail(GDN_ERR_INVALID_ARG, "state_update, replay_count and state are required");
  if (!aligned16(state)) return fail(GDN_ERR_INVALID_ARG, "state is not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(su) & 3u) return fail(GDN_ERR_INVALID_ARG, "state_update is not 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(counts) & 3u) return fail(GDN_ERR_INVALID_ARG, "replay_count is not 4-byte aligned");
  const size_t R = (size_t)Hv + (size_t)Hq * dk + (size_t)Hv * dv;
  if (overlaps(su, (size_t)B * cap * R * 4, state, (size_t)B * Hv * dk * dv * 4))
    return fail(GDN_ERR_INVALID_ARG, "state_update overlaps state");
  gdn::ReplayArgs a{B, Hq, Hv, dk, dv, cap, su, counts, state};
  hipError_t e = gdn::launch_replay(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_replay_state_updates launch");
  return GDN_OK;
}

gdn_status gdn_state_snapshot(const float* src, float* dst, int64_t num_states, int32_t Hv, int32_t dk, int32_t dv,
                              void* stream) {
  if (num_states < 0 || Hv <= 0 || dk <= 0 || dv <= 0)
    return fail(GDN_ERR_INVALID_ARG, "num_states=%lld, Hv=%d, dk=%d, dv=%d", (long long)num_states, Hv, dk, dv);
  if (num_states == 0) return GDN_OK;
  if (src == nullptr || dst == nullptr) return fail(GDN_ERR_INVALID_ARG, "src and dst are required");
  if (!aligned16(src) || !aligned16(dst)) return fail(GDN_ERR_INVALID_ARG, "src/dst are not 16-byte aligned");
  size_t n = (size_t)num_states * Hv * dk * dv;
  if (overlaps(src, n * 4, dst, n * 4)) return fail(GDN_ERR_INVALID_ARG, "snapshot src and dst overlap");
  hipError_t e = gdn::launch_copy(src, dst, n, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_state_snapshot launch");
  return GDN_OK;
}

}  // extern "C"
