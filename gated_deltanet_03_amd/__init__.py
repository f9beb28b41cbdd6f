"""Python binding of libgdn.so, the MI355X Gated DeltaNet engine.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/gdn.h``.  Torch supplies device
memory and the current HIP stream.  There is no fallback: if the library is
missing or fails to load, importing the entry points raises.

Entry points (same names as the C ABI):

``gdn_prefill_chunked``       chunked prefill with explicit initial/final state
``gdn_recurrent_step``        token-by-token step with compact state-update capture
``gdn_replay_state_updates``  replay of captured (decay, key, delta) records
``gdn_state_snapshot``        immutable copy of a state set
``gdn_prefill_workspace_bytes``
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_F16, GDN_BF16 = 0, 1, 2
GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = 0, 1, 2, 3
_DTYPES = {torch.float32: GDN_F32, torch.float16: GDN_F16, torch.bfloat16: GDN_BF16}
EXPORTED = ("gdn_abi_version", "gdn_prefill_workspace_bytes", "gdn_prefill_chunked",
            "gdn_prefill_chunked_states", "gdn_prefill_chunked_ex", "gdn_recurrent_step",
            "gdn_recurrent_step_ex", "gdn_replay_state_updates", "gdn_state_snapshot",
            "gdn_status_string", "gdn_last_error", "gdn_profile_enable", "gdn_profile_collect",
            "gdn_prefill_chunked_noalloc")
GDN_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024


class gdn_prologue(ctypes.Structure):
    _fields_ = [("qk_l2norm", ctypes.c_int32), ("qk_l2norm_eps", ctypes.c_float),
                ("beta_is_logit", ctypes.c_int32), ("gate_A_log", ctypes.c_void_p),
                ("gate_dt_bias", ctypes.c_void_p)]


class Prologue:
    """Input prologue of the *_ex calls: qk_l2norm (with eps), beta given as
    logits, and the gate -exp(A_log[h]) * softplus(g + dt_bias[h]) when A_log
    (fp32 [Hv] on the device) is set.  Tensors are kept alive by this object."""

    def __init__(self, qk_l2norm=False, eps=1e-6, beta_is_logit=False, A_log=None, dt_bias=None):
        self.qk_l2norm, self.eps, self.beta_is_logit = bool(qk_l2norm), float(eps), bool(beta_is_logit)
        self.A_log, self.dt_bias = A_log, dt_bias

    def as_c(self, device):
        for t, n in ((self.A_log, "A_log"), (self.dt_bias, "dt_bias")):
            _need(t, n, torch.float32, device)
        return gdn_prologue(int(self.qk_l2norm), self.eps, int(self.beta_is_logit),
                            None if self.A_log is None else self.A_log.data_ptr(),
                            None if self.dt_bias is None else self.dt_bias.data_ptr())


class gdn_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hv", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdn.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m gated_deltanet_03_amd._build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    shp = ctypes.POINTER(gdn_shape)
    lib.gdn_abi_version.restype = i32
    lib.gdn_abi_version.argtypes = []
    lib.gdn_prefill_workspace_bytes.restype = sz
    lib.gdn_prefill_workspace_bytes.argtypes = [shp, i32, i32]
    lib.gdn_prefill_chunked.restype = i32
    lib.gdn_prefill_chunked.argtypes = [shp, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, vp, sz, vp]
    lib.gdn_prefill_chunked_noalloc.restype = i32
    lib.gdn_prefill_chunked_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, vp]
    lib.gdn_recurrent_step.restype = i32
    lib.gdn_prefill_chunked_states.argtypes = [shp, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, vp, i64, vp,
                                               sz, vp]
    lib.gdn_prefill_chunked_states.restype = i32
    pro = ctypes.POINTER(gdn_prologue)
    lib.gdn_prefill_chunked_ex.argtypes = [shp, pro, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, vp, i64, vp,
                                           sz, vp]
    lib.gdn_prefill_chunked_ex.restype = i32
    lib.gdn_recurrent_step_ex.argtypes = [shp, pro, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, i32, vp, i32, vp, vp]
    lib.gdn_recurrent_step_ex.restype = i32
    lib.gdn_recurrent_step.argtypes = [shp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, i32, vp, i32, vp, vp]
    lib.gdn_replay_state_updates.restype = i32
    lib.gdn_replay_state_updates.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.gdn_state_snapshot.restype = i32
    lib.gdn_state_snapshot.argtypes = [vp, vp, i64, i32, i32, i32, vp]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [i32]
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_profile_enable.restype = i32
    lib.gdn_profile_enable.argtypes = [i32]
    lib.gdn_profile_collect.restype = i32
    lib.gdn_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int32), i32]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != GDN_OK:
        lib = load_library()
        raise GdnError(status, f"{lib.gdn_status_string(status).decode()}: {lib.gdn_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    if device is None or device.type != "cuda":
        return ctypes.c_void_p(0)
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _expect(t, name, numel, at_least=False):
    """Raise ValueError unless tensor t holds exactly (or at least) numel elements.
    The C ABI sees bare pointers, so sizes are checked here, before any call."""
    if t is None:
        return
    n = t.numel()
    if (n < numel) if at_least else (n != numel):
        rel = "at least " if at_least else ""
        raise ValueError(f"{name} has {n} elements, expected {rel}{numel}")


def _check_tokens(sh, q, k, v, g, beta, o, cu_seqlens):
    """Token tensors against the problem description built from q and v."""
    ntok = sh.T if cu_seqlens is not None else sh.B * sh.T
    if tuple(k.shape) != tuple(q.shape):
        raise ValueError(f"k has shape {tuple(k.shape)}, q has {tuple(q.shape)}")
    if v.dim() != q.dim() or tuple(v.shape[:-2]) != tuple(q.shape[:-2]):
        raise ValueError(f"v has shape {tuple(v.shape)}; its leading dims must match q's {tuple(q.shape[:-2])}")
    _expect(v, "v", ntok * sh.Hv * sh.dv)
    for t, n in ((g, "g"), (beta, "beta")):
        if tuple(t.shape) != tuple(v.shape[:-1]):
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {tuple(v.shape[:-1])}")
    if o is not None and tuple(o.shape) != tuple(v.shape):
        raise ValueError(f"o has shape {tuple(o.shape)}, expected {tuple(v.shape)}")
    if cu_seqlens is not None and cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be 1-D [N+1]")


def _check_states(sh, initial_state, stride, final_state):
    """initial_state covers (B-1)*stride + Hv*dk*dv elements; final_state is [B, Hv, dk, dv]."""
    per = sh.Hv * sh.dk * sh.dv
    if stride < 0:
        raise ValueError(f"initial_state_batch_stride={stride} < 0")
    if initial_state is not None and sh.B > 0:
        _expect(initial_state, "initial_state", (sh.B - 1) * stride + per, at_least=True)
    if final_state is not None and tuple(final_state.shape) != (sh.B, sh.Hv, sh.dk, sh.dv):
        raise ValueError(f"final_state has shape {tuple(final_state.shape)}, expected "
                         f"{(sh.B, sh.Hv, sh.dk, sh.dv)}")


def _shape_from(q, k, v, scale, cu_seqlens):
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("dense q must be [B, T, Hq, dk]")
        B, T, Hq, dk = q.shape
    else:
        if q.dim() == 4:
            if q.shape[0] != 1:
                raise ValueError("ragged q must be [1, T, Hq, dk] or [T, Hq, dk]")
            q = q[0]
        T, Hq, dk = q.shape
        B = cu_seqlens.numel() - 1
    Hv, dv = v.shape[-2], v.shape[-1]
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if scale is None:
        scale = dk ** -0.5
    return gdn_shape(B, T, Hq, Hv, dk, dv, float(scale), _DTYPES[q.dtype])


def gdn_prefill_workspace_bytes(shape: gdn_shape, chunk_size: int, ragged: bool) -> int:
    return int(load_library().gdn_prefill_workspace_bytes(ctypes.byref(shape), chunk_size, int(bool(ragged))))


def gdn_prefill_chunked(q, k, v, g, beta, *, scale=None, initial_state=None,
                        initial_state_batch_stride=None, cu_seqlens=None, chunk_size=64,
                        o=None, final_state=None, output_final_state=True, workspace=None):
    """Chunked prefill.  Dense q/k [B,T,Hq,dk], v [B,T,Hv,dv], g/beta [B,T,Hv];
    ragged: the same without B (or B=1) plus cu_seqlens int32 [N+1] on the device.
    Returns (o, final_state or None)."""
    return _prefill(q, k, v, g, beta, scale, initial_state, initial_state_batch_stride, cu_seqlens,
                    chunk_size, o, final_state, output_final_state, workspace, False, None, None)[:2]


def gdn_prefill_chunked_noalloc(q, k, v, g, beta, *, scale=None, initial_state=None,
                                initial_state_batch_stride=None, cu_seqlens=None, chunk_size=64,
                                o=None, final_state=None, output_final_state=True):
    """gdn_prefill_chunked with the library's fixed device scratch array as the
    workspace (the C entry point allocates nothing; pass ``o`` and
    ``final_state`` to allocate nothing here either).  Returns (o, final_state
    or None)."""
    lib = load_library()
    dev = q.device
    sh = _shape_from(q, k, v, scale, cu_seqlens)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _need(initial_state, "initial_state", torch.float32, dev)
    if o is None:
        o = torch.empty(v.shape, dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, dev)
    per = sh.Hv * sh.dk * sh.dv
    if final_state is None and output_final_state:
        final_state = torch.empty((sh.B, sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev)
    if initial_state_batch_stride is None:
        initial_state_batch_stride = 0 if (initial_state is not None and initial_state.shape[0] == 1
                                           and sh.B > 1) else per
    _check_tokens(sh, q, k, v, g, beta, o, cu_seqlens)
    _check_states(sh, initial_state, int(initial_state_batch_stride), final_state)
    _check(lib.gdn_prefill_chunked_noalloc(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                           _ptr(initial_state), int(initial_state_batch_stride),
                                           _ptr(cu_seqlens), int(chunk_size), _ptr(o), _ptr(final_state),
                                           _stream(dev)))
    return o, final_state


def gdn_prefill_chunked_states(q, k, v, g, beta, *, scale=None, initial_state=None,
                               initial_state_batch_stride=None, cu_seqlens=None, chunk_size=64,
                               o=None, final_state=None, output_final_state=True, workspace=None,
                               chunk_states=None, num_chunks=None):
    """Chunked prefill that also returns the state after every chunk:
    chunk_states [sum_s ceil(L_s / chunk_size), Hv, dk, dv] fp32, sequence s's
    chunk j at index sum_{s'<s} ceil(L_s'/chunk_size) + j.  Without
    ``chunk_states`` or ``num_chunks`` the count is taken from the lengths
    (ragged input: one device-to-host read of cu_seqlens).
    Returns (o, final_state or None, chunk_states)."""
    return _prefill(q, k, v, g, beta, scale, initial_state, initial_state_batch_stride, cu_seqlens,
                    chunk_size, o, final_state, output_final_state, workspace, True, chunk_states, num_chunks)


def gdn_prefill_chunked_ex(q, k, v, g, beta, *, prologue=None, scale=None, initial_state=None,
                           initial_state_batch_stride=None, cu_seqlens=None, chunk_size=64, o=None,
                           final_state=None, output_final_state=True, workspace=None, chunk_states=None,
                           num_chunks=None, emit_chunk_states=False):
    """Chunked prefill with the input prologue (a ``Prologue`` or None) and,
    with ``emit_chunk_states`` (or a ``chunk_states`` buffer), the boundary
    states.  Returns (o, final_state or None, chunk_states or None)."""
    emit = emit_chunk_states or chunk_states is not None or num_chunks is not None
    return _prefill(q, k, v, g, beta, scale, initial_state, initial_state_batch_stride, cu_seqlens,
                    chunk_size, o, final_state, output_final_state, workspace, emit, chunk_states, num_chunks,
                    prologue=prologue if prologue is not None else Prologue())


def _prefill(q, k, v, g, beta, scale, initial_state, initial_state_batch_stride, cu_seqlens, chunk_size,
             o, final_state, output_final_state, workspace, emit, chunk_states, num_chunks, prologue=None):
    lib = load_library()
    dev = q.device
    sh = _shape_from(q, k, v, scale, cu_seqlens)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _need(initial_state, "initial_state", torch.float32, dev)
    if o is None:
        o = torch.empty(v.shape, dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, dev)
    per = sh.Hv * sh.dk * sh.dv
    if final_state is None and output_final_state:
        final_state = torch.empty((sh.B, sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev)
    if initial_state_batch_stride is None:
        initial_state_batch_stride = 0 if (initial_state is not None and initial_state.shape[0] == 1
                                           and sh.B > 1) else per
    _check_tokens(sh, q, k, v, g, beta, o, cu_seqlens)
    _check_states(sh, initial_state, int(initial_state_batch_stride), final_state)
    need = gdn_prefill_workspace_bytes(sh, chunk_size, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None, dev)
    common = (ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
              int(initial_state_batch_stride), _ptr(cu_seqlens), int(chunk_size), _ptr(o), _ptr(final_state))
    if prologue is not None:
        pc = prologue.as_c(dev)
        buf = None
        if emit:
            chunk_states, buf = _chunk_buffer(sh, cu_seqlens, chunk_size, chunk_states, num_chunks, dev)
        ncs = 0 if buf is None else int(chunk_states.numel() // max(per, 1))
        _check(lib.gdn_prefill_chunked_ex(common[0], ctypes.byref(pc), *common[1:], _ptr(buf), ncs,
                                          _ptr(workspace), workspace.numel(), _stream(dev)))
        return o, final_state, chunk_states if emit else None
    if not emit:
        _check(lib.gdn_prefill_chunked(*common, _ptr(workspace), workspace.numel(), _stream(dev)))
        return o, final_state, None
    chunk_states, buf = _chunk_buffer(sh, cu_seqlens, chunk_size, chunk_states, num_chunks, dev)
    _check(lib.gdn_prefill_chunked_states(*common, _ptr(buf), int(chunk_states.numel() // max(per, 1)),
                                          _ptr(workspace), workspace.numel(), _stream(dev)))
    return o, final_state, chunk_states


def _chunk_buffer(sh, cu_seqlens, chunk_size, chunk_states, num_chunks, dev):
    """(chunk_states view, buffer with an address) for the boundary states."""
    if chunk_states is not None:
        _need(chunk_states, "chunk_states", torch.float32, dev)
        if chunk_states.dim() != 4 or tuple(chunk_states.shape[1:]) != (sh.Hv, sh.dk, sh.dv):
            raise ValueError(f"chunk_states has shape {tuple(chunk_states.shape)}, expected "
                             f"[num_chunks, {sh.Hv}, {sh.dk}, {sh.dv}]")
        return chunk_states, chunk_states
    if num_chunks is None:
        if cu_seqlens is None:
            num_chunks = sh.B * (-(-sh.T // chunk_size))
        else:
            lens = cu_seqlens.cpu().diff()
            num_chunks = int(((lens + chunk_size - 1) // chunk_size).sum())
    # at least one entry, so the buffer has an address even with no chunks
    buf = torch.empty((max(int(num_chunks), 1), sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device=dev)
    return buf[:int(num_chunks)], buf


def gdn_recurrent_step_ex(q, k, v, g, beta, *, prologue=None, **kw):
    """Recurrent step with the input prologue (a ``Prologue`` or None); the
    other arguments as gdn_recurrent_step.  Returns (o, final_state, state_update)."""
    return gdn_recurrent_step(q, k, v, g, beta, _prologue=prologue if prologue is not None else Prologue(), **kw)


def gdn_recurrent_step(q, k, v, g, beta, *, scale=None, initial_state=None,
                       initial_state_batch_stride=None, cu_seqlens=None, o=None, final_state=None,
                       output_final_state=True, state_update_capacity=0, capture_count=None,
                       state_update_active=1, state_update=None, _prologue=None):
    """Recurrent step with optional compact capture.  Returns (o, final_state, state_update)."""
    lib = load_library()
    dev = q.device
    sh = _shape_from(q, k, v, scale, cu_seqlens)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _need(initial_state, "initial_state", torch.float32, dev)
    _need(capture_count, "capture_count", torch.int32, dev)
    if o is None:
        o = torch.empty(v.shape, dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, dev)
    per = sh.Hv * sh.dk * sh.dv
    if final_state is None and output_final_state:
        final_state = torch.empty((sh.B, sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev)
    if initial_state_batch_stride is None:
        initial_state_batch_stride = 0 if (initial_state is not None and initial_state.shape[0] == 1
                                           and sh.B > 1) else per
    cap = int(state_update_capacity)
    if cap > 0 and state_update is None:
        R = sh.Hv + sh.Hq * sh.dk + sh.Hv * sh.dv
        state_update = torch.empty((sh.B, cap, R), dtype=torch.float32, device=dev)
    _need(state_update, "state_update", torch.float32, dev)
    _check_tokens(sh, q, k, v, g, beta, o, cu_seqlens)
    _check_states(sh, initial_state, int(initial_state_batch_stride), final_state)
    if cap < 0:
        raise ValueError(f"state_update_capacity={cap} < 0")
    if cap > 0:
        if capture_count is None:
            raise ValueError("capture_count is required when state_update_capacity > 0")
        _expect(capture_count, "capture_count", sh.B, at_least=True)
        R = sh.Hv + sh.Hq * sh.dk + sh.Hv * sh.dv
        _expect(state_update, "state_update", sh.B * cap * R, at_least=True)
    rest = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), int(initial_state_batch_stride),
            _ptr(cu_seqlens), _ptr(o), _ptr(final_state), cap, _ptr(capture_count), int(state_update_active),
            _ptr(state_update), _stream(dev))
    if _prologue is None:
        _check(lib.gdn_recurrent_step(ctypes.byref(sh), *rest))
    else:
        pc = _prologue.as_c(dev)
        _check(lib.gdn_recurrent_step_ex(ctypes.byref(sh), ctypes.byref(pc), *rest))
    return o, final_state, state_update


def gdn_replay_state_updates(state, state_update, replay_count, *, Hq, state_update_capacity=None):
    """Replay the first replay_count[b] records of each row onto state (in place)."""
    lib = load_library()
    dev = state.device
    B, Hv, dk, dv = state.shape
    cap = state_update.shape[1] if state_update_capacity is None else int(state_update_capacity)
    _need(state, "state", torch.float32, dev)
    _need(state_update, "state_update", torch.float32, dev)
    _need(replay_count, "replay_count", torch.int32, dev)
    if state.dim() != 4:
        raise ValueError(f"state must be [B, Hv, dk, dv], got shape {tuple(state.shape)}")
    Hq = int(Hq)
    if Hq <= 0 or Hv % Hq != 0:
        raise ValueError(f"Hq={Hq} must be positive and divide Hv={Hv}")
    if cap < 0:
        raise ValueError(f"state_update_capacity={cap} < 0")
    R = Hv + Hq * dk + Hv * dv
    if state_update.dim() == 3 and state_update.shape[-1] != R:
        raise ValueError(f"state_update records hold {state_update.shape[-1]} floats; Hv + Hq*dk + Hv*dv = {R}")
    if cap > 0:
        _expect(state_update, "state_update", B * cap * R, at_least=True)
        _expect(replay_count, "replay_count", B, at_least=True)
    _check(lib.gdn_replay_state_updates(B, int(Hq), Hv, dk, dv, cap, _ptr(state_update), _ptr(replay_count),
                                        _ptr(state), _stream(dev)))
    return state


def gdn_state_snapshot(src, dst=None):
    """Bitwise copy of a [N, Hv, dk, dv] fp32 state set, ordered on the current stream."""
    lib = load_library()
    dev = src.device
    _need(src, "src", torch.float32, dev)
    if dst is None:
        dst = torch.empty_like(src)
    _need(dst, "dst", torch.float32, dev)
    if src.dim() != 4:
        raise ValueError(f"src must be [N, Hv, dk, dv], got shape {tuple(src.shape)}")
    if tuple(dst.shape) != tuple(src.shape):
        raise ValueError(f"dst has shape {tuple(dst.shape)}, src {tuple(src.shape)}")
    N, Hv, dk, dv = src.shape
    _check(lib.gdn_state_snapshot(_ptr(src), _ptr(dst), N, Hv, dk, dv, _stream(dev)))
    return dst


def gdn_profile_enable(on: bool = True) -> None:
    """Turn per-kernel HIP-event timing inside the library on or off."""
    _check(load_library().gdn_profile_enable(int(bool(on))))


def gdn_profile_collect() -> dict:
    """{kernel name: (launches, total ms)} for the kernels timed since the last collect."""
    lib = load_library()
    n = 16
    names = (ctypes.c_char_p * n)()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    k = lib.gdn_profile_collect(names, ms, cnt, n)
    return {names[i].decode(): (int(cnt[i]), float(ms[i])) for i in range(min(k, n))}


__all__ = ["gdn_profile_enable", "gdn_profile_collect", "load_library", "GdnError", "gdn_shape",
           "gdn_prefill_workspace_bytes", "gdn_prefill_chunked", "gdn_prefill_chunked_states",
           "gdn_prefill_chunked_noalloc", "GDN_NOALLOC_SCRATCH_BYTES",
           "gdn_prefill_chunked_ex", "gdn_recurrent_step_ex", "Prologue", "gdn_prologue",
           "gdn_recurrent_step", "gdn_replay_state_updates", "gdn_state_snapshot", "EXPORTED", "LIB_PATH"]
