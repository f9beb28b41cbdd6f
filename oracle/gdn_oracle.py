"""Plain fp64 token-by-token Gated DeltaNet oracle (test infrastructure only).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may use
this module.  It is deliberately slow and literal: one token at a time, one
formula per line, numpy float64 throughout.  Inputs are upcast to float64
*after* they were rounded to the input dtype, so the oracle sees exactly the
values the device sees.

Sources (page title, part of the page):

* [onnxruntime PR 32767, "[WebGPU EP] adds state update capacity support for
  GatedDeltaNet", section "Changes"]: the recurrent path captures, per row, a
  clamped prefix of per-token (decay, shared key, delta) factors whose replay is
  S <- decay * S + outer(key, delta); ``state_update_active = 0`` clears the whole
  capture output; inverse-GQA key sharing (value heads outnumber key heads).
* [executorch issue 23097, "Enable the native Kev example on NVIDIA GPUs ...",
  "Work to cover"]: a prefill with explicit initial and final state, an FP32
  recurrence under 16-bit weights, prefix snapshots reused across batches.
* [executorch issue 23099, "Enable the native Kev example on the WebGPU
  backend", "Work to cover"]: repeated evaluations must leave the prefix state
  unchanged.

The gated delta rule this oracle evaluates (the replay identity of PR 32767
with decay = alpha_t, key = k_t, delta = delta_t):

    alpha_t = exp(g_t)
    delta_t = beta_t * (v_t - (alpha_t * S_{t-1})^T k_t)
    S_t     = alpha_t * S_{t-1} + k_t delta_t^T
    o_t     = scale * S_t^T q_t            (post-update state)

S is [dk, dv] per (sequence, value head); value head h reads key/query head
h // (Hv / Hq) (contiguous groups of value heads share a key head).

Parity status: pinned (tests/test_oracle_pins.py) except the head map above,
which is a convention ("parity unpinned" beyond it).
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a CPU torch tensor handed over by a test
        x = x.detach().to("cpu")
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def record_width(Hq: int, Hv: int, dk: int, dv: int) -> int:
    """Floats per capture record: [decay Hv | key Hq*dk | delta Hv*dv].

    [PR 32767, "Changes"]: one packed float32 output holds decay, shared-key
    and delta factors; the packing order is this library's convention.
    """
    return Hv + Hq * dk + Hv * dv


def sequence_bounds(num_seqs: int, tokens: int, cu_seqlens=None):
    """(start, end) token ranges of each sequence in the packed token axis.

    Dense input: ``num_seqs`` rows of ``tokens`` tokens each.  Packed ragged
    input: ``cu_seqlens`` [N+1] with 0 = cu[0] <= ... <= cu[N] = total tokens;
    empty sequences are allowed.
    """
    if cu_seqlens is None:
        return [(b * tokens, (b + 1) * tokens) for b in range(num_seqs)]
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    assert cu[0] == 0 and all(cu[i] <= cu[i + 1] for i in range(len(cu) - 1))
    return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def _token_update(S, a, kt, vt, b, qt, scale):
    """One token of the gated delta rule, vectorised over value heads.

    S [H, dk, dv]; a, b [H]; kt, qt [H, dk] (key head already mapped); vt [H, dv].
    Returns (S_t, o_t, delta_t).
    """
    u = np.einsum("hij,hi->hj", a[:, None, None] * S, kt)   # (alpha S_{t-1})^T k_t
    delta = b[:, None] * (vt - u)                            # beta (v - ...)
    S_new = a[:, None, None] * S + kt[:, :, None] * delta[:, None, :]   # alpha S + k delta^T
    o = scale * np.einsum("hij,hi->hj", S_new, qt)           # scale S_t^T q_t
    return S_new, o, delta


def recurrent(q, k, v, g, beta, scale, Hq, Hv, cu_seqlens=None, num_seqs=None,
              initial_state=None, initial_state_broadcast=False, heads=None, boundary_every=None):
    """Run the recurrence over every sequence, token by token.

    Layouts (packed tokens): q, k [Ttot, Hq, dk]; v [Ttot, Hv, dv]; g, beta
    [Ttot, Hv].  Dense rows: pass ``num_seqs`` (rows of Ttot/num_seqs tokens).
    ``initial_state`` [N, Hv, dk, dv] (or [1, Hv, dk, dv] with
    ``initial_state_broadcast``); None means zeros.  ``heads`` restricts the
    computation to a subset of value heads (sampled parity at large sizes).

    ``boundary_every`` = C also records the state after every C-th token of
    each sequence and after its last token, i.e. the snapshot of every prefix
    that ends on a chunk boundary ([executorch issue 23097, "Work to cover"]:
    GDN chunk boundaries and retained prefix snapshots).  Sequence s
    contributes ceil(L_s / C) entries, in sequence order.

    Returns dict with
      o        [Ttot, Hv, dv]   (entries of heads not computed are NaN)
      final    [N, Hv, dk, dv]
      alpha    [Ttot, Hv]       per-token decay exp(g)
      delta    [Ttot, Hv, dv]   per-token delta (includes beta)
      boundary [sum_s ceil(L_s/C), Hv, dk, dv] (only with ``boundary_every``)
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    Ttot, _, dk = k.shape
    dv = v.shape[2]
    assert Hv % Hq == 0, "Hv must be a multiple of Hq"
    G = Hv // Hq
    if cu_seqlens is None:
        N = 1 if num_seqs is None else int(num_seqs)
        assert Ttot % N == 0
        bounds = sequence_bounds(N, Ttot // N)
    else:
        bounds = sequence_bounds(0, 0, cu_seqlens)
        N = len(bounds)
        assert bounds[-1][1] == Ttot if N else Ttot == 0
    hs = np.arange(Hv) if heads is None else np.asarray(sorted(heads))
    hk = hs // G                                           # inverse-GQA head map
    s0 = _f64(initial_state)

    o = np.full((Ttot, Hv, dv), np.nan)
    final = np.full((N, Hv, dk, dv), np.nan)
    alpha_all = np.full((Ttot, Hv), np.nan)
    delta_all = np.full((Ttot, Hv, dv), np.nan)
    boundary = []
    for s, (t0, t1) in enumerate(bounds):
        if s0 is None:
            S = np.zeros((len(hs), dk, dv))
        else:
            S = s0[0 if initial_state_broadcast else s][hs].copy()
        for t in range(t0, t1):
            a = np.exp(g[t, hs])
            S, o_t, d_t = _token_update(S, a, k[t, hk], v[t, hs], beta[t, hs], q[t, hk], scale)
            o[t, hs] = o_t
            alpha_all[t, hs] = a
            delta_all[t, hs] = d_t
            if boundary_every and ((t + 1 - t0) % boundary_every == 0 or t == t1 - 1):
                snap = np.full((Hv, dk, dv), np.nan)
                snap[hs] = S
                boundary.append(snap)
        final[s, hs] = S
    out = {"o": o, "final": final, "alpha": alpha_all, "delta": delta_all}
    if boundary_every:
        out["boundary"] = np.stack(boundary) if boundary else np.zeros((0, Hv, dk, dv))
    return out


def prologue(q, k, g, beta, qk_l2norm=False, eps=1e-6, beta_is_logit=False, A_log=None, dt_bias=None):
    """The optional input prologue, in fp64: returns (q, k, g, beta) as the
    recurrence consumes them.

    [executorch issue 23097, "Work to cover"]: reusing a GDN kernel means
    adapting its gate and scaling conventions; the pages give no formulas, so
    the common ones are taken, each switched on separately:
      qk_l2norm:     x / sqrt(sum_i x_i^2 + eps) for every q_t and k_t (last axis)
      beta_is_logit: beta = 1 / (1 + exp(-b))
      A_log [Hv]:    g = -exp(A_log[h]) * softplus(g_in + dt_bias[h]),
                     softplus(x) = log(1 + exp(x)); dt_bias None means 0
    """
    q, k, g, beta = (_f64(x) for x in (q, k, g, beta))
    if qk_l2norm:
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    if beta_is_logit:
        beta = 1.0 / (1.0 + np.exp(-beta))
    if A_log is not None:
        A = _f64(A_log)
        dt = np.zeros_like(A) if dt_bias is None else _f64(dt_bias)
        g = -np.exp(A)[None, :] * np.logaddexp(0.0, g + dt[None, :])   # logaddexp(0, x) = softplus(x)
    return q, k, g, beta


def capture(k, alpha, delta, Hq, Hv, capacity, capture_count, active,
            cu_seqlens=None, num_seqs=None):
    """Expected compact state-update buffer and the mask of specified entries.

    [PR 32767, "Changes"]: for each row b the first n_b tokens are captured,
    n_b = min(max(capture_count[b], 0), capacity, L_b) (the clamp bounds are
    the reading this library takes).  Record c of row b holds, for token start_b + c:
    decay[h] = alpha, key[hk] = k (fp32, stored once per key head), delta[h].
    With ``active == 0`` the whole buffer is zero and every entry is specified;
    when active, uncaptured entries are unspecified (mask False).

    Returns (buffer [N, capacity, R] float64, mask [N, capacity, R] bool).
    """
    k, alpha, delta = _f64(k), _f64(alpha), _f64(delta)
    Ttot, _, dk = k.shape
    dv = delta.shape[2]
    R = record_width(Hq, Hv, dk, dv)
    if cu_seqlens is None:
        N = int(num_seqs)
        bounds = sequence_bounds(N, Ttot // N)
    else:
        bounds = sequence_bounds(0, 0, cu_seqlens)
        N = len(bounds)
    buf = np.zeros((N, capacity, R))
    if not active:
        return buf, np.ones((N, capacity, R), dtype=bool)
    mask = np.zeros((N, capacity, R), dtype=bool)
    counts = np.asarray(capture_count).reshape(-1)
    for b, (t0, t1) in enumerate(bounds):
        n = min(max(int(counts[b]), 0), capacity, t1 - t0)
        for c in range(n):
            t = t0 + c
            rec = np.concatenate([alpha[t], k[t].reshape(-1), delta[t].reshape(-1)])
            buf[b, c] = rec
            mask[b, c] = True
    return buf, mask


def replay(state, state_update, replay_count, Hq, Hv, dk, dv, capacity):
    """Apply the first m_b captured records of each row to ``state``.

    [PR 32767, "Changes" and "DFlash2 Prerequisite"]: after partial acceptance
    the accepted prefix is replayed as S <- decay * S + outer(key, delta);
    m_b = min(max(replay_count[b], 0), capacity).  ``state`` [B, Hv, dk, dv].
    """
    S = _f64(state).copy()
    su = _f64(state_update)
    G = Hv // Hq
    counts = np.asarray(replay_count).reshape(-1)
    for b in range(S.shape[0]):
        m = min(max(int(counts[b]), 0), capacity)
        for c in range(m):
            rec = su[b, c]
            decay = rec[:Hv]
            key = rec[Hv:Hv + Hq * dk].reshape(Hq, dk)
            dlt = rec[Hv + Hq * dk:].reshape(Hv, dv)
            for h in range(Hv):
                S[b, h] = decay[h] * S[b, h] + np.outer(key[h // G], dlt[h])
    return S


def snapshot(src):
    """An immutable copy of a state set ([executorch issue 23099 / 23097],
    "Work to cover": prefix snapshot reused across question batches)."""
    return np.array(_f64(src), copy=True)
