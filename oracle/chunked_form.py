"""The chunked (UT / WY) form of the gated delta rule in fp64 (test infrastructure only).

Only tests may use this module.  It is an independent second algorithm for the
same result as ``gdn_oracle.recurrent`` and serves purely as a cross-check of it:
the recurrence unrolled over a chunk of C tokens with chunk-start state S0
gives, with gamma_i = exp(sum_{j<=i} g_j) over the chunk,

    (I + diag(beta) L) Delta = diag(beta) (V - diag(gamma) K S0),
        L_ij = (gamma_i / gamma_j) k_i . k_j   for j < i, else 0
    O      = scale * (diag(gamma) Q S0 + (Mc * (Q K^T)) Delta),
        Mc_ij = gamma_i / gamma_j for j <= i, else 0
    S_end  = gamma_C S0 + (diag(gamma_C / gamma) K)^T Delta

[executorch issue 23097, "Work to cover": the chunked prefill carries an
explicit state between chunks; chunk boundaries must not change results.]
Steps follow that order; the triangular solve is a library primitive.
"""

from __future__ import annotations

import numpy as np

from .gdn_oracle import _f64, sequence_bounds


def chunked(q, k, v, g, beta, scale, Hq, Hv, chunk, cu_seqlens=None, num_seqs=None,
            initial_state=None):
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    Ttot, _, dk = k.shape
    dv = v.shape[2]
    G = Hv // Hq
    if cu_seqlens is None:
        N = 1 if num_seqs is None else int(num_seqs)
        bounds = sequence_bounds(N, Ttot // N)
    else:
        bounds = sequence_bounds(0, 0, cu_seqlens)
        N = len(bounds)
    s0 = _f64(initial_state)
    o = np.zeros((Ttot, Hv, dv))
    final = np.zeros((N, Hv, dk, dv))
    boundary = []                     # state after each chunk, in sequence order
    for s, (t0, t1) in enumerate(bounds):
        sb = np.zeros((-(-(t1 - t0) // chunk), Hv, dk, dv))
        for h in range(Hv):
            hk = h // G
            S = np.zeros((dk, dv)) if s0 is None else s0[s, h].copy()
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                K, Q, V = k[c0:c1, hk], q[c0:c1, hk], v[c0:c1, h]
                b = beta[c0:c1, h]
                Gc = np.cumsum(g[c0:c1, h])
                ratio = np.exp(Gc[:, None] - Gc[None, :])          # gamma_i / gamma_j
                n = c1 - c0
                L = np.tril(ratio * (K @ K.T), -1)
                rhs = b[:, None] * (V - np.exp(Gc)[:, None] * (K @ S))
                Delta = np.linalg.solve(np.eye(n) + b[:, None] * L, rhs)
                Mc = np.tril(ratio)
                o[c0:c1, h] = scale * (np.exp(Gc)[:, None] * (Q @ S) + (Mc * (Q @ K.T)) @ Delta)
                Kt = np.exp(Gc[-1] - Gc)[:, None] * K
                S = np.exp(Gc[-1]) * S + Kt.T @ Delta
                sb[(c0 - t0) // chunk, h] = S
            final[s, h] = S
        boundary.append(sb)
    return {"o": o, "final": final,
            "boundary": np.concatenate(boundary) if boundary else np.zeros((0, Hv, dk, dv))}
