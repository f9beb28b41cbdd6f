"""Seeded synthetic inputs for the Gated DeltaNet workloads (shared by tests and bench).

This module holds no arithmetic of the method itself: it only draws random
tensors with the distributions and shapes of the workloads and rounds them to
the input dtype on the host, so that the fp64 oracle and the device path see
exactly the same values.  Everything is returned as CPU torch tensors.

Workloads (names used across tests, smoke and bench):

* ``tiny_fp32``      fp32, 1 row x 64 tokens, Hq=Hv=1, dk=dv=16, chunk 16, zero state
* ``qwen_fp16``      fp16, 1 row x 2048 tokens, Hq=2, Hv=6, dk=dv=128, chunk 64,
                     initial state ~ N(0, 0.02^2)
* ``spec_decode``    bf16, 8 ragged rows of 1..7 tokens, Hq=16, Hv=32, dk=dv=128,
                     capture capacity 7, per-row capture counts in {0..7}
* ``long_varlen``    bf16, 4 packed sequences 8192/5000/1031/63, Hq=16, Hv=32,
                     dk=dv=128, chunk 64, per-sequence initial states
* ``prefix_reuse``   bf16, shared 4096-token prefix from zero state, then batches
                     of 16 continuations x 256 tokens branching from its snapshot

Distributions: q, k ~ N(0,1) then L2-normalised per (token, head) in fp64;
v ~ N(0,1); beta = sigmoid(N(0,1)); g = log(alpha) = -softplus(N(0,1));
scale = dk^-1/2; states ~ N(0, 0.02^2).  Draw order: (lengths), q, k, v, x_beta,
x_alpha, initial state, counts.  Seeds: 20261200 + workload index (+ batch index).
"""

from __future__ import annotations

import math

import numpy as np
import torch

WORKLOADS = {
    "tiny_fp32": dict(index=0, dtype="f32", lengths=[64], dense_rows=1, Hq=1, Hv=1, dk=16,
                      dv=16, chunk=16, state_std=0.0),
    "qwen_fp16": dict(index=1, dtype="f16", lengths=[2048], dense_rows=1, Hq=2, Hv=6, dk=128,
                      dv=128, chunk=64, state_std=0.02),
    "spec_decode": dict(index=2, dtype="bf16", lengths=None, rows=8, max_len=7, capacity=7,
                        Hq=16, Hv=32, dk=128, dv=128, chunk=64, state_std=0.02),
    "long_varlen": dict(index=3, dtype="bf16", lengths=[8192, 5000, 1031, 63], Hq=16, Hv=32,
                        dk=128, dv=128, chunk=64, state_std=0.02),
    "prefix_reuse": dict(index=4, dtype="bf16", prefix=4096, batch=16, cont=256, batches=64,
                         Hq=16, Hv=32, dk=128, dv=128, chunk=64, state_std=0.0),
}

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
BASE_SEED = 20261200


def _round(x64: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x64)).to(TORCH_DTYPES[dtype])


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def draw(rng: np.random.Generator, T: int, Hq: int, Hv: int, dk: int, dv: int, dtype: str,
         num_states: int, state_std: float, normalize_qk: bool = True):
    """q, k, v, g, beta, s0 for T packed tokens (CPU tensors, input-dtype rounded)."""
    q = rng.standard_normal((T, Hq, dk))
    k = rng.standard_normal((T, Hq, dk))
    v = rng.standard_normal((T, Hv, dv))
    xb = rng.standard_normal((T, Hv))
    xa = rng.standard_normal((T, Hv))
    if normalize_qk:
        q, k = _unit_rows(q), _unit_rows(k)
    beta = 1.0 / (1.0 + np.exp(-xb))
    g = -np.logaddexp(0.0, xa)                  # log(alpha) = -softplus(x)
    s0 = None
    if state_std > 0.0 and num_states > 0:
        s0 = torch.from_numpy(rng.standard_normal((num_states, Hv, dk, dv)) * state_std).float()
    return dict(q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype),
                g=torch.from_numpy(g).float(), beta=torch.from_numpy(beta).float(), s0=s0)


def make(name: str, batch_index: int = 0, part: str = "prefix", **overrides):
    """Inputs of one named workload (see module docstring).

    ``prefix_reuse`` has two parts: ``part="prefix"`` (seed base+4) and
    ``part="batch"`` with ``batch_index`` i (seed base+4+1+i).
    """
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    seed = BASE_SEED + spec["index"]
    if name == "prefix_reuse" and part != "prefix":
        seed += 1 + batch_index
    rng = np.random.default_rng(seed)
    Hq, Hv, dk, dv, dtype = spec["Hq"], spec["Hv"], spec["dk"], spec["dv"], spec["dtype"]
    out = dict(name=name, seed=seed, dtype=dtype, Hq=Hq, Hv=Hv, dk=dk, dv=dv,
               chunk=spec["chunk"], scale=1.0 / math.sqrt(dk))
    if name == "spec_decode":
        rows = spec["rows"]
        lengths = rng.integers(1, spec["max_len"] + 1, size=rows)
        lengths[1] = spec["max_len"]                 # one full-length row
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        T = int(cu[-1])
        out.update(draw(rng, T, Hq, Hv, dk, dv, dtype, rows, spec["state_std"]))
        cap = spec["capacity"]
        counts = rng.integers(0, cap + 1, size=rows)
        counts[0] = 0                                # zero capture
        counts[1] = cap                              # full capture of the full row
        counts[2] = max(1, int(lengths[2]) - 1) if lengths[2] > 1 else 1   # partial (or full of 1)
        counts[3] = cap + 3                          # over capacity: clamps
        out.update(cu_seqlens=torch.from_numpy(cu), lengths=lengths.tolist(), T=T,
                   capacity=cap, capture_count=torch.from_numpy(counts.astype(np.int32)),
                   num_seqs=rows)
        return out
    if name == "prefix_reuse":
        if part == "prefix":
            T = spec["prefix"]
            out.update(draw(rng, T, Hq, Hv, dk, dv, dtype, 0, 0.0))
            out.update(cu_seqlens=None, lengths=[T], T=T, num_seqs=1)
        else:
            B, L = spec["batch"], spec["cont"]
            T = B * L
            out.update(draw(rng, T, Hq, Hv, dk, dv, dtype, 0, 0.0))
            out.update(cu_seqlens=None, lengths=[L] * B, T=T, num_seqs=B)
        return out
    lengths = list(spec["lengths"])
    T = int(sum(lengths))
    n = len(lengths)
    out.update(draw(rng, T, Hq, Hv, dk, dv, dtype, n, spec["state_std"]))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dense = spec.get("dense_rows")
    out.update(cu_seqlens=None if dense else torch.from_numpy(cu), lengths=lengths, T=T,
               num_seqs=n)
    return out


def random_case(seed: int, lengths, Hq: int, Hv: int, dk: int, dv: int, dtype: str,
                state_std: float = 0.02, dense: bool = False):
    """A free-form case for edge tests: packed ``lengths`` (or dense equal rows)."""
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    out = dict(seed=seed, dtype=dtype, Hq=Hq, Hv=Hv, dk=dk, dv=dv, scale=1.0 / math.sqrt(dk))
    out.update(draw(rng, T, Hq, Hv, dk, dv, dtype, len(lengths), state_std))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    out.update(cu_seqlens=None if dense else torch.from_numpy(cu), lengths=list(lengths), T=T,
               num_seqs=len(lengths))
    return out


def raw_case(seed: int, lengths, Hq: int, Hv: int, dk: int, dv: int, dtype: str,
             state_std: float = 0.02, dense: bool = False):
    """Inputs in the form the input prologue consumes (raw projections):
    q, k ~ N(0,1) * U(0.5, 2) per (token, head), not normalised; v ~ N(0,1);
    ``g`` = gate pre-activation a ~ N(0,1) and ``beta`` = logit b ~ N(0,1), both
    fp32; A_log = log U(1, 16) and dt_bias ~ N(0, 0.5^2) per value head (fp32).
    Draw order: q, k, q/k row scales, v, b, a, A_log, dt_bias, initial state."""
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q = rng.standard_normal((T, Hq, dk))
    k = rng.standard_normal((T, Hq, dk))
    q = q * rng.uniform(0.5, 2.0, (T, Hq, 1))
    k = k * rng.uniform(0.5, 2.0, (T, Hq, 1))
    v = rng.standard_normal((T, Hv, dv))
    b = rng.standard_normal((T, Hv))
    a = rng.standard_normal((T, Hv))
    A_log = np.log(rng.uniform(1.0, 16.0, Hv))
    dt_bias = rng.standard_normal(Hv) * 0.5
    s0 = None
    if state_std > 0.0:
        s0 = torch.from_numpy(rng.standard_normal((len(lengths), Hv, dk, dv)) * state_std).float()
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return dict(seed=seed, dtype=dtype, Hq=Hq, Hv=Hv, dk=dk, dv=dv, scale=1.0 / math.sqrt(dk),
                q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype),
                g=torch.from_numpy(a).float(), beta=torch.from_numpy(b).float(),
                A_log=torch.from_numpy(A_log).float(), dt_bias=torch.from_numpy(dt_bias).float(), s0=s0,
                cu_seqlens=None if dense else torch.from_numpy(cu), lengths=list(lengths), T=T,
                num_seqs=len(lengths))


def random_counts(seed: int, rows: int, capacity: int):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.integers(-2, capacity + 3, size=rows).astype(np.int32))
