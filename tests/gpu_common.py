"""Shared helpers for the GPU parity tests (comparison metrics, device moves)."""

import hashlib

import numpy as np
import torch

DEV = "cuda"

# Tolerances: fp32 inputs max-abs 1e-4; fp16/bf16 inputs relative L2 2e-2
# (computed in fp64) per (sequence, value head) and per partial last chunk;
# capture decay records relative error 4e-7.
TOL_F32_MAXABS = 1e-4
TOL_16_RELL2 = 2e-2
TOL_DECAY_REL = 4e-7


def to_dev(case):
    out = dict(case)
    for key in ("q", "k", "v", "g", "beta", "s0", "cu_seqlens", "capture_count"):
        if out.get(key) is not None:
            out[key] = out[key].to(DEV)
    return out


def f64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_l2(x, ref):
    x, ref = f64(x), f64(ref)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def max_abs(x, ref):
    return float(np.max(np.abs(f64(x) - f64(ref)))) if f64(ref).size else 0.0


def case_bounds(case):
    """(start, end) token ranges of a case's sequences (packed or dense rows)."""
    if case.get("cu_seqlens") is not None:
        cu = [int(x) for x in case["cu_seqlens"].cpu().tolist()]
        return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    n = case["num_seqs"]
    T = case["q"].shape[0] // n
    return [(b * T, (b + 1) * T) for b in range(n)]


def _check_rel(x, ref, what):
    err = rel_l2(x, ref)
    assert err <= TOL_16_RELL2, f"{what}: rel-L2 {err:.3e} > {TOL_16_RELL2}"
    return err


def assert_close(x, ref, dtype, what="", bounds=None, chunk=None, heads=None):
    """The bar for floating point outputs, by input dtype.

    fp32 inputs: max-abs over every element.  fp16/bf16 inputs: relative L2,
    checked locally so that an error confined to one short sequence or one
    partial chunk cannot hide in the norm of a whole tensor:
      * states [N, Hv, dk, dv]: per (sequence, value head);
      * token outputs [tokens, Hv, dv] with ``bounds`` (the sequences' token
        ranges): per (sequence, value head), and with ``chunk`` also on each
        sequence's partial last chunk, per value head;
      * anything else: the whole tensor.
    ``heads`` restricts the local checks to sampled value heads."""
    if dtype == "f32":
        err = max_abs(x, ref)
        say(f"  {what}: max-abs {err:.3e} (bar {TOL_F32_MAXABS})")
        assert err <= TOL_F32_MAXABS, f"{what}: max-abs {err:.3e} > {TOL_F32_MAXABS}"
        return err
    xa, ra = f64(x), f64(ref)
    assert xa.shape == ra.shape, f"{what}: shape {xa.shape} vs {ra.shape}"
    worst, n = 0.0, 0
    if xa.ndim == 4:
        hs = range(xa.shape[1]) if heads is None else heads
        for i in range(xa.shape[0]):
            for h in hs:
                worst = max(worst, _check_rel(xa[i, h], ra[i, h], f"{what} [{i}, head {h}]"))
                n += 1
    elif xa.ndim == 3 and bounds is not None:
        hs = range(xa.shape[1]) if heads is None else heads
        for s, (t0, t1) in enumerate(bounds):
            if t1 <= t0:
                continue
            tail = t0 + ((t1 - t0) // chunk) * chunk if chunk else t1
            for h in hs:
                worst = max(worst, _check_rel(xa[t0:t1, h], ra[t0:t1, h], f"{what} seq {s} head {h}"))
                n += 1
                if tail < t1 and tail > t0:
                    worst = max(worst, _check_rel(xa[tail:t1, h], ra[tail:t1, h],
                                                  f"{what} seq {s} head {h} partial last chunk [{tail}, {t1})"))
                    n += 1
    else:
        worst = _check_rel(xa, ra, what)
        n = 1
    say(f"  {what}: worst rel-L2 {worst:.3e} over {n} local checks (bar {TOL_16_RELL2})")
    return worst


def sha(t):
    return hashlib.sha256(t.detach().contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()


def say(msg):
    print(msg, flush=True)
