"""Shared helpers for the GPU parity tests (comparison metrics, device moves)."""

import hashlib

import numpy as np
import torch

DEV = "cuda"

# Tolerances: fp32 inputs max-abs 1e-4; fp16/bf16 inputs relative L2 2e-2 per
# tensor (computed in fp64); capture decay records relative error 4e-7.
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


def assert_close(x, ref, dtype, what=""):
    """The bar for floating point outputs, by input dtype."""
    if dtype == "f32":
        err = max_abs(x, ref)
        say(f"  {what}: max-abs {err:.3e} (bar {TOL_F32_MAXABS})")
        assert err <= TOL_F32_MAXABS, f"{what}: max-abs {err:.3e} > {TOL_F32_MAXABS}"
    else:
        err = rel_l2(x, ref)
        say(f"  {what}: rel-L2 {err:.3e} (bar {TOL_16_RELL2})")
        assert err <= TOL_16_RELL2, f"{what}: rel-L2 {err:.3e} > {TOL_16_RELL2}"
    return err


def sha(t):
    return hashlib.sha256(t.detach().contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()


def say(msg):
    print(msg, flush=True)
