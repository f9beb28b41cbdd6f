"""The 16-bit parity bar is applied locally (CPU only): an error confined to one
short sequence or to one sequence's partial last chunk must fail it, even when
it is small against the norm of the whole tensor."""

import numpy as np
import pytest

from gpu_common import assert_close


def _fake(lengths, Hv=4, dv=128, seed=0):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    ref = rng.standard_normal((T, Hv, dv))
    bounds, t = [], 0
    for L in lengths:
        bounds.append((t, t + L))
        t += L
    return ref, bounds


def test_error_on_one_short_sequence_fails():
    ref, bounds = _fake([1, 15, 16, 17, 63, 64, 65, 130, 5000])
    x = ref * (1 + 1e-3)
    t0, t1 = bounds[0]
    x[t0:t1, 2] *= 1.31                      # 31% on the 1-token sequence, one head
    assert np.linalg.norm(x - ref) / np.linalg.norm(ref) < 2e-2   # hidden in the whole-tensor norm
    with pytest.raises(AssertionError, match="seq 0 head 2"):
        assert_close(x, ref, "bf16", "o", bounds=bounds, chunk=64)


def test_error_on_a_partial_last_chunk_fails():
    ref, bounds = _fake([5000, 63])
    x = ref.copy()
    t0, t1 = bounds[0]
    tail = t0 + (5000 // 64) * 64            # the 8-token tail chunk
    x[tail:t1, 1] *= 1.4                     # 40% there, under 2% of the sequence's error norm
    assert np.linalg.norm(x[t0:t1, 1] - ref[t0:t1, 1]) / np.linalg.norm(ref[t0:t1, 1]) < 2e-2
    with pytest.raises(AssertionError, match="partial last chunk"):
        assert_close(x, ref, "bf16", "o", bounds=bounds, chunk=64)


def test_state_error_in_one_head_fails():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((4, 32, 16, 16))
    x = ref.copy()
    x[3, 17] *= 1.1
    with pytest.raises(AssertionError, match=r"\[3, head 17\]"):
        assert_close(x, ref, "f16", "final")


def test_within_tolerance_passes():
    ref, bounds = _fake([1, 15, 65, 200])
    x = ref * (1 + 5e-3)
    assert assert_close(x, ref, "bf16", "o", bounds=bounds, chunk=32) < 2e-2
