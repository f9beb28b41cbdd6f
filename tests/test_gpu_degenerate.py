"""Degenerate cases of the gated delta rule on the GPU, against their closed forms.

* beta = 0, g = 0: nothing is written and nothing decays, so both paths return the
  initial state bit for bit, and o_t = scale * S0^T q_t.
* beta = 0: S_T = exp(sum_t g_t) * S0.
* one token from a zero state: S = beta k v^T and o = scale * beta (q . k) v.
* near-total decay (g = -30 per token): every result stays finite and the state
  is only what the last tokens wrote.
* zero keys: delta = beta v, S = alpha S (keys write nothing), o from the decayed state.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_common import assert_close, case_bounds, f64, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_03_amd as m
    m.load_library()
    return m


def both_paths(gdn, d, scale, C=64):
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    kw = dict(scale=scale, cu_seqlens=d["cu_seqlens"], initial_state=d["s0"])
    o1, f1 = gdn.gdn_prefill_chunked(*args, chunk_size=C, **kw)
    o2, f2, _ = gdn.gdn_recurrent_step(*args, **kw)
    torch.cuda.synchronize()
    return (o1, f1), (o2, f2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_beta_no_decay_keeps_the_state_exactly(gdn, dtype):
    dk = 128 if dtype == "bf16" else 64
    lengths = [70, 5]
    case = gi.random_case(9800, lengths, Hq=2, Hv=4, dk=dk, dv=64, dtype=dtype, state_std=0.5)
    case["beta"] = torch.zeros_like(case["beta"])
    case["g"] = torch.zeros_like(case["g"])
    say(f"case beta=0 g=0 {dtype}")
    d = to_dev(case)
    (o1, f1), (o2, f2) = both_paths(gdn, d, case["scale"])
    assert torch.equal(f1, d["s0"]) and torch.equal(f2, d["s0"])
    # o_t = scale S0^T q_t
    cu = case["cu_seqlens"].tolist()
    q = f64(case["q"])
    S0 = f64(case["s0"])
    ref = np.zeros((sum(lengths), 4, 64))
    for s in range(len(lengths)):
        for t in range(cu[s], cu[s + 1]):
            for h in range(4):
                ref[t, h] = case["scale"] * S0[s, h].T @ q[t, h // 2]
    assert_close(o1, ref, dtype, "prefill o", bounds=case_bounds(case), chunk=64)
    assert_close(o2, ref, dtype, "recurrent o", bounds=case_bounds(case))


def test_zero_beta_is_pure_decay(gdn):
    lengths = [200, 1, 64]
    case = gi.random_case(9801, lengths, Hq=1, Hv=2, dk=64, dv=32, dtype="f32", state_std=0.5)
    case["beta"] = torch.zeros_like(case["beta"])
    say("case beta=0 pure decay")
    d = to_dev(case)
    (_, f1), (_, f2) = both_paths(gdn, d, case["scale"], C=32)
    cu = case["cu_seqlens"].tolist()
    g = f64(case["g"])
    decay = np.stack([np.exp(g[cu[s]:cu[s + 1]].sum(axis=0)) for s in range(len(lengths))])   # [N, Hv]
    ref = decay[:, :, None, None] * f64(case["s0"])
    for f, what in ((f1, "prefill"), (f2, "recurrent")):
        np.testing.assert_allclose(f64(f), ref, rtol=2e-5, atol=1e-30, err_msg=what)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_token_from_zero_state(gdn, dtype):
    dk = 128 if dtype == "bf16" else 32
    case = gi.random_case(9802, [1] * 6, Hq=2, Hv=4, dk=dk, dv=32, dtype=dtype, state_std=0.0)
    say(f"case single token zero state {dtype}")
    d = to_dev(case)
    (o1, f1), (o2, f2) = both_paths(gdn, d, case["scale"])
    q, k, v = f64(case["q"]), f64(case["k"]), f64(case["v"])
    beta = f64(case["beta"])
    S = np.zeros((6, 4, dk, 32))
    o = np.zeros((6, 4, 32))
    for t in range(6):
        for h in range(4):
            S[t, h] = beta[t, h] * np.outer(k[t, h // 2], v[t, h])
            o[t, h] = case["scale"] * beta[t, h] * (q[t, h // 2] @ k[t, h // 2]) * v[t, h]
    for (oo, ff), what in (((o1, f1), "prefill"), ((o2, f2), "recurrent")):
        assert_close(oo, o, dtype, f"{what} o", bounds=case_bounds(case))
        assert_close(ff, S, dtype, f"{what} S")


def test_near_total_decay_stays_finite(gdn):
    lengths = [130, 7]
    case = gi.random_case(9803, lengths, Hq=2, Hv=4, dk=128, dv=128, dtype="bf16", state_std=0.5)
    case["g"] = torch.full_like(case["g"], -30.0)
    say("case g=-30 per token")
    d = to_dev(case)
    (o1, f1), (o2, f2) = both_paths(gdn, d, case["scale"])
    for x in (o1, f1, o2, f2):
        assert torch.isfinite(x).all()
    ref = oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"], 2, 4,
                           cu_seqlens=case["cu_seqlens"], initial_state=case["s0"])
    assert_close(o1, ref["o"], "bf16", "prefill o", bounds=case_bounds(case), chunk=64)
    assert_close(f1, ref["final"], "bf16", "prefill final")
    assert_close(o2, ref["o"], "bf16", "recurrent o", bounds=case_bounds(case))


def test_zero_keys_only_decay(gdn):
    lengths = [90, 3]
    case = gi.random_case(9804, lengths, Hq=1, Hv=2, dk=64, dv=64, dtype="f32", state_std=0.5)
    case["k"] = torch.zeros_like(case["k"])
    say("case zero keys")
    d = to_dev(case)
    (o1, f1), (o2, f2) = both_paths(gdn, d, case["scale"], C=16)
    ref = oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"], 1, 2,
                           cu_seqlens=case["cu_seqlens"], initial_state=case["s0"])
    for (oo, ff), what in (((o1, f1), "prefill"), ((o2, f2), "recurrent")):
        assert_close(oo, ref["o"], "f32", f"{what} o")
        assert_close(ff, ref["final"], "f32", f"{what} final")
