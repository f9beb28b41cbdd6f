"""The input prologue (q/k l2norm, beta from logits, softplus gate) fused into
the prefill and recurrent kernels, against the fp64 oracle applied to the same
raw inputs ([executorch issue 23097, "Work to cover"]: gate and scaling
conventions adapted inside the GDN kernels).
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_common import DEV, assert_close, case_bounds, f64, max_abs, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_03_amd as m
    m.load_library()
    return m


def make_prologue(gdn, case, l2norm=True, logits=True, gate=True, eps=1e-6):
    return gdn.Prologue(qk_l2norm=l2norm, eps=eps, beta_is_logit=logits,
                        A_log=case["A_log"].to(DEV) if gate else None,
                        dt_bias=case["dt_bias"].to(DEV) if gate else None)


def oracle_with(case, l2norm=True, logits=True, gate=True, eps=1e-6, boundary_every=None):
    q, k, g, beta = oracle.prologue(case["q"], case["k"], case["g"], case["beta"], qk_l2norm=l2norm, eps=eps,
                                    beta_is_logit=logits, A_log=case["A_log"] if gate else None,
                                    dt_bias=case["dt_bias"] if gate else None)
    ref = oracle.recurrent(q, k, case["v"], g, beta, case["scale"], case["Hq"], case["Hv"],
                           cu_seqlens=case["cu_seqlens"], initial_state=case["s0"], boundary_every=boundary_every)
    return ref, (q, k, g, beta)


def mixed_case(seed, lengths, Hq, Hv, dk, dv, dtype, l2norm, gate):
    """Raw inputs where a switch is on, ready-made ones where it is off."""
    raw = gi.raw_case(seed, lengths, Hq=Hq, Hv=Hv, dk=dk, dv=dv, dtype=dtype)
    base = gi.random_case(seed + 1, lengths, Hq=Hq, Hv=Hv, dk=dk, dv=dv, dtype=dtype)
    case = dict(raw)
    if not l2norm:
        case["q"], case["k"] = base["q"], base["k"]
    if not gate:
        case["g"], case["beta"] = base["g"], base["beta"]
    return case


@pytest.mark.parametrize("dtype,C,dk,dv", [("bf16", 64, 128, 128), ("f16", 32, 64, 64), ("f32", 16, 64, 32)])
def test_prefill_prologue_matches_oracle(gdn, dtype, C, dk, dv):
    lengths = [150, 1, 64, 33]
    case = gi.raw_case(9100 + C, lengths, Hq=2, Hv=4, dk=dk, dv=dv, dtype=dtype)
    say(f"case prefill prologue {dtype} C={C} dk={dk} dv={dv} lengths={lengths}")
    d = to_dev(case)
    o, fin, cs = gdn.gdn_prefill_chunked_ex(*[d[x] for x in ("q", "k", "v", "g", "beta")],
                                            prologue=make_prologue(gdn, case), scale=case["scale"],
                                            cu_seqlens=d["cu_seqlens"], chunk_size=C, initial_state=d["s0"],
                                            emit_chunk_states=True)
    torch.cuda.synchronize()
    ref, _ = oracle_with(case, boundary_every=C)
    assert_close(o, ref["o"], dtype, "o", bounds=case_bounds(case), chunk=C)
    assert_close(fin, ref["final"], dtype, "final")
    assert_close(cs, ref["boundary"], dtype, "chunk states")


@pytest.mark.parametrize("l2norm,gate", [(True, False), (False, True)])
def test_prefill_prologue_parts(gdn, l2norm, gate):
    lengths = [100, 28]
    case = mixed_case(9200 + 2 * l2norm + gate, lengths, 2, 4, 128, 128, "bf16", l2norm, gate)
    say(f"case prefill prologue part l2norm={l2norm} gate={gate}")
    d = to_dev(case)
    o, fin, _ = gdn.gdn_prefill_chunked_ex(*[d[x] for x in ("q", "k", "v", "g", "beta")],
                                           prologue=make_prologue(gdn, case, l2norm=l2norm, logits=gate, gate=gate),
                                           scale=case["scale"], cu_seqlens=d["cu_seqlens"], chunk_size=64,
                                           initial_state=d["s0"])
    torch.cuda.synchronize()
    ref, _ = oracle_with(case, l2norm=l2norm, logits=gate, gate=gate)
    assert_close(o, ref["o"], "bf16", "o", bounds=case_bounds(case), chunk=64)
    assert_close(fin, ref["final"], "bf16", "final")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 32)])
def test_decode_prologue_with_capture_matches_oracle(gdn, dtype, dk, dv):
    lengths = [1, 7, 3, 5]
    counts = [1, 7, 2, 9]
    cap = 7
    Hq, Hv = 2, 4
    case = gi.raw_case(9300 + dk, lengths, Hq=Hq, Hv=Hv, dk=dk, dv=dv, dtype=dtype)
    say(f"case decode prologue {dtype} lengths={lengths} counts={counts}")
    d = to_dev(case)
    cnt = torch.tensor(counts, dtype=torch.int32, device=DEV)
    o, fin, su = gdn.gdn_recurrent_step_ex(*[d[x] for x in ("q", "k", "v", "g", "beta")],
                                           prologue=make_prologue(gdn, case), scale=case["scale"],
                                           cu_seqlens=d["cu_seqlens"], initial_state=d["s0"],
                                           state_update_capacity=cap, capture_count=cnt, state_update_active=1)
    torch.cuda.synchronize()
    ref, (q, k, g, beta) = oracle_with(case)
    assert_close(o, ref["o"], dtype, "o", bounds=case_bounds(case))
    assert_close(fin, ref["final"], dtype, "final")
    buf, mask = oracle.capture(k, ref["alpha"], ref["delta"], Hq, Hv, cap, counts, 1, cu_seqlens=case["cu_seqlens"])
    su = f64(su)
    # decay: the gate in fp32 has a relative error of a few ulp in g, so exp(g)
    # carries an absolute error of about that times |g| in its logarithm
    dec = mask[:, :, :Hv]
    lg_dev, lg_ref = np.log(su[:, :, :Hv][dec]), np.log(buf[:, :, :Hv][dec])
    err = np.max(np.abs(lg_dev - lg_ref) / (1.0 + np.abs(lg_ref)))
    say(f"  decay: max |log a - g| / (1 + |g|) {err:.3e} (bar 2e-6)")
    assert err <= 2e-6
    key = mask[:, :, Hv:Hv + Hq * dk]
    kerr = float(np.max(np.abs(su[:, :, Hv:Hv + Hq * dk][key] - buf[:, :, Hv:Hv + Hq * dk][key])))
    say(f"  unit keys: max-abs {kerr:.3e} (bar 1e-6)")
    assert kerr <= 1e-6
    # deltas of every captured record, per (record, value head)
    rec = mask[:, :, 0]
    dev_d = su[:, :, Hv + Hq * dk:][rec].reshape(-1, Hv, dv, 1)
    ref_d = buf[:, :, Hv + Hq * dk:][rec].reshape(-1, Hv, dv, 1)
    assert_close(dev_d, ref_d, dtype, "deltas")


def test_identity_prologue_is_the_plain_path(gdn):
    """A zeroed prologue gives bit-identical results to the plain entry points."""
    lengths = [70, 5]
    case = gi.random_case(9400, lengths, Hq=2, Hv=4, dk=128, dv=128, dtype="bf16")
    say("case identity prologue")
    d = to_dev(case)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    kw = dict(scale=case["scale"], cu_seqlens=d["cu_seqlens"], initial_state=d["s0"])
    o1, f1 = gdn.gdn_prefill_chunked(*args, chunk_size=64, **kw)
    o2, f2, _ = gdn.gdn_prefill_chunked_ex(*args, prologue=gdn.Prologue(), chunk_size=64, **kw)
    o3, f3, _ = gdn.gdn_recurrent_step(*args, **kw)
    o4, f4, _ = gdn.gdn_recurrent_step_ex(*args, prologue=gdn.Prologue(), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    assert torch.equal(o3, o4) and torch.equal(f3, f4)


def test_prefill_and_decode_agree_under_prologue(gdn):
    """The two fused prologues (prep kernel vs recurrent kernel) agree in fp32."""
    lengths = [48, 17]
    case = gi.raw_case(9500, lengths, Hq=1, Hv=2, dk=64, dv=32, dtype="f32")
    say("case prefill vs decode prologue f32")
    d = to_dev(case)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    kw = dict(scale=case["scale"], cu_seqlens=d["cu_seqlens"], initial_state=d["s0"])
    pro = make_prologue(gdn, case)
    o1, f1, _ = gdn.gdn_prefill_chunked_ex(*args, prologue=pro, chunk_size=16, **kw)
    o2, f2, _ = gdn.gdn_recurrent_step_ex(*args, prologue=pro, **kw)
    torch.cuda.synchronize()
    err = max(max_abs(o1, o2), max_abs(f1, f2))
    say(f"  chunked vs recurrent: max-abs {err:.3e} (bar 1e-4)")
    assert err <= 1e-4
