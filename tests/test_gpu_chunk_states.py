"""Chunk-boundary states from the chunked prefill, against the fp64 oracle.

Each emitted entry is the state after a prefix that ends on a chunk boundary
(or at the sequence end), i.e. a snapshot that a later call can continue from
([executorch issue 23097, "Work to cover"]: GDN chunk boundaries, prefix
snapshots retained in device memory).  Emission must not change o or the final
state, and each sequence's last entry must equal its final state bit for bit.
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_common import assert_close, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_03_amd as m
    m.load_library()
    return m


def n_chunks(lengths, C):
    return [-(-L // C) for L in lengths]


def run_both(gdn, case, C, **kw):
    d = to_dev(case)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    common = dict(scale=case["scale"], cu_seqlens=d["cu_seqlens"], chunk_size=C, initial_state=d["s0"])
    o, fin, cs = gdn.gdn_prefill_chunked_states(*args, **common, **kw)
    o2, fin2 = gdn.gdn_prefill_chunked(*args, **common)
    torch.cuda.synchronize()
    return o, fin, cs, o2, fin2


@pytest.mark.parametrize("dtype,C,dk,dv", [("bf16", 64, 128, 128), ("f16", 32, 64, 128),
                                           ("f32", 16, 64, 32), ("bf16", 16, 32, 16)])
def test_boundary_states_match_oracle(gdn, dtype, C, dk, dv):
    lengths = [130, 0, 64, 1, 2 * C + 5]           # partial, empty, exact multiple, single token
    Hq, Hv = 2, 4
    case = gi.random_case(8800 + C + dk, lengths, Hq=Hq, Hv=Hv, dk=dk, dv=dv, dtype=dtype)
    say(f"case chunk states {dtype} C={C} dk={dk} dv={dv} lengths={lengths}")
    o, fin, cs, o2, fin2 = run_both(gdn, case, C)
    counts = n_chunks(lengths, C)
    assert cs.shape == (sum(counts), Hv, dk, dv)
    # emission does not change the prefill's results
    assert torch.equal(o, o2) and torch.equal(fin, fin2)
    ref = oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"], Hq, Hv,
                           cu_seqlens=case["cu_seqlens"], initial_state=case["s0"], boundary_every=C)
    assert_close(cs, ref["boundary"], dtype, "chunk states")
    last = np.cumsum(counts) - 1
    for s, L in enumerate(lengths):
        if L:
            assert torch.equal(cs[last[s]], fin[s]), f"sequence {s}: last chunk state != final state"


def test_capacity_limits_and_snapshot_continuation(gdn):
    """Entries at or past the capacity are never written; an emitted state used
    as the initial state of the rest of the sequence reproduces the whole
    sequence's final state and outputs."""
    lengths = [200, 77]
    C, Hq, Hv, dk, dv = 64, 2, 4, 128, 128
    case = gi.random_case(8900, lengths, Hq=Hq, Hv=Hv, dk=dk, dv=dv, dtype="bf16")
    say(f"case chunk states capacity lengths={lengths}")
    d = to_dev(case)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    total = sum(n_chunks(lengths, C))                 # 4 + 2
    cap = 3
    buf = torch.full((total, Hv, dk, dv), 7.0, device=d["s0"].device)
    o, fin, _ = gdn.gdn_prefill_chunked_states(*args, scale=case["scale"], cu_seqlens=d["cu_seqlens"],
                                               chunk_size=C, initial_state=d["s0"], chunk_states=buf[:cap])
    torch.cuda.synchronize()
    assert (buf[cap:] == 7.0).all(), "entries past the capacity were written"
    assert not (buf[:cap] == 7.0).any()
    # continue sequence 0 from the state after 128 tokens (entry 1)
    m = 2 * C
    rest = [d[x][m:lengths[0]].contiguous()[None] for x in ("q", "k", "v", "g", "beta")]
    o_rest, fin_rest = gdn.gdn_prefill_chunked(*rest, scale=case["scale"], chunk_size=C,
                                               initial_state=buf[1:2].contiguous())
    torch.cuda.synchronize()
    assert_close(fin_rest, fin[:1], "bf16", "continued final vs whole")
    assert_close(o_rest[0], o[m:lengths[0]], "bf16", "continued o vs whole", bounds=[(0, lengths[0] - m)], chunk=C)


def test_long_varlen_boundary_states_sampled(gdn):
    """The 14286-token packed workload (lengths 8192, 5000, 1031, 63): every
    chunk state of sampled value heads against the oracle's boundary states."""
    case = gi.make("long_varlen")
    C = case["chunk"]
    say(f"case long_varlen chunk states lengths={case['lengths']} seed={case['seed']}")
    o, fin, cs, o2, fin2 = run_both(gdn, case, C)
    assert torch.equal(o, o2) and torch.equal(fin, fin2)
    heads = [0, 31]
    ref = oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"],
                           case["Hq"], case["Hv"], cu_seqlens=case["cu_seqlens"], initial_state=case["s0"],
                           heads=heads, boundary_every=C)
    assert cs.shape[0] == ref["boundary"].shape[0] == sum(n_chunks(case["lengths"], C))
    assert_close(cs, ref["boundary"], "bf16", "chunk states", heads=heads)
    assert torch.isfinite(cs).all()
