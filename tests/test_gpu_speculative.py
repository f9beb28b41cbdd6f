"""Layer-level speculative decoding on the four entry points.

Draft T tokens per row with one recurrent step that captures every token's
(decay, key, delta) record, accept a prefix of m_b tokens per row (none, some,
all), and rebuild the accepted state by replaying the first m_b records onto the
pre-draft state.  The result must equal the non-speculative path -- m_b
single-token steps from the same state -- bit for bit, for the outputs of the
accepted tokens and for the state, and must match the fp64 oracle run over the
accepted tokens only.  Decoding then continues from the replayed state exactly
as it continues from the non-speculative one.

The flow follows [onnxruntime PR 32767, "[WebGPU EP] adds state update capacity
support for GatedDeltaNet", "Changes"]: compact capture during the draft,
ReplayStateUpdates after partial acceptance, no fallback path.
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


def step(gdn, d, sl, state, scale, **kw):
    """One recurrent call over tokens sl (a slice of the dense [B, T] token axis)."""
    args = [d[x][:, sl].contiguous() for x in ("q", "k", "v", "g", "beta")]
    return gdn.gdn_recurrent_step(*args, scale=scale, initial_state=state, **kw)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_draft_accept_replay_equals_non_speculative(gdn, dtype):
    B, T, Hq, Hv = 6, 7, 2, 4
    dk, dv = (128, 128) if dtype == "bf16" else (64, 32)
    accept = [0, 3, 7, 1, 6, 7]                 # none, partial and full acceptance
    case = gi.random_case(4242 + dk, [T + 1] * B, Hq=Hq, Hv=Hv, dk=dk, dv=dv, dtype=dtype, dense=True)
    say(f"case speculative {dtype} B={B} T={T} accept={accept}")
    c = to_dev(case)
    d = {x: c[x].reshape(B, T + 1, *c[x].shape[1:]) for x in ("q", "k", "v", "g", "beta")}
    scale, s0 = case["scale"], c["s0"]
    draft = slice(0, T)

    # speculative: one T-token step with every token captured
    counts = torch.full((B,), T, dtype=torch.int32, device=s0.device)
    o_spec, _, su = step(gdn, d, draft, s0, scale, state_update_capacity=T, capture_count=counts,
                         state_update_active=1)
    state = s0.clone()
    gdn.gdn_replay_state_updates(state, su, torch.tensor(accept, dtype=torch.int32, device=s0.device), Hq=Hq)

    # non-speculative: single-token steps, keeping every intermediate state
    states = [s0.clone()]
    outs = []
    for t in range(T):
        o_t, st, _ = step(gdn, d, slice(t, t + 1), states[-1], scale)
        outs.append(o_t)
        states.append(st)
    torch.cuda.synchronize()

    for b, m in enumerate(accept):
        assert torch.equal(state[b], states[m][b]), f"row {b}: replayed state != {m} single-token steps"
        for t in range(m):
            assert torch.equal(o_spec[b, t], outs[t][b, 0]), f"row {b}: output of accepted token {t}"

    # the accepted state against the fp64 oracle over exactly the accepted tokens
    for b, m in enumerate(accept):
        if m == 0:
            assert torch.equal(state[b].cpu(), case["s0"][b])
            continue
        rows = slice(b * (T + 1), b * (T + 1) + m)
        sub = {x: case[x][rows] for x in ("q", "k", "v", "g", "beta")}
        ref = oracle.recurrent(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale, Hq, Hv,
                               initial_state=case["s0"][b:b + 1])
        assert_close(state[b:b + 1], ref["final"], dtype, f"row {b} accepted state")
        assert_close(o_spec[b, :m], ref["o"], dtype, f"row {b} accepted outputs", bounds=[(0, m)])

    # decoding continues from the replayed state exactly as from the reference one
    nxt = slice(T, T + 1)
    ref_states = torch.stack([states[m][b] for b, m in enumerate(accept)])
    o_a, s_a, _ = step(gdn, d, nxt, state, scale)
    o_b, s_b, _ = step(gdn, d, nxt, ref_states, scale)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(s_a, s_b)


# Record layouts: R = Hv + Hq dk + Hv dv a multiple of 4 with Hv too (16-byte
# record fields), or not (4-byte fields); 32- and 16-column replay slices.
@pytest.mark.parametrize("Hq,Hv,dk,dv", [(2, 4, 128, 64), (1, 3, 64, 32), (2, 6, 32, 32),
                                         (2, 4, 64, 16), (1, 1, 16, 16)])
def test_ragged_draft_with_capture_limits(gdn, Hq, Hv, dk, dv):
    """Ragged drafts packed by cu_seqlens, capture counts below, at and above the
    row length and the capacity: replaying what was captured reproduces the
    non-speculative state after that many tokens."""
    lengths = [5, 1, 7, 3, 6]
    counts = [2, 1, 9, 0, 6]          # clamped to min(count, capacity, length)
    cap = 6
    case = gi.random_case(5150 + dk + dv + Hv, lengths, Hq=Hq, Hv=Hv, dk=dk, dv=dv, dtype="bf16")
    say(f"case ragged speculative Hq={Hq} Hv={Hv} dk={dk} dv={dv} lengths={lengths} counts={counts} cap={cap}")
    c = to_dev(case)
    args = [c[x] for x in ("q", "k", "v", "g", "beta")]
    cnt = torch.tensor(counts, dtype=torch.int32, device=c["s0"].device)
    o, _, su = gdn.gdn_recurrent_step(*args, scale=case["scale"], initial_state=c["s0"],
                                      cu_seqlens=c["cu_seqlens"], state_update_capacity=cap,
                                      capture_count=cnt, state_update_active=1)
    n = [min(max(x, 0), cap, L) for x, L in zip(counts, lengths)]
    state = c["s0"].clone()
    gdn.gdn_replay_state_updates(state, su, torch.tensor(n, dtype=torch.int32, device=state.device), Hq=Hq)
    torch.cuda.synchronize()
    cu = case["cu_seqlens"].tolist()
    for b, m in enumerate(n):
        if m == 0:
            assert torch.equal(state[b].cpu(), case["s0"][b])
            continue
        rows = slice(cu[b], cu[b] + m)
        sub = {x: c[x][rows].clone() for x in ("q", "k", "v", "g", "beta")}   # fresh, aligned storage
        _, ref_state, _ = gdn.gdn_recurrent_step(sub["q"][None], sub["k"][None], sub["v"][None],
                                                 sub["g"][None], sub["beta"][None], scale=case["scale"],
                                                 initial_state=c["s0"][b:b + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(state[b], ref_state[0]), f"row {b}: replay of {m} records"
