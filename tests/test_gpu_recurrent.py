"""GPU parity of the recurrent step, compact capture, replay and snapshot.

Every device result is compared element by element with the fp64 oracle on the
same seeded, host-rounded inputs (tests/gpu_common.py holds the tolerances).
"""

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_common import DEV, TOL_DECAY_REL, assert_close, case_bounds, f64, say, sha, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = 1234.5


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_03_amd as m
    m.load_library()
    return m


def oracle_run(case, heads=None, broadcast=False):
    s0 = case["s0"]
    return oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"],
                            case["Hq"], case["Hv"], cu_seqlens=case["cu_seqlens"],
                            num_seqs=case["num_seqs"], initial_state=s0, heads=heads,
                            initial_state_broadcast=broadcast)


def dense4(case, t):
    """[B*T, H, d] packed tensor -> [B, T, H, d] dense view for dense workloads."""
    B = case["num_seqs"]
    return t.reshape(B, t.shape[0] // B, *t.shape[1:])


def run_step(gdn, case, **kw):
    d = to_dev(case)
    if d["cu_seqlens"] is None:
        args = [dense4(case, d[x]) for x in ("q", "k", "v", "g", "beta")]
    else:
        args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    o, fin, su = gdn.gdn_recurrent_step(*args, scale=case["scale"], initial_state=d["s0"],
                                        cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o.reshape(-1, case["Hv"], case["dv"]), fin, su


def test_recurrent_tiny_fp32(gdn):
    case = gi.make("tiny_fp32")
    say(f"case tiny_fp32 seed={case['seed']}")
    o, fin, _ = run_step(gdn, case)
    ref = oracle_run(case)
    assert_close(o, ref["o"], "f32", "o")
    assert_close(fin, ref["final"], "f32", "final")


@pytest.fixture(scope="module")
def spec(gdn):
    case = gi.make("spec_decode")
    say(f"case spec_decode seed={case['seed']} lengths={case['lengths']} counts={case['capture_count'].tolist()}")
    cap = case["capacity"]
    R = oracle.record_width(case["Hq"], case["Hv"], case["dk"], case["dv"])
    su = torch.full((case["num_seqs"], cap, R), SENTINEL, device=DEV)
    d = to_dev(case)
    o, fin, su = run_step(gdn, case, state_update_capacity=cap, capture_count=d["capture_count"],
                          state_update_active=1, state_update=su)
    ref = oracle_run(case)
    buf, mask = oracle.capture(case["k"], ref["alpha"], ref["delta"], case["Hq"], case["Hv"], cap,
                               case["capture_count"].numpy(), 1, cu_seqlens=case["cu_seqlens"])
    return dict(case=case, o=o, fin=fin, su=su, ref=ref, buf=buf, mask=mask)


def test_recurrent_spec_decode_outputs(spec):
    assert_close(spec["o"], spec["ref"]["o"], "bf16", "o", bounds=case_bounds(spec["case"]))
    assert_close(spec["fin"], spec["ref"]["final"], "bf16", "final")


def test_capture_records(spec):
    case, su, buf, mask = spec["case"], f64(spec["su"]), spec["buf"], spec["mask"]
    Hq, Hv, dk = case["Hq"], case["Hv"], case["dk"]
    n = [min(max(int(c), 0), case["capacity"], L) for c, L in zip(case["capture_count"].tolist(), case["lengths"])]
    # counts: exactly the clamped prefix is written, nothing else is touched
    for b in range(case["num_seqs"]):
        assert mask[b, :n[b]].all() and not mask[b, n[b]:].any()
    assert np.all(su[~mask] == SENTINEL), "uncaptured entries were written"
    # keys: bit-exact fp32 copies of the input keys at the right (row, slot, key head)
    keys_gpu = su[..., Hv:Hv + Hq * dk][mask[..., Hv:Hv + Hq * dk]]
    keys_ref = buf[..., Hv:Hv + Hq * dk][mask[..., Hv:Hv + Hq * dk]]
    np.testing.assert_array_equal(keys_gpu, keys_ref)
    # decays: relative error within the fp32 exp bound
    dm = mask[..., :Hv]
    rel = np.abs(su[..., :Hv][dm] - buf[..., :Hv][dm]) / np.abs(buf[..., :Hv][dm])
    assert rel.max() <= TOL_DECAY_REL, rel.max()
    # deltas: same bar as o, per (captured record, value head)
    rec = mask[..., 0]
    dv = case["dv"]
    assert_close(su[..., Hv + Hq * dk:][rec].reshape(-1, Hv, dv, 1),
                 buf[..., Hv + Hq * dk:][rec].reshape(-1, Hv, dv, 1), "bf16", "deltas")


def test_inactive_capture_zero_fills_everything(gdn, spec):
    case = spec["case"]
    cap = case["capacity"]
    su = torch.full_like(spec["su"], SENTINEL)
    d = to_dev(case)
    o, fin, su = run_step(gdn, case, state_update_capacity=cap, capture_count=d["capture_count"],
                          state_update_active=0, state_update=su)
    assert torch.count_nonzero(su).item() == 0
    assert torch.equal(o, spec["o"]) and torch.equal(fin, spec["fin"])


def test_replay_matches_oracle_and_recurrent_state(gdn, spec):
    case = spec["case"]
    cap, Hq, Hv, dk, dv = case["capacity"], case["Hq"], case["Hv"], case["dk"], case["dv"]
    n = [min(max(int(c), 0), cap, L) for c, L in zip(case["capture_count"].tolist(), case["lengths"])]
    # accept 0, a partial prefix, or everything captured (m_b <= n_b)
    m = [0 if b % 3 == 0 else (n[b] if b % 3 == 1 else n[b] // 2) for b in range(len(n))]
    say(f"replay counts {m} (captured {n})")
    state = case["s0"].to(DEV).clone()
    gdn.gdn_replay_state_updates(state, spec["su"], torch.tensor(m, dtype=torch.int32, device=DEV), Hq=Hq)
    torch.cuda.synchronize()
    ref = oracle.replay(case["s0"], spec["buf"], m, Hq, Hv, dk, dv, cap)
    assert_close(state, ref, "bf16", "replayed state")
    for b in range(len(m)):
        if m[b] == 0:
            assert torch.equal(state[b].cpu(), case["s0"][b])
    # rows whose whole run was captured and replayed: bitwise equal to the recurrent final state
    full = [b for b in range(len(n)) if m[b] == n[b] == case["lengths"][b] and n[b] > 0]
    say(f"bitwise replay rows {full}")
    assert full, "the workload must contain a fully captured row"
    for b in full:
        assert torch.equal(state[b], spec["fin"][b])


def test_snapshot_is_bitwise_and_never_written(gdn, spec):
    case = spec["case"]
    src = spec["fin"]
    snap = gdn.gdn_state_snapshot(src)
    torch.cuda.synchronize()
    assert torch.equal(snap, src)
    h0 = sha(snap)
    d = to_dev(case)
    for _ in range(4):   # repeated evaluations branching from the snapshot (broadcast row 0)
        gdn.gdn_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=case["scale"],
                               initial_state=snap[:1], initial_state_batch_stride=0,
                               cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert sha(snap) == h0


def test_single_token_calls_equal_one_multi_token_call(gdn):
    case = gi.random_case(77, [12, 12, 12], Hq=2, Hv=4, dk=64, dv=128, dtype="bf16", dense=True)
    say("case chained single-token calls, dense 3x12, dk=64")
    d = to_dev(case)
    B, T = 3, 12
    q, k, v, g, beta = (d[x].reshape(B, T, *d[x].shape[1:]) for x in ("q", "k", "v", "g", "beta"))
    o_all, fin_all, _ = gdn.gdn_recurrent_step(q, k, v, g, beta, scale=case["scale"], initial_state=d["s0"])
    state = d["s0"].clone()
    outs = []
    for t in range(T):
        sl = slice(t, t + 1)
        o_t, state, _ = gdn.gdn_recurrent_step(q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(),
                                               g[:, sl].contiguous(), beta[:, sl].contiguous(),
                                               scale=case["scale"], initial_state=state)
        outs.append(o_t)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), o_all)
    assert torch.equal(state, fin_all)


@pytest.mark.parametrize("dtype,dk,dv,Hq,Hv", [("f16", 128, 128, 2, 6), ("f32", 32, 64, 1, 2),
                                               ("bf16", 16, 16, 4, 4), ("bf16", 128, 32, 1, 3)])
def test_recurrent_shapes_and_empty_rows(gdn, dtype, dk, dv, Hq, Hv):
    lengths = [0, 5, 1, 9, 0, 3]
    case = gi.random_case(300 + dk + dv, lengths, Hq=Hq, Hv=Hv, dk=dk, dv=dv, dtype=dtype)
    say(f"case recurrent {dtype} dk={dk} dv={dv} Hq={Hq} Hv={Hv} lengths={lengths}")
    o, fin, _ = run_step(gdn, case)
    ref = oracle_run(case)
    assert_close(o, ref["o"], dtype, "o", bounds=case_bounds(case))
    assert_close(fin, ref["final"], dtype, "final")
    for b, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(fin[b].cpu(), case["s0"][b])


def test_recurrent_in_place_state_and_broadcast(gdn):
    case = gi.random_case(91, [4, 6], Hq=2, Hv=4, dk=128, dv=128, dtype="bf16")
    say("case in-place / broadcast initial state")
    d = to_dev(case)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    o1, fin1, _ = gdn.gdn_recurrent_step(*args, scale=case["scale"], initial_state=d["s0"],
                                         cu_seqlens=d["cu_seqlens"])
    st = d["s0"].clone()
    o2, fin2, _ = gdn.gdn_recurrent_step(*args, scale=case["scale"], initial_state=st, final_state=st,
                                         cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(fin1, st) and torch.equal(o1, o2)
    # stride 0 broadcast of one state equals the explicit repetition
    one = d["s0"][:1].contiguous()
    o3, fin3, _ = gdn.gdn_recurrent_step(*args, scale=case["scale"], initial_state=one,
                                         initial_state_batch_stride=0, cu_seqlens=d["cu_seqlens"])
    rep = one.repeat(2, 1, 1, 1).contiguous()
    o4, fin4, _ = gdn.gdn_recurrent_step(*args, scale=case["scale"], initial_state=rep,
                                         cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(fin3, fin4)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_rows_match_oracle_and_chunked_prefill(gdn, dtype):
    # rows of many tokens (the 4-deep token ring wraps dozens of times): the
    # recurrent step against the oracle, and against the chunked prefill of the
    # same input (the pages' chunked-equals-recurrent invariant)
    lengths = [130, 64, 1, 97]
    case = gi.random_case(4242, lengths, Hq=2, Hv=4, dk=128, dv=128, dtype=dtype)
    say(f"case long recurrent rows {dtype} lengths={lengths}")
    o, fin, _ = run_step(gdn, case)
    ref = oracle_run(case)
    bounds = case_bounds(case)
    assert_close(o, ref["o"], dtype, "o", bounds=bounds)
    assert_close(fin, ref["final"], dtype, "final")
    d = to_dev(case)
    oc, fc = gdn.gdn_prefill_chunked(*[d[x] for x in ("q", "k", "v", "g", "beta")], scale=case["scale"],
                                     initial_state=d["s0"], cu_seqlens=d["cu_seqlens"], chunk_size=64)
    torch.cuda.synchronize()
    assert_close(oc, ref["o"], dtype, "chunked o", bounds=bounds, chunk=64)
    assert_close(fc, ref["final"], dtype, "chunked final")
    if dtype != "f32":   # fp32: both within max-abs 1e-4 of the oracle above
        assert_close(oc, o.float(), dtype, "chunked vs recurrent o", bounds=bounds, chunk=64)
        assert_close(fc, fin, dtype, "chunked vs recurrent final")
