"""GPU parity of the chunked prefill against the fp64 token-by-token oracle.

Small cases are compared in full; the full-size workloads (2048-token fp16,
14286-token packed bf16, the 4096-token prefix plus batches) are compared on
sampled value heads, which the oracle computes one by one.
"""

import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_common import DEV, assert_close, case_bounds, say, sha, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_03_amd as m
    m.load_library()
    return m


def prefill(gdn, case, chunk, heads_out=True, **kw):
    d = to_dev(case)
    if d["cu_seqlens"] is None:
        B = case["num_seqs"]
        args = [d[x].reshape(B, -1, *d[x].shape[1:]) for x in ("q", "k", "v", "g", "beta")]
    else:
        args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    kw.setdefault("initial_state", d["s0"])
    o, fin = gdn.gdn_prefill_chunked(*args, scale=case["scale"], cu_seqlens=d["cu_seqlens"], chunk_size=chunk,
                                     **kw)
    torch.cuda.synchronize()
    return o.reshape(-1, case["Hv"], case["dv"]), fin


def oracle_run(case, heads=None, s0="case", broadcast=False):
    return oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"],
                            case["Hq"], case["Hv"], cu_seqlens=case["cu_seqlens"], num_seqs=case["num_seqs"],
                            initial_state=case["s0"] if isinstance(s0, str) else s0, heads=heads,
                            initial_state_broadcast=broadcast)


def test_prefill_tiny_fp32_chunk16(gdn):
    case = gi.make("tiny_fp32")
    say(f"case tiny_fp32 prefill chunk 16 seed={case['seed']}")
    o, fin = prefill(gdn, case, case["chunk"])
    ref = oracle_run(case)
    assert_close(o, ref["o"], "f32", "o")
    assert_close(fin, ref["final"], "f32", "final")
    # chunked equals recurrent on the device too
    d = to_dev(case)
    o_r, fin_r, _ = gdn.gdn_recurrent_step(*[d[x].reshape(1, 64, *d[x].shape[1:]) for x in
                                             ("q", "k", "v", "g", "beta")], scale=case["scale"])
    assert_close(o, o_r.reshape(-1, 1, 16), "f32", "chunked vs recurrent o")
    assert_close(fin, fin_r, "f32", "chunked vs recurrent final")


def test_prefill_qwen_fp16(gdn):
    case = gi.make("qwen_fp16")
    say(f"case qwen_fp16 T=2048 Hq=2 Hv=6 seed={case['seed']}")
    o, fin = prefill(gdn, case, case["chunk"])
    ref = oracle_run(case)
    assert_close(o, ref["o"], "f16", "o", bounds=case_bounds(case), chunk=case["chunk"])
    assert_close(fin, ref["final"], "f16", "final")


def test_prefill_long_varlen_sampled_heads(gdn):
    case = gi.make("long_varlen")
    say(f"case long_varlen lengths={case['lengths']} seed={case['seed']}")
    o, fin = prefill(gdn, case, case["chunk"])
    heads = [0, 17, 31]   # key heads 0 and 8 (two value heads of key head 0 differ by decay only)
    ref = oracle_run(case, heads=heads)
    assert_close(o, ref["o"], "bf16", "o", bounds=case_bounds(case), chunk=case["chunk"], heads=heads)
    assert_close(fin, ref["final"], "bf16", "final", heads=heads)
    assert torch.isfinite(o).all() and torch.isfinite(fin).all()


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_prefill_ragged_chunk_boundaries(gdn, chunk, dtype):
    lengths = [0, 1, 15, 16, 17, 63, 64, 65, 130]
    case = gi.random_case(500 + chunk, lengths, Hq=2, Hv=4, dk=64, dv=128, dtype=dtype)
    say(f"case ragged {dtype} chunk={chunk} lengths={lengths}")
    o, fin = prefill(gdn, case, chunk)
    ref = oracle_run(case)
    assert_close(o, ref["o"], dtype, "o", bounds=case_bounds(case), chunk=chunk)
    assert_close(fin, ref["final"], dtype, "final")
    assert torch.equal(fin[0].cpu(), case["s0"][0])        # empty sequence: final = initial


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_ragged_dk128_short_and_partial_chunks(gdn, chunk, dtype):
    """16-bit inputs at dk = dv = 128 and C >= 32 take the transpose-read K^T
    path; short sequences and partial last chunks are checked one by one."""
    lengths = [1, 15, 16, 17, 31, 33, 63, 65, 200]
    case = gi.random_case(520 + chunk, lengths, Hq=2, Hv=4, dk=128, dv=128, dtype=dtype)
    say(f"case ragged dk128 {dtype} chunk={chunk} lengths={lengths}")
    o, fin = prefill(gdn, case, chunk)
    ref = oracle_run(case)
    assert_close(o, ref["o"], dtype, "o", bounds=case_bounds(case), chunk=chunk)
    assert_close(fin, ref["final"], dtype, "final")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_prefill_fp32_dk128(gdn, chunk):
    """The unquantised fp32 baseline at the Qwen-like head size dk = dv = 128:
    ragged sequences (empty, single token, partial and exact chunks), random
    initial states, final and chunk-boundary states, max-abs 1e-4."""
    lengths = [0, 1, 17, 64, 65, 130]
    case = gi.random_case(530 + chunk, lengths, Hq=2, Hv=4, dk=128, dv=128, dtype="f32")
    say(f"case fp32 dk128 chunk={chunk} lengths={lengths}")
    d = to_dev(case)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    o, fin, cs = gdn.gdn_prefill_chunked_states(*args, scale=case["scale"], cu_seqlens=d["cu_seqlens"],
                                                chunk_size=chunk, initial_state=d["s0"])
    o2, fin2 = gdn.gdn_prefill_chunked(*args, scale=case["scale"], cu_seqlens=d["cu_seqlens"], chunk_size=chunk,
                                       initial_state=d["s0"])
    torch.cuda.synchronize()
    ref = oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"], 2, 4,
                           cu_seqlens=case["cu_seqlens"], initial_state=case["s0"], boundary_every=chunk)
    assert_close(o, ref["o"], "f32", "o")
    assert_close(fin, ref["final"], "f32", "final")
    assert_close(cs, ref["boundary"], "f32", "chunk states")
    assert torch.equal(o, o2) and torch.equal(fin, fin2)
    assert torch.equal(fin[0].cpu(), case["s0"][0])


@pytest.mark.parametrize("dk,dv,Hq,Hv", [(16, 16, 1, 1), (32, 64, 2, 2), (128, 32, 1, 4), (64, 16, 3, 6)])
def test_prefill_head_dims(gdn, dk, dv, Hq, Hv):
    case = gi.random_case(600 + dk + dv, [70, 33], Hq=Hq, Hv=Hv, dk=dk, dv=dv, dtype="bf16")
    say(f"case head dims dk={dk} dv={dv} Hq={Hq} Hv={Hv}")
    o, fin = prefill(gdn, case, 64)
    ref = oracle_run(case)
    assert_close(o, ref["o"], "bf16", "o", bounds=case_bounds(case), chunk=64)
    assert_close(fin, ref["final"], "bf16", "final")


def test_prefill_chunk_size_does_not_change_results(gdn):
    case = gi.random_case(700, [200, 77], Hq=2, Hv=4, dk=128, dv=128, dtype="bf16")
    say("case chunk-size independence")
    outs = [prefill(gdn, case, c) for c in (16, 32, 64)]
    for o, fin in outs[1:]:
        assert_close(o, outs[0][0], "bf16", "o across chunk sizes", bounds=case_bounds(case))
        assert_close(fin, outs[0][1], "bf16", "final across chunk sizes")


def test_prefill_split_sequence_carries_state(gdn):
    """Prefill [0, m) then [m, T) from the carried final state equals [0, T)."""
    case = gi.random_case(710, [300], Hq=2, Hv=4, dk=128, dv=128, dtype="bf16")
    say("case split prefill carry")
    o_all, fin_all = prefill(gdn, case, 64)
    m = 100
    first = dict(case, q=case["q"][:m], k=case["k"][:m], v=case["v"][:m], g=case["g"][:m],
                 beta=case["beta"][:m], cu_seqlens=torch.tensor([0, m], dtype=torch.int32), T=m)
    second = dict(case, q=case["q"][m:], k=case["k"][m:], v=case["v"][m:], g=case["g"][m:],
                  beta=case["beta"][m:], cu_seqlens=torch.tensor([0, 300 - m], dtype=torch.int32), T=300 - m)
    o1, f1 = prefill(gdn, first, 64)
    o2, f2 = prefill(gdn, second, 64, initial_state=f1)
    assert_close(torch.cat([o1, o2]), o_all, "bf16", "o split vs whole", bounds=[(0, m), (m, 300)])
    assert_close(f2, fin_all, "bf16", "final split vs whole")


def test_prefill_in_place_final_state(gdn):
    case = gi.random_case(720, [90, 40], Hq=2, Hv=4, dk=128, dv=128, dtype="bf16")
    say("case in-place final state")
    o1, fin1 = prefill(gdn, case, 64)
    st = case["s0"].to(DEV).clone()
    o2, fin2 = prefill(gdn, case, 64, initial_state=st, final_state=st)
    assert torch.equal(o1, o2) and torch.equal(fin1, st)


def test_prefix_snapshot_reuse(gdn):
    """Prefill a 4096-token prefix, snapshot it, run 64 batches of 16 x 256
    branching from the snapshot (stride-0 broadcast); the snapshot stays
    bit-identical after every batch and sampled outputs of batches 0, 31 and 63
    match the oracle continuing from its own prefix state."""
    pre = gi.make("prefix_reuse", part="prefix")
    say(f"case prefix_reuse prefix seed={pre['seed']}")
    _, pfin = prefill(gdn, pre, 64)
    snap = gdn.gdn_state_snapshot(pfin)
    torch.cuda.synchronize()
    h0 = sha(snap)
    heads = [5, 26]
    pref = oracle_run(pre, heads=heads)
    checked = {0, 31, 63}
    for bi in range(64):
        bt = gi.make("prefix_reuse", part="batch", batch_index=bi)
        o, fin = prefill(gdn, bt, 64, initial_state=snap, initial_state_batch_stride=0,
                         output_final_state=False)
        assert sha(snap) == h0, f"snapshot changed after batch {bi}"
        if bi in checked:
            say(f"oracle check batch {bi}")
            ref = oracle_run(bt, heads=heads, s0=pref["final"][:1], broadcast=True)
            assert_close(o, ref["o"], "bf16", f"batch {bi} o", bounds=case_bounds(bt), chunk=64, heads=heads)


@pytest.mark.parametrize("dtype,C", [("bf16", 64), ("f16", 32)])
def test_prefill_many_rows_geometry(gdn, dtype, C):
    """More (row, head, 32-column slice) items than two per CU (40 x 4 x 4 = 640
    > 512) selects the 64-column workgroup geometry; ragged rows, random initial
    states, boundary states included."""
    rng_lengths = [97, 64, 1, 130, 33] * 8
    case = gi.random_case(9600 + C, rng_lengths, Hq=2, Hv=4, dk=128, dv=128, dtype=dtype)
    say(f"case many-rows geometry {dtype} C={C} rows={len(rng_lengths)}")
    d = to_dev(case)
    o, fin, cs = gdn.gdn_prefill_chunked_states(*[d[x] for x in ("q", "k", "v", "g", "beta")], scale=case["scale"],
                                                cu_seqlens=d["cu_seqlens"], chunk_size=C, initial_state=d["s0"])
    torch.cuda.synchronize()
    ref = oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"], 2, 4,
                           cu_seqlens=case["cu_seqlens"], initial_state=case["s0"], boundary_every=C)
    assert_close(o, ref["o"], dtype, "o", bounds=case_bounds(case), chunk=C)
    assert_close(fin, ref["final"], dtype, "final")
    assert_close(cs, ref["boundary"], dtype, "chunk states")
    o2, fin2 = gdn.gdn_prefill_chunked(*[d[x] for x in ("q", "k", "v", "g", "beta")], scale=case["scale"],
                                       cu_seqlens=d["cu_seqlens"], chunk_size=C, initial_state=d["s0"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(fin, fin2)


@pytest.mark.parametrize("nseq", [64, 70])
def test_prefill_many_sequences_plan(gdn, nseq):
    """Up to 64 sequences the prep and state kernels build the chunk plan
    themselves; beyond that a plan kernel writes it to the workspace.  Both
    sides of the limit, with empty and ragged sequences, boundary states
    included."""
    lengths = [(7 * i) % 45 if i % 9 else 0 for i in range(nseq)]
    lengths[nseq // 2] = 130                         # one sequence over several chunks
    C = 32
    case = gi.random_case(9700 + nseq, lengths, Hq=1, Hv=2, dk=32, dv=32, dtype="bf16")
    say(f"case {nseq} sequences, {sum(lengths)} tokens, chunk {C}")
    d = to_dev(case)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    o, fin, cs = gdn.gdn_prefill_chunked_states(*args, scale=case["scale"], cu_seqlens=d["cu_seqlens"], chunk_size=C,
                                                initial_state=d["s0"])
    o2, fin2 = gdn.gdn_prefill_chunked(*args, scale=case["scale"], cu_seqlens=d["cu_seqlens"], chunk_size=C,
                                       initial_state=d["s0"])
    torch.cuda.synchronize()
    ref = oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"], 1, 2,
                           cu_seqlens=case["cu_seqlens"], initial_state=case["s0"], boundary_every=C)
    assert_close(o, ref["o"], "bf16", "o", bounds=case_bounds(case), chunk=C)
    assert_close(fin, ref["final"], "bf16", "final")
    assert_close(cs, ref["boundary"], "bf16", "chunk states")
    assert torch.equal(o, o2) and torch.equal(fin, fin2)
    for b, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(fin[b].cpu(), case["s0"][b])


def test_prefill_many_dense_rows_plan(gdn):
    """Dense rows (no cu_seqlens) beyond the 64-sequence wave plan."""
    B, T = 66, 40
    case = gi.random_case(9800, [T] * B, Hq=1, Hv=2, dk=32, dv=32, dtype="bf16", dense=True)
    say(f"case dense B={B} T={T}")
    o, fin = prefill(gdn, case, 32)
    ref = oracle_run(case)
    assert_close(o, ref["o"], "bf16", "o", bounds=case_bounds(case), chunk=32)
    assert_close(fin, ref["final"], "bf16", "final")
