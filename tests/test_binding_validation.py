"""The Python binding checks every tensor's shape or element count against the
problem description before it calls the library: the C ABI receives bare
pointers, so a short buffer would otherwise be read or written out of bounds on
the device.  CPU tensors only; every case must raise before any library call."""

import pytest
import torch

import gated_deltanet_03_amd as gdn


def tokens(T=40, Hq=2, Hv=4, dk=16, dv=32, dtype=torch.bfloat16, B=None):
    lead = (T,) if B is None else (B, T // B)
    q = torch.zeros(*lead, Hq, dk, dtype=dtype)
    k = torch.zeros_like(q)
    v = torch.zeros(*lead, Hv, dv, dtype=dtype)
    g = torch.zeros(*lead, Hv)
    beta = torch.zeros(*lead, Hv)
    return q, k, v, g, beta


def cu(lengths):
    c = [0]
    for L in lengths:
        c.append(c[-1] + L)
    return torch.tensor(c, dtype=torch.int32)


def test_prefill_token_shapes():
    q, k, v, g, beta = tokens()
    with pytest.raises(ValueError, match="k has shape"):
        gdn.gdn_prefill_chunked(q, k[:-1], v, g, beta, cu_seqlens=cu([20, 20]))
    with pytest.raises(ValueError, match="g has shape"):
        gdn.gdn_prefill_chunked(q, k, v, g[:, :2].contiguous(), beta, cu_seqlens=cu([20, 20]))
    with pytest.raises(ValueError, match="v has shape"):
        gdn.gdn_prefill_chunked(q, k, v[:-3], g, beta, cu_seqlens=cu([20, 20]))
    with pytest.raises(ValueError, match="o has shape"):
        gdn.gdn_prefill_chunked(q, k, v, g, beta, cu_seqlens=cu([20, 20]), o=torch.empty_like(v)[:-1])


def test_prefill_state_sizes():
    q, k, v, g, beta = tokens()
    c = cu([10, 10, 20])
    # 1 < N < B states with the default per-sequence stride: too few
    with pytest.raises(ValueError, match="initial_state has"):
        gdn.gdn_prefill_chunked(q, k, v, g, beta, cu_seqlens=c, initial_state=torch.zeros(2, 4, 16, 32))
    with pytest.raises(ValueError, match="final_state has shape"):
        gdn.gdn_prefill_chunked(q, k, v, g, beta, cu_seqlens=c, final_state=torch.zeros(2, 4, 16, 32))
    with pytest.raises(ValueError, match="chunk_states has shape"):
        gdn.gdn_prefill_chunked_states(q, k, v, g, beta, cu_seqlens=c, chunk_size=16,
                                       chunk_states=torch.zeros(4, 4, 16, 16))


def test_recurrent_capture_sizes():
    q, k, v, g, beta = tokens(T=14, B=2)
    R = 4 + 2 * 16 + 4 * 32
    with pytest.raises(ValueError, match="capture_count has"):
        gdn.gdn_recurrent_step(q, k, v, g, beta, state_update_capacity=3,
                               capture_count=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="state_update has"):
        gdn.gdn_recurrent_step(q, k, v, g, beta, state_update_capacity=3,
                               capture_count=torch.zeros(2, dtype=torch.int32),
                               state_update=torch.zeros(2, 2, R))
    with pytest.raises(ValueError, match="capture_count is required"):
        gdn.gdn_recurrent_step(q, k, v, g, beta, state_update_capacity=3)


def test_replay_sizes():
    st = torch.zeros(2, 4, 16, 32)
    R = 4 + 2 * 16 + 4 * 32
    su = torch.zeros(2, 3, R)
    # a wrong Hq changes the record length
    with pytest.raises(ValueError, match="records hold"):
        gdn.gdn_replay_state_updates(st, su, torch.zeros(2, dtype=torch.int32), Hq=1)
    with pytest.raises(ValueError, match="replay_count has"):
        gdn.gdn_replay_state_updates(st, su, torch.zeros(1, dtype=torch.int32), Hq=2)
    with pytest.raises(ValueError, match="state_update has"):
        gdn.gdn_replay_state_updates(st, su, torch.zeros(2, dtype=torch.int32), Hq=2, state_update_capacity=4)
    with pytest.raises(ValueError, match="divide"):
        gdn.gdn_replay_state_updates(st, su, torch.zeros(2, dtype=torch.int32), Hq=3)


def test_snapshot_sizes():
    with pytest.raises(ValueError, match="dst has shape"):
        gdn.gdn_state_snapshot(torch.zeros(2, 4, 16, 32), torch.zeros(1, 4, 16, 32))
