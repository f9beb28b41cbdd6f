"""The allocation-free prefill (library-held scratch instead of a caller
workspace) against the workspace entry point on the same inputs, on two calls
in a row, the second with a smaller input (the scratch keeps the first call's
contents), through the C ABI."""

import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_common import assert_close, case_bounds, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_03_amd as m
    m.load_library()
    return m


def run_both(gdn, case, chunk):
    d = to_dev(case)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    kw = dict(scale=case["scale"], cu_seqlens=d["cu_seqlens"], chunk_size=chunk, initial_state=d["s0"])
    o1, f1 = gdn.gdn_prefill_chunked(*args, **kw)
    o2 = torch.full_like(o1, float("nan"))
    f2 = torch.full_like(f1, float("nan"))
    gdn.gdn_prefill_chunked_noalloc(*args, **kw, o=o2, final_state=f2)
    torch.cuda.synchronize()
    return (o1, f1), (o2, f2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_prefill_matches_workspace_entry_point(gdn, dtype):
    dk = 128
    big = gi.random_case(7700, [300, 1, 64, 130, 17], Hq=2, Hv=4, dk=dk, dv=128, dtype=dtype)
    small = gi.random_case(7701, [70, 5], Hq=2, Hv=4, dk=dk, dv=128, dtype=dtype)
    for name, case in (("first call, 512 tokens", big), ("second call, smaller", small)):
        say(f"case noalloc {dtype} {name} lengths={case['lengths']}")
        (o1, f1), (o2, f2) = run_both(gdn, case, 64)
        # same kernels on the same inputs: identical to the workspace entry point
        assert torch.equal(o1, o2) and torch.equal(f1, f2), name
        ref = oracle.recurrent(case["q"], case["k"], case["v"], case["g"], case["beta"], case["scale"], 2, 4,
                               cu_seqlens=case["cu_seqlens"], initial_state=case["s0"])
        assert_close(o2, ref["o"], dtype, f"{name} o", bounds=case_bounds(case), chunk=64)
        assert_close(f2, ref["final"], dtype, f"{name} final")


def test_noalloc_rejects_problems_beyond_the_scratch(gdn):
    # 40,000 packed tokens at 32 value heads need about 270 MB of workspace
    T, Hq, Hv, dk, dv = 40000, 16, 32, 128, 128
    q = torch.zeros(T, Hq, dk, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(T, Hv, dv, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(T, Hv, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(gdn.GdnError, match="scratch"):
        gdn.gdn_prefill_chunked_noalloc(q, q, v, g, g, cu_seqlens=cu, chunk_size=64)
