"""The C-ABI library loads, exports what include/gdn.h declares, and rejects bad
arguments on the host before touching the GPU (CPU only: every call here is
built to fail validation, so nothing is ever enqueued)."""

import ctypes
import os
import re

import pytest

import gated_deltanet_03_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

# A 16-byte-aligned address that is never dereferenced (every call below fails
# validation before any HIP call; the assertions check exactly that).
FAKE = ctypes.c_void_p(0x10000)
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return gdn.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(gdn.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.gdn_abi_version() == 1


def shape(**kw):
    d = dict(B=2, T=64, Hq=2, Hv=4, dk=128, dv=128, scale=0.088, dtype=gdn.GDN_BF16)
    d.update(kw)
    return gdn.gdn_shape(**d)


def prefill(lib, sh, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=NULL, stride=0, cu=NULL, chunk=64,
            o=ctypes.c_void_p(0x900000), sout=NULL, ws=NULL, wsb=0):
    return lib.gdn_prefill_chunked(ctypes.byref(sh), q, k, v, g, beta, s0, stride, cu, chunk, o, sout, ws, wsb,
                                   NULL)


def step(lib, sh, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=NULL, stride=0, cu=NULL,
         o=ctypes.c_void_p(0x900000), sout=NULL, cap=0, counts=NULL, active=1, su=NULL):
    return lib.gdn_recurrent_step(ctypes.byref(sh), q, k, v, g, beta, s0, stride, cu, o, sout, cap, counts,
                                  active, su, NULL)


def last(lib):
    return lib.gdn_last_error().decode()


def test_shape_validation(lib):
    assert step(lib, shape(Hv=5)) == gdn.GDN_ERR_INVALID_ARG and "multiple" in last(lib)
    assert step(lib, shape(Hq=0)) == gdn.GDN_ERR_INVALID_ARG
    assert step(lib, shape(dk=96)) == gdn.GDN_ERR_UNSUPPORTED
    assert step(lib, shape(dv=8)) == gdn.GDN_ERR_UNSUPPORTED
    assert step(lib, shape(dtype=7)) == gdn.GDN_ERR_INVALID_ARG
    assert step(lib, shape(B=-1)) == gdn.GDN_ERR_INVALID_ARG
    assert step(lib, shape(scale=float("nan"))) == gdn.GDN_ERR_INVALID_ARG
    assert prefill(lib, shape(), chunk=48) == gdn.GDN_ERR_UNSUPPORTED


def test_pointer_validation(lib):
    assert step(lib, shape(), q=NULL) == gdn.GDN_ERR_INVALID_ARG and "q is NULL" in last(lib)
    assert step(lib, shape(), beta=ctypes.c_void_p(0x10008)) == gdn.GDN_ERR_INVALID_ARG
    assert "aligned" in last(lib)
    # o overlapping an input
    assert step(lib, shape(), o=FAKE) == gdn.GDN_ERR_INVALID_ARG and "overlaps" in last(lib)


def test_capture_validation(lib):
    assert step(lib, shape(), cap=-1) == gdn.GDN_ERR_INVALID_ARG
    assert step(lib, shape(), cap=7, counts=NULL, su=ctypes.c_void_p(0x4000000)) == gdn.GDN_ERR_INVALID_ARG
    assert "capture_count" in last(lib)
    assert step(lib, shape(), cap=7, counts=ctypes.c_void_p(0x5000000), su=NULL) == gdn.GDN_ERR_INVALID_ARG
    assert "state_update" in last(lib)


def test_state_aliasing_validation(lib):
    s = ctypes.c_void_p(0x8000000)
    per = 4 * 128 * 128
    # final overlapping initial is only allowed as the exact in-place form
    assert step(lib, shape(), s0=s, stride=0, sout=s) == gdn.GDN_ERR_INVALID_ARG
    assert step(lib, shape(), s0=s, stride=per + 4, sout=ctypes.c_void_p(0x8000000 + 64)) == \
        gdn.GDN_ERR_INVALID_ARG
    assert step(lib, shape(), s0=s, stride=6, sout=NULL) == gdn.GDN_ERR_INVALID_ARG   # stride % 4
    assert step(lib, shape(), s0=s, stride=-4, sout=NULL) == gdn.GDN_ERR_INVALID_ARG


def test_workspace_validation_and_sizing(lib):
    sh = shape()
    need = gdn.gdn_prefill_workspace_bytes(sh, 64, False)
    # dense: ceil(64/64)*B chunks fit in the bound (B*T/C + B + 1) * Hv blocks
    assert need > 0 and need >= (2 + 2 + 1) * 4 * (2 * 6 * 512 * 2 + 1024)
    assert gdn.gdn_prefill_workspace_bytes(sh, 48, False) == 0
    assert gdn.gdn_prefill_workspace_bytes(shape(dk=96), 64, False) == 0
    rag = gdn.gdn_prefill_workspace_bytes(shape(B=4, T=14286, Hq=16, Hv=32), 64, True)
    max_chunks = 14286 // 64 + 4 + 1
    head = -(-(32 + max_chunks * 8) // 256) * 256      # offsets (B+1, padded to 16 B) + chunk table
    assert rag == head + max_chunks * 32 * (2 * 6 * 512 * 2 + 1024)
    assert prefill(lib, sh, ws=NULL, wsb=0) == gdn.GDN_ERR_INVALID_ARG and "workspace" in last(lib)
    assert prefill(lib, sh, ws=ctypes.c_void_p(0x40000008), wsb=need) == gdn.GDN_ERR_INVALID_ARG


def test_chunk_states_validation(lib):
    sh = shape()
    ws = ctypes.c_void_p(0x40000000)
    wsb = gdn.gdn_prefill_workspace_bytes(sh, 64, False)

    def call(cs, cap):
        return lib.gdn_prefill_chunked_states(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL, 64,
                                              ctypes.c_void_p(0x900000), NULL, cs, cap, ws, wsb, NULL)
    assert call(NULL, 4) == gdn.GDN_ERR_INVALID_ARG and "chunk_states is NULL" in last(lib)
    assert call(ctypes.c_void_p(0x80000000), -1) == gdn.GDN_ERR_INVALID_ARG
    assert call(ctypes.c_void_p(0x80000008), 4) == gdn.GDN_ERR_INVALID_ARG and "aligned" in last(lib)
    # overlapping the workspace, o, or an input
    assert call(ctypes.c_void_p(0x40000000 + 256), 4) == gdn.GDN_ERR_INVALID_ARG and "workspace" in last(lib)
    assert call(ctypes.c_void_p(0x900000), 4) == gdn.GDN_ERR_INVALID_ARG and "overlaps o" in last(lib)
    assert call(FAKE, 4) == gdn.GDN_ERR_INVALID_ARG and "overlaps" in last(lib)
    # a huge capacity is clamped to the chunk bound (no size overflow) and still overlap-checked
    assert call(ctypes.c_void_p(0x40000000 - 1024), 1 << 60) == gdn.GDN_ERR_INVALID_ARG and "workspace" in last(lib)


def test_prologue_validation(lib):
    sh = shape()
    ws = ctypes.c_void_p(0x40000000)
    wsb = gdn.gdn_prefill_workspace_bytes(sh, 64, False)

    def pre(pro):
        return lib.gdn_prefill_chunked_ex(ctypes.byref(sh), ctypes.byref(pro), FAKE, FAKE, FAKE, FAKE, FAKE, NULL,
                                          0, NULL, 64, ctypes.c_void_p(0x900000), NULL, NULL, 0, ws, wsb, NULL)

    def rec(pro):
        return lib.gdn_recurrent_step_ex(ctypes.byref(sh), ctypes.byref(pro), FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 0,
                                         NULL, ctypes.c_void_p(0x900000), NULL, 0, NULL, 1, NULL, NULL)
    for call in (pre, rec):
        assert call(gdn.gdn_prologue(1, -1.0, 0, None, None)) == gdn.GDN_ERR_INVALID_ARG and "eps" in last(lib)
        assert call(gdn.gdn_prologue(1, float("nan"), 0, None, None)) == gdn.GDN_ERR_INVALID_ARG
        assert call(gdn.gdn_prologue(0, 0.0, 0, None, 0x20000)) == gdn.GDN_ERR_INVALID_ARG and "dt_bias" in last(lib)
        assert call(gdn.gdn_prologue(0, 0.0, 1, 0x20002, None)) == gdn.GDN_ERR_INVALID_ARG and "aligned" in last(lib)
        # a valid prologue still fails on the (invalid) shape before anything is enqueued
    bad = gdn.gdn_shape(2, 64, 2, 5, 128, 128, 0.088, gdn.GDN_BF16)
    ok = gdn.gdn_prologue(1, 1e-6, 1, 0x20000, 0x20010)
    assert lib.gdn_recurrent_step_ex(ctypes.byref(bad), ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL,
                                     ctypes.c_void_p(0x900000), NULL, 0, NULL, 1, NULL, NULL) == gdn.GDN_ERR_INVALID_ARG


def test_replay_and_snapshot_validation(lib):
    assert lib.gdn_replay_state_updates(2, 2, 5, 128, 128, 7, FAKE, FAKE, FAKE, NULL) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_replay_state_updates(2, 2, 4, 128, 128, -1, FAKE, FAKE, FAKE, NULL) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_replay_state_updates(2, 2, 4, 100, 128, 7, FAKE, FAKE, FAKE, NULL) == gdn.GDN_ERR_UNSUPPORTED
    assert lib.gdn_replay_state_updates(2, 2, 4, 128, 128, 7, NULL, FAKE, FAKE, NULL) == gdn.GDN_ERR_INVALID_ARG
    # state_update overlapping state
    assert lib.gdn_replay_state_updates(2, 2, 4, 128, 128, 7, FAKE, ctypes.c_void_p(0x7000000), FAKE, NULL) == \
        gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_state_snapshot(FAKE, FAKE, 2, 4, 128, 128, NULL) == gdn.GDN_ERR_INVALID_ARG   # overlap
    assert lib.gdn_state_snapshot(NULL, FAKE, 2, 4, 128, 128, NULL) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_state_snapshot(FAKE, ctypes.c_void_p(0x7000008), 2, 4, 128, 128, NULL) == \
        gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_state_snapshot(FAKE, FAKE, -1, 4, 128, 128, NULL) == gdn.GDN_ERR_INVALID_ARG


def test_status_strings(lib):
    for st in range(4):
        assert lib.gdn_status_string(st)
    assert b"unknown" in lib.gdn_status_string(99)


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """Host-side: a problem whose workspace exceeds the fixed scratch array is
    rejected before any HIP call; an invalid shape is named as such."""
    sh = shape(B=1, T=10_000_000, Hq=16, Hv=32)
    st = lib.gdn_prefill_chunked_noalloc(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 0, FAKE, 64,
                                         ctypes.c_void_p(0x900000), NULL, NULL)
    assert st == gdn.GDN_ERR_UNSUPPORTED and "scratch" in last(lib)
    st = lib.gdn_prefill_chunked_noalloc(ctypes.byref(shape(Hv=5)), FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL, 64,
                                         ctypes.c_void_p(0x900000), NULL, NULL)
    assert st == gdn.GDN_ERR_INVALID_ARG and "multiple" in last(lib)
