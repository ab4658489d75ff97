"""CPU-only checks of the C-ABI library: it loads, exports every symbol the
header declares, its host logic (ladder, split, planner) agrees with the
oracle and the pages' printed values, and invalid arguments are rejected on
the host before any launch (no GPU is touched by these tests)."""
import ctypes

import torch
import json
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpk.h")
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_values.json")))

cpk = pytest.importorskip("chunked_prefill_causal_kv_amd")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpk_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(cpk.LIB_PATH)
    names = _declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n


def test_binding_covers_every_declared_symbol():
    for n in _declared_functions():
        assert callable(getattr(cpk, n)), n


def test_ladder_matches_oracle_and_pages():
    assert cpk.cpk_ladder_rungs(GOLD["ladder"]["W"]) == GOLD["ladder"]["rungs"]
    for W in list(range(1, 600)) + [1024, 2048, 4096, 8192]:
        assert cpk.cpk_ladder_rungs(W) == oracle.ladder_rungs(W)
    for W in (1, 2, 3, 4, 5, 7, 64, 255, 256, 512, 1000):
        for r in range(1, W + 1):
            assert cpk.cpk_ladder_width(W, r) == oracle.ladder_width(W, r)


def test_split_matches_oracle_and_pages():
    for L, rows in GOLD["split_examples"]["cases"].items():
        assert [r for _, r in cpk.cpk_split_chunks(int(L), 512)] == rows
    assert [r for _, r in cpk.cpk_split_chunks(1000, 256)] == GOLD["demo_split"]["chunk_rows"]
    for L in (0, 1, 255, 256, 257, 4000, 20000):
        for W in (1, 7, 256, 512):
            assert cpk.cpk_split_chunks(L, W) == oracle.split_chunks(L, W)


def test_planner_matches_oracle():
    for budget in (0, 1, 64, 65, 2048, 8192):
        for n_dec in (0, 1, 64):
            if n_dec > budget:
                with pytest.raises(cpk.CpkError):
                    cpk.cpk_plan_step(budget, n_dec, 100)
                continue
            for rem in (0, 1, 100, 20000):
                assert cpk.cpk_plan_step(budget, n_dec, rem) == oracle.plan_step(budget, n_dec, rem)


def test_host_logic_rejects_bad_arguments():
    for args in ((0, 1), (512, 0), (512, 513)):
        with pytest.raises(cpk.CpkError) as e:
            cpk.cpk_ladder_width(*args)
        assert e.value.status == cpk.CPK_EINVAL
    with pytest.raises(cpk.CpkError):
        cpk.cpk_ladder_rungs(0)
    with pytest.raises(cpk.CpkError):
        cpk.cpk_split_chunks(-1, 4)


# Validation of device calls: each of these must fail on the host before
# any launch.  The device addresses are fake, so the tests only run where no
# GPU is visible: a validation gap then shows up as CPK_EHIP (no device)
# instead of a launch on bogus pointers.

FAKE = 1 << 20  # 16-byte aligned, never dereferenced
no_gpu = pytest.mark.skipif(__import__("torch").cuda.is_available(),
                            reason="fake device pointers: host-only machines")


def _desc(**kw):
    d = dict(k=FAKE, v=FAKE * 2, seqlens_k=FAKE * 3, batch=2, kv_heads=8, capacity=1024,
             head_dim=128, dtype=cpk.CPK_BF16)
    d.update(kw)
    return cpk.cpk_kv_cache(d["k"], d["v"], d["seqlens_k"], d["batch"], d["kv_heads"],
                            d["capacity"], d["head_dim"], d["dtype"])


def _append(desc, b=0, past=0, rows=4, kn=FAKE, vn=FAKE, real=None):
    return cpk._lib.cpk_kv_append(ctypes.byref(desc), b, kn, vn, past, rows,
                                  rows if real is None else real, None)


@no_gpu
def test_append_validation():
    assert _append(_desc(), past=1020, rows=5) == cpk.CPK_ECAPACITY
    assert _append(_desc(), b=2) == cpk.CPK_EINVAL
    assert _append(_desc(), rows=0) == cpk.CPK_EINVAL
    assert _append(_desc(), rows=4, real=5) == cpk.CPK_EINVAL
    assert _append(_desc(), rows=4, real=0) == cpk.CPK_EINVAL
    assert _append(_desc(), kn=FAKE + 2) == cpk.CPK_EALIGN
    assert _append(_desc(head_dim=96)) == cpk.CPK_EDTYPE
    assert _append(_desc(dtype=7)) == cpk.CPK_EDTYPE
    assert _append(_desc(k=0)) == cpk.CPK_EINVAL
    assert "capacity" in (_append(_desc(), past=1024, rows=1) and cpk.cpk_last_error())


def _attn(desc, Hq=32, past=0, rows=8, real=8, q=FAKE, out=FAKE):
    return cpk._lib.cpk_chunk_attention(q, ctypes.byref(desc), 0, Hq, past, rows, real, 0.0,
                                        out, None)


@no_gpu
def test_attention_validation():
    assert _attn(_desc(), real=9) == cpk.CPK_EINVAL
    assert _attn(_desc(), Hq=30) == cpk.CPK_EINVAL
    assert _attn(_desc(kv_heads=1), Hq=128) == cpk.CPK_EINVAL       # group 128 > 64
    assert _attn(_desc(), past=1020, rows=8) == cpk.CPK_ECAPACITY
    assert _attn(_desc(), q=FAKE + 8) == cpk.CPK_EALIGN
    assert _attn(_desc(), rows=0, real=0) == cpk.CPK_EINVAL


@no_gpu
def test_rewind_and_prefill_validation():
    d = _desc()
    assert cpk._lib.cpk_rewind(ctypes.byref(d), 0, 5, 4, None) == cpk.CPK_EINVAL
    assert cpk._lib.cpk_rewind(ctypes.byref(d), 0, -1, 4, None) == cpk.CPK_EINVAL
    w = ctypes.c_int(0)
    f = cpk._lib.cpk_prefill_chunk
    # real rows above the chunk width
    assert f(FAKE, FAKE, FAKE, ctypes.byref(d), 0, 32, 0, 513, 512, 1, 0.0, FAKE, ctypes.byref(w), None) == cpk.CPK_EINVAL
    # padding 113 -> 171 rows does not fit 1024 - 900
    assert f(FAKE, FAKE, FAKE, ctypes.byref(d), 0, 32, 900, 113, 512, 1, 0.0, FAKE, ctypes.byref(w), None) == cpk.CPK_ECAPACITY
    # without padding it would fit: then the failure must come from elsewhere
    assert f(FAKE, FAKE, FAKE, ctypes.byref(d), 0, 30, 900, 113, 512, 0, 0.0, FAKE, ctypes.byref(w), None) == cpk.CPK_EINVAL


@no_gpu
def test_varlen_validation():
    d = _desc()
    A = ctypes.c_int32
    slots = (A * 2)(0, 0)
    cu = (A * 3)(0, 1, 3)
    past = (A * 2)(10, 20)
    f = cpk._lib.cpk_varlen_step
    # slot used twice
    assert f(FAKE, FAKE, FAKE, ctypes.byref(d), FAKE, FAKE, FAKE, slots, cu, past, 2, 3, 32, 0.0,
             FAKE, FAKE, 1 << 30, None) == cpk.CPK_EINVAL
    slots = (A * 2)(0, 1)
    # cu_rows not ending at total_rows
    assert f(FAKE, FAKE, FAKE, ctypes.byref(d), FAKE, FAKE, FAKE, slots, cu, past, 2, 4, 32, 0.0,
             FAKE, FAKE, 1 << 30, None) == cpk.CPK_EINVAL
    # workspace too small for the decode row
    assert f(FAKE, FAKE, FAKE, ctypes.byref(d), FAKE, FAKE, FAKE, slots, cu, past, 2, 3, 32, 0.0,
             FAKE, FAKE, 16, None) == cpk.CPK_EWORKSPACE
    # capacity
    past = (A * 2)(1024, 20)
    assert f(FAKE, FAKE, FAKE, ctypes.byref(d), FAKE, FAKE, FAKE, slots, cu, past, 2, 3, 32, 0.0,
             FAKE, FAKE, 1 << 30, None) == cpk.CPK_ECAPACITY
    assert cpk.cpk_varlen_workspace_size(64, 32, 16385, 128) == 64 * 32 * 65 * 132 * 4


@no_gpu
def test_roll_validation():
    f = cpk._lib.cpk_roll_append
    # c > C
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, FAKE * 6, 1, 2, 8, 9, 64, cpk.CPK_F16, None) == cpk.CPK_EINVAL
    # output overlaps input
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE, FAKE * 6, 1, 2, 8, 4, 64, cpk.CPK_F16, None) == cpk.CPK_EINVAL
    g = cpk._lib.cpk_roll_attention
    assert g(FAKE, FAKE, FAKE, None, 100, 0, 16, 16, 64, 128, 128, cpk.CPK_F16, 0.0, FAKE,
             None, 0, None) == cpk.CPK_EINVAL
    assert g(FAKE, FAKE, FAKE, None, 10, 0, 16, 16, 64, 32, 128, cpk.CPK_F16, 0.0, FAKE,
             None, 0, None) == cpk.CPK_EINVAL
    # a workspace smaller than the split needs
    assert g(FAKE, FAKE, FAKE, None, 4096, 0, 16, 16, 2048, 256, 128, cpk.CPK_F16, 0.0, FAKE,
             FAKE, 16, None) == cpk.CPK_EWORKSPACE


def test_roll_workspace_size():
    """Rolling workload shapes (16 heads, no GQA, C = 2048, c = 256): 64
    workgroups unsplit, so the 16 key tiles are split 4 ways."""
    f16 = torch.float16
    assert cpk.cpk_roll_workspace_size(16, 16, 2048, 256, 128, f16) == 4 * 256 * 16 * 132 * 4
    assert cpk.cpk_roll_workspace_size(16, 16, 2048, 256, 128, torch.float32) == 0
    # enough workgroups already: no split
    assert cpk.cpk_roll_workspace_size(32, 8, 8192, 4096, 128, torch.bfloat16) == 0
    # never more parts than key tiles
    assert cpk.cpk_roll_workspace_size(1, 1, 128, 64, 64, f16) == 0


def test_attention_kernel_setting():
    """The kernel choice is process-wide, returns the previous setting and
    rejects unknown kinds without changing the setting."""
    prev = cpk.cpk_set_attention_kernel(cpk.ATTN_WIDE)
    try:
        assert prev == cpk.ATTN_AUTO
        assert cpk.cpk_set_attention_kernel(cpk.ATTN_NARROW) == cpk.ATTN_WIDE
        assert cpk.cpk_set_attention_kernel(cpk.ATTN_NARROW_GENERAL) == cpk.ATTN_NARROW
        assert cpk.cpk_set_attention_kernel(cpk.ATTN_NARROW) == cpk.ATTN_NARROW_GENERAL
        with pytest.raises(cpk.CpkError):
            cpk.cpk_set_attention_kernel(4)
        with pytest.raises(cpk.CpkError):
            cpk.cpk_set_attention_kernel(-1)
        with cpk.attention_kernel(cpk.ATTN_WIDE):
            assert cpk.cpk_set_attention_kernel(cpk.ATTN_WIDE) == cpk.ATTN_WIDE
        assert cpk.cpk_set_attention_kernel(cpk.ATTN_AUTO) == cpk.ATTN_NARROW
    finally:
        cpk.cpk_set_attention_kernel(cpk.ATTN_AUTO)


@no_gpu
def test_ring_validation():
    """Ring-buffer entry points reject bad shapes, start indices and aliasing
    on the host (fake aligned pointers, never dereferenced)."""
    F16 = cpk.CPK_F16
    ap = cpk._lib.cpk_ring_append
    big = FAKE * 64   # far from the other fake buffers
    # start outside [0, C)
    assert ap(FAKE, FAKE * 2, big, big * 2, 1, 2, 8, 4, 64, F16, 8, None) == cpk.CPK_EINVAL
    assert ap(FAKE, FAKE * 2, big, big * 2, 1, 2, 8, 4, 64, F16, -1, None) == cpk.CPK_EINVAL
    # c > C
    assert ap(FAKE, FAKE * 2, big, big * 2, 1, 2, 8, 9, 64, F16, 0, None) == cpk.CPK_EINVAL
    # a chunk overlapping a ring
    assert ap(big, FAKE * 2, big, big * 2, 1, 2, 8, 4, 64, F16, 0, None) == cpk.CPK_EINVAL
    # unaligned
    assert ap(FAKE + 8, FAKE * 2, big, big * 2, 1, 2, 8, 4, 64, F16, 0, None) == cpk.CPK_EALIGN
    # bad head dim
    assert ap(FAKE, FAKE * 2, big, big * 2, 1, 2, 8, 4, 96, F16, 0, None) == cpk.CPK_EDTYPE
    at = cpk._lib.cpk_ring_attention
    assert at(FAKE, FAKE, FAKE, None, 4096, 0, 16, 16, 2048, 256, 128, F16, 0.0, 2048, FAKE,
              None, 0, None) == cpk.CPK_EINVAL
    assert at(FAKE, FAKE, FAKE, None, 100, 0, 16, 16, 64, 128, 128, F16, 0.0, 0, FAKE,
              None, 0, None) == cpk.CPK_EINVAL
    vw = cpk._lib.cpk_ring_view
    assert vw(FAKE, FAKE * 2, big, big * 2, 1, 2, 8, 64, F16, 8, None) == cpk.CPK_EINVAL
    assert vw(FAKE, FAKE * 2, FAKE, big * 2, 1, 2, 8, 64, F16, 0, None) == cpk.CPK_EINVAL


@no_gpu
def test_ring_step_validation():
    """cpk_ring_step checks the append's and the attention's arguments on
    the host before anything is launched (fake aligned pointers)."""
    F16 = cpk.CPK_F16
    st = cpk._lib.cpk_ring_step
    big = FAKE * 64
    q, kc, vc, out = FAKE, FAKE * 2, FAKE * 3, FAKE * 4

    def call(q=q, kc=kc, vc=vc, kr=big, vr=big * 2, c=4, C=8, D=64, start=0, abs_end=8):
        return st(q, kc, vc, kr, vr, None, abs_end, 0, 2, 2, C, c, D, F16, 0.0, start, out,
                  None, 0, None)

    assert call(start=8) == cpk.CPK_EINVAL           # start outside [0, C)
    assert call(start=-1) == cpk.CPK_EINVAL
    assert call(kc=None) == cpk.CPK_EINVAL            # no chunk
    assert call(kc=big) == cpk.CPK_EINVAL             # a chunk overlapping a ring
    assert call(vr=big) == cpk.CPK_EINVAL             # the rings overlap
    assert call(vc=FAKE * 3 + 8) == cpk.CPK_EALIGN    # unaligned chunk
    assert call(c=9) == cpk.CPK_EINVAL                # c > C
    assert call(D=96) == cpk.CPK_EDTYPE               # unsupported head dim
    assert call(abs_end=3) == cpk.CPK_EINVAL          # abs_end < c


@no_gpu
def test_ring_step_deferred_validation():
    """The deferred ring step and its flush reject, on the host, shapes that
    do not split, a missing or short workspace, and a carried merge whose
    buffers alias the launch's other buffers (fake aligned pointers, 64 MiB
    apart; every call here fails before a launch)."""
    F16 = cpk.CPK_F16
    M = 1 << 26
    q, kc, vc, kr, vr, out, ws, pws, pout = (M * i for i in range(1, 10))
    Hq = Hkv = 16
    C, c, D = 2048, 256, 128
    need = cpk.cpk_roll_workspace_size(Hq, Hkv, C, c, D, torch.float16)
    assert need > 0
    st = cpk._lib.cpk_ring_step_deferred

    def call(heads=Hq, ws=ws, ws_bytes=need, pws=pws, pout=pout, q=q, mask=None):
        return st(q, kc, vc, kr, vr, mask, C, 0, heads, heads, C, c, D, F16, 0.0, 0, out,
                  ws, ws_bytes, pws, pout, None)

    assert cpk.cpk_roll_workspace_size(64, 64, C, c, D, torch.float16) == 0
    assert call(heads=64, ws=None, ws_bytes=0) == cpk.CPK_EINVAL    # no split
    assert call(ws=None, ws_bytes=0) == cpk.CPK_EINVAL              # no workspace
    assert call(ws_bytes=need - 4) == cpk.CPK_EWORKSPACE
    assert call(pout=None) == cpk.CPK_EINVAL                        # prev_ws alone
    assert call(pws=ws + 4096) == cpk.CPK_EINVAL                    # prev_ws overlaps ws
    assert call(pout=kr + 64) == cpk.CPK_EINVAL                     # prev_out on a ring
    assert call(pout=q) == cpk.CPK_EINVAL                           # prev_out on q
    assert call(pout=ws + 1024) == cpk.CPK_EINVAL                   # prev_out on ws
    assert call(pout=pws) == cpk.CPK_EINVAL                         # prev_out on prev_ws
    assert call(pout=M * 10 + 4096, mask=M * 10) == cpk.CPK_EINVAL   # prev_out on the mask
    assert call(pout=pout + 8) == cpk.CPK_EALIGN
    assert call(pws=pws + 8) == cpk.CPK_EALIGN
    fl = cpk._lib.cpk_roll_flush
    assert fl(ws, need, out, 64, 64, C, c, D, F16, None) == cpk.CPK_EINVAL   # no split
    assert fl(ws, need - 4, out, Hq, Hkv, C, c, D, F16, None) == cpk.CPK_EWORKSPACE
    assert fl(ws, need, ws + 4096, Hq, Hkv, C, c, D, F16, None) == cpk.CPK_EINVAL
    assert fl(None, need, out, Hq, Hkv, C, c, D, F16, None) == cpk.CPK_EINVAL
    assert fl(ws, need, out + 8, Hq, Hkv, C, c, D, F16, None) == cpk.CPK_EALIGN
    assert fl(ws, need, out, Hq, Hkv, C, c, 96, F16, None) == cpk.CPK_EDTYPE


@no_gpu
def test_roll_attention_deferred_validation():
    """The deferred literal-shift attention rejects, on the host, shapes that
    do not split, a missing or short workspace and a carried merge whose
    buffers alias the call's other buffers (fake aligned pointers, 64 MiB
    apart; every call here fails before a launch)."""
    F16 = cpk.CPK_F16
    M = 1 << 26
    q, k, v, out, ws, pws, pout, mask = (M * i for i in range(1, 9))
    Hq = Hkv = 16
    C, c, D = 2048, 256, 128
    need = cpk.cpk_roll_workspace_size(Hq, Hkv, C, c, D, torch.float16)
    f = cpk._lib.cpk_roll_attention_deferred

    def call(heads=Hq, ws=ws, ws_bytes=need, pws=pws, pout=pout, mask=None, abs_end=C):
        return f(q, k, v, mask, abs_end, 0, heads, heads, C, c, D, F16, 0.0, out, ws, ws_bytes,
                 pws, pout, None)

    assert call(heads=64, ws=None, ws_bytes=0) == cpk.CPK_EINVAL    # no split
    assert call(ws=None, ws_bytes=0) == cpk.CPK_EINVAL              # no workspace
    assert call(ws_bytes=need - 4) == cpk.CPK_EWORKSPACE
    assert call(abs_end=c - 1) == cpk.CPK_EINVAL                    # abs_end < c
    assert call(pout=None) == cpk.CPK_EINVAL                        # prev_ws alone
    assert call(pws=ws + 4096) == cpk.CPK_EINVAL                    # prev_ws overlaps ws
    assert call(pout=k + 64) == cpk.CPK_EINVAL                      # prev_out on the cache
    assert call(pout=ws + 1024) == cpk.CPK_EINVAL                   # prev_out on ws
    assert call(pout=mask + 4096, mask=mask) == cpk.CPK_EINVAL      # prev_out on the mask
    assert call(pout=pout + 8) == cpk.CPK_EALIGN


@no_gpu
def test_varlen_phases_validation():
    """cpk_varlen_step_phases takes a nonzero subset of the three phases."""
    f = cpk._lib.cpk_varlen_step_phases
    for bad in (0, 8, -1, 15):
        r = f(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, 1, 1, 8, 0.0, FAKE,
              FAKE, 0, bad, None)
        assert r == cpk.CPK_EINVAL, bad


@no_gpu
def test_paged_validation():
    """Paged caches: block_size a positive multiple of 256, a block table,
    positive counts, at most 512 blocks per sequence, bf16/fp16 only --
    rejected on the host."""
    def desc(bs=256, nb=8, mb=4, dt=cpk.CPK_BF16, table=FAKE):
        return cpk.cpk_paged_cache(FAKE, FAKE * 2, table, FAKE * 3, 2, 4, bs, nb, mb, 128, dt)
    f = cpk._lib.cpk_paged_varlen_step
    args = lambda d: (FAKE, FAKE, FAKE, ctypes.byref(d), FAKE, FAKE, FAKE, None, None, None, 1,
                      1, 16, 0.0, FAKE, FAKE, 0, cpk.PHASE_ALL, None)
    assert f(*args(desc(bs=128))) == cpk.CPK_EINVAL
    assert f(*args(desc(bs=0))) == cpk.CPK_EINVAL
    assert f(*args(desc(nb=0))) == cpk.CPK_EINVAL
    assert f(*args(desc(mb=513))) == cpk.CPK_EINVAL     # table entries staged on chip
    assert f(*args(desc(table=None))) == cpk.CPK_EINVAL
    assert f(*args(desc(dt=cpk.CPK_F32))) == cpk.CPK_EDTYPE


@no_gpu
def test_copy_prefix_validation():
    c = cpk.cpk_kv_cache(FAKE, FAKE * 2, FAKE * 3, 2, 4, 1024, 128, cpk.CPK_BF16)
    f = cpk._lib.cpk_kv_copy_prefix
    assert f(ctypes.byref(c), 0, 0, 10, None) == cpk.CPK_EINVAL      # same slot
    assert f(ctypes.byref(c), 0, 2, 10, None) == cpk.CPK_EINVAL      # slot out of range
    assert f(ctypes.byref(c), 0, 1, 1025, None) == cpk.CPK_EINVAL    # past capacity
    assert f(ctypes.byref(c), 0, 1, -1, None) == cpk.CPK_EINVAL
