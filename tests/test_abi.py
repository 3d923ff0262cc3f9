"""C ABI of libgla.so on the CPU: the library loads, exports every entry point declared in
include/gla.h, and rejects bad arguments on the host before any HIP call (fake, aligned
addresses are used; no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_linear_rnn_chunkwise_amd as gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")
A = 0x10000  # a fake 16-byte aligned device address


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gla.LIB_PATH):
        pytest.fail("libgla.so is not built (run __graft_entry__.build())")
    return gla.load()


def header_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(gla_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_python_exports():
    assert header_functions() == sorted(gla.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", gla.LIB_PATH]).decode()
    exported = set(re.findall(r"\sT\s(gla_\w+)$", out, re.M))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    # the version the header declares
    hdr = open(os.path.join(ROOT, "include", "gla.h")).read()
    declared = int(re.search(r"#define GLA_VERSION (\d+)", hdr).group(1))
    assert gla.version() == declared
    for st, txt in [(0, "ok"), (-1, "invalid argument"), (-2, "unsupported configuration"),
                    (-3, "workspace too small or allocation failed"), (-4, "HIP runtime error")]:
        assert gla.status_string(st) == txt
    assert gla.status_string(12345) == "unknown status"


def desc(**kw):
    d = gla.GlaDesc()
    base = dict(B=2, H=3, L=100, Dk=128, Dv=128, chunk=64, in_dtype=gla.DTYPE_BF16, gate_kind=gla.GATE_CHANNEL,
                q=A, k=A, v=A, log_alpha=A, log_ig=None, initial_state=None, out=A, final_state=None,
                seg_chunks=0, flags=0, workspace=None, workspace_bytes=0)
    base.update(kw)
    for key, val in base.items():
        setattr(d, key, val)
    return d


def status(lib, d):
    n = ctypes.c_size_t(0)
    return lib.gla_workspace_size(ctypes.byref(d), ctypes.byref(n)), n.value


def fwd_status(lib, d):
    # gla_fwd_ex validates before touching HIP; only invalid descriptors are passed here.
    return lib.gla_fwd_ex(ctypes.byref(d), None)


def test_valid_descriptor_plans(lib):
    st, n = status(lib, desc())
    assert st == gla.GLA_OK
    p = gla.plan(desc())
    assert p.tiles_per_chunk == 1 and p.dv_tiles == 2 and p.n_seg >= 1
    assert p.grid_out == 2 * 3 * p.n_seg * 2


@pytest.mark.parametrize("field,value", [
    ("q", None), ("k", None), ("v", None), ("out", None),
    ("B", 0), ("H", -1), ("L", 0), ("Dk", 0), ("Dv", 0), ("chunk", 0), ("seg_chunks", -1), ("flags", 2), ("flags", -1),
    ("in_dtype", 7), ("gate_kind", 9), ("log_alpha", None),
    ("q", A + 2), ("v", A + 8), ("out", A + 4), ("log_alpha", A + 4), ("final_state", A + 12),
    ("initial_state", A + 1), ("log_ig", A + 2),
])
def test_invalid_arguments_rejected_before_hip(lib, field, value):
    d = desc(**{field: value})
    assert status(lib, d)[0] == gla.GLA_ERR_INVALID_ARG
    assert fwd_status(lib, d) == gla.GLA_ERR_INVALID_ARG


def test_gate_pointer_must_match_kind(lib):
    assert fwd_status(lib, desc(gate_kind=gla.GATE_NONE, log_alpha=A)) == gla.GLA_ERR_INVALID_ARG
    assert status(lib, desc(gate_kind=gla.GATE_NONE, log_alpha=None))[0] == gla.GLA_OK


def test_size_overflow_rejected(lib):
    assert status(lib, desc(B=1 << 20, H=1 << 10, L=1 << 20))[0] == gla.GLA_ERR_INVALID_ARG
    assert status(lib, desc(B=2 ** 31 - 1, H=2 ** 31 - 1))[0] == gla.GLA_ERR_INVALID_ARG


def test_null_descriptor_and_outputs(lib):
    assert lib.gla_fwd_ex(None, None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_workspace_size(ctypes.byref(desc()), None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_query_plan(ctypes.byref(desc()), None) == gla.GLA_ERR_INVALID_ARG


def test_headline_entry_point_validates(lib):
    # gla_fwd(q, k, v, log_alpha, out, final_state, B, H, L, Dk, Dv, chunk, stream)
    assert lib.gla_fwd(None, A, A, A, A, None, 1, 1, 64, 128, 128, 64, None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_fwd(A, A, A, A, A, None, 1, 1, 0, 128, 128, 64, None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_fwd(A, A, A, A, A + 4, None, 1, 1, 64, 128, 128, 64, None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_fwd(A, A, A, A, A, None, 1, 1, 64, 96, 128, 64, None) == gla.GLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(Dk=96), dict(Dk=32), dict(Dv=96), dict(Dv=32), dict(chunk=32), dict(chunk=96),
                                dict(chunk=1024), dict(Dv=4160), dict(B=1, H=1, L=(1 << 23) - 1024)])
def test_unsupported_shapes(lib, kw):
    d = desc(**kw)
    assert status(lib, d)[0] == gla.GLA_ERR_UNSUPPORTED
    assert fwd_status(lib, d) == gla.GLA_ERR_UNSUPPORTED


def test_longest_sequence_of_a_slice(lib):
    # one (batch, head) slice is addressed with 32-bit byte offsets: (L + 1024) * max(Dk, Dv) * 4 < 2^32
    assert status(lib, desc(B=1, H=1, L=(1 << 23) - 1025))[0] == gla.GLA_OK
    assert status(lib, desc(B=1, H=1, L=(1 << 23) - 1024))[0] == gla.GLA_ERR_UNSUPPORTED
    assert status(lib, desc(B=1, H=1, L=(1 << 20) - 1025, Dv=1024))[0] == gla.GLA_OK
    assert status(lib, desc(B=1, H=1, L=(1 << 20) - 1024, Dv=1024))[0] == gla.GLA_ERR_UNSUPPORTED


def test_caller_workspace_too_small(lib):
    d = desc(B=1, H=1, L=8192, seg_chunks=16)
    st, need = status(lib, d)
    assert st == gla.GLA_OK and need > 0
    d.workspace, d.workspace_bytes = A, need - 256
    assert fwd_status(lib, d) == gla.GLA_ERR_WORKSPACE


def test_workspace_size_formula(lib):
    # segments: (B*H) * (nseg - 1) local states of Dk*Dv fp32 plus their Dk decays, 256-byte aligned
    # the state of each segment boundary is a sum of sub-segment states: the state grid
    # (B*H * (nseg-1) * nsub * Dv/64) is brought nearest to 512 workgroups for a per-channel
    # gate (768 for scalar gates), with nsub at most the 64-token tiles per segment
    d = desc(B=2, H=2, L=4096, Dk=128, Dv=64, chunk=64, seg_chunks=16)
    p = gla.plan(d)
    assert p.n_seg == 4 and p.seg_chunks == 16
    nss = p.grid_state // 4
    assert nss == 3 * 16  # 16 tiles per segment, want 64 sub-segments per boundary -> 16
    al = lambda x: (x + 255) // 256 * 256
    assert p.workspace_bytes == al(4 * nss * 128 * 64 * 4) + al(4 * nss * 128 * 4)
    p2 = gla.plan(desc(B=1, H=16, L=32768, Dk=128, Dv=128, chunk=64))
    assert p2.n_seg == 8 and p2.grid_state == 16 * 7 * 2 * 2  # 2 sub-segments of 32 tiles
    p3 = gla.plan(desc(B=4, H=8, L=8192, Dk=128, Dv=128, chunk=128, gate_kind=gla.GATE_HEAD_CONST))
    assert p3.n_seg == 4 and p3.grid_state == 32 * 3 * 4 * 2  # scalar gate: 4 sub-segments of 8 tiles
    assert gla.plan(desc(B=2, H=2, L=4096, seg_chunks=64)).workspace_bytes == 0


@pytest.mark.parametrize("B,H,L,Dv,chunk,expect_seg", [
    (8, 16, 2048, 128, 64, 1),     # enough (batch, head, value-tile) work: one segment
    (4, 8, 8192, 128, 128, 4),     # 64 workgroups -> 4 segments
    (1, 16, 32768, 128, 64, 8),    # 32 workgroups -> 8 segments
    (1, 16, 32768, 128, 256, 8),
    (8, 8, 8192, 512, 256, 1),
    (1, 1, 256, 64, 64, 1),        # tiny: not worth segmenting
])
def test_automatic_segmentation(lib, B, H, L, Dv, chunk, expect_seg):
    big = Dv == 512  # the mLSTM-style workload: per-head gate, Dk = 256
    p = gla.plan(desc(B=B, H=H, L=L, Dv=Dv, chunk=chunk, Dk=256 if big else 128,
                      gate_kind=gla.GATE_HEAD if big else gla.GATE_CHANNEL))
    assert p.n_seg == expect_seg
    assert p.tiles_per_chunk == chunk // 64


def test_lds_limit_reported_as_unsupported(lib):
    # the tile-pair form keeps a whole chunk's query tiles in LDS: fp32 operands with a
    # per-channel gate (Dk = 128) or Dk = 256 need more than the 160 KB of a compute unit
    TP = gla.FLAG_TILE_PAIRS
    assert status(lib, desc(Dk=128, chunk=128, in_dtype=gla.DTYPE_F32, flags=TP))[0] == gla.GLA_ERR_UNSUPPORTED
    assert status(lib, desc(Dk=256, chunk=128, in_dtype=gla.DTYPE_F32, gate_kind=gla.GATE_HEAD, flags=TP))[0] == \
        gla.GLA_ERR_UNSUPPORTED
    assert status(lib, desc(Dk=128, chunk=128, in_dtype=gla.DTYPE_F32, gate_kind=gla.GATE_HEAD, flags=TP))[0] == \
        gla.GLA_OK
    # the same shapes without tile pairs walk 64-token tiles and fit
    assert status(lib, desc(Dk=128, chunk=128, in_dtype=gla.DTYPE_F32))[0] == gla.GLA_OK
    assert status(lib, desc(Dk=256, chunk=512, in_dtype=gla.DTYPE_F32))[0] == gla.GLA_OK
    assert status(lib, desc(Dk=128, chunk=64, in_dtype=gla.DTYPE_F32, flags=TP))[0] == gla.GLA_OK
    assert status(lib, desc(Dk=256, chunk=64, in_dtype=gla.DTYPE_F32, flags=TP))[0] == gla.GLA_OK
    for f in (0, TP):
        assert status(lib, desc(Dk=128, chunk=512, flags=f))[0] == gla.GLA_OK
        assert status(lib, desc(Dk=256, chunk=512, flags=f))[0] == gla.GLA_OK


def test_tile_pair_flag_in_plan(lib):
    for chunk in (64, 128, 256, 512):
        p0 = gla.plan(desc(chunk=chunk))
        p1 = gla.plan(desc(chunk=chunk, flags=gla.FLAG_TILE_PAIRS))
        assert p0.tiles_per_chunk == p1.tiles_per_chunk == chunk // 64
        assert p0.tile_pairs == 0 and p1.tile_pairs == (1 if chunk > 64 else 0)
        assert p0.workspace_bytes == 0
        # per-channel gate, tile pairs: keys of the earlier tiles of a chunk go to scratch
        assert p1.workspace_bytes == (0 if chunk == 64 else
                                      (p1.grid_out * (chunk // 64 - 1) * 64 * 128 * 2 + 255) // 256 * 256)


def step_desc(**kw):
    d = gla.GlaStepDesc()
    base = dict(B=2, H=3, Dk=128, Dv=128, in_dtype=gla.DTYPE_BF16, gate_kind=gla.GATE_CHANNEL, q=A, k=A, v=A,
                log_alpha=A, log_ig=None, state=A, out=A)
    base.update(kw)
    for key, val in base.items():
        setattr(d, key, val)
    return d


@pytest.mark.parametrize("field,bad", [("B", 0), ("H", -1), ("Dk", 0), ("Dv", 0), ("in_dtype", 7), ("gate_kind", 9),
                                       ("q", None), ("state", None), ("out", None), ("v", A + 8)])
def test_step_invalid_arguments(lib, field, bad):
    assert lib.gla_step(ctypes.byref(step_desc(**{field: bad})), None) == gla.GLA_ERR_INVALID_ARG


def test_step_gate_pointer_must_match_kind(lib):
    assert lib.gla_step(ctypes.byref(step_desc(gate_kind=gla.GATE_NONE)), None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_step(ctypes.byref(step_desc(log_alpha=None)), None) == gla.GLA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(Dv=96), dict(Dv=4160), dict(Dk=4097)])
def test_step_unsupported(lib, kw):
    assert lib.gla_step(ctypes.byref(step_desc(**kw)), None) == gla.GLA_ERR_UNSUPPORTED


# ------------------------------------------------------------------------------ backward
def bdesc(**kw):
    d = gla.GlaBwdDesc()
    base = dict(B=2, H=3, L=100, Dk=128, Dv=128, in_dtype=gla.DTYPE_BF16, gate_kind=gla.GATE_HEAD, q=A, k=A, v=A,
                log_alpha=A, log_ig=None, initial_state=None, dout=A, dfinal_state=None, dq=A, dk=A, dv=A,
                dlog_alpha=A, dlog_ig=None, dinitial_state=None, workspace=None, workspace_bytes=0)
    base.update(kw)
    for key, val in base.items():
        setattr(d, key, val)
    return d


def bstatus(lib, d):
    n = ctypes.c_size_t(0)
    return lib.gla_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)), n.value


def test_bwd_valid_and_workspace_grows_with_length(lib):
    st, n1 = bstatus(lib, bdesc())
    assert st == gla.GLA_OK and n1 > 0
    st, n2 = bstatus(lib, bdesc(L=1000))
    assert st == gla.GLA_OK and n2 > n1
    for kind, la in ((gla.GATE_NONE, None), (gla.GATE_HEAD_CONST, A), (gla.GATE_CHANNEL, A)):
        st, _ = bstatus(lib, bdesc(gate_kind=kind, log_alpha=la, dlog_alpha=la))
        assert st == gla.GLA_OK
    # the per-channel path's scratch grows with the length too (the log-gate scan rows)
    st, c1 = bstatus(lib, bdesc(gate_kind=gla.GATE_CHANNEL))
    st2, c2 = bstatus(lib, bdesc(gate_kind=gla.GATE_CHANNEL, L=1000))
    assert st == st2 == gla.GLA_OK and c2 > c1


@pytest.mark.parametrize("kw", [dict(dq=None), dict(dout=None), dict(q=None), dict(L=0), dict(dq=A + 4),
                                dict(gate_kind=gla.GATE_NONE, log_alpha=None),  # dlog_alpha without a gate
                                dict(dlog_ig=A),                                  # input-gate grad without one
                                dict(gate_kind=9), dict(in_dtype=7)])
def test_bwd_invalid_arguments(lib, kw):
    assert bstatus(lib, bdesc(**kw))[0] == gla.GLA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(Dk=100), dict(Dv=512), dict(Dk=32), dict(gate_kind=gla.GATE_CHANNEL, Dv=96),
                                dict(B=1, H=1, L=1 << 22, Dk=256),  # a slice past 32-bit byte offsets
                                dict(B=1, H=1, L=1 << 22, Dk=256, gate_kind=gla.GATE_CHANNEL)])
def test_bwd_unsupported(lib, kw):
    assert bstatus(lib, bdesc(**kw))[0] == gla.GLA_ERR_UNSUPPORTED


def test_bwd_rejects_small_workspace_before_launching(lib):
    st, need = bstatus(lib, bdesc())
    d = bdesc(workspace=A, workspace_bytes=need - 256)
    assert lib.gla_bwd(ctypes.byref(d), None) == gla.GLA_ERR_WORKSPACE
