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
    ("B", -1), ("H", -1), ("L", -1), ("Dk", 0), ("Dv", 0), ("chunk", 0), ("seg_chunks", -1), ("flags", 4), ("flags", -1),
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
    assert lib.gla_fwd(A, A, A, A, A, None, 1, 1, -1, 128, 128, 64, None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_fwd(A, A, A, A, A + 4, None, 1, 1, 64, 128, 128, 64, None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_fwd(A, A, A, A, A, None, 1, 1, 64, 24, 128, 64, None) == gla.GLA_ERR_UNSUPPORTED
    assert lib.gla_fwd(A, A, A, A, A, None, 1, 1, 64, 272, 128, 64, None) == gla.GLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(Dk=24), dict(Dk=272), dict(Dk=8), dict(Dv=40), dict(Dv=8), dict(chunk=48),
                                dict(chunk=96), dict(chunk=1024), dict(Dv=4160), dict(Dv=4112),
                                dict(B=1, H=1, L=(1 << 23) - 1024)])
def test_unsupported_shapes(lib, kw):
    d = desc(**kw)
    assert status(lib, d)[0] == gla.GLA_ERR_UNSUPPORTED
    assert fwd_status(lib, d) == gla.GLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("Dk,Dv,gate,s0,fin", [(96, 128, gla.GATE_CHANNEL, False, False), (128, 96, gla.GATE_CHANNEL, True, True),
                                             (16, 48, gla.GATE_HEAD, True, False), (240, 272, gla.GATE_NONE, False, True),
                                             (160, 64, gla.GATE_HEAD_CONST, False, False)])
def test_padded_shapes_plan(lib, Dk, Dv, gate, s0, fin):
    # Dk a multiple of 16 up to 256 and Dv a multiple of 16 run on zero-padded copies: q and
    # k (and a per-channel gate) to the next Dk in {64, 128, 256}, v and the output to the
    # next multiple of 64, the states to both; the workspace holds the copies (256-byte
    # aligned) followed by the padded call's own workspace
    B, H, L = 2, 3, 100
    kw = dict(B=B, H=H, L=L, Dk=Dk, Dv=Dv, gate_kind=gate, log_alpha=None if gate == gla.GATE_NONE else A,
              initial_state=A if s0 else None, final_state=A if fin else None)
    st, n = status(lib, desc(**kw))
    assert st == gla.GLA_OK
    dkp = 64 if Dk <= 64 else (128 if Dk <= 128 else 256)
    dvp = -(-Dv // 64) * 64
    al = lambda x: (x + 255) // 256 * 256
    bhl, bh = B * H * L, B * H
    inner = gla.workspace_size(desc(**dict(kw, Dk=dkp, Dv=dvp)))
    want = 0
    if dkp != Dk:
        want += 2 * al(bhl * dkp * 2) + (al(bhl * dkp * 4) if gate == gla.GATE_CHANNEL else 0)
    if dvp != Dv:
        want += al(bhl * dvp * 2)
    want += (al(bh * dkp * dvp * 4) if s0 else 0) + (al(bhl * dvp * 4) if dvp != Dv else 0)
    want += (al(bh * dkp * dvp * 4) if fin else 0) + al(inner)
    assert n == want
    p = gla.plan(desc(**kw))
    assert p.dv_tiles == dvp // 64 and p.workspace_bytes == n


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
    (1, 1, 1024, 128, 64, 1),      # a walk of 16 tiles stays one segment
    (1, 1, 1088, 128, 64, 17),     # 17 tiles on 2 workgroups: one tile per segment
    (1, 1, 65536, 128, 64, 128),   # short batch, long sequence: 128 segments fill the grid
    (2, 2, 2048, 128, 64, 32),
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


def test_query_tile_flag_in_plan(lib):
    # one workgroup per (batch, head, chunk, query tile, value tile); every chunk is its own
    # segment, whose start state the segment-state kernel and scan materialise
    QT = gla.FLAG_QUERY_TILES
    B, H, L, Dk, Dv = 2, 3, 4096 + 100, 128, 128
    for chunk in (64, 128, 256, 512):
        nc = -(-L // chunk)
        nt = chunk // 64
        for gate in (gla.GATE_CHANNEL, gla.GATE_HEAD):
            p = gla.plan(desc(B=B, H=H, L=L, Dk=Dk, Dv=Dv, chunk=chunk, gate_kind=gate, flags=QT))
            assert p.seg_chunks == 1 and p.n_seg == nc and p.tiles_per_chunk == nt
            assert p.tile_pairs == (1 if nt > 1 else 0) and p.query_tiles == (1 if nt > 1 else 0)
            assert p.grid_out == B * H * nc * (Dv // 64) * nt
            # chunk states: (nc - 1) boundaries, one sub-segment each at this size
            nss = p.grid_state // (B * H * (Dv // 64))
            al = lambda x: (x + 255) // 256 * 256
            ke = al(B * H * nc * (nt - 1) * 64 * Dk * 2) if gate == gla.GATE_CHANNEL else 0
            assert p.workspace_bytes == al(B * H * nss * Dk * Dv * 4) + al(B * H * nss * Dk * 4) + ke
    # seg_chunks other than 0 or 1 contradicts one chunk per segment
    assert status(lib, desc(chunk=128, flags=QT, seg_chunks=2))[0] == gla.GLA_ERR_INVALID_ARG
    assert status(lib, desc(chunk=128, flags=QT, seg_chunks=1))[0] == gla.GLA_OK
    assert status(lib, desc(chunk=128, flags=QT | gla.FLAG_TILE_PAIRS))[0] == gla.GLA_OK
    # the tile-pair LDS limit applies unchanged
    assert status(lib, desc(Dk=128, chunk=128, in_dtype=gla.DTYPE_F32, flags=QT))[0] == gla.GLA_ERR_UNSUPPORTED


def step_desc(**kw):
    d = gla.GlaStepDesc()
    base = dict(B=2, H=3, Dk=128, Dv=128, in_dtype=gla.DTYPE_BF16, gate_kind=gla.GATE_CHANNEL, q=A, k=A, v=A,
                log_alpha=A, log_ig=None, state=A, out=A)
    base.update(kw)
    for key, val in base.items():
        setattr(d, key, val)
    return d


@pytest.mark.parametrize("field,bad", [("B", -1), ("H", -1), ("Dk", 0), ("Dv", 0), ("in_dtype", 7), ("gate_kind", 9),
                                       ("q", None), ("state", None), ("out", None), ("v", A + 8)])
def test_step_invalid_arguments(lib, field, bad):
    assert lib.gla_step(ctypes.byref(step_desc(**{field: bad})), None) == gla.GLA_ERR_INVALID_ARG


def test_step_gate_pointer_must_match_kind(lib):
    assert lib.gla_step(ctypes.byref(step_desc(gate_kind=gla.GATE_NONE)), None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_step(ctypes.byref(step_desc(log_alpha=None)), None) == gla.GLA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(Dv=40), dict(Dv=4160), dict(Dk=4097)])
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


@pytest.mark.parametrize("kw", [dict(dq=None), dict(dout=None), dict(q=None), dict(L=-1), dict(dq=A + 4),
                                dict(gate_kind=gla.GATE_NONE, log_alpha=None),  # dlog_alpha without a gate
                                dict(dlog_ig=A),                                  # input-gate grad without one
                                dict(gate_kind=9), dict(in_dtype=7)])
def test_bwd_invalid_arguments(lib, kw):
    assert bstatus(lib, bdesc(**kw))[0] == gla.GLA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(Dk=100), dict(Dv=1024), dict(Dv=512, in_dtype=gla.DTYPE_F32), dict(Dk=32),
                                dict(gate_kind=gla.GATE_CHANNEL, Dv=96),
                                dict(B=1, H=1, L=1 << 22, Dk=256),  # a slice past 32-bit byte offsets
                                dict(B=1, H=1, L=1 << 22, Dk=256, gate_kind=gla.GATE_CHANNEL)])
def test_bwd_unsupported(lib, kw):
    assert bstatus(lib, bdesc(**kw))[0] == gla.GLA_ERR_UNSUPPORTED


def test_bwd_rejects_small_workspace_before_launching(lib):
    st, need = bstatus(lib, bdesc())
    d = bdesc(workspace=A, workspace_bytes=need - 256)
    assert lib.gla_bwd(ctypes.byref(d), None) == gla.GLA_ERR_WORKSPACE


# ------------------------------------------------------------------------------ binding shape checks
def _cpu_fwd_args(B=2, H=3, L=10, Dk=64, Dv=64):
    import torch

    f = torch.float32
    return dict(q=torch.zeros(B, H, L, Dk, dtype=torch.bfloat16), k=torch.zeros(B, H, L, Dk, dtype=torch.bfloat16),
                v=torch.zeros(B, H, L, Dv, dtype=torch.bfloat16), log_alpha=torch.zeros(B, H, L, Dk, dtype=f),
                log_ig=torch.zeros(B, H, L, dtype=f), initial_state=torch.zeros(B, H, Dk, Dv, dtype=f),
                out=torch.zeros(B, H, L, Dv, dtype=f))


@pytest.mark.parametrize("name,shape", [("k", (2, 3, 9, 64)), ("k", (2, 3, 10, 32)), ("v", (2, 3, 9, 64)),
                                        ("log_alpha", (2, 3, 10, 32)), ("log_alpha", (2, 3, 9)),
                                        ("log_ig", (2, 3, 9)), ("initial_state", (2, 3, 64, 32)),
                                        ("out", (2, 3, 10, 32))])
def test_fwd_rejects_mismatched_shapes_before_device_work(lib, name, shape):
    # the kernels size their memory ranges from q and v: any other tensor of the wrong shape
    # is refused on the host (these CPU tensors would otherwise fail the device check later)
    import torch

    a = _cpu_fwd_args()
    a[name] = torch.zeros(shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=name if name != "log_alpha" else "log_alpha"):
        gla.fwd(a["q"], a["k"], a["v"], a["log_alpha"], log_ig=a["log_ig"], initial_state=a["initial_state"],
                out=a["out"])


@pytest.mark.parametrize("name,shape", [("dout", (2, 3, 9, 64)), ("dfinal_state", (2, 3, 64, 63)),
                                        ("k", (1, 3, 10, 64)), ("log_ig", (2, 3, 11))])
def test_bwd_rejects_mismatched_shapes_before_device_work(lib, name, shape):
    import torch

    a = _cpu_fwd_args()
    a["dout"] = torch.zeros(2, 3, 10, 64)
    a["dfinal_state"] = torch.zeros(2, 3, 64, 64)
    a[name] = torch.zeros(shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=name):
        gla.bwd(a["q"], a["k"], a["v"], a["dout"], a["log_alpha"], log_ig=a["log_ig"],
                initial_state=a["initial_state"], dfinal_state=a["dfinal_state"])


@pytest.mark.parametrize("name,shape", [("k", (2, 3, 32)), ("state", (2, 3, 64, 32)), ("out", (2, 3, 32)),
                                        ("log_ig", (2, 2)), ("log_alpha", (2, 3, 63))])
def test_step_rejects_mismatched_shapes_before_device_work(lib, name, shape):
    import torch

    f = torch.float32
    a = dict(q=torch.zeros(2, 3, 64), k=torch.zeros(2, 3, 64), v=torch.zeros(2, 3, 64),
             state=torch.zeros(2, 3, 64, 64), out=torch.zeros(2, 3, 64), log_ig=torch.zeros(2, 3),
             log_alpha=torch.zeros(2, 3, 64, dtype=f))
    a[name] = torch.zeros(shape, dtype=f)
    with pytest.raises(ValueError, match=name if name != "log_alpha" else "log_alpha"):
        gla.step(a["q"], a["k"], a["v"], a["state"], a["log_alpha"], log_ig=a["log_ig"], out=a["out"])


def test_headline_binding_rejects_mismatched_shapes(lib):
    import torch

    a = _cpu_fwd_args()
    with pytest.raises(ValueError, match="out"):
        gla.fwd_headline(a["q"], a["k"], a["v"], a["log_alpha"], torch.zeros(2, 3, 10, 32), None)


def test_noalloc_rejects_caller_workspace_and_oversized_scratch(lib):
    # gla_fwd_noalloc takes its scratch from the library's fixed per-GPU array: a caller
    # workspace is an invalid argument, and a call whose scratch exceeds the array is refused
    # before any HIP call
    d = desc(workspace=A, workspace_bytes=1 << 20)
    assert lib.gla_fwd_noalloc(ctypes.byref(d), None) == gla.GLA_ERR_INVALID_ARG
    big = desc(B=1, H=16, L=1 << 18, seg_chunks=1)  # one boundary state per 64-token chunk
    need = gla.workspace_size(big)
    assert need > gla.NOALLOC_SCRATCH_BYTES
    assert lib.gla_fwd_noalloc(ctypes.byref(big), None) == gla.GLA_ERR_WORKSPACE
    # validation errors come first, as for gla_fwd_ex
    assert lib.gla_fwd_noalloc(ctypes.byref(desc(q=None)), None) == gla.GLA_ERR_INVALID_ARG
    assert lib.gla_fwd_noalloc(ctypes.byref(desc(Dk=24)), None) == gla.GLA_ERR_UNSUPPORTED
    # a shape run on padded copies whose copies exceed the scratch
    assert lib.gla_fwd_noalloc(ctypes.byref(desc(B=8, H=16, L=2048, Dk=96)), None) == gla.GLA_ERR_WORKSPACE
    assert lib.gla_fwd_noalloc(None, None) == gla.GLA_ERR_INVALID_ARG


def test_noalloc_scratch_limit_matches_header():
    hdr = open(HEADER).read()
    m = re.search(r"#define GLA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == gla.NOALLOC_SCRATCH_BYTES


def delta_desc(**kw):
    d = gla.GlaDeltaDesc()
    base = dict(B=2, H=3, L=100, Dk=128, Dv=128, chunk=64, in_dtype=gla.DTYPE_BF16, gate_kind=gla.GATE_HEAD,
                q=A, k=A, v=A, beta=A, log_alpha=A, initial_state=None, out=A, final_state=None)
    base.update(kw)
    for key, val in base.items():
        setattr(d, key, val)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), gla.GLA_ERR_INVALID_ARG), (dict(beta=None), gla.GLA_ERR_INVALID_ARG),
    (dict(out=None), gla.GLA_ERR_INVALID_ARG), (dict(L=-1), gla.GLA_ERR_INVALID_ARG),
    (dict(gate_kind=gla.GATE_NONE), gla.GLA_ERR_INVALID_ARG),  # gate pointer given without a gate
    (dict(log_alpha=None), gla.GLA_ERR_INVALID_ARG),  # gate kind without a pointer
    (dict(beta=A + 4), gla.GLA_ERR_INVALID_ARG), (dict(in_dtype=7), gla.GLA_ERR_INVALID_ARG),
    (dict(gate_kind=gla.GATE_CHANNEL), gla.GLA_ERR_UNSUPPORTED), (dict(chunk=128), gla.GLA_ERR_UNSUPPORTED),
    (dict(Dk=96), gla.GLA_ERR_UNSUPPORTED), (dict(Dv=96), gla.GLA_ERR_UNSUPPORTED),
    (dict(in_dtype=gla.DTYPE_F32, Dk=128), gla.GLA_ERR_UNSUPPORTED),
])
def test_delta_validation_before_any_hip_call(lib, kw, status):
    assert lib.gla_delta_fwd(ctypes.byref(delta_desc(**kw)), None) == status
    assert lib.gla_delta_fwd(None, None) == gla.GLA_ERR_INVALID_ARG


@pytest.mark.parametrize("name,shape", [("k", (2, 3, 9, 64)), ("beta", (2, 3, 9)), ("log_alpha", (2, 3, 10, 64)),
                                        ("initial_state", (2, 3, 64, 32))])
def test_delta_binding_rejects_mismatched_shapes(lib, name, shape):
    import torch

    a = dict(q=torch.zeros(2, 3, 10, 64), k=torch.zeros(2, 3, 10, 64), v=torch.zeros(2, 3, 10, 64),
             beta=torch.zeros(2, 3, 10), log_alpha=torch.zeros(2, 3, 10), initial_state=torch.zeros(2, 3, 64, 64))
    a[name] = torch.zeros(shape)
    with pytest.raises(ValueError, match=name):
        gla.delta_fwd(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"], initial_state=a["initial_state"])


def mlstm_desc(**kw):
    d = gla.GlaMlstmDesc()
    base = dict(B=2, H=3, L=100, Dk=128, Dv=128, chunk=64, in_dtype=gla.DTYPE_BF16, reserved=0,
                q=A, k=A, v=A, log_f=A, log_i=A, initial_C=None, initial_n=None, initial_m=None, out=A,
                final_C=None, final_n=None, final_m=None)
    base.update(kw)
    for key, val in base.items():
        setattr(d, key, val)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), gla.GLA_ERR_INVALID_ARG), (dict(log_f=None), gla.GLA_ERR_INVALID_ARG),
    (dict(log_i=None), gla.GLA_ERR_INVALID_ARG), (dict(out=None), gla.GLA_ERR_INVALID_ARG),
    (dict(L=-1), gla.GLA_ERR_INVALID_ARG), (dict(Dv=-64), gla.GLA_ERR_INVALID_ARG),
    (dict(reserved=1), gla.GLA_ERR_INVALID_ARG), (dict(in_dtype=7), gla.GLA_ERR_INVALID_ARG),
    (dict(initial_C=A), gla.GLA_ERR_INVALID_ARG),  # an initial state given in part
    (dict(initial_C=A, initial_n=A), gla.GLA_ERR_INVALID_ARG),
    (dict(log_i=A + 4), gla.GLA_ERR_INVALID_ARG), (dict(final_m=A + 8), gla.GLA_ERR_INVALID_ARG),
    (dict(chunk=128), gla.GLA_ERR_UNSUPPORTED), (dict(chunk=32), gla.GLA_ERR_UNSUPPORTED),
    (dict(Dk=96), gla.GLA_ERR_UNSUPPORTED), (dict(Dv=96), gla.GLA_ERR_UNSUPPORTED),
    (dict(Dv=8192), gla.GLA_ERR_UNSUPPORTED), (dict(in_dtype=gla.DTYPE_F32, Dk=128), gla.GLA_ERR_UNSUPPORTED),
])
def test_mlstm_validation_before_any_hip_call(lib, kw, status):
    assert lib.gla_mlstm_fwd(ctypes.byref(mlstm_desc(**kw)), None) == status
    assert lib.gla_mlstm_fwd(None, None) == gla.GLA_ERR_INVALID_ARG


@pytest.mark.parametrize("name,shape", [("k", (2, 3, 9, 64)), ("log_f", (2, 3, 9)), ("log_i", (2, 3, 10, 1)),
                                        ("out", (2, 3, 10, 32))])
def test_mlstm_binding_rejects_mismatched_shapes(lib, name, shape):
    import torch

    a = dict(q=torch.zeros(2, 3, 10, 64), k=torch.zeros(2, 3, 10, 64), v=torch.zeros(2, 3, 10, 64),
             log_f=torch.zeros(2, 3, 10), log_i=torch.zeros(2, 3, 10), out=None)
    a[name] = torch.zeros(shape)
    with pytest.raises(ValueError, match=name):
        gla.mlstm_fwd(a["q"], a["k"], a["v"], a["log_f"], a["log_i"], out=a["out"])


@pytest.mark.parametrize("which,shape", [(0, (2, 3, 64, 32)), (1, (2, 3, 32)), (2, (2, 3, 1))])
def test_mlstm_binding_rejects_mismatched_initial_state(lib, which, shape):
    import torch

    init = [torch.zeros(2, 3, 64, 64), torch.zeros(2, 3, 64), torch.zeros(2, 3)]
    init[which] = torch.zeros(shape)
    z = torch.zeros(2, 3, 10, 64)
    with pytest.raises(ValueError, match="initial"):
        gla.mlstm_fwd(z, z, z, torch.zeros(2, 3, 10), torch.zeros(2, 3, 10), initial_state=tuple(init))


def test_mlstm_desc_layout_matches_header():
    # the ctypes mirror of gla_mlstm_desc: eight int32 fields, then twelve pointers
    assert ctypes.sizeof(gla.GlaMlstmDesc) == 8 * 4 + 12 * 8
    assert gla.GlaMlstmDesc.q.offset == 32


@pytest.mark.parametrize("chunk", [16, 32])
def test_small_chunks_run_as_64_token_tiles(lib, chunk):
    # chunks of 16 and 32 tokens are accepted and planned as 64-token tiles (the same map)
    p = gla.plan(desc(chunk=chunk, L=1000))
    q = gla.plan(desc(chunk=64, L=1000))
    assert (p.tiles_per_chunk, p.n_seg, p.grid_out) == (1, q.n_seg, q.grid_out)
    assert p.tiles_per_chunk == 1


def bwd_desc(**kw):
    d = gla.GlaBwdDesc()
    base = dict(B=2, H=3, L=100, Dk=256, Dv=512, in_dtype=gla.DTYPE_BF16, gate_kind=gla.GATE_HEAD, q=A, k=A, v=A,
                log_alpha=A, log_ig=A, initial_state=None, dout=A, dfinal_state=A, dq=A, dk=A, dv=A,
                dlog_alpha=A, dlog_ig=A, dinitial_state=A, workspace=None, workspace_bytes=0)
    base.update(kw)
    for key, val in base.items():
        setattr(d, key, val)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(), gla.GLA_OK), (dict(gate_kind=gla.GATE_NONE, log_alpha=None, dlog_alpha=None), gla.GLA_OK),
    (dict(gate_kind=gla.GATE_HEAD_CONST), gla.GLA_OK), (dict(Dk=64), gla.GLA_OK),
    (dict(in_dtype=gla.DTYPE_F32), gla.GLA_ERR_UNSUPPORTED), (dict(gate_kind=gla.GATE_CHANNEL), gla.GLA_ERR_UNSUPPORTED),
    (dict(Dv=1024), gla.GLA_ERR_UNSUPPORTED), (dict(Dv=384), gla.GLA_ERR_UNSUPPORTED),
])
def test_backward_dv512_support(lib, kw, status):
    # Dv = 512 is supported for bf16 inputs with a scalar gate or none (value-column halves)
    n = ctypes.c_size_t(0)
    assert lib.gla_bwd_workspace_size(ctypes.byref(bwd_desc(**kw)), ctypes.byref(n)) == status
    if status == gla.GLA_OK:
        assert n.value > 0


# ------------------------------------------------------------------------------ empty calls
# B, H or L of zero: no output rows, and the state after no tokens is the state before them.
# Without a final state to write, an empty call does no device work at all, so it runs here.
@pytest.mark.parametrize("kw", [dict(L=0), dict(B=0), dict(H=0), dict(B=0, L=0)])
def test_empty_calls_plan_nothing(lib, kw):
    d = desc(q=None, k=None, v=None, out=None, log_alpha=None, **kw)  # per-token arrays may be NULL
    st, n = status(lib, d)
    assert st == gla.GLA_OK and n == 0
    p = gla.plan(d)
    assert p.n_seg == 0 and p.grid_out == 0 and p.grid_state == 0 and p.workspace_bytes == 0
    assert fwd_status(lib, d) == gla.GLA_OK
    assert lib.gla_fwd_noalloc(ctypes.byref(d), None) == gla.GLA_OK
    assert lib.gla_fwd(None, None, None, None, None, None, 1, 1, 0, 128, 128, 64, None) == gla.GLA_OK


def test_empty_calls_keep_the_support_matrix_and_argument_checks(lib):
    assert status(lib, desc(L=0, Dk=24))[0] == gla.GLA_ERR_UNSUPPORTED
    assert status(lib, desc(L=0, chunk=48))[0] == gla.GLA_ERR_UNSUPPORTED
    assert status(lib, desc(L=0, in_dtype=7))[0] == gla.GLA_ERR_INVALID_ARG
    assert status(lib, desc(L=0, final_state=A + 4))[0] == gla.GLA_ERR_INVALID_ARG


def test_empty_step_delta_mlstm_backward(lib):
    sd = step_desc(B=0, q=None, k=None, v=None, state=None, out=None)
    assert lib.gla_step(ctypes.byref(sd), None) == gla.GLA_OK
    assert lib.gla_delta_fwd(ctypes.byref(delta_desc(L=0, q=None, k=None, v=None, beta=None, out=None)),
                             None) == gla.GLA_OK
    assert lib.gla_delta_fwd(ctypes.byref(delta_desc(L=0, Dk=96)), None) == gla.GLA_ERR_UNSUPPORTED
    assert lib.gla_mlstm_fwd(ctypes.byref(mlstm_desc(L=0, q=None, k=None, v=None, log_f=None, log_i=None,
                                                     out=None)), None) == gla.GLA_OK
    bd = bdesc(L=0, q=None, k=None, v=None, dout=None, dq=None, dk=None, dv=None, dlog_alpha=None)
    st, n = bstatus(lib, bd)
    assert st == gla.GLA_OK and n == 0
    assert lib.gla_bwd(ctypes.byref(bd), None) == gla.GLA_OK
