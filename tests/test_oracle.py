"""Pins for the fp64 oracle (CPU only).

The pages print no worked example, so the oracle is pinned to things other than itself:
hand-derived values (tests/golden), closed forms, special cases that reduce to textbook
sums, the equivalence of the recurrent, quadratic and chunkwise forms that the pages state
[talk summary, 7:36 and 11:58; Tiled Flash Linear Attention abstract: any chunk size], and
invariants (linearity, head independence, segment consistency).  The last test plants
plausible mistakes in copies of the C source and checks that the pins catch each one.
"""
import json
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from gated_linear_rnn_chunkwise_amd import inputs as gin

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(1234)


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    scale = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def small(B=1, H=2, L=13, Dk=5, Dv=3, gate="channel", input_gate=False, seed=0):
    w = gin.custom(B, H, L, Dk, Dv, 4, dtype="f32", gate=gate, input_gate=input_gate, channel_gate_div=2.0)
    return gin.make_inputs(w, seed=seed)


def _golden_case(case, lib=None):
    q = np.array(case["q"], dtype=np.float64)[None, None]
    k = np.array(case["k"], dtype=np.float64)[None, None]
    v = np.array(case["v"], dtype=np.float64)[None, None]
    la = np.log(np.array(case["alpha"], dtype=np.float64))[None, None]
    li = None if case["input_gate"] is None else np.log(np.array(case["input_gate"], dtype=np.float64))[None, None]
    return oracle.recurrent(q, k, v, "channel", la, li, lib=lib)


def test_golden_hand_worked():
    with open(os.path.join(HERE, "golden", "hand_worked_small.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        out, fin = _golden_case(case)
        np.testing.assert_allclose(out[0, 0], np.array(case["out"]), rtol=0, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(fin[0, 0], np.array(case["final_state"]), rtol=0, atol=1e-14,
                                   err_msg=case["name"])


@pytest.mark.parametrize("alpha", [0.5, 0.9, 0.999])
def test_geometric_closed_form(alpha):
    # Dk = Dv = 1, q = k = v = 1, constant alpha: o_t = sum_{s<=t} alpha^(t-s) = (1 - alpha^(t+1)) / (1 - alpha)
    L = 50
    ones = np.ones((1, 1, L, 1))
    la = np.full((1, 1, L, 1), math.log(alpha))
    out, fin = oracle.recurrent(ones, ones, ones, "channel", la)
    t = np.arange(L)
    ref = (1 - alpha ** (t + 1)) / (1 - alpha)
    np.testing.assert_allclose(out[0, 0, :, 0], ref, rtol=1e-13)
    np.testing.assert_allclose(fin[0, 0, 0, 0], ref[-1], rtol=1e-13)


def test_per_channel_closed_form_distinct_channels():
    # q = k = 1 over two channels with different constant decays, v = 1:
    # o_t = sum_d (1 - a_d^(t+1)) / (1 - a_d); a wrong channel index mixes the two decays.
    L, a = 40, np.array([0.3, 0.8])
    ones_k = np.ones((1, 1, L, 2))
    v = np.ones((1, 1, L, 1))
    la = np.broadcast_to(np.log(a), (1, 1, L, 2)).copy()
    out, _ = oracle.recurrent(ones_k, ones_k, v, "channel", la)
    t = np.arange(L)[:, None]
    ref = ((1 - a[None] ** (t + 1)) / (1 - a[None])).sum(1)
    np.testing.assert_allclose(out[0, 0, :, 0], ref, rtol=1e-13)
    # q selecting one channel at a time recovers each geometric series separately
    q = np.zeros((1, 1, L, 2))
    q[..., 1] = 1.0
    out1, _ = oracle.recurrent(q, ones_k, v, "channel", la)
    np.testing.assert_allclose(out1[0, 0, :, 0], ((1 - a[1] ** (t[:, 0] + 1)) / (1 - a[1])), rtol=1e-13)


@pytest.mark.parametrize("gate", ["none", "channel", "head", "head_const"])
def test_ungated_limit_and_bruteforce(gate):
    d = small(gate=gate)
    if gate == "none":
        out, _ = oracle.recurrent(d["q"], d["k"], d["v"])
        ref = oracle.bruteforce_ungated(d["q"], d["k"], d["v"])
        assert rel(out, ref) < 1e-13
    else:
        # a zero log-gate of any kind is the ungated map
        zero = torch.zeros_like(d["log_alpha"])
        out, _ = oracle.recurrent(d["q"], d["k"], d["v"], gate, zero)
        ref = oracle.bruteforce_ungated(d["q"], d["k"], d["v"])
        assert rel(out, ref) < 1e-13


def test_alpha_zero_keeps_only_current_token():
    d = small(gate="channel", input_gate=True)
    B, H, L, Dk = d["q"].shape
    la = np.full((B, H, L, Dk), -np.inf)
    out, fin = oracle.recurrent(d["q"], d["k"], d["v"], "channel", la, d["log_ig"])
    q, k, v = (oracle.oracle._f64(d[x]) for x in "qkv")
    ig = np.exp(oracle.oracle._f64(d["log_ig"]))
    ref = np.einsum("bhtd,bhtd->bht", q, k)[..., None] * ig[..., None] * v
    assert rel(out, ref) < 1e-14
    ref_fin = np.einsum("bhd,bhc->bhdc", k[:, :, -1] * ig[:, :, -1:], v[:, :, -1])
    assert rel(fin, ref_fin) < 1e-14


def test_single_token():
    d = small(L=1, gate="head", input_gate=True)
    out, fin = oracle.recurrent(d["q"], d["k"], d["v"], "head", d["log_alpha"], d["log_ig"])
    q, k, v = (oracle.oracle._f64(d[x]) for x in "qkv")
    ig = np.exp(oracle.oracle._f64(d["log_ig"]))
    ref = np.einsum("bhtd,bhtd->bht", q, k)[..., None] * ig[..., None] * v
    assert rel(out, ref) < 1e-14


@pytest.mark.parametrize("gate,input_gate", [("none", False), ("channel", False), ("channel", True),
                                             ("head", True), ("head_const", False)])
def test_recurrent_equals_parallel_form(gate, input_gate):
    d = small(L=29, gate=gate, input_gate=input_gate)
    B, H, L, Dk = d["q"].shape
    s0 = RNG.standard_normal((B, H, Dk, d["v"].shape[-1]))
    for init in (None, s0):
        out, _ = oracle.recurrent(d["q"], d["k"], d["v"], gate, d["log_alpha"], d["log_ig"], init)
        ref = oracle.parallel_form(d["q"], d["k"], d["v"], gate, d["log_alpha"], d["log_ig"], init)
        assert rel(out, ref) < 1e-12


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64, 29])
@pytest.mark.parametrize("gate,input_gate", [("channel", True), ("head", True), ("head_const", False),
                                             ("none", False)])
def test_chunk_size_invariance(chunk, gate, input_gate):
    d = small(L=29, gate=gate, input_gate=input_gate)
    out, fin = oracle.recurrent(d["q"], d["k"], d["v"], gate, d["log_alpha"], d["log_ig"])
    cout, cfin = oracle.chunkwise_form(d["q"], d["k"], d["v"], chunk, gate, d["log_alpha"], d["log_ig"])
    assert rel(cout, out) < 1e-12
    assert rel(cfin, fin) < 1e-12


def test_retnet_decay_mask_with_integer_powers():
    # scalar fixed decay: O = ((Q K^T) o M) V with M_ts = gamma^(t-s) for s <= t (integer powers,
    # no running sums), the textbook RetNet parallel form.
    w = gin.custom(1, 3, 31, 6, 4, 8, dtype="f32", gate="head_const")
    d = gin.make_inputs(w)
    out, _ = oracle.recurrent(d["q"], d["k"], d["v"], "head_const", d["log_alpha"])
    q, k, v = (oracle.oracle._f64(d[x]) for x in "qkv")
    gam = np.exp(oracle.oracle._f64(d["log_alpha"]))
    t = np.arange(w.L)
    for h in range(w.H):
        M = np.where(t[:, None] >= t[None, :], gam[h] ** (t[:, None] - t[None, :]).astype(np.float64), 0.0)
        ref = ((q[0, h] @ k[0, h].T) * M) @ v[0, h]
        assert rel(out[0, h], ref) < 1e-13


def test_final_state_closed_form():
    d = small(L=23, gate="channel", input_gate=True)
    _, fin = oracle.recurrent(d["q"], d["k"], d["v"], "channel", d["log_alpha"], d["log_ig"])
    ref = oracle.final_state_closed_form(d["k"], d["v"], "channel", d["log_alpha"], d["log_ig"])
    assert rel(fin, ref) < 1e-13


def test_linearity_in_v_and_q():
    d = small(L=17, gate="channel")
    v2 = torch.randn(d["v"].shape, generator=torch.Generator().manual_seed(5))
    q2 = torch.randn(d["q"].shape, generator=torch.Generator().manual_seed(6))
    o1, _ = oracle.recurrent(d["q"], d["k"], d["v"], "channel", d["log_alpha"])
    o2, _ = oracle.recurrent(d["q"], d["k"], v2, "channel", d["log_alpha"])
    o12, _ = oracle.recurrent(d["q"], d["k"], 2.0 * d["v"].double() - 3.0 * v2.double(), "channel", d["log_alpha"])
    assert rel(o12, 2.0 * o1 - 3.0 * o2) < 1e-13
    o3, _ = oracle.recurrent(q2, d["k"], d["v"], "channel", d["log_alpha"])
    o13, _ = oracle.recurrent(d["q"].double() + q2.double(), d["k"], d["v"], "channel", d["log_alpha"])
    assert rel(o13, o1 + o3) < 1e-13


def test_heads_and_batches_are_independent():
    d = small(B=2, H=3, L=11, gate="channel", input_gate=True)
    out, fin = oracle.recurrent(d["q"], d["k"], d["v"], "channel", d["log_alpha"], d["log_ig"])
    perm = [2, 0, 1]
    pout, pfin = oracle.recurrent(d["q"][:, perm], d["k"][:, perm], d["v"][:, perm], "channel",
                                  d["log_alpha"][:, perm], d["log_ig"][:, perm])
    assert rel(pout, out[:, perm]) == 0.0 and rel(pfin, fin[:, perm]) == 0.0
    one, _ = oracle.recurrent(d["q"][1:, 1:2], d["k"][1:, 1:2], d["v"][1:, 1:2], "channel",
                              d["log_alpha"][1:, 1:2], d["log_ig"][1:, 1:2])
    assert rel(one, out[1:, 1:2]) == 0.0


def test_segment_consistency():
    # running [0, L1) and then [L1, L) from the first part's final state is one full run
    d = small(L=30, gate="channel", input_gate=True)
    L1 = 13
    sl = lambda x, a, b: x[:, :, a:b]
    out, fin = oracle.recurrent(d["q"], d["k"], d["v"], "channel", d["log_alpha"], d["log_ig"])
    o1, f1 = oracle.recurrent(*(sl(d[x], 0, L1) for x in "qkv"), "channel", sl(d["log_alpha"], 0, L1),
                              sl(d["log_ig"], 0, L1))
    o2, f2 = oracle.recurrent(*(sl(d[x], L1, 30) for x in "qkv"), "channel", sl(d["log_alpha"], L1, 30),
                              sl(d["log_ig"], L1, 30), initial_state=f1)
    assert rel(np.concatenate([o1, o2], axis=2), out) < 1e-13
    assert rel(f2, fin) < 1e-13


def test_mlstm_reductions():
    d = small(L=19, gate="head", input_gate=True)
    # zero log input gate == scalar gate without an input gate
    o_a, _ = oracle.recurrent(d["q"], d["k"], d["v"], "head", d["log_alpha"], torch.zeros_like(d["log_ig"]))
    o_b, _ = oracle.recurrent(d["q"], d["k"], d["v"], "head", d["log_alpha"], None)
    assert rel(o_a, o_b) < 1e-15
    # forget gate 1: ungated map with k_t scaled by i_t
    ig = torch.exp(d["log_ig"].double())
    o_c, _ = oracle.recurrent(d["q"], d["k"], d["v"], "head", torch.zeros_like(d["log_alpha"]), d["log_ig"])
    ref = oracle.bruteforce_ungated(d["q"], d["k"].double() * ig[..., None], d["v"])
    assert rel(o_c, ref) < 1e-13


def test_gate_broadcast_kinds_agree():
    d = small(B=2, H=3, L=9, gate="head")
    B, H, L, Dk = d["q"].shape
    full = d["log_alpha"][..., None].expand(B, H, L, Dk).contiguous()
    a, _ = oracle.recurrent(d["q"], d["k"], d["v"], "head", d["log_alpha"])
    b, _ = oracle.recurrent(d["q"], d["k"], d["v"], "channel", full)
    assert rel(a, b) == 0.0
    const = torch.tensor([-0.1, -0.5, -0.01])
    c, _ = oracle.recurrent(d["q"], d["k"], d["v"], "head_const", const)
    e, _ = oracle.recurrent(d["q"], d["k"], d["v"], "head", const[None, :, None].expand(B, H, L).contiguous())
    assert rel(c, e) == 0.0


# ---------------------------------------------------------------------------------------
# Planted mistakes: each mutation of the C source must fail at least one pin.

def _pins_pass(lib) -> bool:
    """A compact subset of the pins above, run against a given compiled oracle."""
    try:
        with open(os.path.join(HERE, "golden", "hand_worked_small.json")) as f:
            gold = json.load(f)
        for case in gold["cases"]:
            out, fin = _golden_case(case, lib)
            if np.max(np.abs(out[0, 0] - np.array(case["out"]))) > 1e-12:
                return False
            if np.max(np.abs(fin[0, 0] - np.array(case["final_state"]))) > 1e-12:
                return False
        for gate, ig in (("channel", True), ("none", False), ("head_const", False)):
            d = small(L=21, gate=gate, input_gate=ig)
            out, fin = oracle.recurrent(d["q"], d["k"], d["v"], gate, d["log_alpha"], d["log_ig"], lib=lib)
            ref = oracle.parallel_form(d["q"], d["k"], d["v"], gate, d["log_alpha"], d["log_ig"])
            if rel(out, ref) > 1e-12:
                return False
            if gate == "none" and rel(out, oracle.bruteforce_ungated(d["q"], d["k"], d["v"])) > 1e-12:
                return False
            rf = oracle.final_state_closed_form(d["k"], d["v"], gate, d["log_alpha"], d["log_ig"])
            if rel(fin, rf) > 1e-12:
                return False
        return True
    except Exception:
        return False


MUTATIONS = [
    ("dropped decay", "Sd[c] = a * Sd[c] + w * vt[c];", "Sd[c] = Sd[c] + w * vt[c];"),
    ("wrong gate sign", "alpha[d] = exp(lat[d]);", "alpha[d] = exp(-lat[d]);"),
    ("wrong gate index", "alpha[d] = exp(lat[d]);", "alpha[d] = exp(lat[0]);"),
    ("dropped input gate", "const double w = ig * kt[d];", "const double w = kt[d];"),
    ("query/key swapped", "const double qd = qt[d];", "const double qd = kt[d];"),
    ("wrong value index", "for (long c = 0; c < Dv; ++c) Sd[c] = a * Sd[c] + w * vt[c];",
     "for (long c = 0; c < Dv; ++c) Sd[c] = a * Sd[c] + w * vt[Dv - 1 - c];"),
    ("read before write", None, None),
    ("state not carried", "const double *lat = log_alpha + (bh * L + t) * Dk;",
     "const double *lat = log_alpha + (bh * L + t) * Dk; memset(S, 0, sizeof(double) * (size_t)(Dk * Dv));"),
]


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass(oracle.oracle._load())


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "gla_oracle.c")).read()
    if old is None:  # read before write: o_t = q_t S_{t-1}; swap the two blocks of the step
        i_w = src.index("            /* write:")
        i_r = src.index("            /* read:")
        i_e = src.index("        }\n        if (final_state)")
        mutated = src[:i_w] + src[i_r:i_e] + src[i_w:i_r] + src[i_e:]
    else:
        assert old in src, "mutation anchor missing: " + name
        mutated = src.replace(old, new, 1)
    assert mutated != src
    mpath = tmp_path / "mut.c"
    mpath.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(mpath), "-lm"])
    lib = oracle.load_library(str(so))
    assert not _pins_pass(lib), "planted mistake not caught: " + name
