"""Pins of the mLSTM oracle (exponential input gate and normaliser), on the CPU.

The Tiled Flash Linear Attention abstract applies its kernels to the mLSTM of Beck et al.
(2024) and contrasts it with a variant whose sigmoid input gate needs less computation; the
pages print neither form.  The oracle follows the cited cell: memory and normaliser decay by
f_t = exp(log_f_t) and take the write with i_t = exp(log_i_t), and the read divides by
max(|q_t . n_t|, 1).  None of these tests compares the oracle with itself: each checks it
against hand-worked values, an independent pairwise (parallel) form, the max-stabilised
recurrence, the chunkwise algorithm, an exact scaling law of the input gate, or the pinned
gated linear recurrence where the normaliser is inactive; a planted-mistake suite shows that
each plausible slip in the C source fails at least one of them.
"""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


def draw(B=2, H=2, L=37, Dk=6, Dv=5, seed=0, ig_scale=1.0, init=False, qk_scale=1.0):
    rng = np.random.default_rng(seed)
    d = dict(q=rng.standard_normal((B, H, L, Dk)) * qk_scale,
             k=rng.standard_normal((B, H, L, Dk)) * qk_scale / np.sqrt(Dk),
             v=rng.standard_normal((B, H, L, Dv)),
             log_f=-np.log1p(np.exp(-(rng.standard_normal((B, H, L)) + 2.0))),
             log_i=rng.standard_normal((B, H, L)) * ig_scale)
    d["init"] = None
    if init:
        C0 = rng.standard_normal((B, H, Dk, Dv)) * 0.5
        n0 = rng.standard_normal((B, H, Dk)) * 0.5
        d["init"] = (C0, n0)
    return d


def run(d, lib=None):
    return oracle.mlstm_recurrent(d["q"], d["k"], d["v"], d["log_f"], d["log_i"], d["init"], lib=lib)


def load_golden():
    with open(os.path.join(HERE, "golden", "mlstm_hand_worked.json")) as f:
        return json.load(f)


def golden_case(case, lib=None):
    t = lambda x: np.asarray(x, dtype=np.float64)[None, None]
    init = None if case["C0"] is None else (t(case["C0"]), t(case["n0"]))
    return oracle.mlstm_recurrent(t(case["q"]), t(case["k"]), t(case["v"]), np.log(t(case["f"])),
                                  np.log(t(case["i"])), init, lib=lib)


@pytest.mark.parametrize("idx", [0, 1])
def test_hand_worked_examples(idx):
    case = load_golden()["cases"][idx]
    h, C, n = golden_case(case)
    assert np.max(np.abs(h[0, 0] - np.array(case["out"]))) <= 1e-14
    assert np.max(np.abs(C[0, 0] - np.array(case["final_C"]))) <= 1e-14
    assert np.max(np.abs(n[0, 0] - np.array(case["final_n"]))) <= 1e-14


@pytest.mark.parametrize("init", [False, True])
@pytest.mark.parametrize("ig_scale", [0.5, 3.0])
def test_pairwise_form_matches_the_recurrence(init, ig_scale):
    d = draw(init=init, ig_scale=ig_scale, seed=1)
    h, _, _ = run(d)
    hp = oracle.mlstm_parallel_form(d["q"], d["k"], d["v"], d["log_f"], d["log_i"], d["init"])
    assert rel(h, hp) <= 1e-12


def _stab_init(init):
    # the unstabilised (C0, n0) as a stabilised triple with an arbitrary exponent m0
    if init is None:
        return None
    C0, n0 = init
    m0 = np.full(C0.shape[:2], 0.7)
    return (C0 * np.exp(-0.7), n0 * np.exp(-0.7), m0)


@pytest.mark.parametrize("init", [False, True])
@pytest.mark.parametrize("ig_scale", [0.5, 8.0])
def test_max_stabilised_recurrence_reads_the_same_values(init, ig_scale):
    # the running maximum only rescales memory, normaliser and the clamp together
    d = draw(init=init, ig_scale=ig_scale, seed=2)
    h, C, n = run(d)
    hs, Cs, ns, ms = oracle.mlstm_stabilized_recurrent(d["q"], d["k"], d["v"], d["log_f"], d["log_i"],
                                                       _stab_init(d["init"]))
    # input gates spread over e^(+-24) make the unstabilised sums cancel: fp64 rounding of
    # terms up to 1e8 times the result bounds the agreement
    assert rel(h, hs) <= (1e-12 if ig_scale < 1 else 1e-9)
    assert rel(C, Cs * np.exp(ms)[..., None, None]) <= 1e-12
    assert rel(n, ns * np.exp(ms)[..., None]) <= 1e-12
    # every stabilised gate factor is at most 1, so the stabilised memory stays bounded
    assert np.all(np.isfinite(Cs))


@pytest.mark.parametrize("chunk", [1, 3, 16, 29, 64])
@pytest.mark.parametrize("init", [False, True])
def test_chunkwise_form_matches_the_recurrence(chunk, init):
    for L in (37, 70):
        d = draw(L=L, init=init, ig_scale=2.0, seed=chunk)
        h, C, n = run(d)
        hc, Cc, nc, mc = oracle.mlstm_chunkwise_form(d["q"], d["k"], d["v"], d["log_f"], d["log_i"], chunk,
                                                     _stab_init(d["init"]))
        assert rel(h, hc) <= 1e-12
        assert rel(C, Cc * np.exp(mc)[..., None, None]) <= 1e-12
        assert rel(n, nc * np.exp(mc)[..., None]) <= 1e-12


def test_input_gate_scaling_law():
    # adding c to every log input gate scales memory and normaliser by e^c; a read whose
    # normaliser exceeds 1 before and after is unchanged, one below 1 in both cases scales by e^c
    d = draw(seed=4, ig_scale=1.0)
    h0, C0, n0 = run(d)
    c = 0.9
    d2 = dict(d)
    d2["log_i"] = d["log_i"] + c
    h1, C1, n1 = run(d2)
    assert rel(C1, np.exp(c) * C0) <= 1e-13 and rel(n1, np.exp(c) * n0) <= 1e-13
    qn0 = np.abs(np.einsum("bhtd,bhtd->bht", d["q"], _running_n(d)))
    big = (qn0 >= 1.0) & (qn0 * np.exp(c) >= 1.0)
    small = (qn0 < 1.0) & (qn0 * np.exp(c) < 1.0)
    assert big.sum() > 10 and small.sum() > 10
    assert np.max(np.abs(h1 - h0)[big]) <= 1e-12 * np.sqrt(np.mean(h0 ** 2))
    assert np.max(np.abs(h1 - np.exp(c) * h0)[small]) <= 1e-12 * np.sqrt(np.mean(h0 ** 2))


def _running_n(d):
    # n_t by its closed form sum_{s<=t} exp(F_t - F_s + log_i_s) k_s (no initial state)
    F = np.cumsum(d["log_f"], axis=2)
    B, H, L, Dk = d["k"].shape
    n = np.zeros((B, H, L, Dk))
    for t in range(L):
        w = np.exp(F[:, :, t:t + 1] - F[:, :, :t + 1] + d["log_i"][:, :, :t + 1])
        n[:, :, t] = np.einsum("bhs,bhsd->bhd", w, d["k"][:, :, :t + 1])
    return n


def test_inactive_normaliser_reduces_to_the_gated_linear_recurrence():
    # with small queries and keys |q_t . n_t| < 1 throughout, so h_t = q_t C_t: the gated
    # linear recurrence with a per-token forget gate and input gate (pinned on its own)
    d = draw(seed=6, qk_scale=0.1)
    assert np.max(np.abs(np.einsum("bhtd,bhtd->bht", d["q"], _running_n(d)))) < 1.0
    h, C, _ = run(d)
    r_out, r_fin = oracle.recurrent(d["q"], d["k"], d["v"], "head", d["log_f"], d["log_i"])
    assert rel(h, r_out) <= 1e-13 and rel(C, r_fin) <= 1e-13


def test_independent_across_batch_and_heads():
    d = draw(B=2, H=3, L=20, seed=7, init=True)
    h, C, n = run(d)
    for b in range(2):
        for hh in range(3):
            sub = {key: val[b:b + 1, hh:hh + 1] for key, val in d.items() if key != "init"}
            sub["init"] = (d["init"][0][b:b + 1, hh:hh + 1], d["init"][1][b:b + 1, hh:hh + 1])
            o, c, nn = run(sub)
            assert rel(o[0, 0], h[b, hh]) == 0.0 and rel(c[0, 0], C[b, hh]) == 0.0


# ---------------------------------------------------------------------------------------
# Planted mistakes in a copy of the C source: each must fail at least one pin.

def _pins_pass(lib) -> bool:
    try:
        for case in load_golden()["cases"]:
            h, C, n = golden_case(case, lib)
            if np.max(np.abs(h[0, 0] - np.array(case["out"]))) > 1e-12:
                return False
            if np.max(np.abs(C[0, 0] - np.array(case["final_C"]))) > 1e-12:
                return False
            if np.max(np.abs(n[0, 0] - np.array(case["final_n"]))) > 1e-12:
                return False
        d = draw(L=21, seed=8, ig_scale=2.0, init=True)
        h, _, _ = run(d, lib)
        hp = oracle.mlstm_parallel_form(d["q"], d["k"], d["v"], d["log_f"], d["log_i"], d["init"])
        return rel(h, hp) <= 1e-12
    except Exception:
        return False


def _source():
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "gla_oracle.c")).read()
    i0 = src.index("int gla_oracle_mlstm(")
    i1 = src.index("/* Number of OpenMP threads")
    return src, i0, i1


MUTATIONS = [
    ("signed normaliser", "const double den = fabs(qn) > 1.0 ? fabs(qn) : 1.0;",
     "const double den = qn > 1.0 ? qn : 1.0;"),
    ("no clamp at one", "const double den = fabs(qn) > 1.0 ? fabs(qn) : 1.0;", "const double den = fabs(qn);"),
    ("no normaliser", "for (long c = 0; c < Dv; ++c) ht[c] /= den;", ""),
    ("normaliser without the input gate", "n[d] = ft * n[d] + w;", "n[d] = ft * n[d] + kt[d];"),
    ("normaliser without the forget gate", "n[d] = ft * n[d] + w;", "n[d] = n[d] + w;"),
    ("sigmoid input gate", "const double it = exp(log_i[bh * L + t]);",
     "const double it = 1.0 / (1.0 + exp(-log_i[bh * L + t]));"),
    ("decay after the write", "Cd[c] = ft * Cd[c] + w * vt[c];", "Cd[c] = ft * (Cd[c] + w * vt[c]);"),
    ("write without the input gate", "const double w = it * kt[d];", "const double w = kt[d];"),
    ("key and query swapped in the read", "ht[c] += qt[d] * Cd[c];", "ht[c] += kt[d] * Cd[c];"),
]


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass(oracle.oracle._load())


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src, i0, i1 = _source()
    body = src[i0:i1]
    assert old in body, "mutation anchor missing: " + name
    if name == "write without the input gate":
        # the normaliser keeps its own (correct) input-gated write
        body = body.replace(old, new, 1).replace("n[d] = ft * n[d] + w;", "n[d] = ft * n[d] + it * kt[d];", 1)
    else:
        body = body.replace(old, new, 1)
    mutated = src[:i0] + body + src[i1:]
    assert mutated != src
    mpath = tmp_path / "mut.c"
    mpath.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(mpath), "-lm"])
    lib = oracle.load_library(str(so))
    assert not _pins_pass(lib), "planted mistake not caught: " + name
