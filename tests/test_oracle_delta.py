"""Pins of the delta-rule oracle (DeltaNet and Gated DeltaNet), on the CPU.

The pages fix the update in words: a writing strength beta_t (Hardware-Efficient Training of
Linear Attention Models, talk summary, 22:36) and one stochastic-gradient step on the
squared error of predicting v_t from k_t, with an identity-plus-rank-one transition and, for
Gated DeltaNet, Mamba-2-style gating (same talk, 31:16).  None of these tests compares the
oracle with itself: each checks it against a hand-worked example, a closed form, an exact
invariant of a gradient step, an independent chunkwise (WY) derivation, or the pinned linear
recurrence in a case where the two rules coincide; a planted-mistake suite shows that each
plausible slip in the C source fails at least one of them.
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


def draw(B=2, H=2, L=37, Dk=8, Dv=5, gated=True, seed=0, s0=True):
    g = torch.Generator().manual_seed(seed)
    unit = lambda x: x / x.norm(dim=-1, keepdim=True)
    d = dict(q=unit(torch.randn(B, H, L, Dk, generator=g, dtype=torch.float64)),
             k=unit(torch.randn(B, H, L, Dk, generator=g, dtype=torch.float64)),
             v=torch.randn(B, H, L, Dv, generator=g, dtype=torch.float64),
             beta=torch.sigmoid(torch.randn(B, H, L, generator=g, dtype=torch.float64)))
    d["log_alpha"] = (torch.nn.functional.logsigmoid(torch.randn(B, H, L, generator=g, dtype=torch.float64) + 2)
                      if gated else None)
    d["s0"] = torch.randn(B, H, Dk, Dv, generator=g, dtype=torch.float64) * 0.3 if s0 else None
    return d


def run(d, lib=None):
    return oracle.delta_recurrent(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], lib=lib)


def golden_case(case, lib=None):
    t = lambda x: torch.tensor(x, dtype=torch.float64)[None, None]
    la = None if case["alpha"] is None else torch.log(t(case["alpha"]))
    return oracle.delta_recurrent(t(case["q"]), t(case["k"]), t(case["v"]), t(case["beta"]), la, None, lib=lib)


def load_golden():
    with open(os.path.join(HERE, "golden", "delta_hand_worked.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("idx", [0, 1])
def test_hand_worked_examples(idx):
    case = load_golden()["cases"][idx]
    out, fin = golden_case(case)
    assert np.max(np.abs(out[0, 0] - np.array(case["out"]))) <= 1e-14
    assert np.max(np.abs(fin[0, 0] - np.array(case["final_state"]))) <= 1e-14


@pytest.mark.parametrize("gated", [False, True])
def test_zero_writing_strength_keeps_the_state(gated):
    # beta = 0: no step is taken; the state only decays: S_t = g_t S0, o_t = q_t S_t
    d = draw(gated=gated)
    d["beta"] = torch.zeros_like(d["beta"])
    out, fin = run(d)
    la = d["log_alpha"] if gated else torch.zeros_like(d["beta"])
    G = torch.exp(torch.cumsum(la, dim=2)).numpy()
    S = d["s0"].numpy()
    ref = np.einsum("bhtd,bhdc->bhtc", d["q"].numpy(), S) * G[..., None]
    assert rel(out, ref) <= 1e-13
    assert rel(fin, S * G[:, :, -1, None, None]) <= 1e-13


def test_orthonormal_keys_with_unit_strength_recall_exactly():
    # keys orthonormal, beta = 1, S0 = 0: each step solves its regression exactly and leaves
    # the other keys' associations untouched, so k_i S_L = v_i for every written pair, and a
    # query equal to an earlier key reads back that key's value
    Dk, L, Dv = 12, 9, 4
    rng = np.random.default_rng(3)
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm[:L]
    v = rng.standard_normal((L, Dv))
    q = np.roll(keys, 2, axis=0)  # q_t = k_{t-2}: reads back v_{t-2} from t >= 2 on
    t = lambda x: torch.tensor(x)[None, None]
    out, fin = oracle.delta_recurrent(t(q), t(keys), t(v), torch.ones(1, 1, L, dtype=torch.float64))
    assert np.max(np.abs(keys @ fin[0, 0] - v)) <= 1e-13
    assert np.max(np.abs(out[0, 0, 2:] - v[:-2])) <= 1e-13


def test_one_step_is_a_gradient_step_on_the_regression_loss():
    # from a random state: 1/2 |k S - v|^2 falls for 0 < beta < 2/|k|^2, rises above it,
    # and beta = 1/|k|^2 fits the pair exactly (the step is exact line search)
    rng = np.random.default_rng(5)
    Dk, Dv = 6, 3
    S0 = rng.standard_normal((Dk, Dv))
    k = rng.standard_normal(Dk) * 0.7
    v = rng.standard_normal(Dv)
    kk = float(k @ k)
    loss = lambda S: 0.5 * float(np.sum((k @ S - v) ** 2))
    t = lambda x: torch.tensor(np.asarray(x, dtype=np.float64))[None, None, None]
    for beta, sign in ((0.3 / kk, -1), (1.0 / kk, -1), (1.9 / kk, -1), (2.2 / kk, +1)):
        _, fin = oracle.delta_recurrent(t(k), t(k), t(v), torch.tensor([[[beta]]], dtype=torch.float64),
                                        None, torch.tensor(S0)[None, None])
        after = loss(fin[0, 0])
        assert (after - loss(S0)) * sign > 0, (beta * kk, after, loss(S0))
        # closed form of the step: the residual shrinks by (1 - beta |k|^2)
        r0, r1 = k @ S0 - v, k @ fin[0, 0] - v
        assert np.max(np.abs(r1 - (1 - beta * kk) * r0)) <= 1e-12
    _, fin = oracle.delta_recurrent(t(k), t(k), t(v), torch.tensor([[[1.0 / kk]]], dtype=torch.float64), None,
                                    torch.tensor(S0)[None, None])
    assert np.max(np.abs(k @ fin[0, 0] - v)) <= 1e-13


def test_scalar_key_closed_form():
    # Dk = 1: s_t = a_t s_{t-1} + beta_t k_t v_t with a_t = alpha_t (1 - beta_t k_t^2), whose
    # solution is s_t = (prod_{r<=t} a_r) s0 + sum_{i<=t} (prod_{i<r<=t} a_r) beta_i k_i v_i
    rng = np.random.default_rng(7)
    L, Dv = 23, 3
    k = rng.standard_normal(L)
    v = rng.standard_normal((L, Dv))
    q = rng.standard_normal(L)
    beta = rng.uniform(0, 1, L)
    la = np.log(rng.uniform(0.5, 1, L))
    s0 = rng.standard_normal(Dv)
    a = np.exp(la) * (1 - beta * k * k)
    ref = np.zeros((L, Dv))
    for t in range(L):
        s = np.prod(a[:t + 1]) * s0
        for i in range(t + 1):
            s = s + np.prod(a[i + 1:t + 1]) * beta[i] * k[i] * v[i]
        ref[t] = q[t] * s
    T = lambda x: torch.tensor(x)[None, None]
    out, fin = oracle.delta_recurrent(T(q[:, None]), T(k[:, None]), T(v), T(beta), T(la), T(s0[None]))
    assert rel(out[0, 0], ref) <= 1e-12
    assert np.max(np.abs(fin[0, 0, 0] - ref[-1] / q[-1])) <= 1e-12


@pytest.mark.parametrize("gated", [False, True])
def test_orthogonal_keys_reduce_to_the_gated_linear_recurrence(gated):
    # with mutually orthogonal keys and a zero initial state every prediction k_t S' is zero,
    # so the delta rule is the gated linear recurrence with input gate beta (pinned elsewhere)
    B, H, L, Dk, Dv = 1, 2, 10, 16, 3
    rng = np.random.default_rng(11)
    keys = np.stack([np.linalg.qr(rng.standard_normal((Dk, Dk)))[0][:L] * rng.uniform(0.5, 2, (L, 1))
                     for _ in range(H)])[None]
    q = rng.standard_normal((B, H, L, Dk))
    v = rng.standard_normal((B, H, L, Dv))
    beta = rng.uniform(0.1, 1, (B, H, L))
    la = np.log(rng.uniform(0.3, 1, (B, H, L))) if gated else None
    out, fin = oracle.delta_recurrent(q, keys, v, beta, la)
    r_out, r_fin = oracle.recurrent(q, keys, v, "head" if gated else "none", la, np.log(beta))
    assert rel(out, r_out) <= 1e-12 and rel(fin, r_fin) <= 1e-12


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 29, 64])
@pytest.mark.parametrize("gated", [False, True])
def test_chunkwise_wy_form_matches_the_recurrence(chunk, gated):
    # the WY (lower-triangular solve) chunkwise form is an exact re-association of the same
    # map for every chunk size, ragged tails included (L = 37 and 70)
    for L in (37, 70):
        d = draw(L=L, gated=gated, seed=chunk)
        out, fin = run(d)
        c_out, c_fin = oracle.delta_chunkwise_form(d["q"], d["k"], d["v"], d["beta"], chunk, d["log_alpha"], d["s0"])
        assert rel(out, c_out) <= 1e-12 and rel(fin, c_fin) <= 1e-12


def test_zero_gate_keeps_only_the_current_write():
    # alpha_t = 0 (log -1e4 underflows to an exact zero): the old state is gone before the
    # token is written, so S_t = beta_t k_t^T v_t and o_t = beta_t (q_t . k_t) v_t
    d = draw(gated=True)
    d["log_alpha"] = torch.full_like(d["log_alpha"], -1e4)
    out, fin = run(d)
    qk = (d["q"] * d["k"]).sum(-1)
    ref = (d["beta"] * qk)[..., None] * d["v"]
    assert rel(out, ref.numpy()) <= 1e-13
    ref_fin = d["beta"][:, :, -1, None, None] * d["k"][:, :, -1, :, None] * d["v"][:, :, -1, None, :]
    assert rel(fin, ref_fin.numpy()) <= 1e-13


def test_linear_in_q_and_independent_across_batch_and_heads():
    d = draw(B=2, H=3, L=20)
    out, _ = run(d)
    d2 = dict(d)
    d2["q"] = d["q"] * 2.5 - 0.0
    out2, _ = run(d2)
    assert rel(out2, 2.5 * out) <= 1e-13
    for b in range(2):
        for h in range(3):
            sub = {key: (None if val is None else val[b:b + 1, h:h + 1]) for key, val in d.items()}
            o, f = run(sub)
            assert rel(o[0, 0], out[b, h]) == 0.0


def test_fixed_per_head_gate_broadcasts():
    d = draw(B=2, H=3, L=15)
    const = torch.tensor([-0.1, -0.5, -0.01], dtype=torch.float64)
    a = oracle.delta_recurrent(d["q"], d["k"], d["v"], d["beta"], const, d["s0"])[0]
    b = oracle.delta_recurrent(d["q"], d["k"], d["v"], d["beta"], const[None, :, None].expand(2, 3, 15).contiguous(),
                               d["s0"])[0]
    assert rel(a, b) == 0.0


# ---------------------------------------------------------------------------------------
# Planted mistakes in a copy of the C source: each must fail at least one pin.

def _delta_pins_pass(lib) -> bool:
    try:
        for case in load_golden()["cases"]:
            out, fin = golden_case(case, lib)
            if np.max(np.abs(out[0, 0] - np.array(case["out"]))) > 1e-12:
                return False
            if np.max(np.abs(fin[0, 0] - np.array(case["final_state"]))) > 1e-12:
                return False
        for gated in (False, True):
            d = draw(L=21, gated=gated, seed=4)
            out, fin = run(d, lib)
            c_out, c_fin = oracle.delta_chunkwise_form(d["q"], d["k"], d["v"], d["beta"], 8, d["log_alpha"], d["s0"])
            if rel(out, c_out) > 1e-12 or rel(fin, c_fin) > 1e-12:
                return False
        return True
    except Exception:
        return False


def _delta_source():
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "gla_oracle.c")).read()
    i0 = src.index("int gla_oracle_delta(")
    i1 = src.index("/* The mLSTM cell")
    return src, i0, i1


DELTA_MUTATIONS = [
    ("dropped writing strength", "const double w = bt * kt[d];", "const double w = kt[d];"),
    ("wrong correction sign", "Sd[c] += w * (vt[c] - pred[c]);", "Sd[c] += w * (vt[c] + pred[c]);"),
    ("no correction (plain linear write)", "Sd[c] += w * (vt[c] - pred[c]);", "Sd[c] += w * vt[c];"),
    ("dropped decay", "for (long i = 0; i < Dk * Dv; ++i) S[i] *= at;", "for (long i = 0; i < Dk * Dv; ++i) S[i] *= 1.0;"),
    ("prediction from the query", "pred[c] += kt[d] * Sd[c];", "pred[c] += qt[d] * Sd[c];"),
    ("decay after the write", "for (long i = 0; i < Dk * Dv; ++i) S[i] *= at;\n", ""),
    ("read before write", None, None),
]


def test_delta_pins_pass_on_the_real_oracle():
    assert _delta_pins_pass(oracle.oracle._load())


@pytest.mark.parametrize("name,old,new", DELTA_MUTATIONS, ids=[m[0] for m in DELTA_MUTATIONS])
def test_planted_delta_mistake_is_caught(tmp_path, name, old, new):
    src, i0, i1 = _delta_source()
    body = src[i0:i1]
    if name == "decay after the write":
        assert old in body
        body = body.replace(old, new, 1)
        anchor = "            /* read: o_t = q_t S_t */"
        body = body.replace(anchor, "            for (long i = 0; i < Dk * Dv; ++i) S[i] *= at;\n" + anchor, 1)
    elif old is None:  # read before write: o_t = q_t S'; move the read ahead of the step
        i_p = body.index("            /* prediction")
        i_r = body.index("            /* read:")
        i_e = body.index("        }\n        if (final_state)")
        body = body[:i_p] + body[i_r:i_e] + body[i_p:i_r] + body[i_e:]
    else:
        assert old in body, "mutation anchor missing: " + name
        body = body.replace(old, new, 1)
    mutated = src[:i0] + body + src[i1:]
    assert mutated != src
    mpath = tmp_path / "mut.c"
    mpath.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(mpath), "-lm"])
    lib = oracle.load_library(str(so))
    assert not _delta_pins_pass(lib), "planted mistake not caught: " + name
