"""Pins for the fp64 oracle's gradients (CPU only).

The backward oracle differentiates each step of the recurrence.  It is pinned to things
other than itself: central finite differences of a scalar loss computed with the forward
oracle (a separate function), textbook causal sums for the ungated case, the identity that
ties the log-decay gradient to the query and key gradients, and planted mistakes in copies
of the C source that these pins must catch.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    scale = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def case(gate, input_gate, B=1, H=2, L=9, Dk=3, Dv=4, seed=0, s0=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, L, Dk))
    k = r.standard_normal((B, H, L, Dk))
    v = r.standard_normal((B, H, L, Dv))
    la = {"none": None, "channel": np.log(r.uniform(0.3, 1.0, (B, H, L, Dk))),
          "head": np.log(r.uniform(0.3, 1.0, (B, H, L))), "head_const": np.log(r.uniform(0.3, 1.0, (H,)))}[gate]
    li = np.log(r.uniform(0.2, 1.0, (B, H, L))) if input_gate else None
    S0 = r.standard_normal((B, H, Dk, Dv)) if s0 else None
    dO = r.standard_normal((B, H, L, Dv))
    dF = r.standard_normal((B, H, Dk, Dv))
    return dict(q=q, k=k, v=v, la=la, li=li, S0=S0, dO=dO, dF=dF)


def loss(c, gate, **over):
    x = dict(c, **over)
    out, fin = oracle.recurrent(x["q"], x["k"], x["v"], gate, x["la"], x["li"], x["S0"])
    return float(np.sum(out * c["dO"]) + np.sum(fin * c["dF"]))


def grads(c, gate, lib=None):
    return oracle.backward(c["q"], c["k"], c["v"], c["dO"], gate, c["la"], c["li"], c["S0"], c["dF"], lib=lib)


def finite_difference(c, gate, name, eps=1e-6):
    x = c[name]
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        g[i] = (loss(c, gate, **{name: xp}) - loss(c, gate, **{name: xm})) / (2 * eps)
    return g


KEYS = {"q": "dq", "k": "dk", "v": "dv", "la": "dlog_alpha", "li": "dlog_ig", "S0": "dinitial_state"}


@pytest.mark.parametrize("gate,input_gate", [("none", False), ("channel", False), ("channel", True),
                                             ("head", True), ("head_const", False)])
def test_gradients_match_finite_differences(gate, input_gate):
    c = case(gate, input_gate)
    g = grads(c, gate)
    for name, key in KEYS.items():
        if c[name] is None:
            assert g[key] is None or name == "S0"
            continue
        fd = finite_difference(c, gate, name)
        assert g[key].shape == fd.shape, name
        assert rel(g[key], fd) < 1e-7, (gate, name, rel(g[key], fd))


def test_ungated_gradients_are_textbook_causal_sums():
    # loss = sum_t dO_t . o_t with o_t = sum_{s<=t} (q_t . k_s) v_s, no initial or final state term
    c = case("none", False, L=11, s0=False)
    c["dF"] = np.zeros_like(c["dF"])
    g = grads(c, "none")
    q, k, v, dO = c["q"][0, 0], c["k"][0, 0], c["v"][0, 0], c["dO"][0, 0]
    L = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for t in range(L):
        for s in range(t + 1):
            w = float(dO[t] @ v[s])
            dq[t] += w * k[s]
            dk[s] += w * q[t]
            dv[s] += float(q[t] @ k[s]) * dO[t]
    assert rel(g["dq"][0, 0], dq) < 1e-13
    assert rel(g["dk"][0, 0], dk) < 1e-13
    assert rel(g["dv"][0, 0], dv) < 1e-13


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_log_decay_gradient_identity(gate):
    # With B_t the running sum of log decays, o_t = sum_s exp(B_t - B_s) i_s (q_t . k_s) v_s
    # + exp(B_t) q_t S0, so d loss / d B_t = q_t * dq_t - k_t * dk_t (+ the final-state term
    # at the last token), and the log-decay gradient is its reverse running sum.
    c = case(gate, True, L=10)
    g = grads(c, gate)
    out, fin = oracle.recurrent(c["q"], c["k"], c["v"], gate, c["la"], c["li"], c["S0"])
    dB = c["q"] * g["dq"] - c["k"] * g["dk"]
    dB[:, :, -1, :] += np.sum(c["dF"] * fin, axis=3)
    dla = np.flip(np.cumsum(np.flip(dB, axis=2), axis=2), axis=2)
    assert rel(oracle.reduce_gate_grad(gate, dla), g["dlog_alpha"]) < 1e-12


# ---------------------------------------------------------------------------------------
# Planted mistakes in the backward: each must fail the finite-difference pin.

BWD_MUTATIONS = [
    ("decay not applied going back", "for (long c = 0; c < Dv; ++c) G[d * Dv + c] *= a;",
     "for (long c = 0; c < Dv; ++c) G[d * Dv + c] *= 1.0;"),
    ("read not added", "for (long c = 0; c < Dv; ++c) G[d * Dv + c] += qt[d] * dOt[c];",
     "for (long c = 0; c < Dv; ++c) G[d * Dv + c] += 0.0 * dOt[c];"),
    ("input gate missing in dk", "dkt[d] = ig * sk;", "dkt[d] = sk;"),
    ("decay gradient from the new state", "sa += G[d * Dv + c] * Sprev[d * Dv + c];",
     "sa += G[d * Dv + c] * St[d * Dv + c];"),
    ("dq from the previous state", "sq += dOt[c] * St[d * Dv + c];", "sq += dOt[c] * Sprev[d * Dv + c];"),
]


def _bwd_pins_pass(lib) -> bool:
    try:
        for gate, ig in (("channel", True), ("head", True)):
            c = case(gate, ig, L=7)
            g = grads(c, gate, lib)
            for name, key in KEYS.items():
                if rel(g[key], finite_difference(c, gate, name)) > 1e-6:
                    return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("name,old,new", BWD_MUTATIONS, ids=[m[0] for m in BWD_MUTATIONS])
def test_planted_backward_mistake_is_caught(tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "gla_oracle.c")).read()
    assert old in src, "mutation anchor missing: " + name
    mutated = src.replace(old, new, 1)
    mpath = tmp_path / "mut.c"
    mpath.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(mpath), "-lm"])
    assert not _bwd_pins_pass(oracle.load_library(str(so))), "planted mistake not caught: " + name


def test_backward_pins_pass_on_the_real_oracle():
    assert _bwd_pins_pass(oracle.oracle._load())
