"""fp64 oracle for the gated linear attention forward pass and the delta rule.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

Forms (all fp64, computed from the exact input values):

* :func:`recurrent` -- the definition: the token recurrence
  ``S_t = diag(alpha_t) S_{t-1} + i_t k_t^T v_t``, ``o_t = q_t S_t`` in plain C
  (``gla_oracle.c``).  A matrix-valued state updated by one rank-1 write and read by one
  vector-matrix product per token [Hardware-Efficient Training of Linear Attention Models,
  talk summary, 4:04 and 7:36]; gates as the data-dependent generalisation [Gated Linear
  Attention Transformers with Hardware-Efficient Training, abstract].
* :func:`parallel_form` -- the quadratic ("parallel") form of the same map: causal
  pairwise scores times values, with the gate entering as a per-channel decay between the
  two positions [talk summary, 7:36].  Tiny inputs only.
* :func:`chunkwise_form` -- the chunkwise algorithm written plainly: split the sequence
  into chunks of ``C`` tokens, carry the state only across chunk boundaries, and inside
  a chunk add the masked pairwise term [talk summary, 11:58; Tiled Flash Linear
  Attention, abstract, for arbitrary chunk sizes].  Tiny inputs only.
* :func:`bruteforce_ungated` -- causal sums ``o_t = sum_{s<=t} (q_t . k_s) v_s`` in
  Python loops, the textbook ungated case.  Tiny inputs only.
* :func:`backward` -- gradients of a scalar loss through the recurrence: reverse-mode
  differentiation of each step of the definition, in C.  The pages train these models
  [talk summary, 7:36 "Challenges in Training Linear Attention"] but print no gradient;
  the derivative of the definition is fixed by the definition itself, and the tests pin it
  by finite differences.

* :func:`delta_recurrent` -- the delta rule (DeltaNet, and Gated DeltaNet with a scalar
  per-token decay), token by token in C (``gla_oracle_delta``): each token takes one
  gradient step of size ``beta_t`` on ``1/2 |k_t S - v_t|^2`` [talk summary, 22:36 and
  31:16].
* :func:`delta_chunkwise_form` -- the same map chunkwise, with the lower-triangular (WY)
  system that turns the product of identity-plus-rank-one transitions into sums
  [talk summary, 31:16].  Tiny inputs only.

* :func:`mlstm_recurrent` -- the mLSTM (the xLSTM's matrix memory) with exponential input
  gate and normaliser, token by token in C (``gla_oracle_mlstm``): ``C_t = f_t C_{t-1} +
  i_t k_t^T v_t``, ``n_t = f_t n_{t-1} + i_t k_t``, ``h_t = q_t C_t / max(|q_t . n_t|, 1)``
  with ``f_t = exp(log_f_t)`` and ``i_t = exp(log_i_t)`` [Tiled Flash Linear Attention,
  abstract: the mLSTM of Beck et al. (2024); its sigmoid-gated variant drops the normaliser].
  The pages print neither the exponential gate nor the normaliser; the form used is the one
  of the cited mLSTM.
* :func:`mlstm_parallel_form`, :func:`mlstm_stabilized_recurrent` and
  :func:`mlstm_chunkwise_form` -- the same map as causal pairwise weights, as the
  max-stabilised token recurrence, and chunkwise with a running maximum of the log
  weights.  Tiny inputs only.

Gate kinds (how a stored gate broadcasts to the per-channel log decay):
``"none"`` (zero), ``"channel"`` ``[B,H,L,Dk]``, ``"head"`` ``[B,H,L]`` (one decay per
head and token), ``"head_const"`` ``[H]`` (one fixed decay per head).  The optional input
gate ``log_ig`` is ``[B,H,L]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GATE_KINDS = ("none", "channel", "head", "head_const")


def build(force: bool = False) -> str:
    """Compile ``gla_oracle.c`` into ``liboracle.so`` with gcc (CPU only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open a compiled oracle library at ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gla_oracle_recurrent.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp] + [ctypes.c_long] * 5
    lib.gla_oracle_recurrent.restype = ctypes.c_int
    lib.gla_oracle_backward.argtypes = [dp] * 14 + [ctypes.c_long] * 5
    lib.gla_oracle_backward.restype = ctypes.c_int
    lib.gla_oracle_delta.argtypes = [dp] * 8 + [ctypes.c_long] * 5
    lib.gla_oracle_delta.restype = ctypes.c_int
    lib.gla_oracle_mlstm.argtypes = [dp] * 10 + [ctypes.c_long] * 5
    lib.gla_oracle_mlstm.restype = ctypes.c_int
    lib.gla_oracle_threads.restype = ctypes.c_int
    lib.gla_oracle_threads.argtypes = []
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            _lib = load_library(build())
    return _lib


def threads() -> int:
    """OpenMP threads :func:`recurrent` runs on."""
    return int(_load().gla_oracle_threads())


def _f64(x):
    """Exact conversion of a torch tensor (bf16/fp32/fp64) or array to a C-contiguous fp64 array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16 -> fp32 -> fp64 is exact
        import torch

        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16 or x.dtype == torch.float16:
            x = x.float()
        x = x.double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def expand_gate(gate_kind: str, log_alpha, B: int, H: int, L: int, Dk: int) -> np.ndarray:
    """Broadcast a stored log gate to the per-channel log decay ``[B,H,L,Dk]`` (fp64)."""
    if gate_kind not in GATE_KINDS:
        raise ValueError("unknown gate kind %r" % (gate_kind,))
    if gate_kind == "none":
        return np.zeros((B, H, L, Dk))
    a = _f64(log_alpha)
    if gate_kind == "channel":
        assert a.shape == (B, H, L, Dk), a.shape
        return a
    if gate_kind == "head":
        assert a.shape == (B, H, L), a.shape
        return np.ascontiguousarray(np.broadcast_to(a[..., None], (B, H, L, Dk)))
    assert a.shape == (H,), a.shape
    return np.ascontiguousarray(np.broadcast_to(a[None, :, None, None], (B, H, L, Dk)))


def recurrent(q, k, v, gate_kind="none", log_alpha=None, log_ig=None, initial_state=None, lib=None):
    """The definition, in C: returns ``(out [B,H,L,Dv], final_state [B,H,Dk,Dv])`` in fp64.
    ``lib`` selects another compiled copy of the oracle (used by tests that plant a mistake
    in a copy of the C source to show the pins catch it)."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    assert k64.shape == q64.shape and v64.shape == (B, H, L, Dv)
    la = expand_gate(gate_kind, log_alpha, B, H, L, Dk)
    li = _f64(log_ig)
    if li is not None:
        assert li.shape == (B, H, L)
    s0 = _f64(initial_state)
    if s0 is not None:
        assert s0.shape == (B, H, Dk, Dv)
    out = np.empty((B, H, L, Dv))
    fin = np.empty((B, H, Dk, Dv))
    dp = ctypes.POINTER(ctypes.c_double)

    def p(a):
        return None if a is None else a.ctypes.data_as(dp)

    rc = (lib or _load()).gla_oracle_recurrent(p(q64), p(k64), p(v64), p(la), p(li), p(s0), p(out), p(fin),
                                      B, H, L, Dk, Dv)
    if rc != 0:
        raise RuntimeError("gla_oracle_recurrent failed (%d)" % rc)
    return out, fin


def reduce_gate_grad(gate_kind: str, g: np.ndarray):
    """Sum a per-channel log-decay gradient ``[B,H,L,Dk]`` over the axes a stored gate of
    ``gate_kind`` is broadcast along (the adjoint of :func:`expand_gate`)."""
    if gate_kind == "none":
        return None
    if gate_kind == "channel":
        return g
    if gate_kind == "head":
        return g.sum(axis=3)
    return g.sum(axis=(0, 2, 3))


def backward(q, k, v, dout, gate_kind="none", log_alpha=None, log_ig=None, initial_state=None, dfinal=None,
             lib=None):
    """Gradients of a scalar loss through the recurrence, in C (reverse-mode differentiation
    of each step; ``gla_oracle_backward``).  ``dout`` [B,H,L,Dv] and ``dfinal`` [B,H,Dk,Dv]
    (or None) are the loss gradients with respect to the outputs.  Returns a dict with
    ``dq``, ``dk`` [B,H,L,Dk], ``dv`` [B,H,L,Dv], ``dlog_alpha`` (the stored gate's layout,
    None without a gate), ``dlog_ig`` [B,H,L] (None without an input gate) and
    ``dinitial_state`` [B,H,Dk,Dv], all fp64."""
    q64, k64, v64, do64 = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    assert k64.shape == q64.shape and v64.shape == (B, H, L, Dv) and do64.shape == (B, H, L, Dv)
    la = expand_gate(gate_kind, log_alpha, B, H, L, Dk)
    li = _f64(log_ig)
    s0, dsf = _f64(initial_state), _f64(dfinal)
    dq, dk = np.empty((B, H, L, Dk)), np.empty((B, H, L, Dk))
    dv, dla = np.empty((B, H, L, Dv)), np.empty((B, H, L, Dk))
    dli = np.empty((B, H, L)) if li is not None else None
    ds0 = np.empty((B, H, Dk, Dv))
    dp = ctypes.POINTER(ctypes.c_double)

    def p(a):
        return None if a is None else a.ctypes.data_as(dp)

    rc = (lib or _load()).gla_oracle_backward(p(q64), p(k64), p(v64), p(la), p(li), p(s0), p(do64), p(dsf), p(dq),
                                              p(dk), p(dv), p(dla), p(dli), p(ds0), B, H, L, Dk, Dv)
    if rc != 0:
        raise RuntimeError("gla_oracle_backward failed (%d)" % rc)
    return dict(dq=dq, dk=dk, dv=dv, dlog_alpha=reduce_gate_grad(gate_kind, dla), dlog_ig=dli, dinitial_state=ds0)


def parallel_form(q, k, v, gate_kind="none", log_alpha=None, log_ig=None, initial_state=None):
    """Quadratic form: ``o_t = sum_{s<=t} sum_d q_td k_sd exp(G_td - G_sd) i_s v_s
    + (q_t * exp(G_t)) S0``, where ``G`` is the inclusive running sum of the log decay
    from the start of the sequence.  Per-channel gates make the mask carry a channel
    index, so the pairwise score keeps its sum over ``d`` inside the decay.
    Returns ``out`` only (fp64).  O(L^2 Dk): tiny inputs."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    la = expand_gate(gate_kind, log_alpha, B, H, L, Dk)
    ig = np.ones((B, H, L)) if log_ig is None else np.exp(_f64(log_ig))
    G = np.cumsum(la, axis=2)  # [B,H,L,Dk]
    out = np.zeros(v64.shape)
    causal = np.tril(np.ones((L, L), dtype=bool))
    for b in range(B):
        for h in range(H):
            # decay[t, s, d] = exp(G_td - G_sd), only used where s <= t (so the exponent is <= 0
            # for gates <= 0); the upper triangle is masked before the exponent is taken.
            diff = G[b, h][:, None, :] - G[b, h][None, :, :]
            diff = np.where(causal[:, :, None], diff, -np.inf)
            scores = np.einsum("td,sd,tsd->ts", q64[b, h], k64[b, h], np.exp(diff))
            out[b, h] = (scores * ig[b, h][None, :]) @ v64[b, h]
            if initial_state is not None:
                s0 = _f64(initial_state)[b, h]
                out[b, h] += (q64[b, h] * np.exp(G[b, h])) @ s0
    return out


def chunkwise_form(q, k, v, chunk: int, gate_kind="none", log_alpha=None, log_ig=None,
                   initial_state=None):
    """Chunkwise algorithm, plainly: for each chunk of ``chunk`` tokens (the last may be
    shorter), with ``b`` the inclusive running sum of the log decay inside the chunk and
    ``g`` its value at the chunk's last token:

        o_t   = (q_t * exp(b_t)) S_in + sum_{s<=t in chunk} [sum_d q_td k_sd exp(b_td - b_sd)] i_s v_s
        S_out = diag(exp(g)) S_in + sum_{s in chunk} (k_s * exp(g - b_s))^T i_s v_s

    Returns ``(out, final_state)`` in fp64."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    la = expand_gate(gate_kind, log_alpha, B, H, L, Dk)
    ig = np.ones((B, H, L)) if log_ig is None else np.exp(_f64(log_ig))
    out = np.zeros((B, H, L, Dv))
    fin = np.zeros((B, H, Dk, Dv))
    s0 = None if initial_state is None else _f64(initial_state)
    for b_ in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if s0 is None else s0[b_, h].copy()
            for c0 in range(0, L, chunk):
                c1 = min(L, c0 + chunk)
                qc, kc, vc = q64[b_, h, c0:c1], k64[b_, h, c0:c1], v64[b_, h, c0:c1]
                ic = ig[b_, h, c0:c1]
                bcum = np.cumsum(la[b_, h, c0:c1], axis=0)  # [n, Dk]
                g = bcum[-1]
                n = c1 - c0
                inter = (qc * np.exp(bcum)) @ S
                intra = np.zeros((n, Dv))
                for t in range(n):
                    for s in range(t + 1):
                        score = np.sum(qc[t] * kc[s] * np.exp(bcum[t] - bcum[s]))
                        intra[t] += score * ic[s] * vc[s]
                out[b_, h, c0:c1] = inter + intra
                S = np.exp(g)[:, None] * S + ((kc * np.exp(g[None, :] - bcum)) * ic[:, None]).T @ vc
            fin[b_, h] = S
    return out, fin


def bruteforce_ungated(q, k, v):
    """Ungated causal sums ``o_t = sum_{s<=t} (q_t . k_s) v_s`` with Python loops (fp64)."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    out = np.zeros((B, H, L, Dv))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                acc = [0.0] * Dv
                for s in range(t + 1):
                    dot = 0.0
                    for d in range(Dk):
                        dot += float(q64[b, h, t, d]) * float(k64[b, h, s, d])
                    for c in range(Dv):
                        acc[c] += dot * float(v64[b, h, s, c])
                out[b, h, t] = acc
    return out


def final_state_closed_form(k, v, gate_kind="none", log_alpha=None, log_ig=None):
    """``S_L = sum_t diag(exp(G_{L-1} - G_t)) i_t k_t^T v_t`` (zero initial state), fp64."""
    k64, v64 = _f64(k), _f64(v)
    B, H, L, Dk = k64.shape
    la = expand_gate(gate_kind, log_alpha, B, H, L, Dk)
    ig = np.ones((B, H, L)) if log_ig is None else np.exp(_f64(log_ig))
    G = np.cumsum(la, axis=2)
    w = np.exp(G[:, :, -1:, :] - G) * ig[..., None]  # [B,H,L,Dk]
    return np.einsum("bhtd,bhtc->bhdc", k64 * w, v64)


# ---------------------------------------------------------------------------------------
# The delta rule (DeltaNet) and its gated form.

def delta_gate(log_alpha, B: int, H: int, L: int):
    """Broadcast a per-token ``[B,H,L]`` or fixed per-head ``[H]`` log decay to ``[B,H,L]``
    (fp64), or None."""
    if log_alpha is None:
        return None
    a = _f64(log_alpha)
    if a.shape == (H,) and (B, H, L) != (H,):
        return np.ascontiguousarray(np.broadcast_to(a[None, :, None], (B, H, L)))
    assert a.shape == (B, H, L), a.shape
    return a


def delta_recurrent(q, k, v, beta, log_alpha=None, initial_state=None, lib=None):
    """The delta rule, token by token in C (``gla_oracle_delta``): with
    ``S' = alpha_t S_{t-1}``, ``S_t = S' + beta_t k_t^T (v_t - k_t S')`` and
    ``o_t = q_t S_t`` -- one gradient step of size beta_t on ``1/2 |k_t S - v_t|^2``
    [Hardware-Efficient Training of Linear Attention Models, talk summary, 22:36 and 31:16].
    ``beta`` is ``[B,H,L]``; ``log_alpha`` ``[B,H,L]``, ``[H]`` or None (DeltaNet).
    Returns ``(out [B,H,L,Dv], final_state [B,H,Dk,Dv])`` in fp64."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    assert k64.shape == q64.shape and v64.shape == (B, H, L, Dv)
    b64 = _f64(beta)
    assert b64.shape == (B, H, L), b64.shape
    la = delta_gate(log_alpha, B, H, L)
    s0 = _f64(initial_state)
    if s0 is not None:
        assert s0.shape == (B, H, Dk, Dv)
    out = np.empty((B, H, L, Dv))
    fin = np.empty((B, H, Dk, Dv))
    dp = ctypes.POINTER(ctypes.c_double)

    def p(a):
        return None if a is None else a.ctypes.data_as(dp)

    rc = (lib or _load()).gla_oracle_delta(p(q64), p(k64), p(v64), p(b64), p(la), p(s0), p(out), p(fin),
                                           B, H, L, Dk, Dv)
    if rc != 0:
        raise RuntimeError("gla_oracle_delta failed (%d)" % rc)
    return out, fin


def delta_chunkwise_form(q, k, v, beta, chunk: int, log_alpha=None, initial_state=None):
    """The delta rule computed chunkwise with the WY representation, plainly (fp64).

    The talk (31:16) names the obstacle -- the cumulative product of identity-plus-rank-one
    transitions -- and the remedy: the WY representation turns that product into a sum,
    so the chunkwise algorithm (11:58) applies.  Written out for one chunk of n tokens
    entering with state ``S0``: with ``b`` the inclusive running sum of the log decay
    inside the chunk and ``g = exp(b)``, every token's update is
    ``S_t = alpha_t S_{t-1} + k_t^T u_t`` with ``u_t = beta_t (v_t - alpha_t k_t S_{t-1})``;
    unrolling, ``S_t = g_t S0 + sum_{i<=t} (g_t / g_i) k_i^T u_i``, so the u_t satisfy the
    unit lower-triangular system

        u_t + beta_t sum_{i<t} (g_t / g_i) (k_t . k_i) u_i = beta_t (v_t - g_t k_t S0),

    i.e. ``(I + A) U = diag(beta) (V - diag(g) K S0)``.  With ``T = (I + A)^-1 diag(beta)``
    (the WY factor): ``U = T V - (T diag(g) K) S0``, and

        O     = diag(g) Q S0 + ((Q K^T) * [g_t / g_i]_{i<=t}) U
        S_out = g_n S0 + (diag(g_n / g) K)^T U .

    Tiny inputs only.  Returns ``(out, final_state)``."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    b64 = _f64(beta)
    la = delta_gate(log_alpha, B, H, L)
    if la is None:
        la = np.zeros((B, H, L))
    s0 = None if initial_state is None else _f64(initial_state)
    out = np.zeros((B, H, L, Dv))
    fin = np.zeros((B, H, Dk, Dv))
    for bb in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if s0 is None else s0[bb, h].copy()
            for c0 in range(0, L, chunk):
                c1 = min(L, c0 + chunk)
                n = c1 - c0
                Q, K, V = q64[bb, h, c0:c1], k64[bb, h, c0:c1], v64[bb, h, c0:c1]
                be = b64[bb, h, c0:c1]
                bcum = np.cumsum(la[bb, h, c0:c1])
                g = np.exp(bcum)
                ratio = np.exp(bcum[:, None] - bcum[None, :])  # g_t / g_i, used where i <= t
                strict = np.tril(np.ones((n, n)), -1)
                incl = np.tril(np.ones((n, n)))
                A = be[:, None] * ratio * (K @ K.T) * strict
                T = np.linalg.solve(np.eye(n) + A, np.diag(be))
                U = T @ V - (T @ (g[:, None] * K)) @ S
                out[bb, h, c0:c1] = (g[:, None] * Q) @ S + ((Q @ K.T) * ratio * incl) @ U
                S = g[-1] * S + ((g[-1] / g)[:, None] * K).T @ U
            fin[bb, h] = S
    return out, fin


# ---------------------------------------------------------------------------------------
# The mLSTM with exponential input gate and normaliser.

def _mlstm_gates(log_f, log_i, B: int, H: int, L: int):
    lf, li = _f64(log_f), _f64(log_i)
    assert lf.shape == (B, H, L) and li.shape == (B, H, L), (lf.shape, li.shape)
    return lf, li


def mlstm_recurrent(q, k, v, log_f, log_i, initial_state=None, lib=None):
    """The mLSTM token recurrence in C (``gla_oracle_mlstm``), unstabilised fp64:
    ``C_t = f_t C_{t-1} + i_t k_t^T v_t``, ``n_t = f_t n_{t-1} + i_t k_t``,
    ``h_t = q_t C_t / max(|q_t . n_t|, 1)``, ``f_t = exp(log_f_t)``, ``i_t = exp(log_i_t)``
    [Tiled Flash Linear Attention, abstract, citing the mLSTM of Beck et al. (2024)].
    ``log_f``, ``log_i``: ``[B,H,L]``.  ``initial_state``: ``(C0 [B,H,Dk,Dv], n0 [B,H,Dk])`` in
    the unstabilised scale, or None.  Returns ``(h [B,H,L,Dv], C_L, n_L)``."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    assert k64.shape == q64.shape and v64.shape == (B, H, L, Dv)
    lf, li = _mlstm_gates(log_f, log_i, B, H, L)
    C0 = n0 = None
    if initial_state is not None:
        C0, n0 = _f64(initial_state[0]), _f64(initial_state[1])
        assert C0.shape == (B, H, Dk, Dv) and n0.shape == (B, H, Dk)
    out = np.empty((B, H, L, Dv))
    finC = np.empty((B, H, Dk, Dv))
    finN = np.empty((B, H, Dk))
    dp = ctypes.POINTER(ctypes.c_double)

    def p(a):
        return None if a is None else a.ctypes.data_as(dp)

    rc = (lib or _load()).gla_oracle_mlstm(p(q64), p(k64), p(v64), p(lf), p(li), p(C0), p(n0), p(out), p(finC),
                                           p(finN), B, H, L, Dk, Dv)
    if rc != 0:
        raise RuntimeError("gla_oracle_mlstm failed (%d)" % rc)
    return out, finC, finN


def mlstm_parallel_form(q, k, v, log_f, log_i, initial_state=None):
    """The mLSTM as causal pairwise weights (fp64, tiny inputs): with ``F`` the running sum
    of ``log_f`` from the sequence start, token s reaches token t >= s with weight
    ``D_ts = exp(F_t - F_s + log_i_s)``; ``W = (Q K^T) * D`` (causal), and
    ``h = (W V + e^F Q C0) / max(|W 1 + e^F Q n0|, 1)`` row by row.  Returns ``h``."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    lf, li = _mlstm_gates(log_f, log_i, B, H, L)
    out = np.zeros((B, H, L, Dv))
    causal = np.tril(np.ones((L, L), dtype=bool))
    for bb in range(B):
        for h in range(H):
            F = np.cumsum(lf[bb, h])
            logD = F[:, None] - F[None, :] + li[bb, h][None, :]
            D = np.where(causal, np.exp(np.where(causal, logD, 0.0)), 0.0)
            Q, K, V = q64[bb, h], k64[bb, h], v64[bb, h]
            W = (Q @ K.T) * D
            num = W @ V
            den = W.sum(axis=1)
            if initial_state is not None:
                C0, n0 = _f64(initial_state[0])[bb, h], _f64(initial_state[1])[bb, h]
                eF = np.exp(F)
                num = num + eF[:, None] * (Q @ C0)
                den = den + eF * (Q @ n0)
            out[bb, h] = num / np.maximum(np.abs(den), 1.0)[:, None]
    return out


def mlstm_stabilized_recurrent(q, k, v, log_f, log_i, initial_state=None):
    """The max-stabilised mLSTM recurrence (fp64, tiny inputs): the running maximum
    ``m_t = max(log_f_t + m_{t-1}, log_i_t)`` rescales memory and normaliser to
    ``C'_t = C_t e^{-m_t}``, ``n'_t = n_t e^{-m_t}``, whose updates take the gates
    ``exp(log_f_t + m_{t-1} - m_t)`` and ``exp(log_i_t - m_t)`` (both at most 1); the read is
    ``q_t C'_t / max(|q_t . n'_t|, e^{-m_t})``, the same value as the unstabilised read.
    ``initial_state``: ``(C0', n0', m0)`` stabilised, or None (``m`` starts at -inf).
    Returns ``(h, C'_L, n'_L, m_L)``."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    lf, li = _mlstm_gates(log_f, log_i, B, H, L)
    out = np.zeros((B, H, L, Dv))
    finC = np.zeros((B, H, Dk, Dv))
    finN = np.zeros((B, H, Dk))
    finM = np.zeros((B, H))
    for bb in range(B):
        for h in range(H):
            if initial_state is None:
                C, n, m = np.zeros((Dk, Dv)), np.zeros(Dk), -np.inf
            else:
                C = _f64(initial_state[0])[bb, h].copy()
                n = _f64(initial_state[1])[bb, h].copy()
                m = float(_f64(initial_state[2])[bb, h])
            for t in range(L):
                m_new = max(lf[bb, h, t] + m, li[bb, h, t])
                fp = np.exp(lf[bb, h, t] + m - m_new)
                ip = np.exp(li[bb, h, t] - m_new)
                kt, vt, qt = k64[bb, h, t], v64[bb, h, t], q64[bb, h, t]
                C = fp * C + ip * np.outer(kt, vt)
                n = fp * n + ip * kt
                m = m_new
                out[bb, h, t] = (qt @ C) / max(abs(qt @ n), np.exp(-m))
            finC[bb, h], finN[bb, h], finM[bb, h] = C, n, m
    return out, finC, finN, finM


def mlstm_chunkwise_form(q, k, v, log_f, log_i, chunk: int, initial_state=None):
    """The stabilised mLSTM computed chunkwise, plainly (fp64, tiny inputs).

    A chunk enters with the stabilised state ``(C', n', m)``.  Inside it, with ``b`` the
    inclusive running sum of ``log_f`` and ``a_s = log_i_s - b_s``, token s reaches row t >= s
    with log weight ``b_t + a_s`` and the entering state reaches it with ``b_t + m``; the row's
    stabiliser is ``m_t = b_t + M_t`` with ``M_t = max(m, max_{s<=t} a_s)``, so every factor
    below is at most 1:

        num_t = e^{m - M_t} q_t C' + sum_{s<=t} e^{a_s - M_t} (q_t . k_s) v_s
        den_t = e^{m - M_t} q_t . n' + sum_{s<=t} e^{a_s - M_t} (q_t . k_s)
        h_t   = num_t / max(|den_t|, e^{-m_t})

    and at the chunk end (``M_e`` the last row's maximum)
    ``C' <- e^{m - M_e} C' + K^T diag(e^{a - M_e}) V``, ``n' <- e^{m - M_e} n' + K^T e^{a - M_e}``,
    ``m <- b_last + M_e``.  This is the chunkwise algorithm [Hardware-Efficient Training of
    Linear Attention Models, talk summary, 11:58] with the mLSTM's running maximum carried
    across chunks.  ``initial_state`` as in :func:`mlstm_stabilized_recurrent`.
    Returns ``(h, C'_L, n'_L, m_L)``."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, L, Dk = q64.shape
    Dv = v64.shape[-1]
    lf, li = _mlstm_gates(log_f, log_i, B, H, L)
    out = np.zeros((B, H, L, Dv))
    finC = np.zeros((B, H, Dk, Dv))
    finN = np.zeros((B, H, Dk))
    finM = np.zeros((B, H))
    for bb in range(B):
        for h in range(H):
            if initial_state is None:
                C, n, m = np.zeros((Dk, Dv)), np.zeros(Dk), -np.inf
            else:
                C = _f64(initial_state[0])[bb, h].copy()
                n = _f64(initial_state[1])[bb, h].copy()
                m = float(_f64(initial_state[2])[bb, h])
            for c0 in range(0, L, chunk):
                c1 = min(L, c0 + chunk)
                Q, K, V = q64[bb, h, c0:c1], k64[bb, h, c0:c1], v64[bb, h, c0:c1]
                b = np.cumsum(lf[bb, h, c0:c1])
                a = li[bb, h, c0:c1] - b
                M = np.maximum(np.maximum.accumulate(a), m)
                inter = np.exp(m - M)
                causal = np.tril(np.ones((c1 - c0, c1 - c0), dtype=bool))
                Wt = np.where(causal, np.exp(np.where(causal, a[None, :] - M[:, None], 0.0)), 0.0)
                P = (Q @ K.T) * Wt
                num = inter[:, None] * (Q @ C) + P @ V
                den = inter * (Q @ n) + P.sum(axis=1)
                out[bb, h, c0:c1] = num / np.maximum(np.abs(den), np.exp(-(b + M)))[:, None]
                Me = M[-1]
                w = np.exp(a - Me)
                e = np.exp(m - Me)
                C = e * C + K.T @ (w[:, None] * V)
                n = e * n + K.T @ w
                m = b[-1] + Me
            finC[bb, h], finN[bb, h], finM[bb, h] = C, n, m
    return out, finC, finN, finM
