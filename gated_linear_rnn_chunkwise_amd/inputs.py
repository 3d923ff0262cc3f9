"""Seeded synthetic workloads for the gated linear attention forward pass.

This module only draws random inputs; it holds none of the method's arithmetic and is
shared by the GPU tests, the oracle tests and the benchmark.  Every tensor is drawn on
the CPU with a ``torch.Generator`` seeded explicitly, so the same (workload, seed) gives
the same bytes on any machine.

Recipe (per workload): draw ``q``, ``k``, ``v`` in that order as fp32 N(0, 1), divide by
``sqrt(scale_dim)`` in fp32, and round to the input dtype (bf16 rounds to nearest even);
then draw the gate pre-activations.  Gates are stored as fp32 logs:

* ``channel``: ``log_alpha = logsigmoid(x) / 16``, ``x ~ N(0, 1)``, ``[B, H, L, Dk]``.
* ``head_const``: ``log_alpha[h] = log(1 - 2^(-5-h))`` rounded to fp32, ``[H]``
  (a fixed decay per head, RetNet style).
* ``head``: ``log_alpha = logsigmoid(a)``, ``a ~ N(3, 1)``, ``[B, H, L]`` and the input
  gate ``log_ig = logsigmoid(b)``, ``b ~ N(0, 1)``, ``[B, H, L]`` (sigmoid forget and
  input gates of the mLSTM variant).
* ``none``: no gate.

mLSTM workloads with exponential input gate and normaliser (``rule == "mlstm"``) draw ``q``
and ``v`` as fp32 N(0, 1) and ``k`` as N(0, 1) / sqrt(Dk) (the cell's key scaling), rounded to
the input dtype, then ``log_f = logsigmoid(a)``, ``a ~ N(3, 1)`` (sigmoid forget gate) and
``log_i ~ N(0, ig_std^2)`` (the exponential input gate's pre-activation), both ``[B, H, L]``
fp32.

Delta-rule workloads (``rule == "delta"``) draw ``q`` and ``k`` uniformly on the unit sphere
(fp32 N(0, 1) rows divided by their L2 norm in fp32, then rounded to the input dtype), ``v``
as above, then the writing strength ``beta = sigmoid(x)``, ``x ~ N(0, 1)``, ``[B, H, L]``
fp32, then the gate (``head``: ``log_alpha = logsigmoid(a)``, ``a ~ N(3, 1)``; Gated
DeltaNet) or none (DeltaNet).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    Dk: int
    Dv: int
    chunk: int
    dtype: str = "bf16"          # q, k, v dtype: "bf16" or "f32"
    gate: str = "none"           # none | channel | head | head_const
    input_gate: bool = False     # log input gate [B, H, L]
    scale_dim: Optional[int] = None  # inputs are N(0,1)/sqrt(scale_dim); default Dk
    final_state: bool = True
    gate_shift: float = 3.0      # mean of the forget pre-activation for gate == "head"
    channel_gate_div: float = 16.0
    rule: str = "linear"         # "linear": S_t = diag(alpha_t) S_{t-1} + i_t k_t^T v_t;
                                 # "delta": the delta rule with writing strength beta_t;
                                 # "mlstm": exponential input gate and normaliser
    ig_std: float = 1.0          # std of the mLSTM log input gate

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.L


# The five workloads the method is measured on (sizes, dtypes, gate kinds and chunk sizes).
WORKLOADS = {
    "ungated_f32_L256": Workload("ungated_f32_L256", 1, 1, 256, 64, 64, 64, dtype="f32", gate="none"),
    "gla_bf16_B8H16L2048": Workload("gla_bf16_B8H16L2048", 8, 16, 2048, 128, 128, 64, gate="channel"),
    "retnet_bf16_B4H8L8192": Workload("retnet_bf16_B4H8L8192", 4, 8, 8192, 128, 128, 128, gate="head_const"),
    "long_gla_bf16_H16L32768_C64": Workload("long_gla_bf16_H16L32768_C64", 1, 16, 32768, 128, 128, 64,
                                             gate="channel"),
    "long_gla_bf16_H16L32768_C256": Workload("long_gla_bf16_H16L32768_C256", 1, 16, 32768, 128, 128, 256,
                                              gate="channel"),
    "mlstm_sig_bf16_B8H8L8192": Workload("mlstm_sig_bf16_B8H8L8192", 8, 8, 8192, 256, 512, 256, gate="head",
                                          input_gate=True, scale_dim=256),
}
HEADLINE = "gla_bf16_B8H16L2048"

# Delta-rule workloads (DeltaNet and Gated DeltaNet) at the headline shape.
DELTA_WORKLOADS = {
    "deltanet_bf16_B8H16L2048": Workload("deltanet_bf16_B8H16L2048", 8, 16, 2048, 128, 128, 64, gate="none",
                                         rule="delta"),
    "gated_deltanet_bf16_B8H16L2048": Workload("gated_deltanet_bf16_B8H16L2048", 8, 16, 2048, 128, 128, 64,
                                               gate="head", rule="delta"),
}

# The mLSTM with exponential input gate and normaliser at the sigmoid-gated mLSTM's head shape.
MLSTM_WORKLOADS = {
    "mlstm_exp_bf16_B8H8L8192": Workload("mlstm_exp_bf16_B8H8L8192", 8, 8, 8192, 256, 512, 64, gate="head",
                                         rule="mlstm"),
}


def _dt(name: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def make_inputs(w: Workload, seed: int = 0, device="cpu") -> dict:
    """Draw the inputs of workload ``w``.  Returns a dict with ``q, k, v`` (input dtype),
    ``log_alpha`` (fp32 or None), ``log_ig`` (fp32 or None) and ``sha256`` of all bytes."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    B, H, L, Dk, Dv = w.B, w.H, w.L, w.Dk, w.Dv
    sd = float(w.scale_dim or Dk)
    div = torch.tensor(math.sqrt(sd), dtype=torch.float32)
    dt = _dt(w.dtype)
    if w.rule == "delta":
        return _make_delta_inputs(w, g, div, dt, device)
    if w.rule == "mlstm":
        return _make_mlstm_inputs(w, g, dt, device)
    q = (torch.randn(B, H, L, Dk, generator=g, dtype=torch.float32) / div).to(dt)
    k = (torch.randn(B, H, L, Dk, generator=g, dtype=torch.float32) / div).to(dt)
    v = (torch.randn(B, H, L, Dv, generator=g, dtype=torch.float32) / div).to(dt)
    la = None
    li = None
    if w.gate == "channel":
        x = torch.randn(B, H, L, Dk, generator=g, dtype=torch.float32)
        la = torch.nn.functional.logsigmoid(x) / w.channel_gate_div
    elif w.gate == "head_const":
        la = torch.tensor([math.log1p(-(2.0 ** (-5 - h))) for h in range(H)], dtype=torch.float64).float()
    elif w.gate == "head":
        a = torch.randn(B, H, L, generator=g, dtype=torch.float32) + w.gate_shift
        la = torch.nn.functional.logsigmoid(a)
    elif w.gate != "none":
        raise ValueError(w.gate)
    if w.input_gate:
        b = torch.randn(B, H, L, generator=g, dtype=torch.float32)
        li = torch.nn.functional.logsigmoid(b)
    h = hashlib.sha256()
    for t in (q, k, v, la, li):
        if t is not None:
            h.update(t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype != torch.bfloat16
                     else t.contiguous().view(torch.int16).numpy().tobytes())
    out = dict(q=q, k=k, v=v, log_alpha=la, log_ig=li, sha256=h.hexdigest())
    if device != "cpu":
        for key in ("q", "k", "v", "log_alpha", "log_ig"):
            if out[key] is not None:
                out[key] = out[key].to(device)
    return out


def _unit_rows(x):
    return x / torch.sqrt((x * x).sum(dim=-1, keepdim=True))


def _make_delta_inputs(w: Workload, g, div, dt, device) -> dict:
    B, H, L, Dk, Dv = w.B, w.H, w.L, w.Dk, w.Dv
    q = _unit_rows(torch.randn(B, H, L, Dk, generator=g, dtype=torch.float32)).to(dt)
    k = _unit_rows(torch.randn(B, H, L, Dk, generator=g, dtype=torch.float32)).to(dt)
    v = (torch.randn(B, H, L, Dv, generator=g, dtype=torch.float32) / div).to(dt)
    beta = torch.sigmoid(torch.randn(B, H, L, generator=g, dtype=torch.float32))
    la = None
    if w.gate == "head":
        la = torch.nn.functional.logsigmoid(torch.randn(B, H, L, generator=g, dtype=torch.float32) + w.gate_shift)
    elif w.gate == "head_const":
        la = torch.tensor([math.log1p(-(2.0 ** (-5 - h))) for h in range(H)], dtype=torch.float64).float()
    elif w.gate != "none":
        raise ValueError("delta-rule workloads take a scalar gate, not %r" % w.gate)
    h = hashlib.sha256()
    for t in (q, k, v, beta, la):
        if t is not None:
            h.update(t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype != torch.bfloat16
                     else t.contiguous().view(torch.int16).numpy().tobytes())
    out = dict(q=q, k=k, v=v, beta=beta, log_alpha=la, log_ig=None, sha256=h.hexdigest())
    if device != "cpu":
        for key in ("q", "k", "v", "beta", "log_alpha"):
            if out[key] is not None:
                out[key] = out[key].to(device)
    return out


def _make_mlstm_inputs(w: Workload, g, dt, device) -> dict:
    B, H, L, Dk, Dv = w.B, w.H, w.L, w.Dk, w.Dv
    kdiv = torch.tensor(math.sqrt(Dk), dtype=torch.float32)
    q = torch.randn(B, H, L, Dk, generator=g, dtype=torch.float32).to(dt)
    k = (torch.randn(B, H, L, Dk, generator=g, dtype=torch.float32) / kdiv).to(dt)
    v = torch.randn(B, H, L, Dv, generator=g, dtype=torch.float32).to(dt)
    lf = torch.nn.functional.logsigmoid(torch.randn(B, H, L, generator=g, dtype=torch.float32) + w.gate_shift)
    li = torch.randn(B, H, L, generator=g, dtype=torch.float32) * w.ig_std
    h = hashlib.sha256()
    for t in (q, k, v, lf, li):
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype != torch.bfloat16
                 else t.contiguous().view(torch.int16).numpy().tobytes())
    out = dict(q=q, k=k, v=v, log_f=lf, log_i=li, log_alpha=None, log_ig=None, sha256=h.hexdigest())
    if device != "cpu":
        for key in ("q", "k", "v", "log_f", "log_i"):
            out[key] = out[key].to(device)
    return out


def custom(B, H, L, Dk, Dv, chunk, dtype="bf16", gate="channel", input_gate=False, **kw) -> Workload:
    """A workload of arbitrary shape with the same value distributions."""
    rule = kw.get("rule", "linear")
    return Workload("custom_B%dH%dL%dDk%dDv%dC%d_%s_%s%s" % (B, H, L, Dk, Dv, chunk, dtype, gate,
                                                           "" if rule == "linear" else "_" + rule),
                    B, H, L, Dk, Dv, chunk, dtype=dtype, gate=gate, input_gate=input_gate, **kw)
