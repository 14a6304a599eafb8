"""Seeded synthetic workloads: shapes, value distributions and decay schedules.

This module only draws inputs.  It holds none of the operator's arithmetic, so
both the HIP path and the fp64 oracle can be fed from it.

Recipe (identical for every workload):
  * ``torch.Generator`` on the CPU seeded with ``seed``;
  * draw q, k, v (then the decode state, if any) as float32 N(0, 1) in that
    order, multiply by the workload's scale in float32;
  * cast to the workload's dtype (bf16 by round-to-nearest-even);
  * gamma is a float32 vector with one entry per head.

The decay schedules follow the multi-scale retention of the RetNet page
(section "Multi-Scale Retention and Network Architecture"): gamma_h =
1 - 2^(-5-h); the long-sequence workload spreads the same exponent range over
32 heads as gamma_h = 1 - 2^(-5 - 4h/31).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    op: str              # "retention_fwd" | "linear_attn_fwd" | "retention_decode_step"
    B: int               # batch (decode: number of sequences N)
    H: int
    T: int               # sequence length (decode: 1)
    dk: int
    dv: int
    chunk: int           # chunk length (0 for decode)
    dtype: str           # "f32" | "bf16"
    scale: float         # multiplier applied to the N(0,1) draws of q, k, v
    gamma: str           # decay schedule name
    state_std: float = 0.0   # decode: std of the N(0, sigma^2) initial state
    steps: int = 1           # decode: consecutive steps timed
    description: str = ""

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "ret_fwd_tiny_f32": Workload(
        "ret_fwd_tiny_f32", "retention_fwd", B=1, H=1, T=256, dk=64, dv=64, chunk=64,
        dtype="f32", scale=1.0 / 8.0, gamma="const0.9",
        description="retention fwd fp32, batch 1, 1 head, T=256, d=64, gamma=0.9, chunk 64"),
    "ret_fwd_mh_f32": Workload(
        "ret_fwd_mh_f32", "retention_fwd", B=4, H=8, T=2048, dk=64, dv=64, chunk=64,
        dtype="f32", scale=1.0 / 8.0, gamma="msr",
        description="retention fwd fp32, batch 4, 8 heads, T=2048, d=64, "
                    "gamma_h=1-2^(-5-h), chunk 64, out + final state"),
    "linattn_elu1_bf16": Workload(
        "linattn_elu1_bf16", "linear_attn_fwd", B=8, H=16, T=8192, dk=64, dv=64,
        chunk=128, dtype="bf16", scale=1.0, gamma="one",
        description="causal linear attention phi=elu+1 with normaliser, bf16 in / fp32 "
                    "accumulate, batch 8, 16 heads, T=8192, d=64, chunk 128"),
    "ret_fwd_long_bf16": Workload(
        "ret_fwd_long_bf16", "retention_fwd", B=1, H=32, T=65536, dk=128, dv=128,
        chunk=128, dtype="bf16", scale=1.0 / math.sqrt(128.0), gamma="msr_spread",
        description="retention fwd bf16 in / fp32 accumulate, batch 1, 32 heads, "
                    "T=65536, d=128, gamma_h=1-2^(-5-4h/31), chunk 128"),
    "decode_bf16": Workload(
        "decode_bf16", "retention_decode_step", B=256, H=32, T=1, dk=128, dv=128, chunk=0,
        dtype="bf16", scale=1.0 / math.sqrt(128.0), gamma="msr_spread", state_std=0.1,
        steps=1000,
        description="recurrent decode step, fp32 state 128x128 per head, 256 sequences x "
                    "32 heads, bf16 q/k/v, 1000 consecutive steps"),
}


def gammas(schedule: str, H: int) -> np.ndarray:
    """Per-head decay values as float32."""
    h = np.arange(H, dtype=np.float64)
    if schedule == "const0.9":
        g = np.full(H, 0.9)
    elif schedule == "one":
        g = np.ones(H)
    elif schedule == "msr":
        g = 1.0 - 2.0 ** (-5.0 - h)
    elif schedule == "msr_spread":
        g = 1.0 - 2.0 ** (-5.0 - 4.0 * h / max(H - 1, 1))
    else:
        raise ValueError(f"unknown gamma schedule {schedule!r}")
    return g.astype(np.float32)


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Draw the workload's inputs on the CPU.

    Returns a dict with ``q``, ``k``, ``v`` (torch CPU tensors in the workload
    dtype), ``gamma`` (float32 numpy, one per head) and, for decode, ``state``
    (float32 torch CPU tensor).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    dt = torch_dtype(w.dtype)
    if w.op == "retention_decode_step":
        qk_shape = (w.B, w.H, w.dk)
        v_shape = (w.B, w.H, w.dv)
    else:
        qk_shape = (w.B, w.H, w.T, w.dk)
        v_shape = (w.B, w.H, w.T, w.dv)
    out = {}
    for name, shape in (("q", qk_shape), ("k", qk_shape), ("v", v_shape)):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if w.scale != 1.0:
            x.mul_(w.scale)
        out[name] = x.to(dt)
    if w.op == "retention_decode_step":
        s = torch.randn((w.B, w.H, w.dk, w.dv), generator=g, dtype=torch.float32)
        s.mul_(w.state_std)
        out["state"] = s
    out["gamma"] = gammas(w.gamma, w.H)
    return out
