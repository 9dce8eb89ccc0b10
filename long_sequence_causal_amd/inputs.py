"""Seeded synthetic inputs and the named workloads.

This module serves both the HIP path's tests and the CPU oracle's; it holds
no arithmetic of the method itself, only shapes, seeds and random draws.

Recipe (the same for every workload):
  * one ``torch.Generator`` on the target device, seeded with the workload's
    seed, draws float32 standard normals in the fixed order q, k, v, S0, dO;
  * q and k are scaled by 1/sqrt(d_k), S0 by its stated standard deviation,
    v and dO are left at unit variance;
  * Q, K, V, dO are then rounded (round-to-nearest-even) to the workload's
    dtype; S0 stays float32;
  * the per-head decay is lambda_h = exp(-2^-(5 + 8 h / H)), h = 0..H-1,
    evaluated in float64 and rounded to float32 (or 1 for the undecayed
    workload); the float32 value is the input of record on both sides.
Tensors larger than one draw are drawn in slabs of whole (b, h) heads, in
index order, so the result depends only on the seed and the shape.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    dtype: str            # "bf16" or "fp32"
    decay: bool           # False: lambda = 1 for every head
    s0_std: float         # 0.0: zero initial state (passed as NULL)
    nseg: int = 1         # independent segments per (b, h) sequence
    backward: bool = False
    seed: int = 0
    note: str = ""


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", B=1, H=2, L=1024, d=64, dtype="fp32", decay=False,
                 s0_std=0.0, seed=1,
                 note="tiny fp32 case, no decay, S0=0"),
        Workload("decay_16k", B=2, H=16, L=16384, d=128, dtype="bf16", decay=True,
                 s0_std=0.0, seed=2,
                 note="per-head decay, bf16 inputs, fp32 state, S0=0"),
        Workload("segment_64k", B=1, H=32, L=65536, d=128, dtype="bf16", decay=True,
                 s0_std=0.02, seed=3,
                 note="one 64K-token segment of a longer sequence, S0 ~ N(0, 0.02^2)"),
        Workload("segmented_1m", B=1, H=16, L=1 << 20, d=128, dtype="bf16", decay=True,
                 s0_std=0.0, nseg=64, seed=4,
                 note="1M tokens as 64 segments of 16384, combined by the state scan"),
        Workload("train_256k", B=1, H=16, L=262144, d=128, dtype="bf16", decay=True,
                 s0_std=0.0, backward=True, seed=2,
                 note="forward + backward, dO ~ N(0,1), dS_end = 0, inputs drawn as the 16K decay case"),
    ]
}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def decay_schedule(H: int, decay: bool = True) -> torch.Tensor:
    """lambda_h = exp(-2^-(5 + 8h/H)) in float64, rounded to float32."""
    if not decay:
        return torch.ones(H, dtype=torch.float32)
    vals = [math.exp(-(2.0 ** (-(5.0 + 8.0 * h / H)))) for h in range(H)]
    return torch.tensor(vals, dtype=torch.float64).to(torch.float32)


def _draw(gen, shape, scale, dtype, device):
    """Standard normals of ``shape`` drawn head by head, scaled, then cast."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1, *shape[-2:]) if len(shape) > 2 else out.view(1, *shape)
    for i in range(flat.shape[0]):
        x = torch.randn(flat.shape[1:], generator=gen, dtype=torch.float32, device=device)
        if scale != 1.0:
            x.mul_(scale)
        flat[i].copy_(x)
    return out


def make_inputs(B: int, H: int, L: int, dk: int, dv: int, *, dtype: str = "bf16",
                decay: bool = True, s0_std: float = 0.0, nseg: int = 1,
                need_dO: bool = False, dS_end_std: float = 0.0, seed: int = 0,
                device="cpu", lam: Optional[torch.Tensor] = None):
    """Draw one seeded input set.

    Returns a dict with q, k, v (dtype), lam [H] float32, S0 ([B,H,nseg,dk,dv]
    float32 or None), dO (dtype or None) and dS_end (float32 or None).
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    td = torch_dtype(dtype)
    qk_scale = 1.0 / math.sqrt(dk)
    q = _draw(gen, (B, H, L, dk), qk_scale, td, dev)
    k = _draw(gen, (B, H, L, dk), qk_scale, td, dev)
    v = _draw(gen, (B, H, L, dv), 1.0, td, dev)
    S0 = None
    if s0_std > 0.0:
        S0 = _draw(gen, (B, H, nseg, dk, dv), float(s0_std), torch.float32, dev)
    dO = _draw(gen, (B, H, L, dv), 1.0, td, dev) if need_dO else None
    dS_end = None
    if dS_end_std > 0.0:
        dS_end = _draw(gen, (B, H, nseg, dk, dv), float(dS_end_std), torch.float32, dev)
    if lam is None:
        lam = decay_schedule(H, decay)
    return {"q": q, "k": k, "v": v, "lam": lam.to(dev), "S0": S0, "dO": dO,
            "dS_end": dS_end}


def gate_logs(lam: torch.Tensor, B: int, L: int, seed: int, device="cpu") -> torch.Tensor:
    """Seeded per-token log-gates g = log(alpha) [B, H, L] float32 for the
    gated recurrence: g[b, h, t] = log(lam_h) * 2 sigmoid(z), z ~ N(0, 1) --
    on average the head's fixed decay, varying per token within
    (2 log lam_h, 0).  A separate generator stream (seed + 7919) leaves the
    other inputs of a seed unchanged."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed) + 7919)
    H = lam.numel()
    z = torch.randn((B, H, L), generator=gen, device=dev, dtype=torch.float32)
    loglam = torch.log(lam.to(dev, torch.float64)).to(torch.float32).view(1, H, 1)
    return (loglam * (2.0 * torch.sigmoid(z))).contiguous()


# Decode workloads: one new token for each of B sequences x H heads, with a
# carried state.  Drawn like the sequence workloads (q, k scaled by
# 1/sqrt(d), v at unit variance, rounded to the dtype), in the order q, k, v,
# S; the state S ~ N(0, s_std^2) fp32 stands for the state a prefill left.
DECODE = {
    "decode_b64": dict(B=64, H=32, d=128, dtype="bf16", s_std=0.02, seed=5,
                       note="one decode step of 64 sequences x 32 heads, d = 128"),
    # 1 GiB of fp32 state, four times the 256 MB last-level cache: a step
    # streams its state from HBM however often it is repeated
    "decode_b512": dict(B=512, H=32, d=128, dtype="bf16", s_std=0.02, seed=6,
                        note="one decode step of 512 sequences x 32 heads, d = 128"),
}


def decode_inputs(name: str, device="cpu"):
    """Inputs of a named decode workload: q, k [B,H,d], v [B,H,d] (dtype),
    lam [H] float32 (the per-head schedule), S [B,H,d,d] float32."""
    w = DECODE[name]
    B, H, d = w["B"], w["H"], w["d"]
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(w["seed"]))
    td = torch_dtype(w["dtype"])
    q = _draw(gen, (B, H, d), 1.0 / math.sqrt(d), td, dev)
    k = _draw(gen, (B, H, d), 1.0 / math.sqrt(d), td, dev)
    v = _draw(gen, (B, H, d), 1.0, td, dev)
    S = _draw(gen, (B, H, d, d), float(w["s_std"]), torch.float32, dev)
    return {"q": q, "k": k, "v": v, "lam": decay_schedule(H).to(dev), "S": S}


def workload_inputs(name: str, device="cpu", **over):
    """Inputs of a named workload (keyword overrides allowed, e.g. L=...)."""
    w = WORKLOADS[name]
    kw = dict(B=w.B, H=w.H, L=w.L, dk=w.d, dv=w.d, dtype=w.dtype, decay=w.decay,
              s0_std=w.s0_std, nseg=1, need_dO=w.backward, seed=w.seed)
    kw.update(over)
    B, H, L, dk, dv = (kw.pop(x) for x in ("B", "H", "L", "dk", "dv"))
    return make_inputs(B, H, L, dk, dv, device=device, **kw)
