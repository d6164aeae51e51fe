"""Seeded synthetic inputs for the KDA forward workloads.

This module only draws random numbers and casts them to the storage types the
library consumes (bf16 as raw uint16 bit patterns, fp32, int32 offsets).  It
holds none of the method's arithmetic, so both the fp64 oracle and the GPU
tests can draw identical bits from it without sharing any computation.

Workload shapes follow the pages' interface description ("How to Use FlashKDA
as a Backend for flash-linear-attention", section "Kernel API and Tensor
Requirements": q/k/v/g bf16 [B,T,H,128], beta bf16 [B,T,H], A_log fp32 [H],
dt_bias fp32 [H,128], lower_bound in [-5,0]; section "State Handling and
Variable-Length Batches": state [N,H,V,K], varlen needs B=1) and the irregular
varlen lengths discussed on the cuLA PR #106 page (1023, 1025, 65537, 64K+kx1K).

Draw order per call (numpy Generator(PCG64(seed)), fp32 standard normals times
the stated standard deviation): q, k, v, g, beta, A_log, dt_bias, initial_state.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

HEAD_DIM = 128  # K = V = 128 is the only head size the interface accepts


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = (u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    return out.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (used for reporting only)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One synthetic KDA forward problem."""

    name: str
    B: int
    T: int
    H: int
    seqlens: Optional[Sequence[int]]  # None => fixed length (N = B)
    lower_bound: float
    scale: float
    init_std: Optional[float]  # None => no initial state
    state_dtype: str  # "fp32" or "bf16"
    want_final: bool
    seed: int
    a_log_std: float = 1.0
    dt_bias_std: float = 0.1
    x_std: float = 1.0  # q, k, v, g, beta
    note: str = ""

    @property
    def N(self) -> int:
        return len(self.seqlens) if self.seqlens is not None else self.B

    @property
    def total_tokens(self) -> int:
        return self.B * self.T

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "B": self.B,
            "T": self.T,
            "H": self.H,
            "D": HEAD_DIM,
            "num_seqs": self.N,
            "seqlens": list(self.seqlens) if self.seqlens is not None else None,
            "lower_bound": self.lower_bound,
            "scale": self.scale,
            "initial_state": None if self.init_std is None else f"{self.state_dtype}~N(0,{self.init_std})",
            "final_state": self.state_dtype if self.want_final else None,
            "seed": self.seed,
        }


def _varlen(name, seqlens, **kw) -> Workload:
    return Workload(name=name, B=1, T=int(sum(seqlens)), seqlens=list(seqlens), **kw)


INV_SQRT_D = 1.0 / math.sqrt(HEAD_DIM)

# The five workloads; "N(0,s)" means standard deviation s.
WORKLOADS = {
    "cfg1": Workload("kda_fwd_B1_T256_H2", B=1, T=256, H=2, seqlens=None, lower_bound=-5.0,
                     scale=INV_SQRT_D, init_std=None, state_dtype="fp32", want_final=True, seed=1),
    "cfg2": Workload("kda_fwd_B2_T4096_H16", B=2, T=4096, H=16, seqlens=None, lower_bound=-3.0,
                     scale=0.125, init_std=0.05, state_dtype="fp32", want_final=True, seed=2),
    "cfg3": _varlen("kda_fwd_varlen7_H16", [1023, 1025, 1, 16, 4097, 8191, 65537], H=16,
                    lower_bound=-5.0, scale=INV_SQRT_D, init_std=0.05, state_dtype="bf16",
                    want_final=True, seed=3),
    "cfg4a": Workload("kda_fwd_B1_T65536_H16", B=1, T=65536, H=16, seqlens=None, lower_bound=-5.0,
                      scale=INV_SQRT_D, init_std=0.05, state_dtype="fp32", want_final=True, seed=4),
    "cfg4b": _varlen("kda_fwd_varlen_65536+5x1024_H16", [65536] + [1024] * 5, H=16, lower_bound=-5.0,
                     scale=INV_SQRT_D, init_std=0.05, state_dtype="fp32", want_final=True, seed=4),
    "cfg5": Workload("kda_fwd_B8_T8192_H32", B=8, T=8192, H=32, seqlens=None, lower_bound=-1.0,
                     scale=INV_SQRT_D, init_std=0.05, state_dtype="fp32", want_final=True, seed=5),
    # the long sequence with slowly decaying state (the gate's lower bound near 0): the regime in
    # which a segment's transition M does not underflow to zero
    "cfg4a_slow": Workload("kda_fwd_B1_T65536_H16_lb0.1", B=1, T=65536, H=16, seqlens=None, lower_bound=-0.1,
                           scale=INV_SQRT_D, init_std=0.05, state_dtype="fp32", want_final=True, seed=4),
    # no decay at all (lower bound 0): no segment's transition M ever vanishes, so every merge
    # multiplies by the M of each earlier segment
    "cfg4a_nodecay": Workload("kda_fwd_B1_T65536_H16_lb0", B=1, T=65536, H=16, seqlens=None, lower_bound=0.0,
                              scale=INV_SQRT_D, init_std=0.05, state_dtype="fp32", want_final=True, seed=4),
}


def custom(B=1, T=64, H=2, seqlens=None, lower_bound=-5.0, scale=INV_SQRT_D, init_std=0.05,
           state_dtype="fp32", want_final=True, seed=0, name="custom", **kw) -> Workload:
    if seqlens is not None:
        return _varlen(name, seqlens, H=H, lower_bound=lower_bound, scale=scale, init_std=init_std,
                       state_dtype=state_dtype, want_final=want_final, seed=seed, **kw)
    return Workload(name, B=B, T=T, H=H, seqlens=None, lower_bound=lower_bound, scale=scale,
                    init_std=init_std, state_dtype=state_dtype, want_final=want_final, seed=seed, **kw)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_inputs(w: Workload) -> dict:
    """Draw the workload's tensors.

    bf16 tensors are returned as uint16 bit patterns, fp32 tensors as float32,
    cu_seqlens as int32 (None for fixed length).  scale and lower_bound are
    returned as the fp32 values a kernel receives.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shp = (w.B, w.T, w.H, HEAD_DIM)
    out = {}
    for name in ("q", "k", "v", "g"):
        out[name] = f32_to_bf16_bits(_normal(rng, shp, w.x_std))
    out["beta"] = f32_to_bf16_bits(_normal(rng, (w.B, w.T, w.H), w.x_std))
    out["A_log"] = _normal(rng, (w.H,), w.a_log_std)
    out["dt_bias"] = _normal(rng, (w.H, HEAD_DIM), w.dt_bias_std)
    if w.init_std is not None:
        s = _normal(rng, (w.N, w.H, HEAD_DIM, HEAD_DIM), w.init_std)
        out["initial_state"] = f32_to_bf16_bits(s) if w.state_dtype == "bf16" else s
    else:
        out["initial_state"] = None
    if w.seqlens is not None:
        cu = np.zeros(len(w.seqlens) + 1, dtype=np.int64)
        cu[1:] = np.cumsum(np.asarray(w.seqlens, dtype=np.int64))
        out["cu_seqlens"] = cu.astype(np.int32)
    else:
        out["cu_seqlens"] = None
    out["scale"] = float(np.float32(w.scale))
    out["lower_bound"] = float(np.float32(w.lower_bound))
    return out


def make_device_inputs(w: Workload, device, rows_per_draw: int = 16) -> dict:
    """Draw a fixed-length workload's tensors on a device, for sizes whose
    host draw would take minutes (billions of elements).

    q, k, v, g, beta and the initial state come from torch's generator of that
    device, seeded with w.seed and drawn in that order: fp32 standard normals
    times the stated standard deviation, rounded to bf16 (nearest, ties to
    even) where the tensor is bf16, drawn over the batch dimension in pieces of
    rows_per_draw rows so that the fp32 draw stays small.  A_log and dt_bias
    are small and come from numpy as in make_inputs (PCG64(w.seed), in that
    order).  Device tensors are torch tensors (bf16 as torch.bfloat16); A_log
    and dt_bias are returned as float32 numpy arrays, to be moved by the
    caller.  A check against the oracle reads the slices it needs back from
    the device: those are the inputs, not results.
    """
    import torch

    if w.seqlens is not None:
        raise ValueError("make_device_inputs draws fixed-length workloads (view the result as B = 1 for varlen)")
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed))

    def draw(shape, std, dtype):
        t = torch.empty(shape, dtype=dtype, device=device)
        for r0 in range(0, shape[0], rows_per_draw):
            r1 = min(shape[0], r0 + rows_per_draw)
            x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen, device=device, dtype=torch.float32)
            if std != 1.0:
                x.mul_(std)
            t[r0:r1] = x.to(dtype)
            del x
        return t

    out = {}
    shp = (w.B, w.T, w.H, HEAD_DIM)
    for name in ("q", "k", "v", "g"):
        out[name] = draw(shp, w.x_std, torch.bfloat16)
    out["beta"] = draw((w.B, w.T, w.H), w.x_std, torch.bfloat16)
    if w.init_std is not None:
        sdt = torch.bfloat16 if w.state_dtype == "bf16" else torch.float32
        out["initial_state"] = draw((w.N, w.H, HEAD_DIM, HEAD_DIM), w.init_std, sdt)
    else:
        out["initial_state"] = None
    rng = np.random.Generator(np.random.PCG64(w.seed))
    out["A_log"] = _normal(rng, (w.H,), w.a_log_std)
    out["dt_bias"] = _normal(rng, (w.H, HEAD_DIM), w.dt_bias_std)
    out["cu_seqlens"] = None
    out["scale"] = float(np.float32(w.scale))
    out["lower_bound"] = float(np.float32(w.lower_bound))
    return out
