"""Seeded synthetic inputs for the RWKV-6 WKV forward operator.

This module only draws random numbers and rounds them to the storage type
the workload asks for.  It holds none of the operator's arithmetic, so both
the CPU oracle (under ``oracle/``) and the HIP path can be fed from it
without sharing any of the computation being checked.

Workloads.  The shapes follow the pages: an image of 224x224 pixels cut into
16x16 patches gives T = 196 tokens at embedding width 192 with 3 heads (the
usage example on the "What is the WKV mechanism" page of deepglint/rwkv-clip,
section "Practical Usage Example"); the head size is 64 (the CUDA-kernels
page, section "Code Example", says 64 is the original head size).  The other
shapes scale the same operator up to a ViT-base-like width, to a 4096-token
text context and to a 64x64-patch image.  No dataset, trained weight or
benchmark item is involved: every tensor is drawn here.

Recipe (identical for every consumer):
  * ``rng = numpy.random.default_rng(seed)`` (PCG64);
  * draw, in this order, r, k, v ~ Normal(0, 0.5^2) and w_raw ~ Uniform(lo, hi),
    each of shape [B, T, C] in float64, then u ~ Normal(0, 0.5^2) of shape [C];
  * if the workload asks for "stuck" channels, draw
    ``rng.choice(C, floor(frac*C), replace=False)`` last and set w_raw of
    those channels to a fixed value for every (b, t);
  * cast to float32; for bf16 workloads round r, k, v, w_raw to bfloat16 by
    round-to-nearest-even.  u always stays float32.

The two older operators draw the same way with their own shapes:
  * RWKV-5 (``random_inputs_wkv5``): r, k, v as above, then w_raw ~
    Uniform(lo, hi) of shape [C] (one decay per channel), then u;
  * RWKV-4 (``random_inputs_wkv4``): k ~ Normal(0, kscale^2) and v ~
    Normal(0, 1) of shape [B, T, C], then the decay rates w ~ Uniform(w_lo,
    w_hi) and the bonuses u ~ Normal(0, 1), both [C] float32; bf16 rounds k
    and v only.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "make_inputs",
    "random_inputs",
    "round_to_bf16",
    "bf16_bits",
    "random_inputs_wkv5",
    "random_inputs_wkv4",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape, mode, storage dtype and draw recipe."""

    name: str
    mode: str            # "causal" or "bidirectional"
    dtype: str           # "f32" or "bf16" (storage type of r, k, v, w_raw)
    B: int
    T: int
    C: int
    H: int
    wraw_lo: float
    wraw_hi: float
    seed: int
    stuck_frac: float = 0.0      # fraction of channels whose w_raw is pinned
    stuck_value: float = 0.0     # the pinned w_raw value
    tolerance: float = 1e-4      # max|y - y_ref| / rms(y_ref)

    @property
    def N(self) -> int:
        return self.C // self.H

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def elements(self) -> int:
        return self.B * self.T * self.C

    def algorithmic_bytes(self) -> int:
        """Bytes the operator must move at minimum: read r, k, v, w_raw and u
        once, write the fp32 output once."""
        isz = 4 if self.dtype == "f32" else 2
        return self.elements * (4 * isz + 4) + self.C * 4

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["N"] = self.N
        return d


WORKLOADS: tuple[Workload, ...] = (
    Workload("tiny-causal-f32", "causal", "f32",
             B=1, T=64, C=128, H=2, wraw_lo=-6.0, wraw_hi=-0.5, seed=0,
             tolerance=1e-4),
    Workload("image-tiny-bidir-f32", "bidirectional", "f32",
             B=32, T=196, C=192, H=3, wraw_lo=-6.0, wraw_hi=-0.5, seed=1,
             tolerance=1e-4),
    Workload("image-base-bidir-bf16", "bidirectional", "bf16",
             B=64, T=196, C=768, H=12, wraw_lo=-6.0, wraw_hi=-0.5, seed=2,
             tolerance=5e-3),
    Workload("text-long-causal-bf16", "causal", "bf16",
             B=8, T=4096, C=2048, H=32, wraw_lo=-8.0, wraw_hi=-1.0, seed=3,
             tolerance=5e-3),
    Workload("image-hires-bidir-bf16", "bidirectional", "bf16",
             B=4, T=4096, C=1024, H=16, wraw_lo=-9.0, wraw_hi=-0.5, seed=4,
             stuck_frac=0.1, stuck_value=-9.0, tolerance=5e-3),
)


def workload(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(f"unknown workload {name!r}; known: {[w.name for w in WORKLOADS]}")


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); the result
    is returned as float32 holding exactly representable bfloat16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32)
    # NaN payloads are never produced by the draws; keep them NaN if present.
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("values are not bfloat16-representable; round first")
    return (bits >> 16).astype(np.uint16)


def random_inputs(B: int, T: int, C: int, H: int, *, seed: int, dtype: str = "f32",
                  wraw_lo: float = -6.0, wraw_hi: float = -0.5,
                  stuck_frac: float = 0.0, stuck_value: float = 0.0,
                  scale: float = 0.5) -> dict:
    """Draw one input set by the recipe in the module docstring.

    Returns a dict of float32 numpy arrays ``r, k, v, w_raw`` of shape
    [B, T, C] and ``u`` of shape [C], plus ``stuck`` (the pinned channel
    indices, possibly empty).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    if H <= 0 or C % H:
        raise ValueError("C must be a positive multiple of H")
    rng = np.random.default_rng(seed)
    shape = (B, T, C)
    r = rng.normal(0.0, scale, size=shape).astype(np.float32)
    k = rng.normal(0.0, scale, size=shape).astype(np.float32)
    v = rng.normal(0.0, scale, size=shape).astype(np.float32)
    w_raw = rng.uniform(wraw_lo, wraw_hi, size=shape).astype(np.float32)
    u = rng.normal(0.0, scale, size=(C,)).astype(np.float32)
    stuck = np.zeros((0,), dtype=np.int64)
    if stuck_frac > 0.0:
        n_stuck = int(math.floor(stuck_frac * C))
        stuck = np.sort(rng.choice(C, n_stuck, replace=False))
        w_raw[:, :, stuck] = np.float32(stuck_value)
    if dtype == "bf16":
        r, k, v, w_raw = (round_to_bf16(a) for a in (r, k, v, w_raw))
    return {"r": r, "k": k, "v": v, "w_raw": w_raw, "u": u, "stuck": stuck}


def make_inputs(w: Workload | str) -> dict:
    """Inputs of one named workload."""
    if isinstance(w, str):
        w = workload(w)
    return random_inputs(w.B, w.T, w.C, w.H, seed=w.seed, dtype=w.dtype,
                         wraw_lo=w.wraw_lo, wraw_hi=w.wraw_hi,
                         stuck_frac=w.stuck_frac, stuck_value=w.stuck_value)


def random_inputs_wkv5(B: int, T: int, C: int, *, seed: int, dtype: str = "f32",
                       wraw_lo: float = -6.0, wraw_hi: float = -0.5, scale: float = 0.5) -> dict:
    """RWKV-5 inputs: r, k, v [B, T, C], one w_raw per channel [C], u [C]."""
    rng = np.random.default_rng(seed)
    r, k, v = (rng.normal(0.0, scale, size=(B, T, C)).astype(np.float32) for _ in range(3))
    w_raw = rng.uniform(wraw_lo, wraw_hi, size=(C,)).astype(np.float32)
    u = rng.normal(0.0, scale, size=(C,)).astype(np.float32)
    if dtype == "bf16":
        r, k, v, w_raw = (round_to_bf16(a) for a in (r, k, v, w_raw))
    elif dtype != "f32":
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    return {"r": r, "k": k, "v": v, "w_raw": w_raw, "u": u}


def random_inputs_wkv4(B: int, T: int, C: int, *, seed: int, dtype: str = "f32", kscale: float = 1.0,
                       w_lo: float = 0.0, w_hi: float = 2.0) -> dict:
    """RWKV-4 inputs: k, v [B, T, C]; decay rates w and bonuses u [C] float32."""
    rng = np.random.default_rng(seed)
    k = (rng.normal(size=(B, T, C)) * kscale).astype(np.float32)
    v = rng.normal(size=(B, T, C)).astype(np.float32)
    w = rng.uniform(w_lo, w_hi, size=(C,)).astype(np.float32)
    u = rng.normal(size=(C,)).astype(np.float32)
    if dtype == "bf16":
        k, v = round_to_bf16(k), round_to_bf16(v)
    elif dtype != "f32":
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    return {"k": k, "v": v, "w": w, "u": u}
