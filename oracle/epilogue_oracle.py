"""Plain float64 reference for the fused output epilogue (TEST ONLY).

After the WKV operator, the block normalises each head's output and gates
it: "RWKV Architecture" on llms.blog, section "RWKV-5 Eagle", applies group
normalisation across the individual heads before the output projection and
gates the output with SiLU; the deepglint/rwkv-clip "What is the WKV
mechanism" page forms the gate g as SiLU of a linear map of the block input
(section "Spatial-Mix Block Generating the WKV Inputs") and, after the WKV
call, normalises the output and multiplies it by g (section "Invocation
Inside a Transformer-Style Block").

Readings (the pages give no formula for the normalisation): group
normalisation with one group per head, i.e. for every (b, t) and head h the
mean and the biased variance (divided by N) over the head's N channels,
(y - mean) / sqrt(var + eps), then a per-channel affine gamma, beta (the
usual group-norm parameters), then the product with g.  g is taken as the
page computes it, after the SiLU; eps is a parameter (the pages give none).
"""
from __future__ import annotations

import numpy as np

from .wkv6_oracle import wkv6_ref


def group_norm_heads(y, H: int, gamma, beta, eps: float) -> np.ndarray:
    """Per-(b, t, head) normalisation of y [B, T, C] with affine gamma, beta [C]."""
    y = np.asarray(y, dtype=np.float64)
    B, T, C = y.shape
    N = C // H
    yh = y.reshape(B, T, H, N)
    mean = yh.mean(axis=-1, keepdims=True)
    var = ((yh - mean) ** 2).mean(axis=-1, keepdims=True)
    z = ((yh - mean) / np.sqrt(var + eps)).reshape(B, T, C)
    return z * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def wkv6_gn_ref(r, k, v, w_raw, u, g, gamma, beta, eps: float, H: int, mode: str = "causal") -> np.ndarray:
    """(GroupNorm_heads(WKV6(r, k, v, w_raw, u)) * gamma + beta) * g, float64 [B, T, C]."""
    y = wkv6_ref(r, k, v, w_raw, u, H, mode)
    return group_norm_heads(y, H, gamma, beta, eps) * np.asarray(g, np.float64)
