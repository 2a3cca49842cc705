"""Precision study of the chunked evaluation with 16-bit matrix operands
(CPU only; a study, not a test and not part of the oracle).

It evaluates the chunked algebra the forward kernels use -- 64-token chunks
cut into 16-token blocks, log2-space prefix sums, the decay split between a
query factor and a key factor, the carried state -- in float64, but rounds
every operand a matrix-core product would take to the chosen 16-bit format
(RNE), so that the error of that choice can be measured against the float64
oracle at the workloads' own shapes before any kernel is written.

Operand choices studied (``--fmt``):
  f16     every derived operand (decayed queries and keys, the score tile,
          the state, the value rows) rounded once to IEEE half precision;
  bf16    the same with bfloat16 (8-bit significand);
  bf16x2  every derived operand carried as a bfloat16 pair (hi + lo), the
          value rows (exact bf16 inputs) as one part.

Decay split: the off-diagonal score tiles of key block I and query block J
(I < J) use the factors 2^(Lex_t - E_(J-1)) on the query and
2^(E_(J-1) - Lin_i) on the key (E_b: prefix at the end of block b), both at
most 1; the diagonal tiles use a reference at the block's middle token, so
their factors stay within 2^(+-half the block's decay).  The state product
uses r 2^Lex (at most 1) and the state update k 2^(Ltot - Lin) (at most 1).

Usage: python tests/precision_study.py --workload image-base-bidir-bf16 --items 8 --fmt f16
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from linear_attention_rnn_amd import inputs as I  # noqa: E402

LOG2E = 1.4426950408889634


def rnd(x, fmt):
    """Round to the 16-bit operand format (float64 in, float64 out)."""
    if fmt == "f16":
        return x.astype(np.float16).astype(np.float64)
    if fmt == "bf16":
        return I.round_to_bf16(x.astype(np.float32)).astype(np.float64)
    if fmt == "bf16x2":
        hi = I.round_to_bf16(x.astype(np.float32)).astype(np.float64)
        lo = I.round_to_bf16((x - hi).astype(np.float32)).astype(np.float64)
        return hi + lo
    raise ValueError(fmt)


def f32(x):
    return x.astype(np.float32).astype(np.float64)


EXACT = set()   # operand classes left unrounded (for attributing the error): qk, A, rho, S, eta


def rc(x, fmt, cls):
    return x if cls in EXACT else rnd(x, fmt)


def sweep(R, K, V, W, U, fmt, with_u):
    """One causal sweep over [n, T, N] arrays (float64 holding the inputs'
    exact values); returns y [n, T, N]."""
    n, T, N = R.shape
    L, BL = 64, 16
    Y = np.zeros_like(R)
    S = np.zeros((n, N, N))
    vfmt = "f16" if fmt == "f16" else "bf16"
    for c0 in range(0, T, L):
        c1 = min(T, c0 + L)
        Lc = c1 - c0
        r, k, v = R[:, c0:c1], K[:, c0:c1], V[:, c0:c1]
        lam = f32(-LOG2E * np.exp(W[:, c0:c1]))           # log2 decay per token and channel
        lin = f32(np.cumsum(lam, axis=1))                 # inclusive prefix (fp32 scan)
        lex = lin - lam
        nb = (Lc + BL - 1) // BL
        E = [lin[:, min(Lc, BL * (b + 1)) - 1] for b in range(nb)]      # block ends, [n, N]
        vq = rnd(v, vfmt)
        y = np.zeros((n, Lc, N))
        # in-chunk scores, block by block
        A = np.zeros((n, Lc, Lc))
        for J in range(nb):
            t0, t1 = BL * J, min(Lc, BL * (J + 1))
            start = E[J - 1] if J > 0 else np.zeros((n, N))
            for Ib in range(J + 1):
                i0, i1 = BL * Ib, min(Lc, BL * (Ib + 1))
                if Ib < J:
                    q = rc(r[:, t0:t1] * np.exp2(lex[:, t0:t1] - start[:, None]), fmt, "qk")
                    kk = rc(k[:, i0:i1] * np.exp2(start[:, None] - lin[:, i0:i1]), fmt, "qk")
                    A[:, t0:t1, i0:i1] = np.einsum("ntc,nic->nti", q, kk)
                else:
                    mid = lin[:, min(t1 - 1, t0 + BL // 2 - 1)]
                    q = rc(r[:, t0:t1] * np.exp2(lex[:, t0:t1] - mid[:, None]), fmt, "qk")
                    kk = rc(k[:, i0:i1] * np.exp2(mid[:, None] - lin[:, i0:i1]), fmt, "qk")
                    a = np.einsum("ntc,nic->nti", q, kk)
                    m = np.tril(np.ones((t1 - t0, i1 - i0)), -1)
                    A[:, t0:t1, i0:i1] = a * m
        if with_u:
            d = f32(np.einsum("ntc,c,ntc->nt", r, U, k))
            A[:, np.arange(Lc), np.arange(Lc)] += d
        y += np.einsum("nti,nim->ntm", rc(f32(A), fmt, "A"), vq)
        # inter-chunk: r 2^Lex times the carried state
        rho = rc(r * np.exp2(lex), fmt, "rho")
        y += np.einsum("ntc,ncm->ntm", rho, rc(f32(S), fmt, "S"))
        # state update: S <- 2^Ltot S + (k 2^(Ltot - Lin))^T V
        tot = lin[:, -1]
        eta = rc(k * np.exp2(tot[:, None] - lin), fmt, "eta")
        S = f32(np.exp2(tot)[:, :, None] * S + np.einsum("nic,nim->ncm", eta, vq))
        Y[:, c0:c1] = y
    return Y


def emulate(x, H, mode, fmt):
    def heads(a):
        B, T, C = a.shape
        return np.asarray(a, np.float64).reshape(B, T, H, C // H).transpose(0, 2, 1, 3).reshape(B * H, T, C // H)

    R, K, V, W = (heads(x[key]) for key in ("r", "k", "v", "w_raw"))
    B, T, C = x["r"].shape
    U = np.asarray(x["u"], np.float64).reshape(H, C // H)
    Y = np.zeros_like(R)
    for h in range(H):
        sl = slice(h, None, H)
        Y[sl] = sweep(R[sl], K[sl], V[sl], W[sl], U[h], fmt, True)
        if mode == "bidirectional":
            rev = lambda a: a[sl][:, ::-1]  # noqa: E731
            Y[sl] += sweep(rev(R), rev(K), rev(V), rev(W), U[h], fmt, False)[:, ::-1]
    return Y.reshape(B, H, T, C // H).transpose(0, 2, 1, 3).reshape(B, T, C)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="image-base-bidir-bf16")
    ap.add_argument("--items", type=int, default=4, help="batch items evaluated")
    ap.add_argument("--fmt", default="f16", choices=["f16", "bf16", "bf16x2"])
    ap.add_argument("--exact", default="", help="comma-separated operand classes left unrounded")
    a = ap.parse_args()
    EXACT.update(x for x in a.exact.split(",") if x)
    from oracle import wkv6_ref

    w = I.workload(a.workload)
    x = I.make_inputs(w)
    nb = min(a.items, w.B)
    xs = {key: (val[:nb] if getattr(val, "ndim", 0) == 3 else val) for key, val in x.items()}
    y = emulate(xs, w.H, w.mode, a.fmt)
    y_ref = wkv6_ref(xs["r"], xs["k"], xs["v"], xs["w_raw"], xs["u"], w.H, w.mode)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = np.abs(y - y_ref)
    print(f"{a.workload} items={nb} fmt={a.fmt} exact={a.exact or '-'}: max|dy|/rms = {err.max() / rms:.3e}  "
          f"rms(dy)/rms = {np.sqrt(np.mean(err ** 2)) / rms:.3e}", flush=True)


if __name__ == "__main__":
    main()
