"""Precision study of the chunked backward decomposition with split-bf16
matrix operands (CPU only; a study, not a test and not part of the oracle).

It evaluates, in float64, the chunked form of the backward the MFMA kernels
use -- chunk-entry states swept forward, then the chunks in reverse with the
adjoint G: Bm = dY V^T, A = q kap^T, dr, dk, dv, G_in = G' + q^T dY, and the
decay gradient from P_j = <G_j, S_j> (the chunk-boundary inner product plus
in-chunk suffix sums of r dr - k dk) -- and rounds every operand a
matrix-core product would take to a sum of bf16 parts (RNE), so that the
number of parts each product needs can be chosen against the float64
oracle's adjoint before any kernel is written.

Part counts (``--parts``): 2 for every derived operand, or 3 for the
operands of the dr / dk / state / adjoint products (``--parts 3``); v is an
exact bf16 input and always one part.

Usage: python tests/precision_study_backward.py --parts 3
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from linear_attention_rnn_amd import inputs as I  # noqa: E402

LOG2E = 1.4426950408889634


def bf(x):
    return I.round_to_bf16(np.asarray(x, np.float32)).astype(np.float64)


def parts(x, n):
    out, r = [], np.asarray(x, np.float64)
    for _ in range(n):
        h = bf(r)
        out.append(h)
        r = r - h
    return out


def mm(a, b, na, nb):
    """a @ b with operands split into na / nb bf16 parts; keeps the part
    products of order < max(na, nb), as the kernels do."""
    pa, pb = parts(a, na), parts(b, nb)
    acc = 0.0
    for d in range(max(na, nb) - 1, -1, -1):
        for i in range(d + 1):
            j = d - i
            if i < na and j < nb:
                acc = acc + pa[i] @ pb[j]
    return acc


def f32(x):
    return np.asarray(x, np.float32).astype(np.float64)


def causal_chunked(R, K, V, WR, U, DY, use_u, P, L=64):
    """One causal direction for one (batch, head): [T, N] arrays."""
    T, N = R.shape
    lam2 = f32(-LOG2E * np.exp(WR))
    lamn = -np.exp(WR)
    nch = (T + L - 1) // L
    Sst, S = [], np.zeros((N, N))
    for m in range(nch):
        sl = slice(m * L, min(T, (m + 1) * L))
        lin = np.cumsum(lam2[sl], 0)
        tot = lin[-1]
        Sst.append(f32(S))
        S = f32(np.exp2(tot)[:, None] * S + mm((K[sl] * np.exp2(tot - lin)).T, V[sl], P, 1))
    dR, dK, dV, dW = (np.zeros_like(R) for _ in range(4))
    dU = np.zeros(N)
    G, Pend = np.zeros((N, N)), np.zeros(N)
    for m in range(nch - 1, -1, -1):
        sl = slice(m * L, min(T, (m + 1) * L))
        n = sl.stop - sl.start
        r, k, v, dy = R[sl], K[sl], V[sl], DY[sl]
        lin = f32(np.cumsum(lam2[sl], 0))
        lex = lin - lam2[sl]
        Gp = f32(np.exp2(lin[-1])[:, None] * G)
        kap, q = k * np.exp2(-lin), r * np.exp2(lex)
        Bm = f32(mm(dy, v.T, P, 1))
        lower = np.tril(np.ones((n, n)), -1)
        A = f32(mm(q, kap.T, P, P)) * lower
        diag = np.diag(Bm).copy()
        if use_u:
            A[np.arange(n), np.arange(n)] = f32(np.sum(r * U * k, 1))
        dr = f32(np.exp2(lex) * f32(mm(Bm * lower, kap, P, P) + mm(dy, Sst[m].T, P, P)))
        dk = f32(np.exp2(-lin) * f32(mm((Bm * lower).T, q, P, P) + mm(v, Gp.T, 1, P)))
        if use_u:
            dr = dr + U * k * diag[:, None]
            dk = dk + U * r * diag[:, None]
            dU += np.sum(r * k * diag[:, None], 0)
        dv = mm(A.T, dy, P, P) + mm(kap, Gp, P, P)
        Gin = f32(Gp + mm(q.T, dy, P, P))
        x = r * dr - k * dk
        suf = np.cumsum(x[::-1], 0)[::-1]
        dlam = Pend + (suf - x) - k * dk + (U * r * k * diag[:, None] if use_u else 0.0)
        dR[sl], dK[sl], dV[sl], dW[sl] = dr, dk, f32(dv), dlam * lamn[sl]
        Pend = np.sum(Gin * Sst[m], 1)
        G = Gin
    return dR, dK, dV, dW, dU


def chunked_backward(x, dy, H, mode, P):
    from oracle.wkv6_oracle import merge_heads, split_heads

    R, K, V, WR, DY = (split_heads(a, H) for a in (x["r"], x["k"], x["v"], x["w_raw"], dy))
    B, Hh, T, N = R.shape
    Uh = np.asarray(x["u"], np.float64).reshape(Hh, N)
    out = {key: np.zeros((B, Hh, T, N)) for key in "rkvw"}
    du = np.zeros((Hh, N))
    for b in range(B):
        for h in range(Hh):
            res = causal_chunked(R[b, h], K[b, h], V[b, h], WR[b, h], Uh[h], DY[b, h], True, P)
            for key, val in zip("rkvw", res[:4]):
                out[key][b, h] += val
            du[h] += res[4]
            if mode == "bidirectional":
                rv = lambda a: a[b, h][::-1]  # noqa: E731
                e = causal_chunked(rv(R), rv(K), rv(V), rv(WR), Uh[h], rv(DY), False, P)
                for key, val in zip("rkvw", e[:4]):
                    out[key][b, h] += val[::-1]
    return {"r": merge_heads(out["r"]), "k": merge_heads(out["k"]), "v": merge_heads(out["v"]),
            "w_raw": merge_heads(out["w"]), "u": du.reshape(-1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--parts", type=int, default=3, choices=[2, 3])
    a = ap.parse_args()
    from oracle import wkv6_ref_backward

    for (B, T, C, H, mode, lo, hi) in [(2, 150, 128, 2, "causal", -6, -1), (2, 196, 128, 2, "bidirectional", -9, -0.5),
                                       (1, 700, 64, 1, "causal", -9, -2)]:
        x = I.random_inputs(B, T, C, H, seed=5, dtype="bf16", wraw_lo=lo, wraw_hi=hi)
        dy = np.random.default_rng(6).normal(0, 0.5, size=x["r"].shape).astype(np.float32).astype(np.float64)
        ref = wkv6_ref_backward(x["r"], x["k"], x["v"], x["w_raw"], x["u"], dy, H, mode)
        got = chunked_backward(x, dy, H, mode, a.parts)
        msg = []
        for key in ("r", "k", "v", "u", "w_raw"):
            sc = np.sqrt(np.mean(ref[key] ** 2))
            if key == "w_raw":   # the scale the GPU tests use for dw_raw
                sc = max(sc, np.sqrt(np.mean((x["k"] * ref["k"] * np.exp(x["w_raw"].astype(np.float64))) ** 2)))
            msg.append(f"d{key} {np.max(np.abs(got[key] - ref[key])) / sc:.2e}")
        print(f"B{B} T{T} {mode} w_raw in [{lo}, {hi}] parts={a.parts}: " + "  ".join(msg), flush=True)


if __name__ == "__main__":
    main()
