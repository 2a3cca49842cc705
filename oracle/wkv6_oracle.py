"""Plain float64 reference for the RWKV-6 WKV forward operator (TEST ONLY).

What is computed, for each batch item b and head h (head h owns the
contiguous channels [h*N, (h+1)*N) of the [B, T, C] tensors, C = H*N):

* per-token, per-channel decay  w_t[c] = exp(-exp(w_raw_t[c])).  The wrapper
  on the "What is the WKV mechanism" page of deepglint/rwkv-clip (section
  "CUDA Wrapper (Image Side)") hands the kernel minus the exponential of w,
  and the kernel takes the exponential of that again (CUDA-kernels page,
  section "Kernel Architecture and Launch Configuration"); the decay is data
  dependent per token in RWKV-6 ("RWKV Architecture" page on llms.blog,
  section "RWKV-6 Finch", dynamic time decay).
* an N x N state whose rows are indexed by the key/receptance channel c and
  whose columns by the value channel n ("RWKV Architecture" page, section
  "RWKV-5 Eagle", matrix state updated by decay plus the outer product of
  k and v).  From a zero state, per token t:
      y_t[n]  = sum_c r_t[c] * ( S[c, n] + u[c] * k_t[c] * v_t[n] )
      S[c, n] = w_t[c] * S[c, n] + k_t[c] * v_t[n]
  (CUDA-kernels page, section "Forward Pass Implementation in
  kernel_forward": the kernel forms the outer product of k and v, decays the
  running state by w before adding that product, and in the past-to-future
  pass adds r times (u times the product plus the state) to y.)  So a past
  token i < t reaches t with weight prod_{j=i+1}^{t-1} w_j and the current
  token with weight u.
* bidirectional mode adds a future-to-past sweep from a second zero state,
  with no u term and the output read before the update, so only strictly
  later tokens contribute:
      y_t[n] += sum_c r_t[c] * S'[c, n];   S'[c, n] = w_t[c] * S'[c, n] + k_t[c] * v_t[n]
  (same page and section, "Future-to-Past Pass"; its summary says u is used
  only in the past-to-future sweep and that the first sweep gathers the
  future tokens.)  The two sweeps' contributions are summed.

Readings taken where the pages are silent or garbled are the ones the test
suite pins: decay exp(-exp(w_raw)) (one page's example code writes exp(w),
which would give decays above one and is taken as garbled); the
future-to-past sum is exclusive of the current token; the initial states are
zero; u has one value per channel; the output is always float32-or-wider.
"""
from __future__ import annotations

import numpy as np

MODES = ("causal", "bidirectional")


def _check_mode(mode: str) -> bool:
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}, got {mode!r}")
    return mode == "bidirectional"


def decay(w_raw) -> np.ndarray:
    """w = exp(-exp(w_raw)) in float64.  w_raw = -inf gives w = 1 exactly and
    w_raw = +inf gives w = 0 exactly."""
    return np.exp(-np.exp(np.asarray(w_raw, dtype=np.float64)))


def split_heads(x, H: int) -> np.ndarray:
    """[B, T, C] -> [B, H, T, N] in float64, head h = channels [hN, (h+1)N)."""
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    if C % H:
        raise ValueError("C must be a multiple of H")
    return np.ascontiguousarray(x.reshape(B, T, H, C // H).transpose(0, 2, 1, 3))


def merge_heads(x) -> np.ndarray:
    """[B, H, T, N] -> [B, T, C]."""
    B, H, T, N = x.shape
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(B, T, H * N))


def wkv6_ref(r, k, v, w_raw, u, H: int, mode: str = "causal") -> np.ndarray:
    """Recurrent float64 evaluation; returns y as [B, T, C] float64.

    Loops over t in Python, vectorised over (b, h); O(B*H*T*N^2) work.
    """
    bidir = _check_mode(mode)
    R = split_heads(r, H)
    K = split_heads(k, H)
    V = split_heads(v, H)
    W = np.exp(-np.exp(split_heads(w_raw, H)))
    B, Hh, T, N = R.shape
    U = np.asarray(u, dtype=np.float64).reshape(Hh, N)
    Y = np.zeros((B, Hh, T, N), dtype=np.float64)
    S = np.zeros((B, Hh, N, N), dtype=np.float64)   # S[b, h, c, n]
    for t in range(T):
        kv = K[:, :, t, :, None] * V[:, :, t, None, :]
        # y_t = r_t . (S + diag(u) kv)
        bonus = (R[:, :, t, :] * U[None] * K[:, :, t, :]).sum(-1)
        Y[:, :, t, :] = (R[:, :, t, None, :] @ S)[:, :, 0, :] + bonus[..., None] * V[:, :, t, :]
        S *= W[:, :, t, :, None]
        S += kv
    if bidir:
        S[...] = 0.0
        for t in range(T - 1, -1, -1):
            Y[:, :, t, :] += (R[:, :, t, None, :] @ S)[:, :, 0, :]
            S *= W[:, :, t, :, None]
            S += K[:, :, t, :, None] * V[:, :, t, None, :]
    return merge_heads(Y)


def wkv6_bruteforce(r, k, v, w_raw, u, H: int, mode: str = "causal") -> np.ndarray:
    """Explicit pairwise sum: y_t[n] = sum_{i} sum_c r_t[c] g_{t,i}[c] k_i[c] v_i[n]
    with g_{t,t} = u, g_{t,i} = prod of w_j over j strictly between i and t
    (formed factor by factor, an empty product being one), i < t only in
    causal mode.  No running state; O(T^3 N + T^2 N^2) per (b, h).  Intended
    for T of a few tokens."""
    bidir = _check_mode(mode)
    R = split_heads(r, H)
    K = split_heads(k, H)
    V = split_heads(v, H)
    W = decay(split_heads(w_raw, H))
    B, Hh, T, N = R.shape
    U = np.asarray(u, dtype=np.float64).reshape(Hh, N)
    Y = np.zeros((B, Hh, T, N), dtype=np.float64)
    for t in range(T):
        for i in range(T):
            if i == t:
                g = np.broadcast_to(U[None], (B, Hh, N))
            elif i < t or bidir:
                lo, hi = min(i, t), max(i, t)
                g = np.ones((B, Hh, N), dtype=np.float64)
                for j in range(lo + 1, hi):
                    g = g * W[:, :, j, :]
            else:
                continue
            coef = (R[:, :, t, :] * g * K[:, :, i, :]).sum(-1)      # [B, H]
            Y[:, :, t, :] += coef[..., None] * V[:, :, i, :]
    return merge_heads(Y)
