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

* state passing (causal only): the state is the operator's entire memory,
  updated token by token and kept between calls at inference ("RWKV
  Architecture" page, section "The Recurrent Inference Formulation"; the
  yarian.com RWKV page, section "7. Hidden State = Persistent Memory").  So a
  causal call may start from a given state S instead of zero and hand back
  the state after its last token; cutting a sequence anywhere and passing the
  state across the cut changes nothing.

Readings taken where the pages are silent or garbled are the ones the test
suite pins: decay exp(-exp(w_raw)) (one page's example code writes exp(w),
which would give decays above one and is taken as garbled); the
future-to-past sum is exclusive of the current token; the initial states are
zero unless a causal call passes one; u has one value per channel; the
output is always float32-or-wider.
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


def _state_arg(state_in, B: int, H: int, N: int, bidir: bool, return_state: bool) -> np.ndarray:
    if bidir and (state_in is not None or return_state):
        raise ValueError("state passing is defined for causal mode only")
    if state_in is None:
        return np.zeros((B, H, N, N), dtype=np.float64)
    S = np.array(state_in, dtype=np.float64)   # a copy
    if S.shape != (B, H, N, N):
        raise ValueError(f"state_in must be [B, H, N, N] = {(B, H, N, N)}, got {S.shape}")
    return S


def wkv6_ref(r, k, v, w_raw, u, H: int, mode: str = "causal", state_in=None,
             return_state: bool = False):
    """Recurrent float64 evaluation; returns y as [B, T, C] float64.

    Loops over t in Python, vectorised over (b, h); O(B*H*T*N^2) work.
    Causal mode may start from ``state_in`` ([B, H, N, N], entry [b, h, c, n]
    for key channel c and value channel n; zero if None); with
    ``return_state`` it returns (y, state after the last token).
    """
    bidir = _check_mode(mode)
    R = split_heads(r, H)
    K = split_heads(k, H)
    V = split_heads(v, H)
    W = np.exp(-np.exp(split_heads(w_raw, H)))
    B, Hh, T, N = R.shape
    U = np.asarray(u, dtype=np.float64).reshape(Hh, N)
    Y = np.zeros((B, Hh, T, N), dtype=np.float64)
    S = _state_arg(state_in, B, Hh, N, bidir, return_state)   # S[b, h, c, n]
    for t in range(T):
        kv = K[:, :, t, :, None] * V[:, :, t, None, :]
        # y_t = r_t . (S + diag(u) kv)
        bonus = (R[:, :, t, :] * U[None] * K[:, :, t, :]).sum(-1)
        Y[:, :, t, :] = (R[:, :, t, None, :] @ S)[:, :, 0, :] + bonus[..., None] * V[:, :, t, :]
        S *= W[:, :, t, :, None]
        S += kv
    if return_state:
        return merge_heads(Y), S
    if bidir:
        S[...] = 0.0
        for t in range(T - 1, -1, -1):
            Y[:, :, t, :] += (R[:, :, t, None, :] @ S)[:, :, 0, :]
            S *= W[:, :, t, :, None]
            S += K[:, :, t, :, None] * V[:, :, t, None, :]
    return merge_heads(Y)


def wkv6_bruteforce(r, k, v, w_raw, u, H: int, mode: str = "causal", state_in=None) -> np.ndarray:
    """Explicit pairwise sum: y_t[n] = sum_{i} sum_c r_t[c] g_{t,i}[c] k_i[c] v_i[n]
    with g_{t,t} = u, g_{t,i} = prod of w_j over j strictly between i and t
    (formed factor by factor, an empty product being one), i < t only in
    causal mode.  A causal ``state_in`` S0 adds
    sum_c r_t[c] (prod_{j<t} w_j[c]) S0[c, n].  No running state;
    O(T^3 N + T^2 N^2) per (b, h).  Intended for T of a few tokens."""
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
    if state_in is not None:
        S0 = _state_arg(state_in, B, Hh, N, bidir, False)
        for t in range(T):
            g = np.ones((B, Hh, N), dtype=np.float64)
            for j in range(t):
                g = g * W[:, :, j, :]
            Y[:, :, t, :] += np.einsum("bhc,bhc,bhcn->bhn", R[:, :, t, :], g, S0)
    return merge_heads(Y)


def _causal_backward(R, K, V, W, WR, U, DY, use_u: bool):
    """Adjoint of the causal recurrence for one direction, arrays [B, H, T, N]
    (float64).  Returns dR, dK, dV, dWR (gradient w.r.t. w_raw) and dU [H, N].

    With S_t the state after token t and G_t = dL/dS_t:
      dr_t[c] = sum_n dy_t[n] (S_{t-1}[c, n] + u[c] k_t[c] v_t[n])
      G_{t-1} = w_t[c] G_t[c, n] + r_t[c] dy_t[n]          (G_{T-1} = 0)
      dk_t[c] = sum_n G_t[c, n] v_t[n] + r_t[c] u[c] (dy_t . v_t)
      dv_t[n] = sum_c G_t[c, n] k_t[c] + (sum_c r_t[c] u[c] k_t[c]) dy_t[n]
      dw_t[c] = sum_n G_t[c, n] S_{t-1}[c, n]
    and w = exp(-exp(w_raw)) gives dw_raw = dw * w * (-exp(w_raw))."""
    B, H, T, N = R.shape
    Uu = U[None] if use_u else np.zeros_like(U)[None]
    S = np.zeros((B, H, N, N))
    states = np.zeros((B, H, T, N, N))          # S_{t-1} for every t
    dR = np.zeros_like(R)
    for t in range(T):
        states[:, :, t] = S
        dyv = (DY[:, :, t] * V[:, :, t]).sum(-1)                      # [B, H]
        dR[:, :, t] = np.einsum("bhcn,bhn->bhc", S, DY[:, :, t]) + Uu * K[:, :, t] * dyv[..., None]
        S = W[:, :, t, :, None] * S + K[:, :, t, :, None] * V[:, :, t, None, :]
    G = np.zeros((B, H, N, N))
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dW = np.zeros_like(W)
    dU = np.zeros((H, N))
    for t in range(T - 1, -1, -1):
        dyv = (DY[:, :, t] * V[:, :, t]).sum(-1)
        ruk = (R[:, :, t] * Uu * K[:, :, t]).sum(-1)                   # [B, H]
        dK[:, :, t] = np.einsum("bhcn,bhn->bhc", G, V[:, :, t]) + R[:, :, t] * Uu * dyv[..., None]
        dV[:, :, t] = np.einsum("bhcn,bhc->bhn", G, K[:, :, t]) + ruk[..., None] * DY[:, :, t]
        dW[:, :, t] = np.einsum("bhcn,bhcn->bhc", G, states[:, :, t])
        if use_u:
            dU += (R[:, :, t] * K[:, :, t] * dyv[..., None]).sum(0)
        G = W[:, :, t, :, None] * G + R[:, :, t, :, None] * DY[:, :, t, None, :]
    dWR = dW * W * (-np.exp(WR))
    return dR, dK, dV, dWR, dU


def wkv6_ref_backward(r, k, v, w_raw, u, dy, H: int, mode: str = "causal") -> dict:
    """Gradients of L = sum(y * dy) with respect to r, k, v, w_raw and u, for
    y = wkv6_ref(r, k, v, w_raw, u, H, mode); float64, by the adjoint of the
    recurrence (the pages' CUDA kernel has a backward kernel alongside the
    forward one, CUDA-kernels page, section "Backward Pass Gradient
    Computation"; its steps are not given, so this is derived here).

    Returns {"r", "k", "v", "w_raw": [B, T, C], "u": [C]}.  Bidirectional mode
    adds the gradients of the later-token sum: the causal adjoint of the
    time-reversed sequence without the u term.
    """
    bidir = _check_mode(mode)
    R, K, V, WR, DY = (split_heads(x, H) for x in (r, k, v, w_raw, dy))
    W = np.exp(-np.exp(WR))
    B, Hh, T, N = R.shape
    U = np.asarray(u, dtype=np.float64).reshape(Hh, N)
    dR, dK, dV, dWR, dU = _causal_backward(R, K, V, W, WR, U, DY, True)
    if bidir:
        rev = lambda X: X[:, :, ::-1]
        eR, eK, eV, eWR, _ = _causal_backward(rev(R), rev(K), rev(V), rev(W), rev(WR), U, rev(DY), False)
        dR += rev(eR)
        dK += rev(eK)
        dV += rev(eV)
        dWR += rev(eWR)
    return {"r": merge_heads(dR), "k": merge_heads(dK), "v": merge_heads(dV), "w_raw": merge_heads(dWR),
            "u": dU.reshape(-1)}
