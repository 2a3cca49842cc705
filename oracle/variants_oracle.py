"""Plain float64 references for the two older WKV operators (TEST ONLY).

* RWKV-5 ("RWKV Architecture" page on llms.blog, section "RWKV-5 Eagle"):
  the matrix-state operator of RWKV-6 with a decay that is a learned
  per-channel vector instead of a per-token input.  That section writes the
  state update with the decay exp(-w); RWKV-6 ("RWKV-6 Finch", dynamic time
  decay) only made w depend on the token.  So the RWKV-5 output is the
  RWKV-6 definition with w_t = w for every t.  The decay is given in the
  same pre-transform form as for RWKV-6: w[c] = exp(-exp(w_raw[c])), i.e. the
  section's w is exp(w_raw).

* RWKV-4 (same page, section "The Fundamental Mathematical Duality": the
  baseline WKV formula, and "The Recurrent Inference Formulation"): a
  vector-valued, normalised operator, one independent recurrence per channel
  c, with a non-negative decay rate w[c] and a bonus u[c] for the current
  token:

      WKV_t = ( sum_{i<t} e^{-(t-1-i) w + k_i} v_i + e^{u + k_t} v_t )
              / ( sum_{i<t} e^{-(t-1-i) w + k_i}     + e^{u + k_t} )

  evaluated here in the recurrent form the page gives for it, with numerator
  and denominator states a, b starting at zero:

      WKV_t = (a_{t-1} + e^{u+k_t} v_t) / (b_{t-1} + e^{u+k_t})
      a_t = e^{-w} a_{t-1} + e^{k_t} v_t,   b_t = e^{-w} b_{t-1} + e^{k_t}

  Readings: the formula is causal (the pages give no bidirectional RWKV-4);
  w and u are per-channel vectors of length C and are taken as given (the
  page calls w non-negative; nothing here depends on that); the first token
  (t = 1 in the page's numbering, 0 here) sees empty sums.  Plain float64
  exponentials: inputs need |k|, |u + k| below about 700.
"""
from __future__ import annotations

import numpy as np

from .wkv6_oracle import wkv6_ref


def wkv5_ref(r, k, v, w_raw, u, H: int, mode: str = "causal") -> np.ndarray:
    """RWKV-5: the RWKV-6 operator with the decay w_raw[c] ([C] values, laid
    out [H, N]) used for every token.  Returns y as [B, T, C] float64."""
    r = np.asarray(r)
    w = np.asarray(w_raw, dtype=np.float64).reshape(-1)
    if w.size != r.shape[2]:
        raise ValueError("w_raw must hold C values")
    w_t = np.broadcast_to(w, r.shape)   # w_t = w for every batch item and token
    return wkv6_ref(r, k, v, w_t, u, H, mode)


def wkv4_ref(k, v, w, u) -> np.ndarray:
    """RWKV-4 causal WKV of [B, T, C] inputs k, v with per-channel w, u ([C]).

    One token at a time, vectorised over (b, c); returns [B, T, C] float64.
    """
    K = np.asarray(k, dtype=np.float64)
    V = np.asarray(v, dtype=np.float64)
    B, T, C = K.shape
    W = np.asarray(w, dtype=np.float64).reshape(C)
    U = np.asarray(u, dtype=np.float64).reshape(C)
    if V.shape != K.shape:
        raise ValueError("k and v must have the same shape")
    decay = np.exp(-W)
    a = np.zeros((B, C))
    b = np.zeros((B, C))
    out = np.zeros((B, T, C))
    for t in range(T):
        cur = np.exp(U + K[:, t])
        out[:, t] = (a + cur * V[:, t]) / (b + cur)
        ek = np.exp(K[:, t])
        a = decay * a + ek * V[:, t]
        b = decay * b + ek
    return out
