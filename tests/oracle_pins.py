"""Checks that pin a WKV-6 forward implementation to facts that do not come
from the implementation itself: closed forms, a hand-worked example,
invariants and brute force.  Each ``pin_*`` takes ``impl(r, k, v, w_raw, u,
H, mode) -> y`` (numpy in, numpy out) and raises AssertionError when the
implementation violates the fact.

The definition pinned is the one on the CUDA-kernels page of
deepglint/rwkv-clip, section "Forward Pass Implementation in kernel_forward"
(state decays by w, then gains k^T v; y reads r times (u k^T v + state); a
future-to-past sweep adds the strictly later tokens), with decay
w = exp(-exp(w_raw)) from the "What is the WKV mechanism" page, section
"CUDA Wrapper (Image Side)", and the matrix state of the "RWKV Architecture"
page, sections "RWKV-5 Eagle" and "RWKV-6 Finch".
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MODES = ("causal", "bidirectional")


def draw(B, T, C, H, seed, wlo=-3.0, whi=0.5):
    rng = np.random.default_rng(seed)
    r = rng.normal(size=(B, T, C))
    k = rng.normal(size=(B, T, C))
    v = rng.normal(size=(B, T, C))
    w_raw = rng.uniform(wlo, whi, size=(B, T, C))
    u = rng.normal(size=(C,))
    return r, k, v, w_raw, u


def heads(x, H):
    B, T, C = x.shape
    return x.reshape(B, T, H, C // H)


def close(a, b, rtol=1e-11, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} (scale {scale:.3e})"


# --------------------------------------------------------------------- pins

def pin_single_token(impl):
    """T = 1: y_0 = (sum_c r_0[c] u[c] k_0[c]) v_0 in both modes."""
    for seed, (B, C, H) in enumerate([(2, 8, 2), (1, 64, 1), (3, 12, 3)]):
        r, k, v, w_raw, u = draw(B, 1, C, H, seed)
        coef = (heads(r, H) * heads(k, H) * u.reshape(H, C // H)).sum(-1)   # [B,1,H]
        expect = (coef[..., None] * heads(v, H)).reshape(B, 1, C)
        for mode in MODES:
            close(impl(r, k, v, w_raw, u, H, mode), expect, what=f"T=1 {mode}")


def pin_no_decay_causal(impl):
    """w = 1 (w_raw = -inf), u = 0: y_t = r_t . sum_{i<t} k_i^T v_i, the running
    sum taken with numpy.cumsum."""
    B, T, C, H = 2, 9, 8, 2
    r, k, v, _, _ = draw(B, T, C, H, 11)
    w_raw = np.full((B, T, C), -np.inf)
    u = np.zeros(C)
    y = impl(r, k, v, w_raw, u, H, "causal")
    R, K, V = heads(r, H), heads(k, H), heads(v, H)
    outer = K[..., :, None] * V[..., None, :]                  # [B,T,H,N,N]
    incl = np.cumsum(outer, axis=1)
    excl = np.concatenate([np.zeros_like(incl[:, :1]), incl[:, :-1]], axis=1)
    expect = np.einsum("bthc,bthcn->bthn", R, excl).reshape(B, T, C)
    close(y, expect, what="no-decay causal")


def pin_no_decay_bidirectional(impl):
    """w = 1, u = 0, bidirectional: y_t = r_t . (sum_i k_i^T v_i - k_t^T v_t)."""
    B, T, C, H = 2, 7, 8, 2
    r, k, v, _, _ = draw(B, T, C, H, 12)
    w_raw = np.full((B, T, C), -np.inf)
    u = np.zeros(C)
    y = impl(r, k, v, w_raw, u, H, "bidirectional")
    R, K, V = heads(r, H), heads(k, H), heads(v, H)
    outer = K[..., :, None] * V[..., None, :]
    total = outer.sum(axis=1, keepdims=True)
    expect = np.einsum("bthc,bthcn->bthn", R, total - outer).reshape(B, T, C)
    close(y, expect, what="no-decay bidirectional")


def pin_zero_decay(impl):
    """w = 0 (w_raw = +inf): only the neighbours survive.  Causal:
    y_t = r_t.(k_{t-1}^T v_{t-1} + diag(u) k_t^T v_t); bidirectional also adds
    r_t . k_{t+1}^T v_{t+1}."""
    B, T, C, H = 2, 6, 8, 2
    r, k, v, _, u = draw(B, T, C, H, 13)
    w_raw = np.full((B, T, C), np.inf)
    R, K, V = heads(r, H), heads(k, H), heads(v, H)
    U = u.reshape(H, C // H)
    own = ((R * U * K).sum(-1))[..., None] * V
    prev = np.zeros_like(own)
    prev[:, 1:] = (R[:, 1:] * K[:, :-1]).sum(-1)[..., None] * V[:, :-1]
    nxt = np.zeros_like(own)
    nxt[:, :-1] = (R[:, :-1] * K[:, 1:]).sum(-1)[..., None] * V[:, 1:]
    close(impl(r, k, v, w_raw, u, H, "causal"), (own + prev).reshape(B, T, C), what="w=0 causal")
    close(impl(r, k, v, w_raw, u, H, "bidirectional"), (own + prev + nxt).reshape(B, T, C),
          what="w=0 bidirectional")


def pin_constant_decay(impl):
    """Decay constant in time (the RWKV-5 case): token i reaches t with weight
    w^(|t-i|-1), computed with explicit powers."""
    B, T, C, H = 1, 10, 6, 2
    r, k, v, _, u = draw(B, T, C, H, 14)
    rng = np.random.default_rng(15)
    wr = rng.uniform(-3.0, 0.5, size=(C,))
    w_raw = np.broadcast_to(wr, (B, T, C)).copy()
    w = np.exp(-np.exp(wr)).reshape(H, C // H)
    R, K, V = heads(r, H), heads(k, H), heads(v, H)
    U = u.reshape(H, C // H)
    for mode in MODES:
        expect = np.zeros((B, T, H, C // H))
        for t in range(T):
            for i in range(T):
                if i == t:
                    g = U
                elif i < t or mode == "bidirectional":
                    g = np.power(w, abs(t - i) - 1)
                else:
                    continue
                expect[:, t] += (R[:, t] * g * K[:, i]).sum(-1)[..., None] * V[:, i]
        close(impl(r, k, v, w_raw, u, H, mode), expect.reshape(B, T, C), what=f"const decay {mode}")


def pin_short_sequences(impl):
    """Hand expansions for T = 2 and T = 3 with random values."""
    B, C, H = 2, 6, 1
    r, k, v, w_raw, u = draw(B, 3, C, H, 16)
    w = np.exp(-np.exp(w_raw))
    o = lambda i: k[:, i, :, None] * v[:, i, None, :]             # [B,C,C]
    ro = lambda t, M: np.einsum("bc,bcn->bn", r[:, t], M)
    ud = lambda i: u[None, :, None] * o(i)
    # T = 2
    y2c = np.stack([ro(0, ud(0)), ro(1, o(0) + ud(1))], axis=1)
    y2b = np.stack([ro(0, ud(0) + o(1)), ro(1, o(0) + ud(1))], axis=1)
    close(impl(r[:, :2], k[:, :2], v[:, :2], w_raw[:, :2], u, H, "causal"), y2c, what="T=2 causal")
    close(impl(r[:, :2], k[:, :2], v[:, :2], w_raw[:, :2], u, H, "bidirectional"), y2b,
          what="T=2 bidirectional")
    # T = 3
    w1 = w[:, 1, :, None]
    y3c = np.stack([ro(0, ud(0)), ro(1, o(0) + ud(1)), ro(2, w1 * o(0) + o(1) + ud(2))], axis=1)
    y3b = np.stack([ro(0, ud(0) + o(1) + w1 * o(2)), ro(1, o(0) + ud(1) + o(2)),
                    ro(2, w1 * o(0) + o(1) + ud(2))], axis=1)
    close(impl(r, k, v, w_raw, u, H, "causal"), y3c, what="T=3 causal")
    close(impl(r, k, v, w_raw, u, H, "bidirectional"), y3b, what="T=3 bidirectional")


def load_golden(name="hand_worked_T3_N2.txt"):
    vals = {}
    with open(os.path.join(GOLDEN_DIR, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line or "=" not in line:
                continue
            key, rhs = (s.strip() for s in line.split("=", 1))
            rows = [[float(x) for x in row.split()] for row in rhs.split(";")]
            vals[key] = np.array(rows, dtype=np.float64)
    return vals


def pin_hand_worked(impl):
    """The hand-worked example in tests/golden (exact rationals)."""
    g = load_golden()
    T, N = g["r"].shape
    r, k, v = (g[x].reshape(1, T, N) for x in ("r", "k", "v"))
    w_raw = np.log(-np.log(g["w"])).reshape(1, T, N)
    u = g["u"].reshape(N)
    for mode in MODES:
        close(impl(r, k, v, w_raw, u, 1, mode), g[f"y_{mode}"].reshape(1, T, N),
              rtol=1e-13, what=f"hand-worked {mode}")


def _u_term(r, k, v, u, H):
    B, T, C = r.shape
    coef = (heads(r, H) * heads(k, H) * u.reshape(H, C // H)).sum(-1)
    return (coef[..., None] * heads(v, H)).reshape(B, T, C)


def pin_reversal(impl):
    """Reversing the sequence swaps the two sweeps: with R = reversal in t,
    y_bid(Rx) = R y_bid(x) and y_caus(Rx) - U(Rx) = R (y_bid(x) - y_caus(x)),
    U being the u term."""
    B, T, C, H = 2, 11, 8, 2
    r, k, v, w_raw, u = draw(B, T, C, H, 17)
    rev = lambda a: a[:, ::-1].copy()
    yb = impl(r, k, v, w_raw, u, H, "bidirectional")
    yc = impl(r, k, v, w_raw, u, H, "causal")
    ybR = impl(rev(r), rev(k), rev(v), rev(w_raw), u, H, "bidirectional")
    ycR = impl(rev(r), rev(k), rev(v), rev(w_raw), u, H, "causal")
    close(ybR, rev(yb), what="reversal bidirectional")
    close(ycR - _u_term(rev(r), rev(k), rev(v), u, H), rev(yb - yc), what="reversal sweeps")


def pin_endpoint_decays(impl):
    """w_0 and w_{T-1} never reach y: no token lies before the first or after
    the last, and a token does not decay itself."""
    B, T, C, H = 2, 8, 8, 2
    r, k, v, w_raw, u = draw(B, T, C, H, 18)
    w2 = w_raw.copy()
    w2[:, 0] += 1.7
    w2[:, -1] -= 2.3
    for mode in MODES:
        close(impl(r, k, v, w2, u, H, mode), impl(r, k, v, w_raw, u, H, mode),
              what=f"endpoint decays {mode}")


def pin_layout(impl):
    """Head h owns channels [hN, (h+1)N): permuting heads permutes the channel
    blocks of y; batch items are independent; a value column only reaches the
    same output column."""
    B, T, C, H = 3, 7, 12, 3
    N = C // H
    r, k, v, w_raw, u = draw(B, T, C, H, 19)
    perm = [2, 0, 1]
    cperm = np.concatenate([np.arange(h * N, (h + 1) * N) for h in perm])
    for mode in MODES:
        y = impl(r, k, v, w_raw, u, H, mode)
        yp = impl(r[..., cperm], k[..., cperm], v[..., cperm], w_raw[..., cperm], u[cperm], H, mode)
        close(yp, y[..., cperm], what=f"head permutation {mode}")
        y1 = impl(r[1:2], k[1:2], v[1:2], w_raw[1:2], u, H, mode)
        close(y1, y[1:2], what=f"batch independence {mode}")
        v2 = v.copy()
        v2[..., 5] += 3.0
        d = impl(r, k, v2, w_raw, u, H, mode) - y
        mask = np.ones(C, bool)
        mask[5] = False
        assert np.max(np.abs(d[..., mask])) < 1e-12, f"value column leak {mode}"
        assert np.max(np.abs(d[..., 5])) > 1e-3, f"value column dead {mode}"


def pin_linearity(impl):
    """y is linear in r, in k and in v, and affine in u."""
    B, T, C, H = 2, 6, 8, 2
    r, k, v, w_raw, u = draw(B, T, C, H, 20)
    r2, k2, v2, _, u2 = draw(B, T, C, H, 21)
    a, b = 0.75, -1.25
    for mode in MODES:
        f = lambda R=r, K=k, V=v, U=u: impl(R, K, V, w_raw, U, H, mode)
        close(f(R=a * r + b * r2), a * f(R=r) + b * f(R=r2), what=f"linear r {mode}")
        close(f(K=a * k + b * k2), a * f(K=k) + b * f(K=k2), what=f"linear k {mode}")
        close(f(V=a * v + b * v2), a * f(V=v) + b * f(V=v2), what=f"linear v {mode}")
        close(f(U=a * u + (1 - a) * u2), a * f(U=u) + (1 - a) * f(U=u2), what=f"affine u {mode}")


def pin_bruteforce(impl, brute):
    """Agreement with the explicit pairwise sum on tiny random inputs."""
    for seed, (B, T, C, H) in enumerate([(1, 1, 1, 1), (2, 5, 2, 1), (1, 8, 8, 2),
                                         (2, 7, 4, 4), (1, 6, 64, 1), (3, 4, 12, 3)]):
        r, k, v, w_raw, u = draw(B, T, C, H, 100 + seed)
        for mode in MODES:
            close(impl(r, k, v, w_raw, u, H, mode), brute(r, k, v, w_raw, u, H, mode),
                  rtol=1e-12, what=f"bruteforce {mode} {(B, T, C, H)}")


PINS = {
    "single_token": pin_single_token,
    "no_decay_causal": pin_no_decay_causal,
    "no_decay_bidirectional": pin_no_decay_bidirectional,
    "zero_decay": pin_zero_decay,
    "constant_decay": pin_constant_decay,
    "short_sequences": pin_short_sequences,
    "hand_worked": pin_hand_worked,
    "reversal": pin_reversal,
    "endpoint_decays": pin_endpoint_decays,
    "layout": pin_layout,
    "linearity": pin_linearity,
}


def violated_pins(impl, brute=None):
    """Names of the pins the implementation fails (empty list = all hold)."""
    bad = []
    for name, pin in PINS.items():
        try:
            pin(impl)
        except (AssertionError, FloatingPointError, ValueError):
            bad.append(name)
    if brute is not None:
        try:
            pin_bruteforce(impl, brute)
        except AssertionError:
            bad.append("bruteforce")
    return bad



# ------------------------------------------------------- state passing pins
#
# For causal calls that start from a given state and return the final state
# ("RWKV Architecture" page, section "The Recurrent Inference Formulation":
# the state is all the operator keeps between steps).  Each ``spin_*`` takes
# ``impl_state(r, k, v, w_raw, u, H, S0) -> (y, S_end)`` with S0 of shape
# [B, H, N, N] (entry [b, h, c, n]: key channel c, value channel n).

def draw_state(B, H, N, seed):
    return np.random.default_rng(seed).normal(size=(B, H, N, N))


def spin_state_alone(impl_state):
    """k = 0 (nothing is added): S0 only decays.  y_t = r_t diag(prod_{j<t} w_j) S0
    and S_end = diag(prod_{all j} w_j) S0, with the products formed here by an
    exclusive cumulative product over time."""
    for seed, (B, T, C, H) in enumerate([(1, 5, 4, 1), (2, 6, 8, 2), (1, 3, 64, 1)]):
        r, k, v, w_raw, u = draw(B, T, C, H, 200 + seed)
        k = np.zeros_like(k)
        N = C // H
        S0 = draw_state(B, H, N, 300 + seed)
        W = np.exp(-np.exp(heads(w_raw, H)))                        # [B, T, H, N]
        P = np.concatenate([np.ones((B, 1, H, N)), np.cumprod(W, axis=1)[:, :-1]], axis=1)
        expect = np.einsum("bthc,bthc,bhcn->bthn", heads(r, H), P, S0).reshape(B, T, C)
        S_expect = np.prod(W, axis=1)[..., None] * S0
        y, S_end = impl_state(r, k, v, w_raw, u, H, S0)
        close(y, expect, what=f"state alone y {(B, T, C, H)}")
        close(S_end, S_expect, what=f"state alone S_end {(B, T, C, H)}")


def spin_state_superposition(impl_state):
    """The state's contribution is separate from the tokens': the result from
    S0 equals the result from zero plus the result of S0 alone (k = 0); the
    same holds for the final state."""
    for seed, (B, T, C, H) in enumerate([(2, 7, 8, 2), (1, 4, 64, 1)]):
        r, k, v, w_raw, u = draw(B, T, C, H, 210 + seed)
        S0 = draw_state(B, H, C // H, 310 + seed)
        y, S = impl_state(r, k, v, w_raw, u, H, S0)
        y0, S0end = impl_state(r, k, v, w_raw, u, H, np.zeros_like(S0))
        ys, Ss = impl_state(r, np.zeros_like(k), v, w_raw, u, H, S0)
        close(y, y0 + ys, what="superposition y")
        close(S, S0end + Ss, what="superposition S_end")


def spin_state_split(impl_state):
    """Cutting the sequence anywhere and passing the state across the cut gives
    the same y and final state (a property of any recurrence on a state)."""
    for seed, (B, T, C, H) in enumerate([(2, 9, 8, 2), (1, 6, 64, 1)]):
        r, k, v, w_raw, u = draw(B, T, C, H, 220 + seed)
        S0 = draw_state(B, H, C // H, 320 + seed)
        y, S_end = impl_state(r, k, v, w_raw, u, H, S0)
        for cut in range(0, T + 1):
            a = [x[:, :cut] for x in (r, k, v, w_raw)]
            b = [x[:, cut:] for x in (r, k, v, w_raw)]
            y1, S1 = impl_state(*a, u, H, S0)
            y2, S2 = impl_state(*b, u, H, S1)
            close(np.concatenate([y1, y2], axis=1), y, what=f"split at {cut}: y")
            close(S2, S_end, what=f"split at {cut}: S_end")


def spin_state_zero_is_stateless(impl_state, impl):
    """A zero initial state gives the stateless causal result."""
    for seed, (B, T, C, H) in enumerate([(2, 6, 8, 2), (1, 5, 64, 1)]):
        r, k, v, w_raw, u = draw(B, T, C, H, 230 + seed)
        y, _ = impl_state(r, k, v, w_raw, u, H, np.zeros((B, H, C // H, C // H)))
        close(y, impl(r, k, v, w_raw, u, H, "causal"), what="zero state")


STATE_PINS = {
    "state_alone": spin_state_alone,
    "state_superposition": spin_state_superposition,
    "state_split": spin_state_split,
}


def violated_state_pins(impl_state):
    bad = []
    for name, pin in STATE_PINS.items():
        try:
            pin(impl_state)
        except (AssertionError, FloatingPointError, ValueError):
            bad.append(name)
    return bad
