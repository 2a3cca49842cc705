"""The RWKV-5 and RWKV-4 oracles against facts that do not come from them.

RWKV-5 (one decay per channel for every token) is checked against the
definition written with powers of the decay instead of running products and
against a geometric-series closed form.  RWKV-4 (the normalised per-channel
operator) is checked against a hand-worked example, the explicit-sum form of
its definition on tiny inputs, closed forms and invariants.  Each planted
mistake below must break at least one of the checks.
"""
import os

import numpy as np
import pytest

from oracle import wkv4_ref, wkv5_ref, wkv6_ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rwkv4_hand_worked_T3.txt")


# ---------------------------------------------------------------- RWKV-5
def wkv5_powers(r, k, v, w_raw, u, H, mode):
    """y_t = sum_{i<t} r_t diag(w^(t-1-i)) k_i^T v_i + r_t diag(u) k_t^T v_t
    (+ sum_{i>t} r_t diag(w^(i-1-t)) k_i^T v_i), with w = exp(-exp(w_raw)):
    with a fixed decay the product over the tokens strictly between i and t
    is a power of w."""
    r, k, v = (np.asarray(a, np.float64) for a in (r, k, v))
    B, T, C = r.shape
    w = np.exp(-np.exp(np.asarray(w_raw, np.float64).reshape(C)))
    u = np.asarray(u, np.float64).reshape(C)
    N = C // H
    y = np.zeros((B, T, C))
    for b in range(B):
        for h in range(H):
            sl = slice(h * N, (h + 1) * N)
            for t in range(T):
                for i in range(T):
                    if i < t:
                        g = np.power(w[sl], t - 1 - i)
                    elif i == t:
                        g = u[sl]
                    elif mode == "bidirectional":
                        g = np.power(w[sl], i - 1 - t)
                    else:
                        continue
                    y[b, t, sl] += np.sum(r[b, t, sl] * g * k[b, i, sl]) * v[b, i, sl]
    return y


def draw5(B, T, C, seed):
    rng = np.random.default_rng(seed)
    r, k, v = (rng.normal(size=(B, T, C)) for _ in range(3))
    w_raw = rng.uniform(-3.0, 0.5, size=C)
    u = rng.normal(size=C)
    return r, k, v, w_raw, u


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_wkv5_matches_power_form(mode):
    for seed, (B, T, C, H) in enumerate([(1, 1, 4, 1), (2, 6, 8, 2), (1, 8, 12, 3)]):
        x = draw5(B, T, C, 300 + seed)
        np.testing.assert_allclose(wkv5_ref(*x, H, mode), wkv5_powers(*x, H, mode), rtol=1e-12, atol=1e-12)


def test_wkv5_geometric_closed_form():
    """One channel, r = k = v = 1, u = 0: y_t = sum_{i<t} w^(t-1-i) = (1 - w^t) / (1 - w)."""
    T = 9
    w = 0.3
    w_raw = np.array([np.log(-np.log(w))])
    one = np.ones((1, T, 1))
    y = wkv5_ref(one, one, one, w_raw, np.zeros(1), 1)[0, :, 0]
    t = np.arange(T)
    np.testing.assert_allclose(y, (1 - w ** t) / (1 - w), rtol=1e-13, atol=1e-15)


WKV5_MUTANTS = {
    # the decay of channel c taken from another channel (reversed order)
    "channels_reversed": lambda r, k, v, w, u, H, mode: wkv6_ref(
        r, k, v, np.broadcast_to(np.asarray(w, np.float64)[::-1], np.shape(r)), u, H, mode),
    # the [H, N] layout of the decay read as [N, H]
    "layout_transposed": lambda r, k, v, w, u, H, mode: wkv6_ref(
        r, k, v, np.broadcast_to(np.asarray(w, np.float64).reshape(-1, H).T.reshape(-1), np.shape(r)), u, H, mode),
    # a sign slip in the decay transform: exp(-exp(-w_raw))
    "decay_sign_slip": lambda r, k, v, w, u, H, mode: wkv6_ref(
        r, k, v, np.broadcast_to(-np.asarray(w, np.float64), np.shape(r)), u, H, mode),
}


@pytest.mark.parametrize("name", sorted(WKV5_MUTANTS))
def test_wkv5_pins_catch_planted_mistakes(name):
    bad = WKV5_MUTANTS[name]
    x = draw5(1, 6, 8, 310)
    assert not np.allclose(bad(*x, 2, "causal"), wkv5_powers(*x, 2, "causal"), rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------- RWKV-4
def wkv4_sums(k, v, w, u):
    """The definition as written: explicit sums with the exponent
    -(t-1-i) w + k_i for each earlier token i, exp(u + k_t) for t itself."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    B, T, C = k.shape
    w, u = np.asarray(w, np.float64), np.asarray(u, np.float64)
    out = np.zeros((B, T, C))
    for t in range(T):
        num = np.exp(u + k[:, t]) * v[:, t]
        den = np.exp(u + k[:, t])
        for i in range(t):
            e = np.exp(-(t - 1 - i) * w + k[:, i])
            num = num + e * v[:, i]
            den = den + e
        out[:, t] = num / den
    return out


def load_rwkv4_golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                key, rhs = line.split("=", 1)
                vals[key.strip()] = np.array([float(x) for x in rhs.split()])
    return vals


def draw4(B, T, C, seed, kscale=1.0):
    rng = np.random.default_rng(seed)
    k = rng.normal(size=(B, T, C)) * kscale
    v = rng.normal(size=(B, T, C))
    w = rng.uniform(0.0, 2.0, size=C)
    u = rng.normal(size=C)
    return k, v, w, u


def pin4_golden(f):
    g = load_rwkv4_golden()
    y = f(g["k"].reshape(1, 3, 1), g["v"].reshape(1, 3, 1), g["w"], g["u"])[0, :, 0]
    np.testing.assert_allclose(y, [1.0, 5.0 / 3.0, 15.0 / 7.0], rtol=1e-13)
    np.testing.assert_allclose(g["wkv"], [1.0, 5.0 / 3.0, 15.0 / 7.0], rtol=1e-15)


def pin4_sums(f):
    for seed, (B, T, C) in enumerate([(1, 1, 3), (2, 7, 4), (1, 12, 2)]):
        x = draw4(B, T, C, 400 + seed, kscale=2.0)
        np.testing.assert_allclose(f(*x), wkv4_sums(*x), rtol=1e-12, atol=1e-12)


def pin4_first_token(f):
    k, v, w, u = draw4(3, 1, 5, 410)
    np.testing.assert_allclose(f(k, v, w, u), v, rtol=1e-14)


def pin4_constant_values(f):
    """Every output is a weighted mean of v: constant values come back."""
    k, _, w, u = draw4(2, 20, 6, 411, kscale=3.0)
    v = np.broadcast_to(np.linspace(-2.0, 3.0, 6), k.shape)
    np.testing.assert_allclose(f(k, v, w, u), v, rtol=1e-12, atol=1e-12)


def pin4_key_shift(f):
    """Adding a constant to every k of a channel scales numerator and
    denominator alike."""
    k, v, w, u = draw4(2, 15, 4, 412)
    shift = np.array([5.0, -7.0, 0.5, 11.0])
    np.testing.assert_allclose(f(k + shift, v, w, u), f(k, v, w, u), rtol=1e-11, atol=1e-12)


def pin4_no_memory(f):
    """w = inf: only the previous token (weight e^{k_{t-1}}, never decayed)
    and the current one (e^{u + k_t}) remain."""
    k, v, _, u = draw4(1, 10, 3, 413)
    y = f(k, v, np.full(3, np.inf), u)
    e_prev, e_cur = np.exp(k[:, :-1]), np.exp(u + k[:, 1:])
    np.testing.assert_allclose(y[:, 1:], (e_prev * v[:, :-1] + e_cur * v[:, 1:]) / (e_prev + e_cur), rtol=1e-12)
    np.testing.assert_allclose(y[:, 0], v[:, 0], rtol=1e-14)


PINS4 = {"golden": pin4_golden, "sums": pin4_sums, "first_token": pin4_first_token,
         "constant_values": pin4_constant_values, "key_shift": pin4_key_shift, "no_memory": pin4_no_memory}


@pytest.mark.parametrize("name", sorted(PINS4))
def test_wkv4_holds_pin(name):
    PINS4[name](wkv4_ref)


def _wkv4_variant(k, v, w, u, *, decay_before=False, bonus_k=True, den_cur=True, out_after=False, num_only_u=False):
    K, V = np.asarray(k, np.float64), np.asarray(v, np.float64)
    B, T, C = K.shape
    d = np.exp(-np.asarray(w, np.float64))
    a = np.zeros((B, C))
    b = np.zeros((B, C))
    out = np.zeros((B, T, C))
    for t in range(T):
        cur = np.exp(u + K[:, t]) if bonus_k else np.exp(u) * np.ones_like(K[:, t])
        ek = np.exp(K[:, t])
        if out_after:
            a = d * a + ek * V[:, t]
            b = d * b + ek
        cur_den = (np.exp(K[:, t]) if num_only_u else cur) if den_cur else 0.0
        out[:, t] = (a + cur * V[:, t]) / (b + cur_den)
        if not out_after:
            if decay_before:
                a = d * (a + ek * V[:, t])
                b = d * (b + ek)
            else:
                a = d * a + ek * V[:, t]
                b = d * b + ek
    return out


WKV4_MUTANTS = {
    "decay_one_step_too_many": dict(decay_before=True),
    "bonus_without_key": dict(bonus_k=False),
    "denominator_without_current": dict(den_cur=False),
    "output_after_update": dict(out_after=True),
    "u_in_numerator_only": dict(num_only_u=True),
}


@pytest.mark.parametrize("name", sorted(WKV4_MUTANTS))
def test_wkv4_pins_catch_planted_mistakes(name):
    bad = lambda k, v, w, u: _wkv4_variant(k, v, w, u, **WKV4_MUTANTS[name])
    failed = []
    for pin_name, pin in PINS4.items():
        try:
            pin(bad)
        except AssertionError:
            failed.append(pin_name)
    assert failed, f"mutant {name} passes every pin"


def test_wkv4_unmutated_variant_is_the_oracle():
    x = draw4(2, 9, 5, 420)
    np.testing.assert_allclose(_wkv4_variant(*x), wkv4_ref(*x), rtol=1e-14)
