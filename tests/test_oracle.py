"""The CPU oracle against facts that do not come from the oracle itself.

Every pin in ``oracle_pins`` must hold for the recurrent oracle and for the
brute-force evaluator, the two must agree on tiny random inputs, and each
plausible mistake planted in a copy of the recurrence (a dropped term, a
wrong sign or index, a transposed operand) must break at least one pin --
which is what makes the pins worth trusting.
"""
import numpy as np
import pytest

from oracle import wkv6_bruteforce, wkv6_ref, decay
from tests import oracle_pins as P


@pytest.mark.parametrize("name", sorted(P.PINS))
def test_oracle_holds_pin(name):
    P.PINS[name](wkv6_ref)


@pytest.mark.parametrize("name", sorted(P.PINS))
def test_bruteforce_holds_pin(name):
    P.PINS[name](wkv6_bruteforce)


def test_oracle_matches_bruteforce():
    P.pin_bruteforce(wkv6_ref, wkv6_bruteforce)


def test_decay_endpoints():
    assert decay(-np.inf) == 1.0
    assert decay(np.inf) == 0.0
    assert abs(decay(np.log(np.log(2.0))) - 0.5) < 1e-15
    w = decay(np.linspace(-9.0, -0.5, 101))
    assert np.all((w > 0.0) & (w < 1.0)) and np.all(np.diff(w) < 0)


def test_oracle_input_dtypes_widened():
    r, k, v, w_raw, u = P.draw(1, 5, 8, 2, 3)
    y64 = wkv6_ref(r, k, v, w_raw, u, 2, "bidirectional")
    f32 = [a.astype(np.float32) for a in (r, k, v, w_raw, u)]
    y32 = wkv6_ref(*f32, 2, "bidirectional")
    y64b = wkv6_ref(*[a.astype(np.float64) for a in f32], 2, "bidirectional")
    assert y32.dtype == np.float64
    np.testing.assert_array_equal(y32, y64b)
    assert np.max(np.abs(y32 - y64)) < 1e-5


def test_oracle_rejects_bad_mode_and_shape():
    r, k, v, w_raw, u = P.draw(1, 3, 8, 2, 4)
    with pytest.raises(ValueError):
        wkv6_ref(r, k, v, w_raw, u, 2, "sideways")
    with pytest.raises(ValueError):
        wkv6_ref(r, k, v, w_raw, u, 3, "causal")


# ------------------------------------------------------------------ mutants

def _mutant(kind):
    """A copy of the recurrence with exactly one planted mistake."""

    def impl(r, k, v, w_raw, u, H, mode):
        B, T, C = r.shape
        N = C // H
        hs = lambda x: np.asarray(x, np.float64).reshape(B, T, H, N).transpose(0, 2, 1, 3)
        if kind == "strided_heads":   # channel c assigned to head c % H
            hs = lambda x: np.asarray(x, np.float64).reshape(B, T, N, H).transpose(0, 3, 1, 2)
        R, K, V, WR = hs(r), hs(k), hs(v), hs(w_raw)
        U = np.asarray(u, np.float64).reshape(H, N)
        if kind == "strided_heads":
            U = np.asarray(u, np.float64).reshape(N, H).T
        W = np.exp(-np.exp(WR))
        if kind == "decay_exp_only":          # w = exp(-w_raw)
            W = np.exp(-WR)
        if kind == "decay_sign":              # w = exp(+exp(w_raw))... clipped to stay finite
            W = np.exp(np.minimum(np.exp(WR), 5.0))
        Y = np.zeros((B, H, T, N))
        S = np.zeros((B, H, N, N))
        for t in range(T):
            kv = K[:, :, t, :, None] * V[:, :, t, None, :]
            Uu = 0.0 if kind == "drop_u" else U[None, :, :, None]
            if kind == "update_before_read":
                S = W[:, :, t, :, None] * S + kv
                Y[:, :, t] = np.einsum("bhc,bhcn->bhn", R[:, :, t], S + Uu * kv - kv)
                continue
            if kind == "transposed_state":
                Y[:, :, t] = np.einsum("bhn,bhcn->bhc", R[:, :, t], S) + \
                    np.einsum("bhc,bhcn->bhn", R[:, :, t], Uu * kv)
            else:
                Y[:, :, t] = np.einsum("bhc,bhcn->bhn", R[:, :, t], S + Uu * kv)
            if kind == "decay_after_add":
                S = W[:, :, t, :, None] * (S + kv)
            elif kind == "decay_value_index":
                S = W[:, :, t, None, :] * S + kv
            elif kind == "decay_prev_token":
                S = (W[:, :, t - 1, :, None] if t > 0 else 1.0) * S + kv
            else:
                S = W[:, :, t, :, None] * S + kv
        if mode == "bidirectional":
            S = np.zeros((B, H, N, N))
            for t in range(T - 1, -1, -1):
                kv = K[:, :, t, :, None] * V[:, :, t, None, :]
                if kind == "inclusive_reverse":       # the literal list order
                    S = W[:, :, t, :, None] * S + kv
                    Y[:, :, t] += np.einsum("bhc,bhcn->bhn", R[:, :, t], S)
                    continue
                extra = U[None, :, :, None] * kv if kind == "u_both_sweeps" else 0.0
                Y[:, :, t] += np.einsum("bhc,bhcn->bhn", R[:, :, t], S + extra)
                S = W[:, :, t, :, None] * S + kv
        return Y.transpose(0, 2, 1, 3).reshape(B, T, C)

    return impl


MUTANTS = ["strided_heads", "decay_exp_only", "decay_sign", "drop_u", "update_before_read",
           "transposed_state", "decay_after_add", "decay_value_index", "decay_prev_token",
           "inclusive_reverse", "u_both_sweeps"]


def test_unmutated_copy_holds_all_pins():
    assert P.violated_pins(_mutant("none")) == []


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    bad = P.violated_pins(_mutant(kind))
    assert bad, f"mutant {kind} passed every pin"


# ------------------------------------------------------------ state passing

def _ref_state(r, k, v, w_raw, u, H, S0):
    return wkv6_ref(r, k, v, w_raw, u, H, "causal", state_in=S0, return_state=True)


@pytest.mark.parametrize("name", sorted(P.STATE_PINS))
def test_oracle_holds_state_pin(name):
    P.STATE_PINS[name](_ref_state)


def test_oracle_zero_state_is_stateless():
    P.spin_state_zero_is_stateless(_ref_state, wkv6_ref)


def test_bruteforce_with_state_matches_oracle():
    """The explicit pairwise sum with an initial state (its own formula for
    the state term) agrees with the recurrence, and holds the closed form."""
    for seed, (B, T, C, H) in enumerate([(1, 1, 2, 1), (2, 5, 4, 2), (1, 6, 64, 1)]):
        r, k, v, w_raw, u = P.draw(B, T, C, H, 400 + seed)
        S0 = P.draw_state(B, H, C // H, 500 + seed)
        P.close(wkv6_bruteforce(r, k, v, w_raw, u, H, "causal", state_in=S0),
                _ref_state(r, k, v, w_raw, u, H, S0)[0], rtol=1e-12, what="bruteforce with state")
    P.spin_state_alone(lambda r, k, v, w_raw, u, H, S0: (
        wkv6_bruteforce(r, k, v, w_raw, u, H, "causal", state_in=S0),
        _ref_state(r, k, v, w_raw, u, H, S0)[1]))


def test_state_passing_is_causal_only():
    r, k, v, w_raw, u = P.draw(1, 3, 8, 2, 5)
    with pytest.raises(ValueError):
        wkv6_ref(r, k, v, w_raw, u, 2, "bidirectional", state_in=np.zeros((1, 2, 4, 4)))
    with pytest.raises(ValueError):
        wkv6_ref(r, k, v, w_raw, u, 2, "causal", state_in=np.zeros((1, 2, 4, 5)))


def _state_mutant(kind):
    """A copy of the causal recurrence with a state and one planted mistake."""

    def impl(r, k, v, w_raw, u, H, S0):
        B, T, C = r.shape
        N = C // H
        hs = lambda x: np.asarray(x, np.float64).reshape(B, T, H, N).transpose(0, 2, 1, 3)
        R, K, V, W = hs(r), hs(k), hs(v), np.exp(-np.exp(hs(w_raw)))
        U = np.asarray(u, np.float64).reshape(H, N)
        S = np.array(S0, np.float64)
        if kind == "state_transposed":
            S = S.transpose(0, 1, 3, 2).copy()
        if kind == "state_decayed_first" and T > 0:   # S0 decayed by w_0 before token 0 reads it
            S = W[:, :, 0, :, None] * S
        Y = np.zeros((B, H, T, N))
        for t in range(T):
            kv = K[:, :, t, :, None] * V[:, :, t, None, :]
            Y[:, :, t] = np.einsum("bhc,bhcn->bhn", R[:, :, t], S + U[None, :, :, None] * kv)
            if kind == "last_token_not_in_state" and t == T - 1:
                break
            S = W[:, :, t, :, None] * S + kv
        if kind == "state_scaled_twice":
            S = 2.0 * S - np.array(S0, np.float64) * 0.0 + 0.5 * S
        return Y.transpose(0, 2, 1, 3).reshape(B, T, C), S

    return impl


def test_unmutated_state_copy_holds_state_pins():
    assert P.violated_state_pins(_state_mutant("none")) == []


@pytest.mark.parametrize("kind", ["state_transposed", "state_decayed_first", "last_token_not_in_state",
                                  "state_scaled_twice"])
def test_planted_state_mistake_is_caught(kind):
    assert P.violated_state_pins(_state_mutant(kind)), f"state mutant {kind} passed every pin"
