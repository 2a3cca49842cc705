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


# ------------------------------------------------------------------ backward

def _fd_grad(fn, args, name, eps=1e-6):
    """Central differences of fn(**args) with respect to args[name]."""
    x = args[name]
    g = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        a = dict(args)
        xp = x.copy()
        xp[idx] += eps
        a[name] = xp
        fp = fn(**a)
        xm = x.copy()
        xm[idx] -= eps
        a[name] = xm
        g[idx] = (fp - fn(**a)) / (2 * eps)
    return g


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
@pytest.mark.parametrize("shape", [(1, 1, 4, 1), (2, 5, 8, 2), (1, 7, 4, 1)])
def test_backward_matches_finite_differences(mode, shape):
    """The gradients of sum(y * dy) agree with central differences of the
    (pinned) forward oracle: a check that does not use the backward's own
    recurrences."""
    from oracle import wkv6_ref_backward

    B, T, C, H = shape
    r, k, v, w_raw, u = P.draw(B, T, C, H, 600 + T + C)
    dy = np.random.default_rng(700 + T).normal(size=(B, T, C))
    g = wkv6_ref_backward(r, k, v, w_raw, u, dy, H, mode)
    loss = lambda r, k, v, w_raw, u: float((wkv6_ref(r, k, v, w_raw, u, H, mode) * dy).sum())
    args = {"r": r, "k": k, "v": v, "w_raw": w_raw, "u": u}
    for name in args:
        P.close(g[name], _fd_grad(loss, args, name), rtol=1e-7, what=f"d{name} {mode} {shape}")


def test_backward_decay_identity():
    """The decay gradient by the pair-counting identity the GPU kernel uses,
    dlambda_j = sum_{t>j} r dr - sum_{i>=j} k dk + r_j u k_j (dy_j . v_j) and
    dw_raw = dlambda * (-exp(w_raw)), equals the oracle's (which takes
    sum_n G_t S_{t-1} from the states instead)."""
    from oracle import wkv6_ref_backward

    B, T, C, H = 2, 9, 8, 2
    r, k, v, w_raw, u = P.draw(B, T, C, H, 620)
    dy = np.random.default_rng(621).normal(size=(B, T, C))
    g = wkv6_ref_backward(r, k, v, w_raw, u, dy, H, "causal")
    rdr, kdk = r * g["r"], k * g["k"]
    dyv = (P.heads(dy, H) * P.heads(v, H)).sum(-1, keepdims=True)          # [B, T, H, 1]
    bonus = (P.heads(r, H) * u.reshape(H, C // H) * P.heads(k, H) * dyv).reshape(B, T, C)
    after = np.cumsum(rdr[:, ::-1], axis=1)[:, ::-1] - rdr                   # sum over t > j
    from_j = np.cumsum(kdk[:, ::-1], axis=1)[:, ::-1]                       # sum over i >= j
    dlam = after - from_j + bonus
    P.close(dlam * -np.exp(w_raw), g["w_raw"], rtol=1e-12, what="decay identity")


def _bwd_mutant(kind):
    """A copy of the causal adjoint with one planted mistake (dr, dk, dv, dW)."""

    def impl(r, k, v, w_raw, u, dy, H):
        B, T, C = r.shape
        N = C // H
        hs = lambda x: np.asarray(x, np.float64).reshape(B, T, H, N).transpose(0, 2, 1, 3)
        R, K, V, WR, DY = (hs(x) for x in (r, k, v, w_raw, dy))
        W = np.exp(-np.exp(WR))
        U = np.asarray(u, np.float64).reshape(H, N)[None]
        S = np.zeros((B, H, N, N))
        St = np.zeros((B, H, T, N, N))
        dR = np.zeros_like(R)
        for t in range(T):
            St[:, :, t] = S
            dyv = (DY[:, :, t] * V[:, :, t]).sum(-1)[..., None]
            bon = 0.0 if kind == "dr_no_bonus" else U * K[:, :, t] * dyv
            dR[:, :, t] = np.einsum("bhcn,bhn->bhc", S, DY[:, :, t]) + bon
            S = W[:, :, t, :, None] * S + K[:, :, t, :, None] * V[:, :, t, None, :]
        G = np.zeros_like(S)
        dK, dV, dW = np.zeros_like(K), np.zeros_like(V), np.zeros_like(W)
        for t in range(T - 1, -1, -1):
            if kind == "adjoint_updated_first":
                G = W[:, :, t, :, None] * G + R[:, :, t, :, None] * DY[:, :, t, None, :]
            dyv = (DY[:, :, t] * V[:, :, t]).sum(-1)[..., None]
            ruk = (R[:, :, t] * U * K[:, :, t]).sum(-1)[..., None]
            dK[:, :, t] = np.einsum("bhcn,bhn->bhc", G, V[:, :, t]) + R[:, :, t] * U * dyv
            Gv = G.transpose(0, 1, 3, 2) if kind == "dv_transposed" else G
            dV[:, :, t] = np.einsum("bhcn,bhc->bhn", Gv, K[:, :, t]) + ruk * DY[:, :, t]
            Sprev = S if kind == "dw_current_state" else St[:, :, t]
            dW[:, :, t] = np.einsum("bhcn,bhcn->bhc", G, Sprev)
            if kind != "adjoint_updated_first":
                G = W[:, :, t, :, None] * G + R[:, :, t, :, None] * DY[:, :, t, None, :]
        back = lambda X: X.transpose(0, 2, 1, 3).reshape(B, T, C)
        return {"r": back(dR), "k": back(dK), "v": back(dV), "w_raw": back(dW * W * -np.exp(WR))}

    return impl


@pytest.mark.parametrize("kind", ["dr_no_bonus", "adjoint_updated_first", "dv_transposed", "dw_current_state"])
def test_backward_mutant_fails_finite_differences(kind):
    B, T, C, H = 1, 5, 4, 1
    r, k, v, w_raw, u = P.draw(B, T, C, H, 640)
    dy = np.random.default_rng(641).normal(size=(B, T, C))
    g = _bwd_mutant(kind)(r, k, v, w_raw, u, dy, H)
    good = _bwd_mutant("none")(r, k, v, w_raw, u, dy, H)
    loss = lambda r, k, v, w_raw, u: float((wkv6_ref(r, k, v, w_raw, u, H, "causal") * dy).sum())
    args = {"r": r, "k": k, "v": v, "w_raw": w_raw, "u": u}
    bad = []
    for name in ("r", "k", "v", "w_raw"):
        fd = _fd_grad(loss, args, name)
        P.close(good[name], fd, rtol=1e-7, what="unmutated copy")
        if np.max(np.abs(g[name] - fd)) > 1e-6 * max(1.0, np.max(np.abs(fd))):
            bad.append(name)
    assert bad, f"backward mutant {kind} passed the finite-difference check"
