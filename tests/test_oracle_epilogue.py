"""The epilogue oracle (per-head group normalisation, affine, gate) against
facts that do not come from it: a hand-worked example, torch's own
group_norm (float64, on the CPU) as an independent library routine, and
invariants; each planted mistake must break one of them.
"""
import numpy as np
import pytest

from oracle import group_norm_heads, wkv6_gn_ref, wkv6_ref


def test_hand_worked_example():
    # one head of N = 4: y = 1, 2, 3, 6 has mean 3 and biased variance 3.5;
    # with eps = 0.5 the scale is 1/2, so z = -1, -1/2, 0, 3/2; gamma = 1, 2,
    # 1, 1 and beta = 0, 0, 1, 0 give -1, -1, 1, 3/2; times g = 2, 1, 1, -1:
    # -2, -1, 1, -3/2
    y = np.array([[[1.0, 2.0, 3.0, 6.0]]])
    out = group_norm_heads(y, 1, [1.0, 2.0, 1.0, 1.0], [0.0, 0.0, 1.0, 0.0], 0.5) * np.array([2.0, 1.0, 1.0, -1.0])
    np.testing.assert_allclose(out[0, 0], [-2.0, -1.0, 1.0, -1.5], rtol=1e-15)


@pytest.mark.parametrize("H,N", [(1, 4), (3, 64), (12, 64)])
def test_matches_torch_group_norm(H, N):
    import torch

    rng = np.random.default_rng(H * 100 + N)
    B, T, C = 2, 5, H * N
    y = rng.normal(size=(B, T, C)) * rng.uniform(0.1, 10.0, size=(1, T, 1))
    gamma, beta = rng.normal(size=C), rng.normal(size=C)
    ref = torch.nn.functional.group_norm(torch.from_numpy(y.reshape(B * T, C)), H,
                                         torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-3)
    np.testing.assert_allclose(group_norm_heads(y, H, gamma, beta, 1e-3), ref.numpy().reshape(B, T, C),
                               rtol=1e-12, atol=1e-12)


def test_scale_and_shift_of_a_head_do_not_matter():
    rng = np.random.default_rng(7)
    B, T, H, N = 2, 6, 3, 64
    y = rng.normal(size=(B, T, H * N))
    a = rng.uniform(0.5, 4.0, size=(B, T, H, 1))
    c = rng.normal(size=(B, T, H, 1))
    y2 = (y.reshape(B, T, H, N) * a + c).reshape(B, T, H * N)
    one, zero = np.ones(H * N), np.zeros(H * N)
    np.testing.assert_allclose(group_norm_heads(y2, H, one, zero, 0.0), group_norm_heads(y, H, one, zero, 0.0),
                               rtol=1e-10, atol=1e-10)
    z = group_norm_heads(y, H, one, zero, 0.0).reshape(B, T, H, N)
    np.testing.assert_allclose(z.mean(-1), 0.0, atol=1e-13)
    np.testing.assert_allclose((z ** 2).mean(-1), 1.0, rtol=1e-12)


def test_fused_reference_hand_worked_single_token():
    """wkv6_gn_ref through the operator, worked by hand.  With one token the
    operator's output is the u-weighted current token alone, y_0 = (sum_c
    r_0[c] u[c] k_0[c]) v_0, in both modes (no earlier and no later token).
    Here r_0 = (1, 2, 0, 0), u = (0.5, 0.25, 3, 3), k_0 = (1, 1, 0, 0) give
    the weight 1/2 + 1/2 = 1, so y_0 = v_0 = (1, 2, 3, 6), and the worked
    normalisation above (eps = 1/2, gamma = 1, 2, 1, 1, beta = 0, 0, 1, 0,
    gate 2, 1, 1, -1) gives -2, -1, 1, -3/2.  A second head has r scaled by 10
    and u by 1/10, so its weight and its row are the same."""
    r = np.array([[[1.0, 2.0, 0.0, 0.0, 10.0, 20.0, 0.0, 0.0]]])
    k = np.array([[[1.0, 1.0, 0.0, 0.0, 1.0, 1.0, 0.0, 0.0]]])
    u = np.array([0.5, 0.25, 3.0, 3.0, 0.05, 0.025, 7.0, 7.0])
    v = np.array([[[1.0, 2.0, 3.0, 6.0, 1.0, 2.0, 3.0, 6.0]]])
    w_raw = np.array([[[0.3, -1.0, 2.0, -5.0, 0.0, 0.0, 1.0, 1.0]]])   # a single token never decays
    gamma = np.array([1.0, 2.0, 1.0, 1.0] * 2)
    beta = np.array([0.0, 0.0, 1.0, 0.0] * 2)
    g = np.array([[[2.0, 1.0, 1.0, -1.0] * 2]])
    for mode in ("causal", "bidirectional"):
        out = wkv6_gn_ref(r, k, v, w_raw, u, g, gamma, beta, 0.5, 2, mode)
        np.testing.assert_allclose(out[0, 0], [-2.0, -1.0, 1.0, -1.5] * 2, rtol=1e-12)


def test_fused_reference_hand_worked_two_tokens():
    """Two tokens, one head of N = 2, causal: y_0 = (r_0 . u k_0) v_0 and
    y_1 = r_1 . (k_0^T v_0 + diag(u) k_1^T v_1) (the first token reaches the
    second with weight 1: no decay lies strictly between them).  With
    r_0 = (1, 0), k_0 = (1, 0), v_0 = (1, 3), r_1 = (1, 1), k_1 = (0, 2),
    v_1 = (2, 2), u = (1, 1): y_0 = (1, 3) and y_1 = (1 + 4, 3 + 4) = (5, 7).
    Each row has mean m and half-spread d, so with eps = 0 it normalises to
    (-1, +1); gamma = (2, 1), beta = (1, 0), gate (1, -1) give (-1, -1).
    Bidirectional adds r_0 . k_1^T v_1 = 0 to y_0 and nothing to y_1."""
    r = np.array([[[1.0, 0.0], [1.0, 1.0]]])
    k = np.array([[[1.0, 0.0], [0.0, 2.0]]])
    v = np.array([[[1.0, 3.0], [2.0, 2.0]]])
    w_raw = np.array([[[0.7, -0.2], [1.1, 0.4]]])
    u = np.array([1.0, 1.0])
    g = np.array([[[1.0, -1.0], [1.0, -1.0]]])
    for mode in ("causal", "bidirectional"):
        out = wkv6_gn_ref(r, k, v, w_raw, u, g, [2.0, 1.0], [1.0, 0.0], 0.0, 1, mode)
        np.testing.assert_allclose(out[0], [[-1.0, -1.0], [-1.0, -1.0]], rtol=1e-12, atol=1e-12)


def test_fused_reference_is_the_composition():
    rng = np.random.default_rng(8)
    B, T, H = 1, 7, 2
    C = 64 * H
    r, k, v = (rng.normal(size=(B, T, C)) * 0.5 for _ in range(3))
    w_raw = rng.uniform(-6.0, -0.5, size=(B, T, C))
    u, gamma, beta = rng.normal(size=C), rng.normal(size=C), rng.normal(size=C)
    g = rng.normal(size=(B, T, C))
    for mode in ("causal", "bidirectional"):
        y = wkv6_ref(r, k, v, w_raw, u, H, mode)
        want = group_norm_heads(y, H, gamma, beta, 1e-4) * g
        np.testing.assert_array_equal(wkv6_gn_ref(r, k, v, w_raw, u, g, gamma, beta, 1e-4, H, mode), want)


def _mutant(kind, y, H, gamma, beta, eps):
    y = np.asarray(y, np.float64)
    B, T, C = y.shape
    N = C // H
    groups = 1 if kind == "whole_row" else H
    yh = y.reshape(B, T, groups, C // groups)
    mean = yh.mean(-1, keepdims=True)
    ddof = 1 if kind == "unbiased" else 0
    var = ((yh - mean) ** 2).sum(-1, keepdims=True) / (yh.shape[-1] - ddof)
    den = np.sqrt(var) + eps if kind == "eps_outside" else np.sqrt(var + eps)
    z = ((yh - mean) / den).reshape(B, T, C)
    return z * gamma + beta


@pytest.mark.parametrize("kind", ["whole_row", "unbiased", "eps_outside"])
def test_pins_catch_planted_mistakes(kind):
    caught = False
    try:
        y = np.array([[[1.0, 2.0, 3.0, 6.0]]])
        out = _mutant(kind, y, 1, np.array([1.0, 2.0, 1.0, 1.0]), np.array([0.0, 0.0, 1.0, 0.0]), 0.5)
        np.testing.assert_allclose(out[0, 0] * np.array([2.0, 1.0, 1.0, -1.0]), [-2.0, -1.0, 1.0, -1.5], rtol=1e-15)
    except AssertionError:
        caught = True
    if not caught:   # the hand-worked case has one head: the per-head check needs several
        import torch
        rng = np.random.default_rng(9)
        y = rng.normal(size=(1, 3, 128))
        gamma, beta = rng.normal(size=128), rng.normal(size=128)
        ref = torch.nn.functional.group_norm(torch.from_numpy(y.reshape(3, 128)), 2, torch.from_numpy(gamma),
                                             torch.from_numpy(beta), eps=1e-3).numpy().reshape(1, 3, 128)
        caught = not np.allclose(_mutant(kind, y, 2, gamma, beta, 1e-3), ref, rtol=1e-9, atol=1e-9)
    assert caught


def test_gate_multiplies_after_the_affine():
    """(z gamma + beta) g, not z gamma g + beta: with beta != 0 and g != 1 the
    two differ; the hand-worked example above has beta = 1 on a channel
    whose gate is 1 and beta = 0 elsewhere, so check a channel with both."""
    y = np.array([[[0.0, 2.0]]])
    out = group_norm_heads(y, 1, [1.0, 1.0], [3.0, 3.0], 0.0) * np.array([2.0, 2.0])
    np.testing.assert_allclose(out[0, 0], [(-1.0 + 3.0) * 2.0, (1.0 + 3.0) * 2.0], rtol=1e-15)
