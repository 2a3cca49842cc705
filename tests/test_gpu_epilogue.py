"""Parity of wkv6_fwd_gn (the forward with the per-head group normalisation,
affine and gate fused into its output) with the float64 oracle.

Bound, per element, derived from the forward's own bound: y on the GPU is
within tol_y * rms(y_ref) of the oracle (tol_y = 1e-4 for float32 inputs,
5e-3 for bfloat16 inputs, as the plain forward's parity tests check), and
the normalisation z = (y - mean) / s of a head row with s = sqrt(var + eps)
moves by at most (2 + |z|) * max|dy| / s for a change dy of its row; the
affine and gate scale that by |gamma * g|; the result is then rounded to
bf16 (nearest even: at most 2^-8 of its size), with a little float32
rounding on top:

  |out - ref| <= 2^-8 |ref| + (2 + |z|) tol_y rms(y_ref) / s |gamma g| + 1e-6 (|gamma g| + |beta g|)
"""
import numpy as np
import pytest

from linear_attention_rnn_amd import inputs as I
from oracle import wkv6_gn_ref, wkv6_ref
from tests.gpu_util import device_inputs, say, to_device

pytestmark = pytest.mark.gpu

TOL_Y = {"f32": 1e-4, "bf16": 5e-3}
EPS = 64e-5


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def extras(B, T, C, seed, dtype):
    rng = np.random.default_rng(seed)
    g = rng.normal(size=(B, T, C)).astype(np.float32)
    if dtype == "bf16":
        g = I.round_to_bf16(g)
    gamma = rng.uniform(0.5, 1.5, size=C).astype(np.float32)
    beta = rng.normal(0.0, 0.3, size=C).astype(np.float32)
    return g, gamma, beta


def run_gn(x, g, gamma, beta, H, mode, dtype, eps=EPS):
    import torch
    from linear_attention_rnn_amd import wkv6

    d = device_inputs(x, dtype)
    out = wkv6.fwd_gn(*d, to_device(g, dtype), torch.from_numpy(gamma).cuda(), torch.from_numpy(beta).cuda(),
                      H, mode, eps=eps)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check(tag, x, g, gamma, beta, H, mode, dtype, out, eps=EPS):
    """out against wkv6_gn_ref; the per-element bound needs the operator's y
    and the normalised z of each head row, taken from the oracle as well."""
    ref = wkv6_gn_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], g, gamma, beta, eps, H, mode)
    y = wkv6_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], H, mode)
    B, T, C = y.shape
    yh = y.reshape(B, T, H, 64)
    s = np.sqrt(yh.var(-1) + eps)[..., None]
    z = ((yh - yh.mean(-1, keepdims=True)) / s).reshape(B, T, C)
    s = np.broadcast_to(s, yh.shape).reshape(B, T, C)
    gg = np.abs(gamma * g)
    bound = (2.0 ** -8 * np.abs(ref) + (2.0 + np.abs(z)) * TOL_Y[dtype] * np.sqrt(np.mean(y ** 2)) / s * gg
             + 1e-6 * (gg + np.abs(beta * g)))
    err = np.abs(out - ref)
    ratio = float(np.max(err / bound)) if np.all(np.isfinite(out)) else np.inf
    rel = float(np.max(err) / np.sqrt(np.mean(ref ** 2)))
    say(f"[gn] {tag}: max err/bound {ratio:.3f}  max|d|/rms {rel:.2e}")
    assert ratio <= 1.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
@pytest.mark.parametrize("T", [1, 4, 64, 130])
def test_gn_parity(torch_cuda, T, mode, dtype):
    B, H = 2, 3
    C = 64 * H
    x = I.random_inputs(B, T, C, H, seed=700 + T, dtype=dtype)
    g, gamma, beta = extras(B, T, C, 710 + T, dtype)
    out = run_gn(x, g, gamma, beta, H, mode, dtype)
    check(f"T={T} {mode} {dtype}", x, g, gamma, beta, H, mode, dtype, out)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_gn_segments_and_slow_path(torch_cuda, monkeypatch, mode, dtype):
    """Sequences cut into segments (carries), and decays fast enough that
    chunks take the general path: in the float32 sweeps themselves, for bf16
    through the fix-up kernel and its markers."""
    B, H, T = 1, 2, 64 * 7 + 9
    C = 64 * H
    for G, slow in ((3, False), (None, True), (4, True)):
        if G is None:
            monkeypatch.delenv("WKV6_SEGMENTS", raising=False)
        else:
            monkeypatch.setenv("WKV6_SEGMENTS", str(G))
        x = I.random_inputs(B, T, C, H, seed=720, dtype=dtype)
        if slow:
            x["w_raw"] = np.random.default_rng(721).choice(np.array([-9.0, -0.5, 1.0, 1.5], np.float32),
                                                           size=x["w_raw"].shape)
        g, gamma, beta = extras(B, T, C, 722, dtype)
        out = run_gn(x, g, gamma, beta, H, mode, dtype)
        check(f"segments {G} slow {slow} {mode} {dtype}", x, g, gamma, beta, H, mode, dtype, out)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gn_repeated_calls_reuse_clean_markers(torch_cuda, dtype):
    """A call with chunks on the general path (bf16: the fix-up path and its
    markers), then one without, on workspace memory the allocator hands
    back: the second is still right."""
    B, H, T = 2, 2, 200
    C = 64 * H
    x = I.random_inputs(B, T, C, H, seed=730, dtype=dtype)
    x["w_raw"][:, 100:110] = 1.5
    g, gamma, beta = extras(B, T, C, 731, dtype)
    check("slow call", x, g, gamma, beta, H, "bidirectional", dtype, run_gn(x, g, gamma, beta, H, "bidirectional", dtype))
    x2 = I.random_inputs(B, T, C, H, seed=732, dtype=dtype)
    check("fast call after", x2, g, gamma, beta, H, "bidirectional", dtype,
          run_gn(x2, g, gamma, beta, H, "bidirectional", dtype))


def test_gn_image_base_shape_full(torch_cuda):
    """Full image-base size (B = 64, T = 196, C = 768, H = 12, bidirectional,
    bf16) in one call; every batch item checked against the oracle."""
    B, T, C, H = 64, 196, 768, 12
    x = I.random_inputs(B, T, C, H, seed=740, dtype="bf16")
    g, gamma, beta = extras(B, T, C, 741, "bf16")
    out = run_gn(x, g, gamma, beta, H, "bidirectional", "bf16")
    check("image-base, all 64 items", x, g, gamma, beta, H, "bidirectional", "bf16", out)


def test_gn_zero_eps_and_constant_rows(torch_cuda):
    """eps = 0 on ordinary rows; a row with equal values everywhere (all
    inputs zero except the gate) gives beta * g exactly when eps > 0."""
    B, H, T = 1, 2, 70
    C = 64 * H
    x = I.random_inputs(B, T, C, H, seed=750, dtype="f32")
    g, gamma, beta = extras(B, T, C, 751, "f32")
    check("eps 0", x, g, gamma, beta, H, "causal", "f32", run_gn(x, g, gamma, beta, H, "causal", "f32", eps=0.0), eps=0.0)
    z = {key: np.zeros_like(val) for key, val in x.items() if key != "stuck"}
    out = run_gn(z, g, gamma, beta, H, "causal", "f32")
    want = I.round_to_bf16((beta * g).astype(np.float32)).astype(np.float64)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_group_norm_gate_standalone(torch_cuda, dtype):
    """wkv6_group_norm_gate on a given y: the oracle's normalisation and gate
    of that same y, within bf16 rounding of the result (2^-8 of its size)
    plus float32 rounding of the row statistics."""
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    B, T, H = 3, 77, 5
    C = 64 * H
    rng = np.random.default_rng(760)
    y = (rng.normal(size=(B, T, C)) * rng.uniform(0.01, 30.0, size=(B, T, 1))
         + rng.normal(size=(B, T, 1))).astype(np.float32)
    g, gamma, beta = extras(B, T, C, 761, dtype)
    out = wkv6.group_norm_gate(torch.from_numpy(y).cuda(), to_device(g, dtype), torch.from_numpy(gamma).cuda(),
                               torch.from_numpy(beta).cuda(), H, eps=EPS)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    yh = y.astype(np.float64).reshape(B, T, H, 64)
    z = ((yh - yh.mean(-1, keepdims=True)) / np.sqrt(yh.var(-1, keepdims=True) + EPS)).reshape(B, T, C)
    ref = (z * gamma + beta) * g
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * (np.abs(gamma * g) * (1.0 + np.abs(z)) + np.abs(beta * g))
    ratio = float(np.max(np.abs(got - ref) / bound))
    say(f"[gn] standalone {dtype}: max err/bound {ratio:.3f}")
    assert ratio <= 1.0


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_forward_then_group_norm_gate(torch_cuda, mode):
    """The unfused order (wkv6_fwd, then wkv6_group_norm_gate on its y) meets
    the fused epilogue's bound against the oracle."""
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    B, H, T = 2, 3, 300
    C = 64 * H
    x = I.random_inputs(B, T, C, H, seed=770, dtype="bf16")
    g, gamma, beta = extras(B, T, C, 771, "bf16")
    d = device_inputs(x, "bf16")
    y = wkv6.fwd(*d, H, mode)
    out = wkv6.group_norm_gate(y, to_device(g, "bf16"), torch.from_numpy(gamma).cuda(), torch.from_numpy(beta).cuda(),
                               H, eps=EPS)
    torch.cuda.synchronize()
    check(f"two-step {mode}", x, g, gamma, beta, H, mode, "bf16", out.float().cpu().numpy().astype(np.float64))


def test_gn_empty(torch_cuda):
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    z = torch.zeros((2, 0, 128), device="cuda")
    c = torch.ones(128, device="cuda")
    out = wkv6.fwd_gn(z, z, z, z, c, z, c, c, 2, "bidirectional")
    assert out.shape == (2, 0, 128) and out.dtype == torch.bfloat16
