"""Parity of wkv6_bwd (the gradients of sum(y * dy)) with the float64 oracle's
adjoint, through the C ABI.

The backward runs in float32 on the exact input values, so one tolerance
serves both input dtypes: max|g - g_ref| / rms(g_ref) <= 1e-4 for each of
dr, dk, dv, dw_raw and du.
"""
import numpy as np
import pytest

from linear_attention_rnn_amd import inputs as I
from oracle import wkv6_ref_backward
from tests.gpu_util import device_inputs, err_over_rms, say

pytestmark = pytest.mark.gpu

TOL = 1e-4
NAMES = ("r", "k", "v", "w_raw", "u")


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def gpu_bwd(x, dy, H, mode, dtype):
    import torch
    from linear_attention_rnn_amd import wkv6

    d = device_inputs(x, dtype)
    g = wkv6.bwd(*d, torch.from_numpy(np.ascontiguousarray(dy, np.float32)).cuda(), H, mode)
    torch.cuda.synchronize()
    return {name: g[name].double().cpu().numpy() for name in NAMES}


def check(tag, x, dy, H, mode, dtype):
    g = gpu_bwd(x, dy, H, mode, dtype)
    ref = wkv6_ref_backward(x["r"], x["k"], x["v"], x["w_raw"], x["u"], dy, H, mode)
    errs = {name: err_over_rms(g[name], ref[name]) for name in NAMES if name != "w_raw"}
    # dw_raw is a difference of running sums of k dk and r dr (times exp(w_raw));
    # it can be exactly zero (first and last token, T <= 2), so its error is
    # measured against the scale of those terms as well
    scale = max(float(np.sqrt(np.mean(ref["w_raw"] ** 2))),
                float(np.sqrt(np.mean((x["k"] * ref["k"] * np.exp(x["w_raw"].astype(np.float64))) ** 2))))
    dw_err = float(np.max(np.abs(g["w_raw"] - ref["w_raw"]))) if np.all(np.isfinite(g["w_raw"])) else np.inf
    errs["w_raw"] = dw_err / scale if scale > 0 else dw_err   # scale 0: w = 1 everywhere, dw_raw = 0
    say(f"[backward] {tag}: " + "  ".join(f"d{n} {e:.2e}" for n, e in errs.items()))
    for name, e in errs.items():
        assert e <= TOL, f"d{name}: {e:.3e}"


def dy_of(x, seed):
    return np.random.default_rng(seed).normal(0.0, 0.5, size=x["r"].shape).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
@pytest.mark.parametrize("T", [1, 2, 17, 64, 130])
def test_backward_parity(torch_cuda, T, mode, dtype):
    B, H = 2, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=800 + T, dtype=dtype)
    check(f"T={T} {mode} {dtype}", x, dy_of(x, 900 + T), H, mode, dtype)


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_backward_image_shape(torch_cuda, mode):
    """The image-base shape (T = 196, C = 768, H = 12) with a smaller batch."""
    B, T, H = 3, 196, 12
    x = I.random_inputs(B, T, 64 * H, H, seed=81, dtype="bf16")
    check(f"image shape {mode}", x, dy_of(x, 82), H, mode, "bf16")


def test_backward_long_sequence(torch_cuda):
    """Slow decays over 1500 tokens: the running sums behind the decay
    gradient and the state keep their accuracy."""
    B, T, H = 1, 1500, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=83, dtype="f32", wraw_lo=-9.0, wraw_hi=-2.0)
    check("long causal", x, dy_of(x, 84), H, "causal", "f32")


def test_backward_image_hires_full(torch_cuda):
    """The benched image-hires shape (B = 4, T = 4096, C = 1024, H = 16,
    bidirectional, bf16, 10% of channels at w_raw = -9) with the planner's
    own segment count (the sequences are cut into segments there), every
    gradient compared with the oracle over the whole tensor."""
    w = I.workload("image-hires-bidir-bf16")
    x = I.make_inputs(w)
    say(f"[backward] image-hires full: B={w.B} T={w.T} C={w.C} H={w.H}")
    check("image-hires full (default segments)", x, dy_of(x, w.seed + 1000), w.H, w.mode, w.dtype)


@pytest.mark.parametrize("case", ["no_decay", "fast_decay", "mixed"])
def test_backward_decay_extremes(torch_cuda, case):
    B, T, H = 2, 40, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=85, dtype="f32")
    if case == "no_decay":
        x["w_raw"][:] = -np.inf
    elif case == "fast_decay":
        x["w_raw"][:] = 1.5
    else:
        x["w_raw"] = np.random.default_rng(86).choice(
            np.array([-np.inf, -20.0, -4.0, 0.0, 1.5], np.float32), size=x["w_raw"].shape)
    check(f"extremes {case}", x, dy_of(x, 87), H, "bidirectional", "f32")


def test_backward_empty_sequence(torch_cuda):
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    z = torch.zeros((2, 0, 128), device="cuda")
    g = wkv6.bwd(z, z, z, z, torch.ones(128, device="cuda"), z, 2, "bidirectional")
    torch.cuda.synchronize()
    assert g["r"].shape == (2, 0, 128) and torch.count_nonzero(g["u"]).item() == 0


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_backward_segments(torch_cuda, monkeypatch, mode):
    """A sequence cut into segments (state and adjoint carried across the cuts,
    the decay gradient's running sum completed by the later segments) gives
    the one-segment result; ragged last segments included."""
    B, T, H = 1, 300, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=88, dtype="f32", wraw_lo=-6.0, wraw_hi=-1.0)
    dy = dy_of(x, 89)
    got = {}
    for G in (1, 2, 3, 5):
        monkeypatch.setenv("WKV6_BWD_SEGMENTS", str(G))
        check(f"segments {G} {mode}", x, dy, H, mode, "f32")
        got[G] = gpu_bwd(x, dy, H, mode, "f32")
    for G in (2, 3, 5):
        for name in NAMES:
            scale = float(np.sqrt(np.mean(got[1][name] ** 2))) or 1.0
            assert float(np.max(np.abs(got[G][name] - got[1][name]))) / scale <= 1e-4, (G, name)


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_backward_segments_decay_extremes(torch_cuda, monkeypatch, mode):
    """Segment summaries under decays of 1 (w_raw = -inf), 0 to rounding
    (w_raw = 1.5) and between, mixed per token and channel: the carried state,
    adjoint and total decay still give the oracle's gradients."""
    B, T, H = 1, 200, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=90, dtype="f32")
    x["w_raw"] = np.random.default_rng(91).choice(
        np.array([-np.inf, -20.0, -4.0, 0.0, 1.5], np.float32), size=x["w_raw"].shape)
    dy = dy_of(x, 92)
    for G in (1, 3):
        monkeypatch.setenv("WKV6_BWD_SEGMENTS", str(G))
        check(f"segments {G} extremes {mode}", x, dy, H, mode, "f32")


def test_backward_text_long_full(torch_cuda):
    """The benched text-long shape (B = 8, T = 4096, C = 2048, H = 32, causal,
    bf16) with the planner's own choice (unsegmented, on the chunked MFMA
    kernels), every gradient compared with the oracle over the whole tensor."""
    w = I.workload("text-long-causal-bf16")
    x = I.make_inputs(w)
    say(f"[backward] text-long full: B={w.B} T={w.T} C={w.C} H={w.H}")
    check("text-long full (default plan)", x, dy_of(x, w.seed + 1000), w.H, w.mode, w.dtype)
