"""Parity of the two older operators with their float64 oracles, through the
C ABI: wkv5_fwd (RWKV-5, one decay per channel for every token) and
wkv4_fwd (RWKV-4, the normalised per-channel operator).

Tolerances, max|y - y_ref| / rms(y_ref): RWKV-5 runs the RWKV-6 kernels, so
it has their bounds (1e-4 with float32 inputs, 5e-3 with bfloat16 inputs);
it must also equal wkv6_fwd bit for bit when that is given the same decay
for every token.  RWKV-4 runs in float32 on the exact input values (bf16
inputs widen exactly), so one bound serves both dtypes: 1e-4.
"""
import numpy as np
import pytest

from linear_attention_rnn_amd import inputs as I
from oracle import wkv4_ref, wkv5_ref
from tests.gpu_util import err_over_rms, say, to_device

pytestmark = pytest.mark.gpu

TOL5 = {"f32": 1e-4, "bf16": 5e-3}
TOL4 = 1e-4


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def run5(x, H, mode, dtype):
    import torch
    from linear_attention_rnn_amd import wkv6

    d = [to_device(x[key], dtype) for key in ("r", "k", "v", "w_raw")]
    u = torch.from_numpy(x["u"]).cuda()
    y = wkv6.fwd5(*d, u, H, mode)
    torch.cuda.synchronize()
    return y


def run6_broadcast(x, H, mode, dtype):
    """wkv6_fwd with the RWKV-5 decay repeated for every token."""
    import torch
    from linear_attention_rnn_amd import wkv6

    w_t = np.ascontiguousarray(np.broadcast_to(x["w_raw"], x["r"].shape))
    d = [to_device(x[key], dtype) for key in ("r", "k", "v")] + [to_device(w_t, dtype)]
    u = torch.from_numpy(x["u"]).cuda()
    y = wkv6.fwd(*d, u, H, mode)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
@pytest.mark.parametrize("T", [1, 3, 64, 130, 257])
def test_wkv5_parity(torch_cuda, T, mode, dtype):
    B, H = 2, 3
    x = I.random_inputs_wkv5(B, T, 64 * H, seed=500 + T, dtype=dtype)
    y = run5(x, H, mode, dtype).double().cpu().numpy()
    y_ref = wkv5_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], H, mode)
    e = err_over_rms(y, y_ref)
    say(f"[wkv5] T={T} {mode} {dtype}: {e:.3e}")
    assert e <= TOL5[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_wkv5_equals_wkv6_with_a_repeated_decay(torch_cuda, monkeypatch, mode, dtype):
    """The same kernels on the same values: identical bits, with one and with
    several segments per sequence, and for few-token causal calls."""
    B, H = 2, 2
    for T, G in ((3, None), (300, None), (64 * 7 + 5, 3)):
        if G is None:
            monkeypatch.delenv("WKV6_SEGMENTS", raising=False)
        else:
            monkeypatch.setenv("WKV6_SEGMENTS", str(G))
        x = I.random_inputs_wkv5(B, T, 64 * H, seed=510 + T, dtype=dtype)
        assert torch_cuda.equal(run5(x, H, mode, dtype), run6_broadcast(x, H, mode, dtype)), (T, G)


def test_wkv5_image_base_shape_equals_wkv6(torch_cuda):
    """Full image-base size (B = 64, T = 196, C = 768, H = 12, bidirectional,
    bf16), in the launch configuration the benchmark times."""
    x = I.random_inputs_wkv5(64, 196, 768, seed=520, dtype="bf16")
    y5 = run5(x, 12, "bidirectional", "bf16")
    assert torch_cuda.equal(y5, run6_broadcast(x, 12, "bidirectional", "bf16"))
    # and a few (batch item) slices against the oracle
    for b in (0, 37, 63):
        sl = {key: (val[b:b + 1] if val.ndim == 3 else val) for key, val in x.items()}
        y_ref = wkv5_ref(sl["r"], sl["k"], sl["v"], sl["w_raw"], sl["u"], 12, "bidirectional")
        e = err_over_rms(y5[b:b + 1].double().cpu().numpy(), y_ref)
        say(f"[wkv5] image-base item {b}: {e:.3e}")
        assert e <= TOL5["bf16"]


def run4(x, dtype):
    import torch
    from linear_attention_rnn_amd import wkv6

    k, v = to_device(x["k"], dtype), to_device(x["v"], dtype)
    w, u = torch.from_numpy(x["w"]).cuda(), torch.from_numpy(x["u"]).cuda()
    y = wkv6.fwd4(k, v, w, u)
    torch.cuda.synchronize()
    return y.double().cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C", [(2, 1, 64), (2, 7, 100), (3, 200, 64), (1, 1000, 64), (4, 333, 1000)])
def test_wkv4_parity(torch_cuda, B, T, C, dtype):
    """(1, 1000, 64) runs in 15 segments; (4, 333, 1000) in one."""
    x = I.random_inputs_wkv4(B, T, C, seed=600 + T + C, dtype=dtype, kscale=2.0)
    y = run4(x, dtype)
    y_ref = wkv4_ref(x["k"], x["v"], x["w"], x["u"])
    e = err_over_rms(y, y_ref)
    say(f"[wkv4] B={B} T={T} C={C} {dtype}: {e:.3e}")
    assert e <= TOL4


@pytest.mark.parametrize("case", ["large_keys", "no_decay", "no_memory", "tiny_bonus"])
def test_wkv4_extremes(torch_cuda, case):
    """Keys up to +-60 (e^60 overflows no float32 sum here only because of
    the running rescaling), w = 0 (plain running mean), w = inf (previous
    token only), u = -30 (the current token almost ignored)."""
    B, T, C = 2, 700, 128
    x = I.random_inputs_wkv4(B, T, C, seed=610, dtype="f32")
    if case == "large_keys":
        x["k"] = np.random.default_rng(611).uniform(-60.0, 60.0, size=x["k"].shape).astype(np.float32)
    elif case == "no_decay":
        x["w"][:] = 0.0
    elif case == "no_memory":
        x["w"][:] = np.inf
    else:
        x["u"][:] = -30.0
    y = run4(x, "f32")
    y_ref = wkv4_ref(x["k"], x["v"], x["w"], x["u"])
    e = err_over_rms(y, y_ref)
    say(f"[wkv4] extremes {case}: {e:.3e}")
    assert e <= TOL4


def test_wkv4_text_shape_full(torch_cuda):
    """B = 8, T = 4096, C = 1024 bf16 (the RWKV-4 benchmark's token count;
    the sequences run in segments): every output against the oracle."""
    x = I.random_inputs_wkv4(8, 4096, 1024, seed=620, dtype="bf16")
    y = run4(x, "bf16")
    e = err_over_rms(y, wkv4_ref(x["k"], x["v"], x["w"], x["u"]))
    say(f"[wkv4] text shape, all outputs: {e:.3e}")
    assert e <= TOL4


def test_wkv4_odd_channel_count_segmented(torch_cuda):
    """An odd channel count (one channel per thread even for bf16) over many
    segments, several channel blocks."""
    x = I.random_inputs_wkv4(3, 1000, 777, seed=621, dtype="bf16", kscale=2.0)
    y = run4(x, "bf16")
    e = err_over_rms(y, wkv4_ref(x["k"], x["v"], x["w"], x["u"]))
    say(f"[wkv4] B=3 T=1000 C=777 bf16: {e:.3e}")
    assert e <= TOL4


@pytest.mark.parametrize("G", [None, 1, 2, 7, 64])
def test_wkv4_segments_staged_summaries(torch_cuda, monkeypatch, G):
    """bf16 with C a multiple of 8: the segment summaries stage k and v
    through LDS.  C = 264 leaves 8 live channels in the second block of 256;
    T = 4097 in 64 segments of 65 tokens leaves a last segment of 2 (a single
    staged group, so the groups read ahead lie past its end)."""
    if G is not None:
        monkeypatch.setenv("WKV4_SEGMENTS", str(G))
    x = I.random_inputs_wkv4(2, 4097, 264, seed=622, dtype="bf16", kscale=2.0)
    y = run4(x, "bf16")
    e = err_over_rms(y, wkv4_ref(x["k"], x["v"], x["w"], x["u"]))
    say(f"[wkv4] B=2 T=4097 C=264 bf16 segments={G}: {e:.3e}")
    assert e <= TOL4


def test_wkv4_empty(torch_cuda):
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    z = torch.zeros((2, 0, 64), device="cuda")
    y = wkv6.fwd4(z, z, torch.zeros(64, device="cuda"), torch.zeros(64, device="cuda"))
    assert y.shape == (2, 0, 64)
