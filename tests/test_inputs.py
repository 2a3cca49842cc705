"""The seeded input generator: determinism, distributions, bf16 rounding."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_amd import inputs as I


def test_workload_table():
    names = [w.name for w in I.WORKLOADS]
    assert len(names) == len(set(names)) == 5
    for w in I.WORKLOADS:
        assert w.C == w.H * 64 and w.N == 64
        assert w.mode in ("causal", "bidirectional") and w.dtype in ("f32", "bf16")
    assert I.workload("image-tiny-bidir-f32").T == 196   # 14 x 14 patches
    assert I.workload("image-hires-bidir-bf16").T == 4096  # 64 x 64 patches
    with pytest.raises(KeyError):
        I.workload("nope")


def test_algorithmic_bytes():
    w = I.workload("image-base-bidir-bf16")
    assert w.algorithmic_bytes() == 64 * 196 * 768 * 12 + 768 * 4
    w = I.workload("tiny-causal-f32")
    assert w.algorithmic_bytes() == 64 * 128 * 20 + 128 * 4


def test_deterministic_per_seed():
    a = I.random_inputs(2, 9, 128, 2, seed=7)
    b = I.random_inputs(2, 9, 128, 2, seed=7)
    c = I.random_inputs(2, 9, 128, 2, seed=8)
    for key in ("r", "k", "v", "w_raw", "u"):
        np.testing.assert_array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])


def test_distributions():
    x = I.random_inputs(4, 256, 256, 4, seed=3, wraw_lo=-6.0, wraw_hi=-0.5)
    for key in ("r", "k", "v"):
        assert x[key].dtype == np.float32 and x[key].shape == (4, 256, 256)
        assert abs(float(x[key].mean())) < 0.01
        assert abs(float(x[key].std()) - 0.5) < 0.01
    w = x["w_raw"]
    assert w.min() >= -6.0 and w.max() <= -0.5
    assert abs(float(w.mean()) - (-3.25)) < 0.02
    assert x["u"].shape == (256,)


def test_stuck_channels_recipe():
    w = I.workload("image-hires-bidir-bf16")
    # small copy of the recipe: same draws, reduced T
    x = I.random_inputs(w.B, 8, w.C, w.H, seed=w.seed, dtype="bf16", wraw_lo=w.wraw_lo,
                        wraw_hi=w.wraw_hi, stuck_frac=w.stuck_frac, stuck_value=w.stuck_value)
    st = x["stuck"]
    assert len(st) == 102 and len(np.unique(st)) == 102
    assert np.all(x["w_raw"][:, :, st] == -9.0)
    others = np.setdiff1d(np.arange(w.C), st)
    # bf16 spacing near 9 is 1/16, so draws within 1/32 of -9 also round to -9
    assert np.mean(x["w_raw"][:, :, others] == -9.0) < 0.01


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=100000).astype(np.float32),
                        np.array([1.0, -1.0, 0.0, 3.0e38, 1e-40, 1.00390625, 1.01171875],
                                 np.float32)])
    ours = I.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)
    bits = I.bf16_bits(ours)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(back, ours)
    with pytest.raises(ValueError):
        I.bf16_bits(np.array([1.0 + 2 ** -20], np.float32))


def test_bf16_workload_values_are_representable():
    x = I.random_inputs(1, 16, 128, 2, seed=2, dtype="bf16")
    for key in ("r", "k", "v", "w_raw"):
        assert not np.any(x[key].view(np.uint32) & 0xFFFF)
    assert x["u"].dtype == np.float32


def test_rwkv5_inputs():
    a = I.random_inputs_wkv5(2, 7, 128, seed=5, dtype="bf16", wraw_lo=-4.0, wraw_hi=-1.0)
    b = I.random_inputs_wkv5(2, 7, 128, seed=5, dtype="bf16", wraw_lo=-4.0, wraw_hi=-1.0)
    assert a["w_raw"].shape == (128,) and a["r"].shape == (2, 7, 128) and a["u"].shape == (128,)
    for key in ("r", "k", "v", "w_raw", "u"):
        np.testing.assert_array_equal(a[key], b[key])
    for key in ("r", "k", "v", "w_raw"):   # bf16-exact; u stays float32
        assert not np.any(a[key].view(np.uint32) & 0xFFFF)
    assert np.all((a["w_raw"] >= -4.0) & (a["w_raw"] <= -1.0))
    with pytest.raises(ValueError):
        I.random_inputs_wkv5(1, 2, 64, seed=0, dtype="f16")


def test_rwkv4_inputs():
    x = I.random_inputs_wkv4(3, 50, 40, seed=6, dtype="bf16", kscale=2.0, w_lo=0.5, w_hi=1.5)
    assert x["k"].shape == x["v"].shape == (3, 50, 40) and x["w"].shape == x["u"].shape == (40,)
    for key in ("k", "v"):
        assert not np.any(x[key].view(np.uint32) & 0xFFFF)
    assert np.any(x["w"].view(np.uint32) & 0xFFFF)   # w and u stay float32
    assert np.all((x["w"] >= 0.5) & (x["w"] <= 1.5))
    y = I.random_inputs_wkv4(3, 50, 40, seed=6, dtype="f32", kscale=2.0)
    assert 1.7 < float(np.std(y["k"])) < 2.3
    with pytest.raises(ValueError):
        I.random_inputs_wkv4(1, 2, 8, seed=0, dtype="int8")
