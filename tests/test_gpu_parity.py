"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Tolerances, max|y - y_ref| / rms(y_ref): 1e-4 for float32 inputs and 5e-3
for bfloat16 inputs (the bf16 values themselves are the oracle's inputs, so
the bound measures kernel error only).  Any non-finite output fails.
"""
import numpy as np
import pytest

from linear_attention_rnn_amd import inputs as I
from oracle import wkv6_ref
from tests.gpu_util import err_over_rms, gpu_fwd, say, device_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 5e-3}

WORKLOADS = ["tiny-causal-f32", "image-tiny-bidir-f32", "image-base-bidir-bf16", "text-long-causal-bf16",
             "image-hires-bidir-bf16"]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_full_parity(torch_cuda, name):
    """Every output of the full-size launch against the oracle over every
    (batch, head) pair: the global max|y - y_ref| over all B*T*C outputs
    divided by the global rms of y_ref.  Per-head maxima are printed for
    diagnosis."""
    w = I.workload(name)
    x = I.make_inputs(w)
    say(f"[parity] {name}: B={w.B} T={w.T} C={w.C} H={w.H} {w.mode} {w.dtype}")
    y = gpu_fwd(x, w.H, w.mode, w.dtype)
    say(f"[parity] {name}: GPU done, running the oracle")
    y_ref = wkv6_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], w.H, w.mode)
    e = err_over_rms(y, y_ref)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    per_head = np.abs(y - y_ref).reshape(w.B, w.T, w.H, 64).max(axis=(0, 1, 3)) / rms
    say(f"[parity] {name}: max|dy|/rms = {e:.3e} (tol {w.tolerance:g}); worst head {int(per_head.argmax())} "
        f"{per_head.max():.3e}, best head {per_head.min():.3e}")
    assert e <= w.tolerance


SHAPES_T = [1, 2, 3, 15, 16, 17, 31, 63, 64, 65, 127, 128, 129, 196, 257]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
@pytest.mark.parametrize("T", SHAPES_T)
def test_ragged_lengths(torch_cuda, T, mode, dtype):
    B, H = 2, 3
    x = I.random_inputs(B, T, 64 * H, H, seed=1000 + T, dtype=dtype)
    y = gpu_fwd(x, H, mode, dtype)
    y_ref = wkv6_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], H, mode)
    e = err_over_rms(y, y_ref)
    say(f"[ragged] T={T} {mode} {dtype}: {e:.3e}")
    assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ["no_decay", "near_one", "fast_decay", "mixed_extremes"])
@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_decay_extremes(torch_cuda, case, mode, dtype):
    """w_raw = -inf (w = 1), w_raw = -20 (w within 2e-9 of 1), w_raw = 1.5
    (the documented upper end, w = 0.011), and a mix per element (every value
    exact in bf16).  Four items over 150 tokens run in three segments, so the
    general sweeps also run from segment carries."""
    B, T, H = 2, 150, 2
    C = 64 * H
    x = I.random_inputs(B, T, C, H, seed=77, dtype=dtype)
    rng = np.random.default_rng(78)
    if case == "no_decay":
        x["w_raw"][:] = -np.inf
    elif case == "near_one":
        x["w_raw"][:] = -20.0
    elif case == "fast_decay":
        x["w_raw"][:] = 1.5
    else:
        x["w_raw"] = rng.choice(np.array([-np.inf, -20.0, -9.0, -0.5, 0.0, 1.0, 1.5], np.float32),
                                size=(B, T, C)).astype(np.float32)
    y = gpu_fwd(x, H, mode, dtype)
    y_ref = wkv6_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], H, mode)
    e = err_over_rms(y, y_ref)
    say(f"[extremes] {case} {mode} {dtype}: {e:.3e}")
    assert e <= TOL[dtype]


@pytest.mark.parametrize("B,H", [(64, 12), (40, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_many_slow_items(torch_cuda, B, H, mode, dtype):
    """Every third (batch, head) item decays fast enough (w_raw = 1.5) that its
    chunks need the general sweeps, among 768 and 2560 items: the fix-up
    launch recomputes exactly the marked items and leaves the others'
    outputs as the fast kernel wrote them."""
    T = 70
    C = 64 * H
    x = I.random_inputs(B, T, C, H, seed=91, dtype=dtype)
    item = np.arange(B)[:, None] * H + np.arange(H)[None, :]
    slow = (item % 3 == 1)                      # [B, H]
    mask = np.repeat(slow, 64, axis=1)[:, None, :]   # [B, 1, C]
    x["w_raw"] = np.where(mask, np.float32(1.5), x["w_raw"]).astype(np.float32)
    y = gpu_fwd(x, H, mode, dtype)
    y_ref = wkv6_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], H, mode)
    e = err_over_rms(y, y_ref)
    say(f"[slow items] B={B} H={H} {mode} {dtype}: {e:.3e}")
    assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reversal_invariant_on_gpu(torch_cuda, dtype):
    """Reversing the sequence reverses the bidirectional output."""
    B, T, H = 2, 200, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=5, dtype=dtype)
    xr = {key: (np.ascontiguousarray(val[:, ::-1]) if val.ndim == 3 else val) for key, val in x.items()}
    y = gpu_fwd(x, H, "bidirectional", dtype)
    yr = gpu_fwd(xr, H, "bidirectional", dtype)
    scale = float(np.sqrt(np.mean(y ** 2)))
    assert np.max(np.abs(yr[:, ::-1] - y)) / scale <= TOL[dtype]


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_deterministic_and_overwrites_poisoned_output(torch_cuda, mode):
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    B, T, H = 3, 300, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=9, dtype="bf16")
    d = device_inputs(x, "bf16")
    before = [t.clone() for t in d]
    out = torch.full((B, T, 64 * H), float("nan"), device="cuda")
    y1 = wkv6.fwd(*d, H, mode, out=out).clone()
    out.fill_(float("nan"))
    y2 = wkv6.fwd(*d, H, mode, out=out).clone()
    torch.cuda.synchronize()
    assert torch.isfinite(y1).all()
    assert torch.equal(y1, y2)
    for a, b in zip(before, d):
        assert torch.equal(a, b), "inputs modified"


def test_runs_on_a_side_stream(torch_cuda):
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    B, T, H = 2, 130, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=11, dtype="f32")
    d = device_inputs(x, "f32")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = wkv6.fwd(*d, H, "bidirectional", stream=s)
    s.synchronize()
    y_ref = wkv6_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], H, "bidirectional")
    assert err_over_rms(y.double().cpu().numpy(), y_ref) <= TOL["f32"]


def test_concurrent_host_threads(torch_cuda):
    """Four host threads call the library at once, each on its own stream with
    its own inputs, in calls that take a workspace from the shared per-device
    pool (two items only, so the sequences are cut into segments).  Every
    result equals the same call made alone, bit for bit."""
    torch = torch_cuda
    import threading
    from linear_attention_rnn_amd import wkv6

    B, T, H = 1, 64 * 6 + 7, 2
    ds = [device_inputs(I.random_inputs(B, T, 64 * H, H, seed=300 + i, dtype="bf16"), "bf16")
          for i in range(4)]
    alone = [wkv6.fwd(*d, H, "bidirectional") for d in ds]
    torch.cuda.synchronize()
    results, errors = [None] * 4, []
    start = threading.Barrier(4)

    def worker(i):
        try:
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(5):
                    y = wkv6.fwd(*ds[i], H, "bidirectional", stream=s)
            s.synchronize()
            results[i] = y
        except Exception as e:   # reported below, on the test's thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for i in range(4):
        assert results[i] is not None and torch.equal(results[i], alone[i]), i


def test_empty_problem_on_gpu(torch_cuda):
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    z = torch.zeros((2, 0, 128), device="cuda")
    y = wkv6.fwd(z, z, z, z, torch.zeros(128, device="cuda"), 2, "bidirectional")
    assert y.shape == (2, 0, 128)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_segment_count_invariance(torch_cuda, monkeypatch, mode, dtype):
    """Cutting each sequence into G segments (carries combined from per-segment
    summaries) gives the oracle's result for every G, including a ragged last
    segment.  The error is also checked on the tokens after the first chunk,
    where the carries act, and the G = 1 and G = 8 outputs must differ in
    rounding (evidence that the segment path really ran)."""
    B, T, H = 1, 64 * 7 + 5, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=21, dtype=dtype)
    y_ref = wkv6_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], H, mode)
    outs = {}
    for G in (1, 2, 3, 5, 8):
        monkeypatch.setenv("WKV6_SEGMENTS", str(G))
        y = gpu_fwd(x, H, mode, dtype)
        outs[G] = y
        e = err_over_rms(y, y_ref)
        scale = float(np.sqrt(np.mean(y_ref ** 2)))
        e_tail = float(np.max(np.abs(y[:, 64:] - y_ref[:, 64:]))) / scale
        say(f"[segments] G={G} {mode} {dtype}: all {e:.3e}  after chunk 0 {e_tail:.3e}")
        assert e <= TOL[dtype] and e_tail <= TOL[dtype]
    assert not np.array_equal(outs[1], outs[8])
