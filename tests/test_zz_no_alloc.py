"""wkv6_fwd_noalloc (the forward with its workspace in the library's static
per-device scratch array, for callers that cannot allocate) against wkv6_fwd
through the C ABI: two calls in a row on one stream, the second with a
smaller input, both on segmented paths (few (batch, head) pairs, long
sequences), so the segment summaries really go through the scratch array.
The planner gives both entry points the same segment count at these sizes,
so the outputs must agree bit for bit; both are also checked against the
oracle at the parity bound."""
import numpy as np
import pytest

from linear_attention_rnn_amd import inputs as I
from oracle import wkv6_ref
from tests.gpu_util import device_inputs, err_over_rms, say

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 5e-3}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_fwd_twice(torch_cuda, mode, dtype):
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    for B, T, H, seed in ((2, 64 * 9 + 11, 3, 610), (1, 64 * 4 + 3, 2, 611)):   # second call smaller
        x = I.random_inputs(B, T, 64 * H, H, seed=seed, dtype=dtype)
        d = device_inputs(x, dtype)
        say(f"[noalloc] B={B} T={T} H={H} {mode} {dtype}")
        y_na = wkv6.fwd_noalloc(*d, H, mode)
        y = wkv6.fwd(*d, H, mode)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y), "noalloc differs from wkv6_fwd"
        e = err_over_rms(y_na.double().cpu().numpy(), wkv6_ref(x["r"], x["k"], x["v"], x["w_raw"], x["u"], H, mode))
        say(f"[noalloc] B={B} T={T}: max|dy|/rms = {e:.3e}")
        assert e <= TOL[dtype]


def test_noalloc_caps_segments_at_full_size(torch_cuda):
    """image-hires (64 pairs, T = 4096, bidirectional, bf16): the planned
    segments fit the 32 MiB scratch, and the result matches wkv6_fwd's."""
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    w = I.workload("image-hires-bidir-bf16")
    x = I.make_inputs(w)
    d = device_inputs(x, w.dtype)
    y_na = wkv6.fwd_noalloc(*d, w.H, w.mode)
    y = wkv6.fwd(*d, w.H, w.mode)
    torch.cuda.synchronize()
    scale = float(torch.sqrt(torch.mean(y.double() ** 2)))
    diff = float(torch.max(torch.abs(y_na.double() - y.double()))) / scale
    say(f"[noalloc] image-hires: max|d|/rms vs wkv6_fwd = {diff:.3e}")
    assert diff <= TOL[w.dtype]
