"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph).

Each graph is replayed several times; between replays the program changes
the captured inputs with its own eager work and synchronises, and every
replay must equal, bit for bit, the eager call on the same inputs (the same
kernels on the same data).  Captured: an unsegmented bidirectional forward
(no workspace), a segmented causal forward through wkv6_fwd_noalloc (its
workspace is the static scratch array, so nothing is allocated under
capture), an 8-step single-token decode loop passing the state between
two buffers, and the RWKV-5 and RWKV-4 forwards on shapes that need no
workspace.
"""
import numpy as np
import pytest

from linear_attention_rnn_amd import inputs as I
from tests.gpu_util import device_inputs, say, to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _static(torch, x, dtype, dev=device_inputs):
    return [t.clone() for t in dev(x, dtype)]


def _refill(static, x, dtype, dev=device_inputs):
    for dst, src in zip(static, dev(x, dtype)):
        dst.copy_(src)


def _replay_and_compare(torch, graph, static, out, eager, draw, dtype, label, dev=device_inputs):
    for rep in range(REPLAYS):
        x = draw(rep)
        _refill(static, x, dtype, dev)     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu() for t in out]
        want = [t.cpu() for t in eager(static)]
        for g, w in zip(got, want):
            assert torch.equal(g, w), f"{label}: replay {rep} differs from the eager call"
        say(f"[graph] {label}: replay {rep} equals the eager call")


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_forward_under_capture(torch_cuda, mode):
    """B*H = 768 items: one segment per sequence, no workspace."""
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    B, T, H = 64, 150, 12
    C = 64 * H
    draw = lambda rep: I.random_inputs(B, T, C, H, seed=700 + rep, dtype="bf16")
    static = _static(torch, draw(0), "bf16")
    y = torch.empty(B, T, C, dtype=torch.float32, device="cuda")
    wkv6.fwd(*static, H, mode, out=y)          # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wkv6.fwd(*static, H, mode, out=y)
    _replay_and_compare(torch, g, static, [y], lambda s: [wkv6.fwd(*s, H, mode)], draw, "bf16",
                        f"fwd {mode}")


def test_noalloc_segmented_under_capture(torch_cuda):
    """Four items over 1000 tokens: the sequences run in segments, whose
    summaries live in the static scratch array of wkv6_fwd_noalloc."""
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    B, T, H = 2, 1000, 2
    C = 64 * H
    draw = lambda rep: I.random_inputs(B, T, C, H, seed=710 + rep, dtype="bf16")
    static = _static(torch, draw(0), "bf16")
    y = torch.empty(B, T, C, dtype=torch.float32, device="cuda")
    wkv6.fwd_noalloc(*static, H, "causal", out=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wkv6.fwd_noalloc(*static, H, "causal", out=y)
    _replay_and_compare(torch, g, static, [y], lambda s: [wkv6.fwd_noalloc(*s, H, "causal")], draw,
                        "bf16", "fwd_noalloc causal, segmented")


def test_decode_loop_under_capture(torch_cuda):
    """Eight single-token steps from a given state, the state handed from
    step to step through two buffers, captured as one graph."""
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    B, H, STEPS = 4, 4, 8
    C = 64 * H

    def draw(rep):
        x = I.random_inputs(B, STEPS, C, H, seed=720 + rep, dtype="f32")
        x["s0"] = np.random.default_rng(730 + rep).normal(0.0, 0.5, size=(B, H, 64, 64)).astype(np.float32)
        return x

    def dev(x):
        r, k, v, w, u = device_inputs(x, "f32")
        return [r, k, v, w, u, torch.from_numpy(x["s0"]).cuda()]

    static = [t.clone() for t in dev(draw(0))]
    ys = [torch.empty(B, 1, C, dtype=torch.float32, device="cuda") for _ in range(STEPS)]
    sa = torch.empty(B, H, 64, 64, dtype=torch.float32, device="cuda")
    sb = torch.empty_like(sa)

    def loop(s, y_bufs, bufs):
        r, k, v, w, u, s0 = s
        cur = s0
        for t in range(STEPS):
            nxt = bufs[t % 2]
            sl = slice(t, t + 1)
            step = [a[:, sl].contiguous() for a in (r, k, v, w)]
            wkv6.fwd_state(*step, u, H, s_in=cur, out=y_bufs[t], s_out=nxt)
            cur = nxt
        return cur

    loop(static, ys, (sa, sb))             # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s_end = loop(static, ys, (sa, sb))

    def eager(s):
        yb = [torch.empty_like(t) for t in ys]
        bufs = (torch.empty_like(sa), torch.empty_like(sa))
        return yb + [loop(s, yb, bufs)]

    for rep in range(REPLAYS):
        x = draw(rep)
        for dst, src in zip(static, dev(x)):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.cpu() for t in ys] + [s_end.cpu()]
        want = [t.cpu() for t in eager(static)]
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"decode loop: replay {rep} differs from the eager loop"
        say(f"[graph] decode loop: replay {rep} equals the eager loop")


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_fwd5_under_capture(torch_cuda, mode):
    """RWKV-5 (one decay per channel), B*H = 768 items, no workspace."""
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    B, T, H = 64, 150, 12
    C = 64 * H
    assert wkv6.fwd_workspace_bytes(B, T, C, H, mode, True) == 0
    draw = lambda rep: I.random_inputs_wkv5(B, T, C, seed=740 + rep, dtype="bf16")
    static = _static(torch, draw(0), "bf16")
    y = torch.empty(B, T, C, dtype=torch.float32, device="cuda")
    wkv6.fwd5(*static, H, mode, out=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wkv6.fwd5(*static, H, mode, out=y)
    _replay_and_compare(torch, g, static, [y], lambda s: [wkv6.fwd5(*s, H, mode)], draw, "bf16",
                        f"fwd5 {mode}")


def _dev4(x, dtype):
    import torch

    return ([to_device(x[key], dtype) for key in ("k", "v")]
            + [torch.from_numpy(np.ascontiguousarray(x[key], np.float32)).cuda() for key in ("w", "u")])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd4_under_capture(torch_cuda, dtype):
    """RWKV-4 over 196 tokens of 64 x 768 channels: one pass, no segments and
    so no workspace (bf16 takes the LDS-staged output kernel)."""
    torch = torch_cuda
    from linear_attention_rnn_amd import wkv6

    B, T, C = 64, 196, 768
    draw = lambda rep: I.random_inputs_wkv4(B, T, C, seed=750 + rep, dtype=dtype)
    static = _static(torch, draw(0), dtype, _dev4)
    y = torch.empty(B, T, C, dtype=torch.float32, device="cuda")
    wkv6.fwd4(*static, out=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wkv6.fwd4(*static, out=y)
    _replay_and_compare(torch, g, static, [y], lambda s: [wkv6.fwd4(*s)], draw, dtype,
                        f"fwd4 {dtype}", _dev4)
