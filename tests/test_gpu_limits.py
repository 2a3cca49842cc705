"""The largest sequence the forward accepts, end to end.

The kernels address one (batch item, head) slice with 32-bit byte offsets,
and the library accepts T up to (2^31 - 1 - 4096) / (4 C).  At C = 64 that
is T = 8,388,591 tokens in one item (a single head, so the call is cut into
the most segments).  With w_raw = -0.5 every token's weight falls by a
factor 0.545 per token of distance, so the outputs near either end of the
sequence are fixed, to far below the tolerance (0.545^128 < 1e-33), by the
256 tokens around them: the float64 oracle run on those windows is the
reference.  Inputs are drawn on the device from a seeded generator and the
windows copied back; nothing the library computes feeds the reference.
"""
import numpy as np
import pytest

from oracle import wkv6_ref
from tests.gpu_util import err_over_rms, say

pytestmark = pytest.mark.gpu

C, H = 64, 1
T_MAX = (2 ** 31 - 1 - 4096) // (4 * C)
WIN = 256


@pytest.fixture(scope="module")
def big_inputs():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = torch.Generator(device="cuda")
    g.manual_seed(900)
    shape = (1, T_MAX, C)
    r, k, v = (torch.randn(shape, generator=g, device="cuda").mul_(0.5).to(torch.bfloat16) for _ in range(3))
    w = torch.full(shape, -0.5, device="cuda", dtype=torch.bfloat16)
    u = (torch.randn(C, generator=g, device="cuda") * 0.5).contiguous()
    return r, k, v, w, u


def window(t, lo, hi):
    return t[:, lo:hi].float().cpu().numpy().astype(np.float32)


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_longest_sequence(big_inputs, mode):
    import torch
    from linear_attention_rnn_amd import wkv6

    r, k, v, w, u = big_inputs
    say(f"[limits] T = {T_MAX}, C = {C}, {mode}: running")
    y = wkv6.fwd(r, k, v, w, u, H, mode)
    torch.cuda.synchronize()
    un = u.cpu().numpy()
    for lo, hi, keep in ((0, WIN, slice(0, WIN // 2)), (T_MAX - WIN, T_MAX, slice(WIN // 2, WIN))):
        xs = [window(t, lo, hi) for t in (r, k, v, w)]
        ref = wkv6_ref(*xs, un, H, mode)[:, keep]
        got = y[:, lo:hi].double().cpu().numpy()[:, keep]
        e = err_over_rms(got, ref)
        say(f"[limits] {mode} tokens {lo}..{hi}: {e:.2e}")
        assert e <= 5e-3


def test_one_token_more_is_refused():
    from linear_attention_rnn_amd import wkv6

    A = 0x10000
    p = [A + 0x100000 * i for i in range(6)]
    assert wkv6.fwd_raw(1, T_MAX + 1, C, H, *p, 0, 1, 0) == wkv6.ERR_UNSUPPORTED


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_longest_sequence_backward(big_inputs, mode):
    """The backward on the same sequence.  dr, dk and dv of a token depend on
    its neighbourhood only (the state and the adjoint decay like y), so the
    oracle's gradients on the two end windows are the reference.  The causal
    decay gradient sums over every later token, so it is checked in the last
    window only (all of its later tokens lie there); the bidirectional one
    also sums over every earlier token (the reversed problem's later ones),
    so no window holds all its terms and it is left out, as is du (a sum
    over the whole sequence)."""
    import torch
    from linear_attention_rnn_amd import wkv6
    from oracle import wkv6_ref_backward

    r, k, v, w, u = big_inputs
    g = torch.Generator(device="cuda")
    g.manual_seed(901)
    dy = (torch.randn(r.shape, generator=g, device="cuda") * 0.5).contiguous()
    say(f"[limits] backward T = {T_MAX}, {mode}: running")
    grads = wkv6.bwd(r, k, v, w, u, dy, H, mode)
    torch.cuda.synchronize()
    un = u.cpu().numpy()
    for lo, hi, keep, names in ((0, WIN, slice(0, WIN // 2), ("r", "k", "v")),
                                (T_MAX - WIN, T_MAX, slice(WIN // 2, WIN),
                                 ("r", "k", "v") + (("w_raw",) if mode == "causal" else ()))):
        xs = [window(t, lo, hi) for t in (r, k, v, w)]
        ref = wkv6_ref_backward(*xs, un, dy[:, lo:hi].cpu().numpy(), H, mode)
        for name in names:
            got = grads[name][:, lo:hi].double().cpu().numpy()[:, keep]
            e = err_over_rms(got, ref[name][:, keep])
            say(f"[limits] backward {mode} d{name} tokens {lo}..{hi}: {e:.2e}")
            assert e <= 1e-4
