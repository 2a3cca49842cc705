"""Parity of the chunked MFMA backward (bf16 inputs, one workgroup per
(batch, head)) with the float64 oracle's adjoint, through the C ABI.

The library takes that path for bf16 calls whose (batch, head) pairs run
unsegmented over long enough sequences; here WKV6_BWD_CHUNKED=1 forces it
and WKV6_BWD_SEGMENTS=1 forces one segment for the small shapes (an autouse
fixture), and WKV6_BWD_CHUNKED=0 selects the token-serial kernels for
comparison.  Items with a 16-token block that decays by 2^-24 or more in
some channel are recomputed by the token-serial kernels.  Same bound as the
other backward tests: max|g - g_ref| / rms(g_ref) <= 1e-4.
"""
import numpy as np
import pytest

from linear_attention_rnn_amd import inputs as I
from tests.gpu_util import say
from tests.test_gpu_backward import NAMES, check, dy_of, gpu_bwd, torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def chunked(monkeypatch):
    monkeypatch.setenv("WKV6_BWD_CHUNKED", "1")
    monkeypatch.setenv("WKV6_BWD_SEGMENTS", "1")


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
@pytest.mark.parametrize("T", [1, 2, 17, 63, 64, 65, 130, 300])
def test_chunked_parity(torch_cuda, T, mode):
    B, H = 2, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=1800 + T, dtype="bf16")
    check(f"chunked T={T} {mode}", x, dy_of(x, 1900 + T), H, mode, "bf16")


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_chunked_matches_token_serial(torch_cuda, monkeypatch, mode):
    """The two kernel families agree to rounding on the same inputs."""
    B, T, H = 3, 259, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=1950, dtype="bf16", wraw_lo=-8.0, wraw_hi=-0.5)
    dy = dy_of(x, 1951)
    a = gpu_bwd(x, dy, H, mode, "bf16")
    monkeypatch.setenv("WKV6_BWD_CHUNKED", "0")
    b = gpu_bwd(x, dy, H, mode, "bf16")
    for name in NAMES:
        scale = float(np.sqrt(np.mean(b[name] ** 2))) or 1.0
        e = float(np.max(np.abs(a[name] - b[name]))) / scale
        say(f"[chunked] vs token-serial {mode} d{name}: {e:.2e}")
        assert e <= 1e-4, (name, e)


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_chunked_slow_items_fall_back(torch_cuda, mode):
    """Items whose decays leave the chunked path's range (here one item with
    w_raw = 1.5 in some channels, one with decays of exactly 1) are
    recomputed by the token-serial kernels; the others stay chunked."""
    B, T, H = 2, 150, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=1960, dtype="bf16")
    x["w_raw"][1, :, 5:64:7] = 1.5          # item (b=1, h=0): fast decays in some channels
    x["w_raw"][0, :, 64:] = -np.inf         # item (b=0, h=1): no decay
    check(f"chunked slow items {mode}", x, dy_of(x, 1961), H, mode, "bf16")


@pytest.mark.parametrize("mode", ["causal", "bidirectional"])
def test_chunked_image_base_full(torch_cuda, mode):
    """The image-base shape (B = 64, T = 196, C = 768, H = 12, bf16): 768
    items, unsegmented, on the chunked kernels; every gradient compared over
    the whole tensor."""
    w = I.workload("image-base-bidir-bf16")
    x = I.make_inputs(w)
    check(f"chunked image-base full {mode}", x, dy_of(x, w.seed + 1000), w.H, mode, w.dtype)


def test_chunked_long_text_rows(torch_cuda):
    """Text-long rows (T = 4096, C = 2048, H = 32, causal, bf16, w_raw in
    [-8, -1]) with two batch items, unsegmented: 64 chunks carried through
    the stored states and the adjoint."""
    w = I.workload("text-long-causal-bf16")
    x = I.random_inputs(2, w.T, w.C, w.H, seed=w.seed, dtype="bf16", wraw_lo=-8.0, wraw_hi=-1.0)
    check("chunked text-long rows (B=2)", x, dy_of(x, w.seed + 1000), w.H, "causal", "bf16")


def test_chunked_item_slow_in_reverse_only(torch_cuda):
    """An item whose fast decays fill one 16-token block of the reversed
    sweep but straddle two blocks of the forward one (T = 150 is not a
    multiple of 16, so the blocks of the two directions differ): only the
    reverse direction flags it, after the forward direction's chunked kernel
    has already written its gradients; the token-serial kernels then
    recompute the whole item.  Here tokens 118..133 (reversed-sweep block
    [118, 134)) decay by 2^-1.7 each in one channel: 2^-27.2 in that block,
    2^-17 and 2^-10.2 in the forward blocks [112, 128) and [128, 144)."""
    B, T, H = 2, 150, 2
    x = I.random_inputs(B, T, 64 * H, H, seed=1970, dtype="bf16", wraw_lo=-8.0, wraw_hi=-2.0)
    w_fast = float(np.log(1.7 / np.log2(np.e)))
    x["w_raw"][1, 118:134, 64 + 7] = I.round_to_bf16(np.float32(w_fast))
    check("chunked slow in the reverse direction only", x, dy_of(x, 1971), H, "bidirectional", "bf16")
