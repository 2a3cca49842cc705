"""The library's workspace pool keeps at most WKV6_WORKSPACE_KEEP_BYTES of
freed workspace per device once the stream has synchronised, and
wkv6_trim_workspace hands the rest back."""
import pytest

from linear_attention_rnn_amd import inputs as I
from tests.gpu_util import device_inputs, say

pytestmark = pytest.mark.gpu


def test_pool_keeps_at_most_the_bound_and_trims(monkeypatch):
    import torch
    from linear_attention_rnn_amd import wkv6

    assert torch.cuda.is_available()
    # bidirectional fused-epilogue calls keep the reverse rows in a B*T*C*4
    # byte workspace: 16 * 2048 * 2048 * 4 = 268 MB, above the 256 MiB bound
    B, T, H = 16, 2048, 32
    C = 64 * H
    x = I.random_inputs(B, T, C, H, seed=640, dtype="bf16")
    d = device_inputs(x, "bf16")
    g = d[0]
    one = torch.ones(C, device="cuda")
    for _ in range(2):
        wkv6.fwd_gn(*d, g, one, one * 0, H, "bidirectional")
    torch.cuda.synchronize()
    held = wkv6.workspace_reserved_bytes()
    say(f"[workspace] after two 268 MB workspace calls and a synchronize: pool holds {held / 2**20:.1f} MiB")
    assert held <= wkv6.WORKSPACE_KEEP_BYTES
    # a segmented call's small workspace (below the bound) stays in the pool
    # for the next call, until trimmed
    xs = I.random_inputs(1, 1000, 128, 2, seed=641, dtype="bf16")
    need = wkv6.fwd_workspace_bytes(1, 1000, 128, 2, "causal", True)
    assert need > 0
    wkv6.fwd(*device_inputs(xs, "bf16"), 2, "causal")
    torch.cuda.synchronize()
    kept = wkv6.workspace_reserved_bytes()
    say(f"[workspace] after a call taking {need} B: pool holds {kept} B")
    assert need <= kept <= wkv6.WORKSPACE_KEEP_BYTES
    wkv6.trim_workspace()
    assert wkv6.workspace_reserved_bytes() == 0
