"""Argument checks of the Python binding that run before any library call.
No GPU and no built library are needed: the library loader is replaced by
one that fails the test if it is reached."""
import pytest
import torch

from linear_attention_rnn_amd import wkv6


class FakeGpuTensor:
    """A host tensor that reports itself as a contiguous tensor on cuda:0,
    so the binding's input checks pass without a GPU."""

    def __init__(self, t, device="cuda:0"):
        self._t = t
        self.device = torch.device(device)
        self.is_cuda = True
        self.shape = t.shape
        self.dtype = t.dtype

    def dim(self):
        return self._t.dim()

    def numel(self):
        return self._t.numel()

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return 0x10000


@pytest.fixture
def no_library(monkeypatch):
    def fail():
        raise AssertionError("the library was called")

    monkeypatch.setattr(wkv6, "lib", fail)


def inputs(B=1, T=4, C=64, dtype=torch.float32, device="cuda:0"):
    x = [FakeGpuTensor(torch.zeros(B, T, C, dtype=dtype), device) for _ in range(4)]
    return x + [FakeGpuTensor(torch.zeros(C), device)]


@pytest.mark.parametrize("call", ["fwd", "fwd5", "fwd_gn", "fwd4", "fwd_state", "fwd_state_s_out"])
def test_host_output_buffer_is_refused(no_library, call):
    """A host tensor passed as an output buffer raises ValueError before any
    library call (its address would otherwise reach the kernels' stores)."""
    B, T, C = 1, 4, 64
    r, k, v, w, u = inputs(B, T, C)
    host = torch.empty(B, T, C)
    with pytest.raises(ValueError):
        if call == "fwd":
            wkv6.fwd(r, k, v, w, u, 1, out=host, stream=0)
        elif call == "fwd5":
            w5 = FakeGpuTensor(torch.zeros(C))
            wkv6.fwd5(r, k, v, w5, u, 1, out=host, stream=0)
        elif call == "fwd_gn":
            one = FakeGpuTensor(torch.ones(C))
            wkv6.fwd_gn(r, k, v, w, u, r, one, one, 1, out=torch.empty(B, T, C, dtype=torch.bfloat16),
                        stream=0)
        elif call == "fwd4":
            one = FakeGpuTensor(torch.ones(C))
            wkv6.fwd4(k, v, one, one, out=host, stream=0)
        elif call == "fwd_state":
            wkv6.fwd_state(r, k, v, w, u, 1, out=host, stream=0)
        else:
            wkv6.fwd_state(r, k, v, w, u, 1, out=FakeGpuTensor(torch.empty(B, T, C)), s_out=torch.empty(B, 1, 64, 64),
                           stream=0)


def test_output_on_another_gpu_is_refused(no_library):
    r, k, v, w, u = inputs()
    other = FakeGpuTensor(torch.empty(1, 4, 64), device="cuda:1")
    with pytest.raises(ValueError):
        wkv6.fwd(r, k, v, w, u, 1, out=other, stream=0)


def test_inputs_on_two_gpus_are_refused(no_library):
    r, k, v, w, u = inputs()
    k = FakeGpuTensor(torch.zeros(1, 4, 64), device="cuda:1")
    with pytest.raises(ValueError):
        wkv6.fwd(r, k, v, w, u, 1, stream=0)
