"""Helpers shared by the GPU tests: move seeded inputs to the device, call the
HIP path through the C ABI binding, and measure the error against the
oracle as max|y - y_ref| / rms(y_ref)."""
from __future__ import annotations

import os
import sys

import numpy as np

from linear_attention_rnn_amd import inputs as I


def say(*a):
    """Print a progress/result line; also append it to $WKV6_TEST_LOG if set."""
    print(*a, flush=True)
    sys.stdout.flush()
    path = os.environ.get("WKV6_TEST_LOG")
    if path:
        with open(path, "a") as f:
            f.write(" ".join(str(x) for x in a) + "\n")


def to_device(x: np.ndarray, dtype: str):
    import torch

    if dtype == "bf16":
        bits = I.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def device_inputs(x: dict, dtype: str):
    import torch

    return ([to_device(x[key], dtype) for key in ("r", "k", "v", "w_raw")]
            + [torch.from_numpy(np.ascontiguousarray(x["u"], np.float32)).cuda()])


def gpu_fwd(x: dict, H: int, mode: str, dtype: str, out=None) -> np.ndarray:
    import torch
    from linear_attention_rnn_amd import wkv6

    d = device_inputs(x, dtype)
    y = wkv6.fwd(*d, H, mode, out=out)
    torch.cuda.synchronize()
    return y.double().cpu().numpy()


def err_over_rms(y: np.ndarray, y_ref: np.ndarray) -> float:
    y_ref = np.asarray(y_ref, np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    return float(np.max(np.abs(y - y_ref))) / max(rms, 1e-30)


def head_slice(x: dict, b: int, h: int, N: int = 64) -> dict:
    """Inputs of one (batch item, head) pair as a B = 1, H = 1 problem."""
    sl = slice(h * N, (h + 1) * N)
    return {"r": x["r"][b:b + 1, :, sl], "k": x["k"][b:b + 1, :, sl], "v": x["v"][b:b + 1, :, sl],
            "w_raw": x["w_raw"][b:b + 1, :, sl], "u": x["u"][sl]}
