"""ctypes binding of libwkv6.so (C ABI in include/wkv6.h).

Argument marshalling only: every step of the WKV-6 forward runs in the
library's HIP kernels.  PyTorch provides device memory and the current HIP
stream.  There is no fallback: if the library is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libwkv6.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "wkv6.h")

MODE_CAUSAL = 0
MODE_BIDIRECTIONAL = 1
DTYPE_F32 = 0
DTYPE_BF16 = 1
OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED = 2
ERR_MISALIGNED = 3
ERR_HIP = 4

_MODES = {"causal": MODE_CAUSAL, "bidirectional": MODE_BIDIRECTIONAL}

_lib = None


class WKV6Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"wkv6_fwd failed with status {status}: {message}")
        self.status = status


def header_functions() -> list[str]:
    """Names of the functions include/wkv6.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(wkv\d_\w+)\s*\(", text, flags=re.M)


def lib() -> ctypes.CDLL:
    """Load libwkv6.so (once).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with `python -m linear_attention_rnn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        L.wkv6_fwd.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                               ctypes.c_int, ctypes.c_int, vp]
        L.wkv6_fwd.restype = ctypes.c_int
        L.wkv5_fwd.argtypes = L.wkv6_fwd.argtypes
        L.wkv5_fwd.restype = ctypes.c_int
        L.wkv6_fwd_noalloc.argtypes = L.wkv6_fwd.argtypes
        L.wkv6_fwd_noalloc.restype = ctypes.c_int
        L.wkv6_fwd_gn.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                  ctypes.c_int, ctypes.c_int, vp]
        L.wkv6_fwd_gn.restype = ctypes.c_int
        L.wkv6_group_norm_gate.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_int, vp]
        L.wkv6_group_norm_gate.restype = ctypes.c_int
        L.wkv4_fwd.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, ctypes.c_int, vp]
        L.wkv4_fwd.restype = ctypes.c_int
        L.wkv6_fwd_state.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_int, vp]
        L.wkv6_fwd_state.restype = ctypes.c_int
        L.wkv6_bwd.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                               ctypes.c_int, ctypes.c_int, vp]
        L.wkv6_bwd.restype = ctypes.c_int
        L.wkv6_status_str.argtypes = [ctypes.c_int]
        L.wkv6_status_str.restype = ctypes.c_char_p
        L.wkv6_last_error.argtypes = []
        L.wkv6_last_error.restype = ctypes.c_char_p
        L.wkv6_abi_version.argtypes = []
        L.wkv6_abi_version.restype = ctypes.c_int
        L.wkv6_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
        L.wkv6_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.wkv6_workspace_reserved_bytes.argtypes = []
        L.wkv6_workspace_reserved_bytes.restype = ctypes.c_size_t
        L.wkv6_trim_workspace.argtypes = []
        L.wkv6_trim_workspace.restype = ctypes.c_int
        _lib = L
    return _lib


WORKSPACE_KEEP_BYTES = 256 << 20   # WKV6_WORKSPACE_KEEP_BYTES


def fwd_workspace_bytes(B: int, T: int, C: int, H: int, mode: str = "causal", bf16: bool = True) -> int:
    """Workspace bytes a wkv6_fwd call of these sizes takes (host arithmetic)."""
    return lib().wkv6_fwd_workspace_bytes(B, T, C, H, _MODES[mode], DTYPE_BF16 if bf16 else DTYPE_F32)


def workspace_reserved_bytes() -> int:
    """Bytes the current device's workspace pool holds now."""
    return lib().wkv6_workspace_reserved_bytes()


def trim_workspace() -> None:
    """Hand the unused blocks of the current device's workspace pool back."""
    st = lib().wkv6_trim_workspace()
    if st != OK:
        raise WKV6Error(st, f"{status_str(st)}: {last_error()}")


def abi_version() -> int:
    return lib().wkv6_abi_version()


def status_str(status: int) -> str:
    return lib().wkv6_status_str(status).decode()


def last_error() -> str:
    return lib().wkv6_last_error().decode()


def fwd_raw(B: int, T: int, C: int, H: int, r: int, k: int, v: int, w_raw: int, u: int,
            y: int, mode: int, dtype: int, stream: int = 0) -> int:
    """Direct call with integer addresses; returns the status code."""
    return lib().wkv6_fwd(B, T, C, H, r, k, v, w_raw, u, y, mode, dtype, stream)


def fwd_noalloc_raw(B: int, T: int, C: int, H: int, r: int, k: int, v: int, w_raw: int, u: int,
                    y: int, mode: int, dtype: int, stream: int = 0) -> int:
    """Direct call of wkv6_fwd_noalloc (workspace in the library's static
    scratch array) with integer addresses."""
    return lib().wkv6_fwd_noalloc(B, T, C, H, r, k, v, w_raw, u, y, mode, dtype, stream)


def fwd5_raw(B: int, T: int, C: int, H: int, r: int, k: int, v: int, w_raw: int, u: int,
             y: int, mode: int, dtype: int, stream: int = 0) -> int:
    """Direct call of wkv5_fwd (w_raw: C values) with integer addresses."""
    return lib().wkv5_fwd(B, T, C, H, r, k, v, w_raw, u, y, mode, dtype, stream)


def fwd_gn_raw(B: int, T: int, C: int, H: int, r: int, k: int, v: int, w_raw: int, u: int, g: int,
               gamma: int, beta: int, eps: float, out: int, mode: int, dtype: int, stream: int = 0) -> int:
    """Direct call of wkv6_fwd_gn with integer addresses."""
    return lib().wkv6_fwd_gn(B, T, C, H, r, k, v, w_raw, u, g, gamma, beta, eps, out, mode, dtype, stream)


def fwd4_raw(B: int, T: int, C: int, k: int, v: int, w: int, u: int, y: int, dtype: int,
             stream: int = 0) -> int:
    """Direct call of wkv4_fwd with integer addresses."""
    return lib().wkv4_fwd(B, T, C, k, v, w, u, y, dtype, stream)


def fwd_state_raw(B: int, T: int, C: int, H: int, r: int, k: int, v: int, w_raw: int, u: int,
                  y: int, s_in: int, s_out: int, dtype: int, stream: int = 0) -> int:
    """Direct call of wkv6_fwd_state with integer addresses (0 = NULL)."""
    return lib().wkv6_fwd_state(B, T, C, H, r, k, v, w_raw, u, y, s_in, s_out, dtype, stream)


def _check_inputs(r, k, v, w_raw, u, w_static=False):
    import torch

    if r.dim() != 3:
        raise ValueError("r must be [B, T, C]")
    B, T, C = r.shape
    for name, t in (("k", k), ("v", v), ("w_raw", w_raw)):
        if name == "w_raw" and w_static:
            if t.numel() != C or t.dtype != r.dtype:
                raise ValueError("w_raw must hold C values of r's dtype")
        elif t.shape != r.shape or t.dtype != r.dtype:
            raise ValueError(f"{name} must match r in shape and dtype")
    if r.dtype == torch.float32:
        dtype = DTYPE_F32
    elif r.dtype == torch.bfloat16:
        dtype = DTYPE_BF16
    else:
        raise ValueError("r, k, v, w_raw must be float32 or bfloat16")
    if u.dtype != torch.float32 or u.numel() != C:
        raise ValueError("u must be float32 with C elements")
    for name, t in (("r", r), ("k", k), ("v", v), ("w_raw", w_raw), ("u", u)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        if t.device != r.device:
            raise ValueError(f"{name} must be on the same GPU as r")
    return B, T, C, dtype


def _check_out(t, shape, dtype, device, name: str):
    """A caller-supplied output buffer: a contiguous tensor of the given shape
    and dtype on the inputs' GPU.  A host tensor would hand the kernels a host
    address to store through, so it is refused here, before any library call."""
    if (not getattr(t, "is_cuda", False) or t.device != device or tuple(t.shape) != tuple(shape)
            or t.dtype != dtype or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {list(shape)} on {device}")


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def fwd_state(r, k, v, w_raw, u, H: int, s_in=None, want_state: bool = True, out=None,
              s_out=None, stream=None):
    """Causal y = WKV6(r, k, v, w_raw, u) starting from state ``s_in``.

    s_in: None (zero state) or a contiguous float32 CUDA tensor [B, H, 64, 64]
    (entry [b, h, c, n]: key channel c, value channel n).  Returns (y, s_out)
    with s_out the state after the last token (None if ``want_state`` is
    false and no ``s_out`` buffer is given).
    """
    import torch

    B, T, C, dtype = _check_inputs(r, k, v, w_raw, u)
    shape = (B, H, 64, 64)
    if s_in is not None and (s_in.shape != shape or s_in.dtype != torch.float32 or not s_in.is_cuda
                             or not s_in.is_contiguous()):
        raise ValueError("s_in must be a contiguous float32 GPU tensor [B, H, 64, 64]")
    if s_in is not None and s_in.device != r.device:
        raise ValueError("s_in must be on the inputs' GPU")
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=r.device)
    else:
        _check_out(out, (B, T, C), torch.float32, r.device, "out")
    if s_out is None and want_state:
        s_out = torch.empty(shape, dtype=torch.float32, device=r.device)
    elif s_out is not None:
        _check_out(s_out, shape, torch.float32, r.device, "s_out")
    st = fwd_state_raw(B, T, C, H, r.data_ptr(), k.data_ptr(), v.data_ptr(), w_raw.data_ptr(),
                       u.data_ptr(), out.data_ptr(), 0 if s_in is None else s_in.data_ptr(),
                       0 if s_out is None else s_out.data_ptr(), dtype,
                       _stream_handle(stream, r.device))
    if st != OK:
        raise WKV6Error(st, f"{status_str(st)}: {last_error()}")
    return out, s_out


def fwd(r, k, v, w_raw, u, H: int, mode: str = "causal", out=None, stream=None):
    """y = WKV6(r, k, v, w_raw, u) on the GPU.

    r, k, v, w_raw: contiguous CUDA tensors [B, T, C] of one dtype (float32 or
    bfloat16); u: contiguous float32 [C]; returns (or fills ``out``) a float32
    [B, T, C] tensor.  Runs on ``stream`` (default: torch's current stream).
    """
    import torch

    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    B, T, C, dtype = _check_inputs(r, k, v, w_raw, u)
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=r.device)
    else:
        _check_out(out, (B, T, C), torch.float32, r.device, "out")
    st = fwd_raw(B, T, C, H, r.data_ptr(), k.data_ptr(), v.data_ptr(), w_raw.data_ptr(),
                 u.data_ptr(), out.data_ptr(), _MODES[mode], dtype, _stream_handle(stream, r.device))
    if st != OK:
        raise WKV6Error(st, f"{status_str(st)}: {last_error()}")
    return out


def fwd_noalloc(r, k, v, w_raw, u, H: int, mode: str = "causal", out=None, stream=None):
    """fwd() through wkv6_fwd_noalloc: the library allocates nothing (segment
    summaries go to its static per-device scratch array).  Calls that may
    overlap on one GPU race on that array."""
    import torch

    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    B, T, C, dtype = _check_inputs(r, k, v, w_raw, u)
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=r.device)
    else:
        _check_out(out, (B, T, C), torch.float32, r.device, "out")
    st = fwd_noalloc_raw(B, T, C, H, r.data_ptr(), k.data_ptr(), v.data_ptr(), w_raw.data_ptr(),
                         u.data_ptr(), out.data_ptr(), _MODES[mode], dtype, _stream_handle(stream, r.device))
    if st != OK:
        raise WKV6Error(st, f"{status_str(st)}: {last_error()}")
    return out


def fwd5(r, k, v, w_raw, u, H: int, mode: str = "causal", out=None, stream=None):
    """y = WKV5(r, k, v, w_raw, u): fwd with one decay for every token.

    w_raw: contiguous CUDA tensor of C values (dtype of r), laid out [H, 64];
    every token decays by exp(-exp(w_raw)).  Everything else as fwd.
    """
    import torch

    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    B, T, C, dtype = _check_inputs(r, k, v, w_raw, u, w_static=True)
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=r.device)
    else:
        _check_out(out, (B, T, C), torch.float32, r.device, "out")
    st = fwd5_raw(B, T, C, H, r.data_ptr(), k.data_ptr(), v.data_ptr(), w_raw.data_ptr(),
                  u.data_ptr(), out.data_ptr(), _MODES[mode], dtype, _stream_handle(stream, r.device))
    if st != OK:
        raise WKV6Error(st, f"{status_str(st)}: {last_error()}")
    return out


def fwd_gn(r, k, v, w_raw, u, g, gamma, beta, H: int, mode: str = "causal", eps: float = 64e-5,
           out=None, stream=None):
    """bf16 [B, T, C] = (GroupNorm over each head's 64 channels of fwd(...))
    * gamma + beta, times the gate g ([B, T, C], dtype of r); gamma, beta:
    float32 [C].  y itself is never written."""
    import torch

    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    B, T, C, dtype = _check_inputs(r, k, v, w_raw, u)
    if g.shape != r.shape or g.dtype != r.dtype or not g.is_cuda or not g.is_contiguous():
        raise ValueError("g must be a contiguous GPU tensor like r")
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t.dtype != torch.float32 or t.numel() != C or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor of C values")
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.bfloat16, device=r.device)
    else:
        _check_out(out, (B, T, C), torch.bfloat16, r.device, "out")
    st = fwd_gn_raw(B, T, C, H, r.data_ptr(), k.data_ptr(), v.data_ptr(), w_raw.data_ptr(), u.data_ptr(),
                    g.data_ptr(), gamma.data_ptr(), beta.data_ptr(), float(eps), out.data_ptr(), _MODES[mode],
                    dtype, _stream_handle(stream, r.device))
    if st != OK:
        raise WKV6Error(st, f"{status_str(st)}: {last_error()}")
    return out


def group_norm_gate(y, g, gamma, beta, H: int, eps: float = 64e-5, out=None, stream=None):
    """bf16 [B, T, C] = (GroupNorm over each head's 64 channels of y) * gamma
    + beta, times the gate g: the epilogue of fwd_gn as a pass of its own.
    y: float32 [B, T, C]; g: [B, T, C] float32 or bfloat16; gamma, beta:
    float32 [C]."""
    import torch

    if y.dim() != 3 or y.dtype != torch.float32:
        raise ValueError("y must be a float32 [B, T, C] tensor")
    B, T, C = y.shape
    if g.shape != y.shape or g.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("g must be [B, T, C] float32 or bfloat16")
    for name, t in (("y", y), ("g", g)):
        if not t.is_cuda or not t.is_contiguous() or t.device != y.device:
            raise ValueError(f"{name} must be a contiguous tensor on y's GPU")
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t.dtype != torch.float32 or t.numel() != C or not t.is_cuda or not t.is_contiguous() or t.device != y.device:
            raise ValueError(f"{name} must be a contiguous float32 tensor of C values on y's GPU")
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.bfloat16, device=y.device)
    else:
        _check_out(out, (B, T, C), torch.bfloat16, y.device, "out")
    dtype = DTYPE_BF16 if g.dtype == torch.bfloat16 else DTYPE_F32
    st = lib().wkv6_group_norm_gate(B, T, C, H, y.data_ptr(), g.data_ptr(), gamma.data_ptr(), beta.data_ptr(),
                                    float(eps), out.data_ptr(), dtype, _stream_handle(stream, y.device))
    if st != OK:
        raise WKV6Error(st, f"{status_str(st)}: {last_error()}")
    return out


def fwd4(k, v, w, u, out=None, stream=None):
    """RWKV-4 WKV of k, v ([B, T, C], float32 or bfloat16) with per-channel
    float32 decay rates w and bonuses u ([C]); returns float32 [B, T, C]."""
    import torch

    if k.dim() != 3 or v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must be [B, T, C] tensors of one dtype")
    B, T, C = k.shape
    if k.dtype == torch.float32:
        dtype = DTYPE_F32
    elif k.dtype == torch.bfloat16:
        dtype = DTYPE_BF16
    else:
        raise ValueError("k and v must be float32 or bfloat16")
    for name, t in (("w", w), ("u", u)):
        if t.dtype != torch.float32 or t.numel() != C:
            raise ValueError(f"{name} must be float32 with C elements")
    for name, t in (("k", k), ("v", v), ("w", w), ("u", u)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=k.device)
    else:
        _check_out(out, (B, T, C), torch.float32, k.device, "out")
    st = fwd4_raw(B, T, C, k.data_ptr(), v.data_ptr(), w.data_ptr(), u.data_ptr(), out.data_ptr(), dtype,
                  _stream_handle(stream, k.device))
    if st != OK:
        raise WKV6Error(st, f"{status_str(st)}: {last_error()}")
    return out


def bwd_raw(B: int, T: int, C: int, H: int, r: int, k: int, v: int, w_raw: int, u: int, dy: int,
            dr: int, dk: int, dv: int, dw_raw: int, du: int, mode: int, dtype: int, stream: int = 0) -> int:
    """Direct call of wkv6_bwd with integer addresses."""
    return lib().wkv6_bwd(B, T, C, H, r, k, v, w_raw, u, dy, dr, dk, dv, dw_raw, du, mode, dtype, stream)


def bwd(r, k, v, w_raw, u, dy, H: int, mode: str = "causal", stream=None) -> dict:
    """Gradients of sum(y * dy) for y = fwd(r, k, v, w_raw, u, H, mode).

    dy: contiguous float32 CUDA tensor [B, T, C].  Returns a dict of float32
    tensors: "r", "k", "v", "w_raw" ([B, T, C]) and "u" ([C]).
    """
    import torch

    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    B, T, C, dtype = _check_inputs(r, k, v, w_raw, u)
    if dy.shape != (B, T, C) or dy.dtype != torch.float32 or not dy.is_cuda or not dy.is_contiguous():
        raise ValueError("dy must be a contiguous float32 GPU tensor [B, T, C]")
    g = {name: torch.empty((B, T, C), dtype=torch.float32, device=r.device) for name in ("r", "k", "v", "w_raw")}
    g["u"] = torch.empty((C,), dtype=torch.float32, device=r.device)
    st = bwd_raw(B, T, C, H, r.data_ptr(), k.data_ptr(), v.data_ptr(), w_raw.data_ptr(), u.data_ptr(),
                 dy.data_ptr(), g["r"].data_ptr(), g["k"].data_ptr(), g["v"].data_ptr(), g["w_raw"].data_ptr(),
                 g["u"].data_ptr(), _MODES[mode], dtype, _stream_handle(stream, r.device))
    if st != OK:
        raise WKV6Error(st, f"{status_str(st)}: {last_error()}")
    return g
