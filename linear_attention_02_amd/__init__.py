"""Linear attention with phi(x) = elu(x) + 1 on AMD Instinct MI355X (gfx950).

Thin Python binding of ``liblinattn.so`` (C ABI in ``include/linattn.h``).
This module only checks and marshals arguments -- shapes, dtypes, device
pointers, the current HIP stream, workspace allocation through PyTorch's
allocator -- and calls the library; every arithmetic step runs in the HIP
kernels.  There is no fallback: if the library is missing or no GPU is
present, calls raise.

    forward(q, k, v, causal=True)               -> o
    forward_state(q, k, v, S0=None, z0=None)    -> (o, S_N, z_N)   causal, carries state
    backward(q, k, v, grad_out, causal=True)    -> (dq, dk, dv)
    forward_train(q, k, v, causal=True)         -> (o, workspace)  saves what backward_train reads
    backward_train(q, k, v, o, grad_out, ws)    -> (dq, dk, dv)
    decode_step(S, z, q, k, v)                  -> o               updates S, z in place
    decode_step_strided(S, z, q, k, v)          -> o               q, k, v as strided row views

q, k: [B, H, N, 64]; v: [B, H, N, 64]; float32 or bfloat16, contiguous, CUDA.
Each call runs on the device of its tensors, on that device's current stream
unless ``stream`` is given.  ``linear_attention_02_amd.autograd.linear_attention``
wraps forward_train and backward_train as a torch.autograd.Function.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

__all__ = ["forward", "forward_noalloc", "forward_state", "backward", "forward_train", "backward_train",
           "decode_step", "decode_step_strided", "workspace_bytes", "state_workspace_bytes", "backward_workspace_bytes",
           "train_workspace_bytes", "lib", "LinattnError", "timer", "set_segments", "plan_segments", "LIB_PATH",
           "HEADER_PATH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# LINATTN_LIB selects another in-tree build (e.g. the 32-token-chunk walk
# variant of ``python -m linear_attention_02_amd.build --walk-tiles 2 --out ...``).
LIB_PATH = os.environ.get("LINATTN_LIB") or os.path.join(_HERE, "liblinattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "linattn.h")

F32, BF16 = 0, 1
STATUS = {0: "LINATTN_OK", 1: "LINATTN_ERR_NULL", 2: "LINATTN_ERR_SHAPE", 3: "LINATTN_ERR_DTYPE",
          4: "LINATTN_ERR_ALIGN", 5: "LINATTN_ERR_ALIAS", 6: "LINATTN_ERR_WORKSPACE", 7: "LINATTN_ERR_HIP",
          8: "LINATTN_ERR_ARG"}


class LinattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status
        self.name = STATUS.get(status, str(status))


_lib = None


def lib() -> ctypes.CDLL:
    """Loads liblinattn.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LinattnError(8, f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                                  "or python -m linear_attention_02_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.linattn_version.restype = i
        L.linattn_version.argtypes = []
        L.linattn_status_string.restype = ctypes.c_char_p
        L.linattn_status_string.argtypes = [i]
        L.linattn_last_error.restype = ctypes.c_char_p
        L.linattn_last_error.argtypes = []
        L.linattn_forward_workspace_bytes.restype = sz
        L.linattn_forward_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.linattn_forward_state_workspace_bytes.restype = sz
        L.linattn_forward_state_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.linattn_forward.restype = i
        L.linattn_forward.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
        L.linattn_forward_noalloc.restype = i
        L.linattn_forward_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
        L.linattn_forward_state.restype = i
        L.linattn_forward_state.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp, vp, vp, vp, vp, sz, vp]
        L.linattn_backward_workspace_bytes.restype = sz
        L.linattn_backward_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.linattn_backward.restype = i
        L.linattn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
        L.linattn_backward_after_forward.restype = i
        L.linattn_backward_after_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
        L.linattn_train_workspace_bytes.restype = sz
        L.linattn_train_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.linattn_forward_train.restype = i
        L.linattn_forward_train.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
        L.linattn_backward_train.restype = i
        L.linattn_backward_train.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
        L.linattn_decode_step_strided.restype = i
        L.linattn_decode_step_strided.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, ctypes.c_longlong, vp]
        L.linattn_decode_step.restype = i
        L.linattn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
        L.linattn_timer_enable.restype = None
        L.linattn_timer_enable.argtypes = [i]
        L.linattn_timer_reset.restype = None
        L.linattn_timer_reset.argtypes = []
        L.linattn_timer_read.restype = i
        L.linattn_timer_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_long)]
        L.linattn_timer_names.restype = sz
        L.linattn_timer_names.argtypes = [ctypes.c_char_p, sz]
        L.linattn_set_segments.restype = i
        L.linattn_set_segments.argtypes = [i]
        L.linattn_plan_segments.restype = i
        L.linattn_plan_segments.argtypes = [i, i, i, i, i]
        _lib = L
    return _lib


def declared_functions() -> list:
    """Names of the functions include/linattn.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(linattn_[a-z_0-9]+)\s*\(", text)))


def _raise(rc: int):
    if rc != 0:
        msg = lib().linattn_last_error().decode()
        raise LinattnError(rc, msg or STATUS.get(rc, str(rc)))


def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise LinattnError(3, f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _check_cuda(*ts):
    device = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise LinattnError(8, "tensors must be on a GPU device (no CPU fallback exists)")
        if not t.is_contiguous():
            raise LinattnError(8, "tensors must be contiguous")
        if device is None:
            device = t.device
        elif t.device != device:
            raise LinattnError(8, f"tensors must be on one device (found {device} and {t.device})")


def _stream(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _call(device, fn, *args):
    """Calls a library entry point with ``device`` as the current HIP device
    (the library launches on the current device) and raises on an error status."""
    with _torch().cuda.device(device):
        _raise(fn(*args))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def workspace_bytes(B: int, H: int, N: int, dtype, causal: bool) -> int:
    dt = F32 if str(dtype).endswith("float32") else BF16
    return int(lib().linattn_forward_workspace_bytes(B, H, N, 64, 64, dt, int(bool(causal))))


def state_workspace_bytes(B: int, H: int, N: int, dtype) -> int:
    dt = F32 if str(dtype).endswith("float32") else BF16
    return int(lib().linattn_forward_state_workspace_bytes(B, H, N, 64, 64, dt))


def _alloc_ws(nbytes: int, device, workspace):
    torch = _torch()
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.device != device or not workspace.is_contiguous():
            raise LinattnError(8, "workspace must be a contiguous tensor on the inputs' device")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise LinattnError(6, f"workspace needs {nbytes} bytes")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _check_like(name: str, t, ref):
    """A caller-supplied output must match ``ref`` in shape and dtype: the
    library sizes every access from the input's shape and element type."""
    if t is None:
        return
    if tuple(t.shape) != tuple(ref.shape):
        raise LinattnError(2, f"{name} must have shape {tuple(ref.shape)}, got {tuple(t.shape)}")
    if t.dtype != ref.dtype:
        raise LinattnError(3, f"{name} must be {ref.dtype}, got {t.dtype}")


def _check_state(name: str, t, numel: int):
    """A state buffer is float32 with exactly ``numel`` elements."""
    if t is None:
        return
    torch = _torch()
    if t.dtype != torch.float32:
        raise LinattnError(3, f"{name} must be float32, got {t.dtype}")
    if t.numel() != numel:
        raise LinattnError(2, f"{name} must have {numel} elements, got {t.numel()}")


def _shape(q, k, v):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise LinattnError(2, f"expected q, k [B,H,N,C] and v [B,H,N,M]; got {tuple(q.shape)}, "
                              f"{tuple(k.shape)}, {tuple(v.shape)}")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise LinattnError(3, "q, k and v must share one dtype")
    B, H, N, C = q.shape
    return B, H, N, C, v.shape[3]


def forward(q, k, v, causal: bool = True, out=None, workspace=None, stream=None):
    """Chunked parallel forward; returns o [B,H,N,M] in the input dtype."""
    torch = _torch()
    B, H, N, C, M = _shape(q, k, v)
    dt = _dt(q)
    _check_like("out", out, v)
    _check_cuda(q, k, v, out)
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    nbytes = int(lib().linattn_forward_workspace_bytes(B, H, N, C, M, dt, int(bool(causal))))
    ws = _alloc_ws(nbytes, q.device, workspace)
    _call(q.device, lib().linattn_forward, _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, C, M, dt,
          int(bool(causal)), _ptr(ws), nbytes, _stream(stream, q.device))
    return out


def forward_noalloc(q, k, v, causal: bool = True, out=None, stream=None):
    """``forward`` through linattn_forward_noalloc: the library's static device
    scratch instead of a workspace (nothing is allocated when ``out`` is given)."""
    torch = _torch()
    B, H, N, C, M = _shape(q, k, v)
    dt = _dt(q)
    _check_like("out", out, v)
    _check_cuda(q, k, v, out)
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    _call(q.device, lib().linattn_forward_noalloc, _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, C, M, dt,
          int(bool(causal)), _stream(stream, q.device))
    return out


def forward_state(q, k, v, S0=None, z0=None, out=None, S_out=None, z_out=None, workspace=None, stream=None,
                  return_state: bool = True):
    """Causal forward from state (S0, z0) (zero if None); returns (o, S_N, z_N).

    S0/S_out: [B*H, C, M] float32 (or [B, H, C, M]); z0/z_out: [B*H, C] float32.
    """
    torch = _torch()
    B, H, N, C, M = _shape(q, k, v)
    dt = _dt(q)
    _check_like("out", out, v)
    for name, t, n in (("S0", S0, B * H * C * M), ("z0", z0, B * H * C), ("S_out", S_out, B * H * C * M),
                       ("z_out", z_out, B * H * C)):
        _check_state(name, t, n)
    _check_cuda(q, k, v, S0, z0, out, S_out, z_out)
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    if return_state and S_out is None:
        S_out = torch.empty((B * H, C, M), dtype=torch.float32, device=q.device)
        z_out = torch.empty((B * H, C), dtype=torch.float32, device=q.device)
    nbytes = int(lib().linattn_forward_state_workspace_bytes(B, H, N, C, M, dt))
    ws = _alloc_ws(nbytes, q.device, workspace)
    _call(q.device, lib().linattn_forward_state, _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, C, M, dt, _ptr(S0),
          _ptr(z0), _ptr(S_out), _ptr(z_out), _ptr(ws), nbytes, _stream(stream, q.device))
    return out, S_out, z_out


def backward_workspace_bytes(B: int, H: int, N: int, dtype, causal: bool) -> int:
    dt = F32 if str(dtype).endswith("float32") else BF16
    return int(lib().linattn_backward_workspace_bytes(B, H, N, 64, 64, dt, int(bool(causal))))


def backward(q, k, v, grad_out, causal: bool = True, dq=None, dk=None, dv=None, workspace=None, stream=None,
             after_forward: bool = False):
    """Gradients of ``forward`` (zero initial state) for dL/dO = grad_out; returns (dq, dk, dv).

    after_forward=True: ``workspace`` (sized by backward_workspace_bytes) was last
    written by ``forward`` on the same q, k, v and causal flag, and the segment
    records it holds are reused instead of recomputed.
    """
    torch = _torch()
    B, H, N, C, M = _shape(q, k, v)
    if grad_out.shape != v.shape or grad_out.dtype != v.dtype:
        raise LinattnError(2, "grad_out must match v in shape and dtype")
    dt = _dt(q)
    _check_like("dq", dq, q)
    _check_like("dk", dk, k)
    _check_like("dv", dv, v)
    _check_cuda(q, k, v, grad_out, dq, dk, dv)
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=v.dtype, device=v.device) if dv is None else dv
    nbytes = int(lib().linattn_backward_workspace_bytes(B, H, N, C, M, dt, int(bool(causal))))
    if after_forward and workspace is None:
        raise LinattnError(8, "after_forward needs the workspace the forward used")
    ws = _alloc_ws(nbytes, q.device, workspace)
    fn = lib().linattn_backward_after_forward if after_forward else lib().linattn_backward
    _call(q.device, fn, _ptr(q), _ptr(k), _ptr(v), _ptr(grad_out), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, C, M, dt,
          int(bool(causal)), _ptr(ws), nbytes, _stream(stream, q.device))
    return dq, dk, dv


def train_workspace_bytes(B: int, H: int, N: int, dtype, causal: bool) -> int:
    dt = F32 if str(dtype).endswith("float32") else BF16
    return int(lib().linattn_train_workspace_bytes(B, H, N, 64, 64, dt, int(bool(causal))))


def forward_train(q, k, v, causal: bool = True, out=None, workspace=None, stream=None):
    """``forward`` for a training step; returns (o, workspace).

    The workspace (sized by train_workspace_bytes) then holds what
    ``backward_train`` reads: the segment records and, for bf16 causal calls,
    1/den per token.  o equals ``forward``'s bit for bit.
    """
    torch = _torch()
    B, H, N, C, M = _shape(q, k, v)
    dt = _dt(q)
    _check_like("out", out, v)
    _check_cuda(q, k, v, out)
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    nbytes = int(lib().linattn_train_workspace_bytes(B, H, N, C, M, dt, int(bool(causal))))
    ws = _alloc_ws(nbytes, q.device, workspace)
    _call(q.device, lib().linattn_forward_train, _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, C, M, dt,
          int(bool(causal)), _ptr(ws), nbytes, _stream(stream, q.device))
    return out, ws


def backward_train(q, k, v, o, grad_out, workspace, causal: bool = True, dq=None, dk=None, dv=None, stream=None):
    """Gradients after ``forward_train`` on the same q, k, v and causal flag,
    with its output ``o`` and ``workspace``; returns (dq, dk, dv)."""
    torch = _torch()
    B, H, N, C, M = _shape(q, k, v)
    if grad_out.shape != v.shape or grad_out.dtype != v.dtype:
        raise LinattnError(2, "grad_out must match v in shape and dtype")
    _check_like("o", o, v)
    if o is None:
        raise LinattnError(1, "backward_train needs the forward's output o")
    dt = _dt(q)
    _check_like("dq", dq, q)
    _check_like("dk", dk, k)
    _check_like("dv", dv, v)
    _check_cuda(q, k, v, o, grad_out, dq, dk, dv)
    nbytes = int(lib().linattn_train_workspace_bytes(B, H, N, C, M, dt, int(bool(causal))))
    if nbytes > 0 and workspace is None:
        raise LinattnError(8, "backward_train needs the workspace forward_train used")
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=v.dtype, device=v.device) if dv is None else dv
    ws = _alloc_ws(nbytes, q.device, workspace)
    _call(q.device, lib().linattn_backward_train, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(grad_out), _ptr(dq),
          _ptr(dk), _ptr(dv), B, H, N, C, M, dt, int(bool(causal)), _ptr(ws), nbytes, _stream(stream, q.device))
    return dq, dk, dv


def decode_step(S, z, q, k, v, out=None, stream=None):
    """One recurrent step for BH heads; S [BH,C,M] and z [BH,C] float32 are updated in place.

    q, k: [BH, C]; v: [BH, M] in float32 or bfloat16.  Returns o [BH, M] float32.
    """
    torch = _torch()
    if q.dim() != 2 or v.dim() != 2:
        raise LinattnError(2, "q, k must be [BH, C] and v [BH, M]")
    BH, C = q.shape
    M = v.shape[1]
    if k.shape != q.shape or v.shape[0] != BH:
        raise LinattnError(2, "decode_step shape mismatch")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise LinattnError(3, "q, k and v must share one dtype")
    dt = _dt(q)
    _check_state("S", S, BH * C * M)
    _check_state("z", z, BH * C)
    _check_state("out", out, BH * M)
    _check_cuda(S, z, q, k, v, out)
    if out is None:
        out = torch.empty((BH, M), dtype=torch.float32, device=q.device)
    _call(q.device, lib().linattn_decode_step, _ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), BH, C, M, dt,
          _stream(stream, q.device))
    return out


class timer:
    """Per-kernel HIP-event timing inside the library (measurement support)."""

    @staticmethod
    def enable(on: bool = True):
        lib().linattn_timer_enable(int(bool(on)))

    @staticmethod
    def reset():
        lib().linattn_timer_reset()

    @staticmethod
    def read(kernel: str) -> Tuple[float, int]:
        ms = ctypes.c_double(0.0)
        n = ctypes.c_long(0)
        if lib().linattn_timer_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)) != 0:
            return 0.0, 0
        return ms.value, n.value

    @staticmethod
    def names() -> list:
        n = lib().linattn_timer_names(None, 0)
        buf = ctypes.create_string_buffer(n + 1)
        lib().linattn_timer_names(buf, n + 1)
        return [s for s in buf.value.decode().split(";") if s]


def set_segments(n: int) -> int:
    """Forces the number of sequence segments per head (0 = automatic); returns the previous value."""
    return int(lib().linattn_set_segments(int(n)))


def plan_segments(B: int, H: int, N: int, dtype, causal: bool) -> int:
    dt = F32 if str(dtype).endswith("float32") else BF16
    return int(lib().linattn_plan_segments(B, H, N, dt, int(bool(causal))))


def decode_step_strided(S, z, q, k, v, out=None, stream=None):
    """decode_step for q, k, v given as [BH, 64] views that share one row
    stride (e.g. column slices of a [BH, 3 * 64] projection output)."""
    torch = _torch()
    for t in (q, k, v):
        if t.dim() != 2 or t.stride(1) != 1:
            raise LinattnError(2, "q, k, v must be 2-D with unit column stride")
    stride = q.stride(0)
    if k.stride(0) != stride or v.stride(0) != stride:
        raise LinattnError(2, "q, k and v must share one row stride")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise LinattnError(3, "q, k and v must share one dtype")
    _dt(q)
    BH, C = q.shape
    M = v.shape[1]
    if k.shape != q.shape or v.shape[0] != BH:
        raise LinattnError(2, "decode_step_strided shape mismatch")
    _check_state("S", S, BH * C * M)
    _check_state("z", z, BH * C)
    _check_state("out", out, BH * M)
    _check_cuda(S, z, out)
    for t in (q, k, v):
        if not t.is_cuda:
            raise LinattnError(8, "tensors must be on a GPU device (no CPU fallback exists)")
    if any(t.device != S.device for t in (q, k, v)):
        raise LinattnError(8, "q, k, v and the state must be on one device")
    if out is None:
        out = torch.empty((BH, M), dtype=torch.float32, device=q.device)
    _call(q.device, lib().linattn_decode_step_strided, _ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), BH,
          C, M, _dt(q), int(stride), _stream(stream, q.device))
    return out
