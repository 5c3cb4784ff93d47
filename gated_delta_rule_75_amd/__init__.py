"""libkda: the Kimi Delta Attention recurrence on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI declared in include/kda.h.  It only
checks dtypes, shapes, contiguity and devices, allocates outputs with torch
(device memory and streams are all torch provides here) and passes raw
pointers plus the current HIP stream; every step of the recurrence runs in the
HIP kernels of libkda.so.  There is no fallback: importing works without a
GPU, but any call needs the built library and a GPU, and raises otherwise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "KDAError", "lib", "library_path", "kda_version", "kda_status_string",
    "chunk_fwd", "chunk_fwd_workspace_size", "chunk_fwd_workspace_min", "chunk_fwd_checkpointed",
    "chunk_fwd_fused", "chunk_fwd_noalloc", "kcp_scan", "kcp_workspace_size", "kcp_workspace_min", "decode_step",
    "decode_step_fused", "decode_replay",
    "KDA_BF16", "KDA_F32",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")
_lib = None

KDA_BF16, KDA_F32 = 0, 1
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_WORKSPACE_TOO_SMALL", 4: "KDA_ERR_HIP"}

# Every symbol include/kda.h declares.
SYMBOLS = ("kda_version", "kda_status_string", "kda_chunk_fwd_workspace_size",
           "kda_chunk_fwd_workspace_min", "kda_chunk_fwd", "kda_chunk_fwd_checkpointed",
           "kda_kcp_workspace_size", "kda_kcp_workspace_min", "kda_kcp_scan",
           "kda_decode_step", "kda_decode_replay", "kda_chunk_fwd_fused", "kda_decode_step_fused",
           "kda_chunk_fwd_noalloc", "kda_noalloc_scratch_bytes")


class KDAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {_STATUS.get(status, status)}")


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libkda.so with argument types set (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libkda.so is not built ({_LIB_PATH}); run "
                          "python -m gated_delta_rule_75_amd.build")
    L = ctypes.CDLL(_LIB_PATH)
    i, i64, f, vp, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    L.kda_version.argtypes = []
    L.kda_version.restype = i
    L.kda_status_string.argtypes = [i]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_chunk_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i64]
    L.kda_chunk_fwd_workspace_size.restype = sz
    L.kda_chunk_fwd_workspace_min.argtypes = [i, i, i, i, i, i, i64]
    L.kda_chunk_fwd_workspace_min.restype = sz
    L.kda_chunk_fwd.argtypes = [i, i, i, i, i, f, i, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                vp, sz, vp]
    L.kda_chunk_fwd.restype = i
    L.kda_chunk_fwd_noalloc.argtypes = [i, i, i, i, i, f, i, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp]
    L.kda_chunk_fwd_noalloc.restype = i
    L.kda_noalloc_scratch_bytes.argtypes = []
    L.kda_noalloc_scratch_bytes.restype = sz
    L.kda_chunk_fwd_fused.argtypes = L.kda_chunk_fwd.argtypes
    L.kda_chunk_fwd_fused.restype = i
    L.kda_chunk_fwd_checkpointed.argtypes = [i, i, i, i, i, f, i, i64, vp, vp, vp, vp, vp, vp, vp,
                                             vp, vp, vp, i, vp, vp, i64, vp, sz, vp]
    L.kda_chunk_fwd_checkpointed.restype = i
    L.kda_kcp_workspace_size.argtypes = [i, i, i, i, i, i64, i]
    L.kda_kcp_workspace_size.restype = sz
    L.kda_kcp_workspace_min.argtypes = [i, i, i, i, i, i64, i]
    L.kda_kcp_workspace_min.restype = sz
    L.kda_kcp_scan.argtypes = [i, i, i, i, i, f, i64, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                               sz, vp]
    L.kda_kcp_scan.restype = i
    L.kda_decode_step.argtypes = [i, i, i, i, i, f, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_decode_step.restype = i
    L.kda_decode_step_fused.argtypes = L.kda_decode_step.argtypes
    L.kda_decode_step_fused.restype = i
    L.kda_decode_replay.argtypes = [i, i, i, i, i, i, f, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_decode_replay.restype = i
    _lib = L
    return L


def kda_version() -> int:
    return lib().kda_version()


def kda_status_string(status: int) -> str:
    return lib().kda_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise KDAError(fn, status)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v/z must be bfloat16 or float32, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libkda tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("libkda tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("libkda tensors must share one device")
    return dev


def _need(name: str, t, shape, dtype) -> None:
    """A tensor the caller supplies must have exactly this shape and dtype.
    Checked before any device or contiguity check, so a wrong buffer is
    refused on the host whatever it holds."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def _need_workspace(ws) -> None:
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check_inputs(q, k, v, g, beta, z, fused: bool = False):
    """fused: g, beta are the pre-activations a, b, in q's dtype."""
    dt = _dt(q)
    for name, t in (("k", k), ("v", v), ("z", z)):
        if t is not None and t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype {q.dtype}")
    if fused:
        if g.dtype != q.dtype or beta.dtype != q.dtype:
            raise TypeError(f"a and b must have q's dtype {q.dtype}")
    elif g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("g and beta must be float32")
    T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (T, H, dv):
        raise ValueError("q, k, g must be [T, H, dk] and v [T, H, dv]")
    if beta.shape != (T, H) or (z is not None and z.shape != v.shape):
        raise ValueError("beta must be [T, H] and z like v")
    return dt, T, H, dk, dv


def chunk_fwd_workspace_size(dtype: int, H: int, dk: int, dv: int, chunk: int, num_seqs: int,
                             T_total: int) -> int:
    """Bytes of workspace with which a prefill runs in one pass (the fastest)."""
    return int(lib().kda_chunk_fwd_workspace_size(dtype, H, dk, dv, chunk, num_seqs, T_total))


def chunk_fwd_workspace_min(dtype: int, H: int, dk: int, dv: int, chunk: int, num_seqs: int,
                            T_total: int) -> int:
    """The smallest workspace a prefill accepts (time slabs of one chunk)."""
    return int(lib().kda_chunk_fwd_workspace_min(dtype, H, dk, dv, chunk, num_seqs, T_total))


def _workspace_bytes(full: int, least: int, limit: Optional[int]) -> int:
    """The workspace to allocate: the full size, or at most `limit` bytes."""
    if full == 0 or least == 0:
        raise KDAError("workspace size query", 2)
    if limit is None or limit >= full:
        return full
    if limit < least:
        raise ValueError(f"max_workspace_bytes={limit} is below the minimum {least}")
    return int(limit)


def chunk_fwd(q, k, v, g, beta, cu_seqlens: Optional[torch.Tensor] = None, z=None,
              initial_state=None, output_final_state: bool = True, chunk: int = 64,
              scale: float = 1.0, y: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None,
              max_workspace_bytes: Optional[int] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Prefill over packed sequences; returns (y, final_state or None).  The
    workspace (1-D uint8 device tensor) is allocated when not given: the full
    size, or at most max_workspace_bytes (time slabs; at least
    chunk_fwd_workspace_min bytes)."""
    return _chunk_fwd(False, q, k, v, g, beta, cu_seqlens, z, initial_state, output_final_state,
                      chunk, scale, y, final_state, workspace, max_workspace_bytes)


def chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens: Optional[torch.Tensor] = None, z=None,
                      initial_state=None, chunk: int = 64, scale: float = 1.0,
                      y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None):
    """chunk_fwd through kda_chunk_fwd_noalloc: no workspace, the library's own
    per-GPU scratch instead.  y and final_state are allocated here when not
    given (the C call itself allocates nothing); both are returned."""
    dt, T, H, dk, dv = _check_inputs(q, k, v, g, beta, z)
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    N = cu_seqlens.numel() - 1 if cu_seqlens is not None else 1
    _need("y", y, (T, H, dv), q.dtype)
    _need("initial_state", initial_state, (N, H, dk, dv), torch.float32)
    _need("final_state", final_state, (N, H, dk, dv), torch.float32)
    dev = _dev(q, k, v, g, beta, z, cu_seqlens, initial_state, y, final_state)
    if y is None:
        y = torch.empty(T, H, dv, dtype=q.dtype, device=dev)
    if final_state is None:
        final_state = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
    st = lib().kda_chunk_fwd_noalloc(dt, H, dk, dv, chunk, scale, N, T, _ptr(cu_seqlens), _ptr(q),
                                     _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(z),
                                     _ptr(initial_state), _ptr(final_state), _ptr(y), _stream(dev))
    _check("kda_chunk_fwd_noalloc", st)
    return y, final_state


def chunk_fwd_fused(q, k, v, a, b, cu_seqlens: Optional[torch.Tensor] = None, z=None,
                    initial_state=None, output_final_state: bool = True, chunk: int = 64,
                    scale: float = 1.0, y: Optional[torch.Tensor] = None,
                    final_state: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    max_workspace_bytes: Optional[int] = None):
    """chunk_fwd on raw inputs: q, k unnormalised, a [T, H, dk] and b [T, H] the
    decay and beta pre-activations in q's dtype (g = -5 sigmoid(a), beta =
    sigmoid(b), unit q and k formed in the kernel)."""
    return _chunk_fwd(True, q, k, v, a, b, cu_seqlens, z, initial_state, output_final_state,
                      chunk, scale, y, final_state, workspace, max_workspace_bytes)


def _chunk_fwd(fused, q, k, v, g, beta, cu_seqlens, z, initial_state, output_final_state, chunk,
               scale, y, final_state, workspace, max_workspace_bytes=None):
    dt, T, H, dk, dv = _check_inputs(q, k, v, g, beta, z, fused)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be 1-D with at least two offsets")
        N = cu_seqlens.numel() - 1
    else:
        N = 1
    _need("y", y, (T, H, dv), q.dtype)
    _need("initial_state", initial_state, (N, H, dk, dv), torch.float32)
    _need("final_state", final_state, (N, H, dk, dv), torch.float32)
    _need_workspace(workspace)
    dev = _dev(q, k, v, g, beta, z, cu_seqlens, initial_state, y, final_state, workspace)
    if y is None:
        y = torch.empty(T, H, dv, dtype=q.dtype, device=dev)
    if final_state is None and output_final_state:
        final_state = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
    if workspace is None:
        need = _workspace_bytes(chunk_fwd_workspace_size(dt, H, dk, dv, chunk, N, T),
                                chunk_fwd_workspace_min(dt, H, dk, dv, chunk, N, T),
                                max_workspace_bytes)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    fn = "kda_chunk_fwd_fused" if fused else "kda_chunk_fwd"
    st = getattr(lib(), fn)(dt, H, dk, dv, chunk, scale, N, T, _ptr(cu_seqlens), _ptr(q),
                            _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(z),
                            _ptr(initial_state), _ptr(final_state), _ptr(y), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(dev))
    _check(fn, st)
    return y, final_state


def chunk_fwd_checkpointed(q, k, v, g, beta, interval: int, cu_seqlens=None, z=None,
                           initial_state=None, chunk: int = 64, scale: float = 1.0,
                           max_workspace_bytes: Optional[int] = None):
    """Prefill that also saves the state every `interval` tokens of each sequence.
    Returns (y, final_state, checkpoints [T // interval, H, dk, dv] (rows past
    offsets[-1] unused), offsets int32 [N + 1] (device))."""
    dt, T, H, dk, dv = _check_inputs(q, k, v, g, beta, z)
    N = cu_seqlens.numel() - 1 if cu_seqlens is not None else 1
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if interval <= 0 or interval % chunk != 0:
        raise ValueError("interval must be a positive multiple of the chunk")
    _need("initial_state", initial_state, (N, H, dk, dv), torch.float32)
    dev = _dev(q, k, v, g, beta, z, cu_seqlens, initial_state)
    y = torch.empty(T, H, dv, dtype=q.dtype, device=dev)
    fs = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
    cap = max(T // interval, 1)
    ck = torch.empty(cap, H, dk, dv, dtype=torch.float32, device=dev)
    offs = torch.empty(N + 1, dtype=torch.int32, device=dev)
    need = _workspace_bytes(chunk_fwd_workspace_size(dt, H, dk, dv, chunk, N, T),
                            chunk_fwd_workspace_min(dt, H, dk, dv, chunk, N, T), max_workspace_bytes)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().kda_chunk_fwd_checkpointed(dt, H, dk, dv, chunk, scale, N, T, _ptr(cu_seqlens),
                                          _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(z),
                                          _ptr(initial_state), _ptr(fs), _ptr(y), interval,
                                          _ptr(ck), _ptr(offs), cap, _ptr(ws), need, _stream(dev))
    _check("kda_chunk_fwd_checkpointed", st)
    return y, fs, ck, offs


def kcp_workspace_size(dtype: int, H: int, dk: int, dv: int, chunk: int, T: int,
                       num_segments: int) -> int:
    """Bytes of workspace with which a KCP scan forms its chunk products once."""
    return int(lib().kda_kcp_workspace_size(dtype, H, dk, dv, chunk, T, num_segments))


def kcp_workspace_min(dtype: int, H: int, dk: int, dv: int, chunk: int, T: int,
                      num_segments: int) -> int:
    """The smallest workspace a KCP scan accepts (pairs and entering states plus
    one chunk per head)."""
    return int(lib().kda_kcp_workspace_min(dtype, H, dk, dv, chunk, T, num_segments))


def kcp_scan(q, k, v, g, beta, num_segments: int, z=None, initial_state=None, chunk: int = 64,
             scale: float = 1.0, workspace: Optional[torch.Tensor] = None,
             y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
             max_workspace_bytes: Optional[int] = None):
    """One long sequence split into segments composed by a prefix scan; returns
    (y, final_state).  The workspace is allocated when not given: the full
    size, or at most max_workspace_bytes."""
    dt, T, H, dk, dv = _check_inputs(q, k, v, g, beta, z)
    if not 1 <= num_segments <= max(T, 1):
        raise ValueError("num_segments must lie in [1, T]")
    _need("y", y, (T, H, dv), q.dtype)
    _need("initial_state", initial_state, (1, H, dk, dv), torch.float32)
    _need("final_state", final_state, (1, H, dk, dv), torch.float32)
    _need_workspace(workspace)
    dev = _dev(q, k, v, g, beta, z, initial_state, workspace, y, final_state)
    if workspace is None:
        need = _workspace_bytes(kcp_workspace_size(dt, H, dk, dv, chunk, T, num_segments),
                                kcp_workspace_min(dt, H, dk, dv, chunk, T, num_segments),
                                max_workspace_bytes)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty(T, H, dv, dtype=q.dtype, device=dev)
    if final_state is None:
        final_state = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    st = lib().kda_kcp_scan(dt, H, dk, dv, chunk, scale, T, num_segments, _ptr(q), _ptr(k),
                            _ptr(v), _ptr(g), _ptr(beta), _ptr(z), _ptr(initial_state),
                            _ptr(final_state), _ptr(y), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(dev))
    _check("kda_kcp_scan", st)
    return y, final_state


def decode_step(q, k, v, g, beta, state, z=None, scale: float = 1.0,
                y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per request; q, k, g: [N, H, dk], v, z: [N, H, dv], beta [N, H],
    state fp32 [N, H, dk, dv] updated in place.  Returns y [N, H, dv]."""
    return _decode_step(False, q, k, v, g, beta, state, z, scale, y)


def decode_step_fused(q, k, v, a, b, state, z=None, scale: float = 1.0,
                      y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_step on raw inputs (q, k unnormalised; a [N, H, dk], b [N, H] the
    gate pre-activations in q's dtype)."""
    return _decode_step(True, q, k, v, a, b, state, z, scale, y)


def _decode_step(fused, q, k, v, g, beta, state, z, scale, y):
    dt, N, H, dk, dv = _check_inputs(q, k, v, g, beta, z, fused)
    if state is None:
        raise ValueError("state is required")
    _need("state", state, (N, H, dk, dv), torch.float32)
    _need("y", y, (N, H, dv), q.dtype)
    dev = _dev(q, k, v, g, beta, z, state, y)
    if y is None:
        y = torch.empty(N, H, dv, dtype=q.dtype, device=dev)
    fn = "kda_decode_step_fused" if fused else "kda_decode_step"
    st = getattr(lib(), fn)(dt, N, H, dk, dv, scale, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                            _ptr(beta), _ptr(z), _ptr(state), _ptr(y), _stream(dev))
    _check(fn, st)
    return y


def decode_replay(q, k, v, g, beta, state, accepted=None, z=None, scale: float = 1.0,
                  want_y: bool = True, y: Optional[torch.Tensor] = None):
    """Speculative-decoding replay.  q, k, g: [N, Td, H, dk]; v, z: [N, Td, H, dv];
    beta [N, Td, H]; state fp32 [N, H, dk, dv] (overwritten with the state after
    accepted[n] tokens when `accepted` (int32 [N]) is given).  Returns y
    [N, Td, H, dv] or None."""
    dt = _dt(q)
    N, Td, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("k", k), ("v", v), ("z", z)):
        if t is not None and t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype {q.dtype}")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (N, Td, H, dv) or \
            beta.shape != (N, Td, H) or (z is not None and z.shape != v.shape):
        raise ValueError("replay inputs must be [N, Td, H, d] (beta [N, Td, H])")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("g and beta must be float32")
    _need("state", state, (N, H, dk, dv), torch.float32)
    _need("accepted", accepted, (N,), torch.int32)
    _need("y", y, (N, Td, H, dv), q.dtype)
    if not want_y and y is not None:
        raise ValueError("y given with want_y=False")
    if not want_y and accepted is None:
        raise ValueError("a replay needs outputs (want_y) or accepted lengths")
    dev = _dev(q, k, v, g, beta, z, state, accepted, y)
    if want_y and y is None:
        y = torch.empty(N, Td, H, dv, dtype=q.dtype, device=dev)
    if not want_y:
        y = None
    st = lib().kda_decode_replay(dt, N, Td, H, dk, dv, scale, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                 _ptr(beta), _ptr(z), _ptr(accepted), _ptr(state), _ptr(y),
                                 _stream(dev))
    _check("kda_decode_replay", st)
    return y
