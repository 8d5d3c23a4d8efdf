"""ctypes binding of libssd (include/ssd.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  torch supplies device memory and the current stream; nothing
here computes on the host.  If libssd.so is missing the import fails loudly --
there is no fallback path.

Python names follow the C entry points (ssd_chunk_scan_fwd, ssd_chunk_cumsum,
...).  They take torch tensors already resident on the GPU and enqueue on
torch's current stream (or the stream passed in).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libssd.so")

SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP = range(5)
SSD_F32, SSD_BF16 = 0, 1


class SSDError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libssd: {msg} (status {status})")
        self.status = status


class SSDInvalidArgument(SSDError, ValueError):
    pass


class SSDUnsupported(SSDError, NotImplementedError):
    pass


class SSDWorkspaceError(SSDError, ValueError):
    pass


class ssd_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("nseq", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class ssd_workspace_layout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_size_t), ("nc_max", ctypes.c_int64),
                ("acum_offset", ctypes.c_size_t), ("dtq_offset", ctypes.c_size_t),
                ("states_offset", ctypes.c_size_t), ("hprev_offset", ctypes.c_size_t),
                ("chunk_table_offset", ctypes.c_size_t), ("chunk_dir_offset", ctypes.c_size_t)]


EXPORTS = ["ssd_workspace_size", "ssd_get_workspace_layout", "ssd_chunk_scan_fwd",
           "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan",
           "ssd_step", "ssd_conv1d_silu", "ssd_gate_rmsnorm", "ssd_fused_fwd",
           "ssd_fused_fwd_train", "ssd_fused_states_size", "ssd_fused_bwd_workspace_size",
           "ssd_fused_bwd",
           "ssd_status_string", "ssd_version"]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libssd.so not built at {LIB_PATH}; run "
                          "`python -c 'import __graft_entry__ as g; g.build()'` first")
    lib = ctypes.CDLL(LIB_PATH)
    p, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dims_p = ctypes.POINTER(ssd_dims)
    lib.ssd_workspace_size.restype = sz
    lib.ssd_workspace_size.argtypes = [dims_p, i32]
    lib.ssd_get_workspace_layout.restype = i32
    lib.ssd_get_workspace_layout.argtypes = [dims_p, i32, ctypes.POINTER(ssd_workspace_layout)]
    lib.ssd_chunk_scan_fwd.restype = i32
    lib.ssd_chunk_scan_fwd.argtypes = [p, p, p, p, p, p, i32, p, p, p, p, dims_p, p, sz, p]
    lib.ssd_chunk_cumsum.restype = i32
    lib.ssd_chunk_cumsum.argtypes = [p, p, i32, p, dims_p, p, sz, p]
    lib.ssd_chunk_state.restype = i32
    lib.ssd_chunk_state.argtypes = [p, p, i32, dims_p, p, sz, p]
    lib.ssd_state_passing.restype = i32
    lib.ssd_state_passing.argtypes = [p, p, i32, dims_p, p, sz, p]
    lib.ssd_chunk_scan.restype = i32
    lib.ssd_chunk_scan.argtypes = [p, p, p, p, p, i32, dims_p, p, sz, p]
    lib.ssd_step.restype = i32
    lib.ssd_step.argtypes = [p, p, p, p, p, p, p, p, dims_p, p]
    i64 = ctypes.c_int64
    lib.ssd_conv1d_silu.restype = i32
    lib.ssd_conv1d_silu.argtypes = [p, i64, p, p, i32, p, i64, i64, i64, i64, p, i64, i32, p]
    lib.ssd_gate_rmsnorm.restype = i32
    lib.ssd_gate_rmsnorm.argtypes = [p, p, p, ctypes.c_float, p, i64, i64, i32, p]
    lib.ssd_fused_fwd.restype = i32
    lib.ssd_fused_fwd.argtypes = [p, p, p, p, p, p, p, p, p, p, dims_p, p]
    lib.ssd_fused_fwd_train.restype = i32
    lib.ssd_fused_fwd_train.argtypes = [p, p, p, p, p, p, p, p, p, p, p, sz, dims_p, p]
    lib.ssd_fused_states_size.restype = sz
    lib.ssd_fused_states_size.argtypes = [dims_p]
    lib.ssd_fused_bwd_workspace_size.restype = sz
    lib.ssd_fused_bwd_workspace_size.argtypes = [dims_p]
    lib.ssd_fused_bwd.restype = i32
    lib.ssd_fused_bwd.argtypes = [p, p, p, p, p, p, p, p, sz, p, p, p, p, p, p, p, p, p, dims_p,
                                  p, sz, p]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [i32]
    lib.ssd_version.restype = i32
    lib.ssd_version.argtypes = []
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def ssd_status_string(status: int) -> str:
    return _lib.ssd_status_string(int(status)).decode()


def ssd_version() -> int:
    return int(_lib.ssd_version())


def _check(status: int) -> None:
    if status == SSD_OK:
        return
    msg = ssd_status_string(status)
    if status == SSD_ERR_INVALID_ARG:
        raise SSDInvalidArgument(status, msg)
    if status == SSD_ERR_UNSUPPORTED:
        raise SSDUnsupported(status, msg)
    if status == SSD_ERR_WORKSPACE:
        raise SSDWorkspaceError(status, msg)
    raise SSDError(status, msg)


def make_dims(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, ngroups: int,
              nseq: int = 0, io_dtype: int = SSD_BF16) -> ssd_dims:
    return ssd_dims(batch, seqlen, nheads, headdim, dstate, ngroups, nseq, io_dtype, 0)


def ssd_workspace_size(dims: ssd_dims, chunk_len: int) -> int:
    return int(_lib.ssd_workspace_size(ctypes.byref(dims), int(chunk_len)))


def ssd_get_workspace_layout(dims: ssd_dims, chunk_len: int) -> ssd_workspace_layout:
    out = ssd_workspace_layout()
    _check(_lib.ssd_get_workspace_layout(ctypes.byref(dims), int(chunk_len), ctypes.byref(out)))
    return out


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "tensor is not on the GPU")
    if not t.is_contiguous():
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "tensor is not contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def ssd_chunk_scan_fwd(x, dt, A, B, C, D, chunk_len, init_state, cu_seqlens, y, final_state,
                       dims, workspace, stream=None) -> None:
    _check(_lib.ssd_chunk_scan_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                   int(chunk_len), _ptr(init_state), _ptr(cu_seqlens), _ptr(y),
                                   _ptr(final_state), ctypes.byref(dims), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def ssd_chunk_cumsum(dt, A, chunk_len, cu_seqlens, dims, workspace, stream=None) -> None:
    _check(_lib.ssd_chunk_cumsum(_ptr(dt), _ptr(A), int(chunk_len), _ptr(cu_seqlens),
                                 ctypes.byref(dims), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def ssd_chunk_state(x, B, chunk_len, dims, workspace, stream=None) -> None:
    _check(_lib.ssd_chunk_state(_ptr(x), _ptr(B), int(chunk_len), ctypes.byref(dims),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)))


def ssd_state_passing(init_state, final_state, chunk_len, dims, workspace, stream=None) -> None:
    _check(_lib.ssd_state_passing(_ptr(init_state), _ptr(final_state), int(chunk_len),
                                  ctypes.byref(dims), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def ssd_chunk_scan(x, B, C, D, y, chunk_len, dims, workspace, stream=None) -> None:
    _check(_lib.ssd_chunk_scan(_ptr(x), _ptr(B), _ptr(C), _ptr(D), _ptr(y), int(chunk_len),
                               ctypes.byref(dims), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)))


def ssd_step(x, dt, A, B, C, D, state, y, dims, stream=None) -> None:
    _check(_lib.ssd_step(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(state),
                         _ptr(y), ctypes.byref(dims), _stream(stream)))


def ssd_fused_fwd(x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state, dims,
                  stream=None) -> None:
    _check(_lib.ssd_fused_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                              _ptr(init_state), _ptr(cu_seqlens), _ptr(y), _ptr(final_state),
                              ctypes.byref(dims), _stream(stream)))


def ssd_fused_states_size(dims) -> int:
    return int(_lib.ssd_fused_states_size(ctypes.byref(dims)))


def ssd_fused_bwd_workspace_size(dims) -> int:
    return int(_lib.ssd_fused_bwd_workspace_size(ctypes.byref(dims)))


def ssd_fused_fwd_train(x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state, chunk_states,
                        states_bytes, dims, stream=None) -> None:
    _check(_lib.ssd_fused_fwd_train(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                    _ptr(init_state), _ptr(cu_seqlens), _ptr(y),
                                    _ptr(final_state), _ptr(chunk_states), int(states_bytes),
                                    ctypes.byref(dims), _stream(stream)))


def ssd_fused_bwd(x, dt, A, B, C, D, cu_seqlens, chunk_states, states_bytes, dy, dfinal, dx, ddt,
                  dA, dB, dC, dD, dinit, dims, workspace, workspace_bytes, stream=None) -> None:
    _check(_lib.ssd_fused_bwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                              _ptr(cu_seqlens), _ptr(chunk_states), int(states_bytes), _ptr(dy),
                              _ptr(dfinal), _ptr(dx), _ptr(ddt), _ptr(dA), _ptr(dB), _ptr(dC),
                              _ptr(dD), _ptr(dinit), ctypes.byref(dims), _ptr(workspace),
                              int(workspace_bytes), _stream(stream)))


def _raw_ptr(t: Optional[torch.Tensor], offset_elems: int = 0):
    """Device address of t's storage start + offset (t may be a strided view)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "tensor is not on the GPU")
    return ctypes.c_void_p(t.data_ptr() + offset_elems * t.element_size()) if t.numel() else None


def ssd_conv1d_silu(inp, in_stride, weight, bias, kernel_width, out, out_stride, batch, seqlen,
                    nseq, cu_seqlens, channels, io_dtype, stream=None) -> None:
    """inp / out: tensors whose first element is channel 0 of token 0 (row
    strides given in elements, so they may be column slices of wider rows)."""
    _check(_lib.ssd_conv1d_silu(_raw_ptr(inp), int(in_stride), _ptr(weight), _ptr(bias),
                                int(kernel_width), _raw_ptr(out), int(out_stride), int(batch),
                                int(seqlen), int(nseq), _ptr(cu_seqlens), int(channels),
                                int(io_dtype), _stream(stream)))


def ssd_gate_rmsnorm(y, z, weight, eps, out, tokens, width, io_dtype, stream=None) -> None:
    _check(_lib.ssd_gate_rmsnorm(_ptr(y), _ptr(z), _ptr(weight), float(eps), _ptr(out),
                                 int(tokens), int(width), int(io_dtype), _stream(stream)))
