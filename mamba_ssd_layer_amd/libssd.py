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


# SSD_NOALLOC_SCRATCH_BYTES of include/ssd.h: the largest workspace of
# ssd_chunk_scan_fwd_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ["ssd_workspace_size", "ssd_get_workspace_layout", "ssd_chunk_scan_fwd",
           "ssd_chunk_scan_fwd_noalloc",
           "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan",
           "ssd_step", "ssd_conv1d_silu", "ssd_gate_rmsnorm", "ssd_fused_fwd",
           "ssd_fused_fwd_train", "ssd_fused_states_size", "ssd_fused_bwd_workspace_size",
           "ssd_fused_fwd_split", "ssd_fused_split_workspace_size", "ssd_fused_split_seg_len",
           "ssd_fused_fwd_split_train",
           "ssd_chunk_scan_bwd", "ssd_chunk_scan_bwd_workspace_size",
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
    lib.ssd_chunk_scan_fwd_noalloc.restype = i32
    lib.ssd_chunk_scan_fwd_noalloc.argtypes = [p, p, p, p, p, p, i32, p, p, p, p, dims_p, p]
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
    lib.ssd_fused_fwd_split.restype = i32
    lib.ssd_fused_fwd_split.argtypes = [p, p, p, p, p, p, p, p, p, ctypes.c_int64, dims_p, p, sz,
                                        p]
    lib.ssd_fused_fwd_split_train.restype = i32
    lib.ssd_fused_fwd_split_train.argtypes = [p, p, p, p, p, p, p, p, p, p, sz, ctypes.c_int64,
                                              dims_p, p, sz, p]
    lib.ssd_fused_split_workspace_size.restype = sz
    lib.ssd_fused_split_workspace_size.argtypes = [dims_p, ctypes.c_int64]
    lib.ssd_fused_split_seg_len.restype = ctypes.c_int64
    lib.ssd_fused_split_seg_len.argtypes = [dims_p]
    lib.ssd_chunk_scan_bwd.restype = i32
    lib.ssd_chunk_scan_bwd.argtypes = [p] * 17 + [dims_p, p, sz, p]
    lib.ssd_chunk_scan_bwd_workspace_size.restype = sz
    lib.ssd_chunk_scan_bwd_workspace_size.argtypes = [dims_p]
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
    if not isinstance(t, torch.Tensor):
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "expected a torch tensor")
    if not t.is_cuda:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "tensor is not on the GPU")
    if not t.is_contiguous():
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "tensor is not contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _io_torch(dims) -> torch.dtype:
    return torch.bfloat16 if dims.io_dtype == SSD_BF16 else torch.float32


def _sizes(dims):
    """(T, H, P, N, G, rows) of a dims struct (T = tokens, rows = sequences)."""
    T = dims.seqlen if dims.nseq > 0 else dims.batch * dims.seqlen
    rows = dims.nseq if dims.nseq > 0 else dims.batch
    return T, dims.nheads, dims.headdim, dims.dstate, dims.ngroups, rows


def _t(t: Optional[torch.Tensor], dtype: torch.dtype, numel: int, name: str,
       optional: bool = False) -> Optional[torch.Tensor]:
    """t after checking that it is present (unless optional), of dtype `dtype`
    and of exactly `numel` elements: the C entry points see only a pointer,
    so a wrong dtype or size would make the kernels read or write past the
    buffer.  Where it lives is checked when its pointer is taken (_ptrs)."""
    if t is None:
        if optional or numel == 0:
            return None
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG,
                                 f"{name} must hold {numel} elements, got {t.numel()}")
    return t


def _ptrs(*ts):
    """Device pointers of already checked tensors (None stays None)."""
    return [_ptr(t) for t in ts]


def _cu(cu: Optional[torch.Tensor], dims):
    if dims.nseq > 0:
        return _t(cu, torch.int32, dims.nseq + 1, "cu_seqlens")
    if cu is not None:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG,
                                 "cu_seqlens given for a fixed-length batch (dims.nseq == 0)")
    return None


def _bytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _fwd(dims, x=None, dt=None, A=None, B=None, C=None, D=None, y=None, need=()):
    """The forward's token tensors, checked against dims; those named in
    `need` must be present."""
    T, H, P, N, G, _ = _sizes(dims)
    io = _io_torch(dims)
    f32 = torch.float32
    opt = lambda k: k not in need
    return (_t(x, io, T * H * P, "x", opt("x")), _t(dt, f32, T * H, "dt", opt("dt")),
            _t(A, f32, H, "A", opt("A")), _t(B, io, T * G * N, "B", opt("B")),
            _t(C, io, T * G * N, "C", opt("C")), _t(D, f32, H, "D", optional=True),
            _t(y, io, T * H * P, "y", opt("y")))


ALL = ("x", "dt", "A", "B", "C", "y")


def _state(t, dims, name):
    T, H, P, N, G, rows = _sizes(dims)
    return _t(t, torch.float32, rows * H * P * N, name, optional=True)


def ssd_chunk_scan_fwd(x, dt, A, B, C, D, chunk_len, init_state, cu_seqlens, y, final_state,
                       dims, workspace, stream=None) -> None:
    ts = _fwd(dims, x, dt, A, B, C, D, y, need=ALL)
    hi, cu, hf = _state(init_state, dims, "init_state"), _cu(cu_seqlens, dims), \
        _state(final_state, dims, "final_state")
    px, pdt, pA, pB, pC, pD, py, phi, pcu, phf, pws = _ptrs(*ts, hi, cu, hf, workspace)
    _check(_lib.ssd_chunk_scan_fwd(px, pdt, pA, pB, pC, pD, int(chunk_len), phi, pcu, py, phf,
                                   ctypes.byref(dims), pws, _bytes(workspace), _stream(stream)))


def ssd_chunk_scan_fwd_noalloc(x, dt, A, B, C, D, chunk_len, init_state, cu_seqlens, y,
                               final_state, dims, stream=None) -> None:
    ts = _fwd(dims, x, dt, A, B, C, D, y, need=ALL)
    hi, cu, hf = _state(init_state, dims, "init_state"), _cu(cu_seqlens, dims), \
        _state(final_state, dims, "final_state")
    px, pdt, pA, pB, pC, pD, py, phi, pcu, phf = _ptrs(*ts, hi, cu, hf)
    _check(_lib.ssd_chunk_scan_fwd_noalloc(px, pdt, pA, pB, pC, pD, int(chunk_len), phi, pcu, py,
                                           phf, ctypes.byref(dims), _stream(stream)))


def ssd_chunk_cumsum(dt, A, chunk_len, cu_seqlens, dims, workspace, stream=None) -> None:
    _, dt, A, _, _, _, _ = _fwd(dims, dt=dt, A=A, need=("dt", "A"))
    pdt, pA, pcu, pws = _ptrs(dt, A, _cu(cu_seqlens, dims), workspace)
    _check(_lib.ssd_chunk_cumsum(pdt, pA, int(chunk_len), pcu, ctypes.byref(dims), pws,
                                 _bytes(workspace), _stream(stream)))


def ssd_chunk_state(x, B, chunk_len, dims, workspace, stream=None) -> None:
    x, _, _, B, _, _, _ = _fwd(dims, x=x, B=B, need=("x", "B"))
    px, pB, pws = _ptrs(x, B, workspace)
    _check(_lib.ssd_chunk_state(px, pB, int(chunk_len), ctypes.byref(dims), pws,
                                _bytes(workspace), _stream(stream)))


def ssd_state_passing(init_state, final_state, chunk_len, dims, workspace, stream=None) -> None:
    phi, phf, pws = _ptrs(_state(init_state, dims, "init_state"),
                          _state(final_state, dims, "final_state"), workspace)
    _check(_lib.ssd_state_passing(phi, phf, int(chunk_len), ctypes.byref(dims), pws,
                                  _bytes(workspace), _stream(stream)))


def ssd_chunk_scan(x, B, C, D, y, chunk_len, dims, workspace, stream=None) -> None:
    x, _, _, B, C, D, y = _fwd(dims, x=x, B=B, C=C, D=D, y=y, need=("x", "B", "C", "y"))
    px, pB, pC, pD, py, pws = _ptrs(x, B, C, D, y, workspace)
    _check(_lib.ssd_chunk_scan(px, pB, pC, pD, py, int(chunk_len), ctypes.byref(dims), pws,
                               _bytes(workspace), _stream(stream)))


def ssd_step(x, dt, A, B, C, D, state, y, dims, stream=None) -> None:
    # one token per sequence: T = rows = dims.batch
    ts = _fwd(dims, x, dt, A, B, C, D, y, need=ALL)
    T, H, P, N, G, rows = _sizes(dims)
    st = _t(state, torch.float32, rows * H * P * N, "state")
    px, pdt, pA, pB, pC, pD, py, pst = _ptrs(*ts, st)
    _check(_lib.ssd_step(px, pdt, pA, pB, pC, pD, pst, py, ctypes.byref(dims), _stream(stream)))


def ssd_fused_fwd(x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state, dims,
                  stream=None) -> None:
    ts = _fwd(dims, x, dt, A, B, C, D, y, need=ALL)
    hi, cu, hf = _state(init_state, dims, "init_state"), _cu(cu_seqlens, dims), \
        _state(final_state, dims, "final_state")
    px, pdt, pA, pB, pC, pD, py, phi, pcu, phf = _ptrs(*ts, hi, cu, hf)
    _check(_lib.ssd_fused_fwd(px, pdt, pA, pB, pC, pD, phi, pcu, py, phf, ctypes.byref(dims),
                              _stream(stream)))


def ssd_fused_fwd_split(x, dt, A, B, C, D, init_state, y, final_state, seg_len, dims, workspace,
                        stream=None) -> None:
    if dims.nseq > 0:
        raise SSDUnsupported(SSD_ERR_UNSUPPORTED, "the split forward takes fixed-length batches")
    ts = _fwd(dims, x, dt, A, B, C, D, y, need=ALL)
    hi, hf = _state(init_state, dims, "init_state"), _state(final_state, dims, "final_state")
    need = ssd_fused_split_workspace_size(dims, seg_len)
    ws = _t(workspace, torch.uint8, _bytes(workspace), "workspace", optional=need == 0)
    if need and _bytes(ws) < need:
        raise SSDWorkspaceError(SSD_ERR_WORKSPACE, f"workspace has {_bytes(ws)} bytes, needs {need}")
    px, pdt, pA, pB, pC, pD, py, phi, phf, pws = _ptrs(*ts, hi, hf, ws)
    _check(_lib.ssd_fused_fwd_split(px, pdt, pA, pB, pC, pD, phi, py, phf, int(seg_len),
                                    ctypes.byref(dims), pws, _bytes(ws), _stream(stream)))


def ssd_fused_fwd_split_train(x, dt, A, B, C, D, init_state, y, final_state, chunk_states,
                              states_bytes, seg_len, dims, workspace, stream=None) -> None:
    if dims.nseq > 0:
        raise SSDUnsupported(SSD_ERR_UNSUPPORTED, "the split forward takes fixed-length batches")
    ts = _fwd(dims, x, dt, A, B, C, D, y, need=ALL)
    hi, hf = _state(init_state, dims, "init_state"), _state(final_state, dims, "final_state")
    need = ssd_fused_split_workspace_size(dims, seg_len)
    ws = _t(workspace, torch.uint8, _bytes(workspace), "workspace", optional=need == 0)
    if need and _bytes(ws) < need:
        raise SSDWorkspaceError(SSD_ERR_WORKSPACE, f"workspace has {_bytes(ws)} bytes, needs {need}")
    if chunk_states is None:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "chunk_states is required")
    if int(states_bytes) > _bytes(chunk_states):
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "states_bytes exceeds its buffer")
    px, pdt, pA, pB, pC, pD, py, phi, phf, pcs, pws = _ptrs(*ts, hi, hf, chunk_states, ws)
    _check(_lib.ssd_fused_fwd_split_train(px, pdt, pA, pB, pC, pD, phi, py, phf, pcs,
                                          int(states_bytes), int(seg_len), ctypes.byref(dims),
                                          pws, _bytes(ws), _stream(stream)))


def ssd_fused_split_workspace_size(dims, seg_len) -> int:
    return int(_lib.ssd_fused_split_workspace_size(ctypes.byref(dims), int(seg_len)))


def ssd_fused_split_seg_len(dims) -> int:
    return int(_lib.ssd_fused_split_seg_len(ctypes.byref(dims)))


def ssd_fused_states_size(dims) -> int:
    return int(_lib.ssd_fused_states_size(ctypes.byref(dims)))


def ssd_fused_bwd_workspace_size(dims) -> int:
    return int(_lib.ssd_fused_bwd_workspace_size(ctypes.byref(dims)))


def ssd_fused_fwd_train(x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state, chunk_states,
                        states_bytes, dims, stream=None) -> None:
    ts = _fwd(dims, x, dt, A, B, C, D, y, need=ALL)
    hi, cu, hf = _state(init_state, dims, "init_state"), _cu(cu_seqlens, dims), \
        _state(final_state, dims, "final_state")
    if chunk_states is not None and int(states_bytes) > _bytes(chunk_states):
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "states_bytes exceeds its buffer")
    px, pdt, pA, pB, pC, pD, py, phi, pcu, phf, pcs = _ptrs(*ts, hi, cu, hf, chunk_states)
    _check(_lib.ssd_fused_fwd_train(px, pdt, pA, pB, pC, pD, phi, pcu, py, phf, pcs,
                                    int(states_bytes), ctypes.byref(dims), _stream(stream)))


def ssd_fused_bwd(x, dt, A, B, C, D, cu_seqlens, chunk_states, states_bytes, dy, dfinal, dx, ddt,
                  dA, dB, dC, dD, dinit, dims, workspace, workspace_bytes, stream=None) -> None:
    x, dt, A, B, C, D, _ = _fwd(dims, x, dt, A, B, C, D, need=("x", "dt", "A", "B", "C"))
    T, H, P, N, G, rows = _sizes(dims)
    io, f32 = _io_torch(dims), torch.float32
    outs = (_t(dy, io, T * H * P, "dy"), _state(dfinal, dims, "dfinal"),
            _t(dx, io, T * H * P, "dx"), _t(ddt, f32, T * H, "ddt"), _t(dA, f32, H, "dA"),
            _t(dB, f32, T * G * N, "dB"), _t(dC, f32, T * G * N, "dC"),
            _t(dD, f32, H, "dD", optional=True), _state(dinit, dims, "dinit"))
    if int(states_bytes) > _bytes(chunk_states) or int(workspace_bytes) > _bytes(workspace):
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "byte count exceeds its buffer")
    cu = _cu(cu_seqlens, dims)
    (px, pdt, pA, pB, pC, pD, pcu, pcs, pdy, pdf, pdx, pddt, pdA, pdB, pdC, pdD, pdi,
     pws) = _ptrs(x, dt, A, B, C, D, cu, chunk_states, *outs, workspace)
    _check(_lib.ssd_fused_bwd(px, pdt, pA, pB, pC, pD, pcu, pcs, int(states_bytes), pdy, pdf, pdx,
                              pddt, pdA, pdB, pdC, pdD, pdi, ctypes.byref(dims), pws,
                              int(workspace_bytes), _stream(stream)))


def ssd_chunk_scan_bwd_workspace_size(dims) -> int:
    return int(_lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(dims)))


def ssd_chunk_scan_bwd(x, dt, A, B, C, D, init_state, cu_seqlens, dy, dfinal, dx, ddt, dA, dB, dC,
                       dD, dinit, dims, workspace, workspace_bytes, stream=None) -> None:
    x, dt, A, B, C, D, _ = _fwd(dims, x, dt, A, B, C, D, need=("x", "dt", "A", "B", "C"))
    T, H, P, N, G, rows = _sizes(dims)
    io, f32 = _io_torch(dims), torch.float32
    hi = _state(init_state, dims, "init_state")
    outs = (_t(dy, io, T * H * P, "dy"), _state(dfinal, dims, "dfinal"),
            _t(dx, io, T * H * P, "dx"), _t(ddt, f32, T * H, "ddt"), _t(dA, f32, H, "dA"),
            _t(dB, f32, T * G * N, "dB"), _t(dC, f32, T * G * N, "dC"),
            _t(dD, f32, H, "dD", optional=True), _state(dinit, dims, "dinit"))
    if int(workspace_bytes) > _bytes(workspace):
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "byte count exceeds its buffer")
    cu = _cu(cu_seqlens, dims)
    (px, pdt, pA, pB, pC, pD, phi, pcu, pdy, pdf, pdx, pddt, pdA, pdB, pdC, pdD, pdi,
     pws) = _ptrs(x, dt, A, B, C, D, hi, cu, *outs, workspace)
    _check(_lib.ssd_chunk_scan_bwd(px, pdt, pA, pB, pC, pD, phi, pcu, pdy, pdf, pdx, pddt, pdA,
                                   pdB, pdC, pdD, pdi, ctypes.byref(dims), pws,
                                   int(workspace_bytes), _stream(stream)))


def check_cu_seqlens(cu_host, T: int) -> None:
    """Host-side check of packed-batch offsets (a host copy of cu_seqlens):
    cu[0] == 0, non-decreasing, cu[-1] == T.  The kernels never leave their
    buffers on malformed offsets, but the results would be wrong without an
    error; this turns that case into SSDInvalidArgument."""
    c = [int(v) for v in cu_host]
    if not c or c[0] != 0 or c[-1] != int(T) or any(b < a for a, b in zip(c, c[1:])):
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG,
                                 "cu_seqlens must start at 0, not decrease and end at T")


def _raw_ptr(t: Optional[torch.Tensor], offset_elems: int = 0):
    """Device address of t's storage start + offset (t may be a strided view)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "tensor is not on the GPU")
    return ctypes.c_void_p(t.data_ptr() + offset_elems * t.element_size()) if t.numel() else None


def _span_ok(t: torch.Tensor, rows: int, stride: int, channels: int, name: str) -> None:
    """rows of `stride` elements starting at t's first element, of which the
    first `channels` are used, must lie inside t's storage."""
    if rows == 0:
        return
    need = (rows - 1) * stride + channels
    have = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if need > have:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, f"{name} is smaller than its rows span")


def ssd_conv1d_silu(inp, in_stride, weight, bias, kernel_width, out, out_stride, batch, seqlen,
                    nseq, cu_seqlens, channels, io_dtype, stream=None) -> None:
    """inp / out: tensors whose first element is channel 0 of token 0 (row
    strides given in elements, so they may be column slices of wider rows)."""
    io = torch.bfloat16 if io_dtype == SSD_BF16 else torch.float32
    T = int(seqlen) if int(nseq) > 0 else int(batch) * int(seqlen)
    for t, name, stride in ((inp, "inp", in_stride), (out, "out", out_stride)):
        if t is None:
            if T:
                raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, f"{name} is required")
            continue
        if t.dtype != io:
            raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, f"{name} must be {io}, got {t.dtype}")
        _span_ok(t, T, int(stride), int(channels), name)
    C, K = int(channels), int(kernel_width)
    cu = None
    if int(nseq) > 0:
        cu = _t(cu_seqlens, torch.int32, int(nseq) + 1, "cu_seqlens")
    elif cu_seqlens is not None:
        raise SSDInvalidArgument(SSD_ERR_INVALID_ARG, "cu_seqlens given without nseq")
    pw, pb, pcu = _ptrs(_t(weight, torch.float32, C * K, "weight"),
                        _t(bias, torch.float32, C, "bias", optional=True), cu)
    _check(_lib.ssd_conv1d_silu(_raw_ptr(inp), int(in_stride), pw, pb, K, _raw_ptr(out),
                                int(out_stride), int(batch), int(seqlen), int(nseq), pcu, C,
                                int(io_dtype), _stream(stream)))


def ssd_gate_rmsnorm(y, z, weight, eps, out, tokens, width, io_dtype, stream=None) -> None:
    io = torch.bfloat16 if io_dtype == SSD_BF16 else torch.float32
    n = int(tokens) * int(width)
    py, pz, pw, po = _ptrs(_t(y, io, n, "y"), _t(z, io, n, "z"),
                           _t(weight, torch.float32, int(width), "weight", optional=True),
                           _t(out, io, n, "out"))
    _check(_lib.ssd_gate_rmsnorm(py, pz, pw, float(eps), po, int(tokens), int(width),
                                 int(io_dtype), _stream(stream)))
