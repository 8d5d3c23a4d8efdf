"""mamba_ssd_layer_amd -- Mamba-2 SSD chunked-scan forward on AMD MI355X.

The compute lives in libssd.so (HIP kernels for gfx950 behind the C ABI of
include/ssd.h).  This package is its Python face:

  libssd             ctypes binding, same names as the C entry points
  chunk_scan_fwd()   convenience wrapper: infers the dims from torch tensors,
                     allocates y / final_state / workspace, runs the forward
  SSDForward         a reusable plan (fixed dims, workspace allocated once)
  fused_fwd()        the same forward in one pass per (sequence, head), no workspace
                     (bf16, head dim 64 / 128 / 192 / 256, dstate 64 / 128 / 256)
  step()             one recurrent decode step per sequence, state updated in place
  conv1d_silu()      the causal depthwise conv1d + SiLU before the core
  gate_rmsnorm()     y * SiLU(z), then RMS norm over the channel width, after it

Tensors (GPU, contiguous):
  x [B, L, H, P]   dt [B, L, H] float32   A [H] float32   B, C [B, L, G, N]
  D [H] float32 or None   init_state [B, H, P, N] float32 or None
For a packed variable-length batch pass cu_seqlens (int32 [nseq + 1], GPU),
B = 1 (the leading dim may be dropped), and init_state [nseq, H, P, N].
x, B, C and y are bfloat16 or float32 (all the same).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import libssd
from .libssd import (SSD_BF16, SSD_F32, SSDError, SSDInvalidArgument, SSDUnsupported,
                     SSDWorkspaceError, make_dims)

__all__ = ["libssd", "chunk_scan_fwd", "SSDForward", "SSDTrainForward", "SSDError", "SSDInvalidArgument",
           "SSDUnsupported", "SSDWorkspaceError", "make_dims", "dims_for", "validate_cu_seqlens", "step",
           "conv1d_silu", "gate_rmsnorm", "fused_fwd", "fused_fwd_split", "fused_split_seg_len",
           "make_fused_states", "fused_bwd", "chunk_scan_bwd"]


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG, f"unsupported dtype {t.dtype}")


def validate_cu_seqlens(cu_seqlens: Optional[torch.Tensor], tokens: int) -> None:
    """Checks packed-batch offsets on the host (0 first, non-decreasing, the
    token count last) and raises SSDInvalidArgument otherwise.  The kernels
    stay inside their buffers on malformed offsets but would return wrong
    results without an error.  A tensor is copied to the host (one
    synchronisation) only the first time it is seen in its current version
    (torch bumps a tensor's version on every in-place write, also through
    another view); the mark lives on the tensor object and dies with it."""
    if cu_seqlens is None:
        return
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG, "cu_seqlens must be 1-D int32")
    mark = (cu_seqlens._version, int(tokens))
    if getattr(cu_seqlens, "_libssd_checked", None) == mark:
        return
    libssd.check_cu_seqlens(cu_seqlens.cpu().tolist(), tokens)
    cu_seqlens._libssd_checked = mark


def dims_for(x: torch.Tensor, B: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None):
    """ssd_dims from tensor shapes (see the module docstring)."""
    if cu_seqlens is not None:
        if x.dim() == 4:
            if x.shape[0] != 1:
                raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG,
                                         "packed batches have a leading dim of 1")
            _, T, H, P = x.shape
        else:
            T, H, P = x.shape
        G, N = B.shape[-2], B.shape[-1]
        nseq = cu_seqlens.numel() - 1
        return make_dims(1, T, H, P, N, G, nseq, _io_dtype(x))
    if x.dim() != 4 or B.dim() != 4:
        raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG, "x and B must be 4-D")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return make_dims(b, L, H, P, N, G, 0, _io_dtype(x))


class SSDForward:
    """A plan for one set of dims: the workspace is allocated once and every
    call enqueues the four stages on the current stream."""

    def __init__(self, dims, chunk_len: int, device="cuda"):
        self.dims = dims
        self.chunk_len = int(chunk_len)
        self.layout = libssd.ssd_get_workspace_layout(dims, chunk_len)
        self.workspace = torch.empty(self.layout.total_bytes, dtype=torch.uint8, device=device)
        self.nrows = dims.nseq if dims.nseq > 0 else dims.batch

    def __call__(self, x, dt, A, B, C, D=None, init_state=None, cu_seqlens=None, y=None,
                 final_state=None, want_final: bool = True, stream=None):
        if cu_seqlens is not None:
            validate_cu_seqlens(cu_seqlens, self.dims.seqlen)
        if y is None:
            y = torch.empty_like(x)
        if final_state is None and want_final:
            final_state = torch.empty((self.nrows, self.dims.nheads, self.dims.headdim,
                                       self.dims.dstate), dtype=torch.float32, device=x.device)
        libssd.ssd_chunk_scan_fwd(x, dt, A, B, C, D, self.chunk_len, init_state, cu_seqlens, y,
                                  final_state, self.dims, self.workspace, stream)
        return y, final_state

    # per-stage calls on the plan's workspace (for checks and timing)
    def cumsum(self, dt, A, cu_seqlens=None, stream=None):
        if cu_seqlens is not None:
            validate_cu_seqlens(cu_seqlens, self.dims.seqlen)
        libssd.ssd_chunk_cumsum(dt, A, self.chunk_len, cu_seqlens, self.dims, self.workspace,
                                stream)

    def state(self, x, B, stream=None):
        libssd.ssd_chunk_state(x, B, self.chunk_len, self.dims, self.workspace, stream)

    def passing(self, init_state, final_state, stream=None):
        libssd.ssd_state_passing(init_state, final_state, self.chunk_len, self.dims,
                                 self.workspace, stream)

    def scan(self, x, B, C, D, y, stream=None):
        libssd.ssd_chunk_scan(x, B, C, D, y, self.chunk_len, self.dims, self.workspace, stream)

    def saved_states(self) -> torch.Tensor:
        """The hprev buffer of the workspace as bytes: with chunk_len 64 and bf16
        io it holds, after a call, the state entering every 64-token chunk in the
        layout fused_bwd takes as chunk_states (the chunk-parallel way to get
        them for a few long sequences)."""
        if self.chunk_len != 64 or self.dims.io_dtype != SSD_BF16:
            raise SSDUnsupported(libssd.SSD_ERR_UNSUPPORTED,
                                 "saved states need chunk_len 64 and bf16 io")
        n = libssd.ssd_fused_states_size(self.dims)
        if n == 0:
            raise SSDUnsupported(libssd.SSD_ERR_UNSUPPORTED, "shape outside the one-pass forward")
        off = self.layout.hprev_offset
        return self.workspace[off:off + n]

    def view(self, name: str) -> torch.Tensor:
        """A typed view of one workspace buffer (acum, dtq, states, hprev,
        chunk_table, chunk_dir) in its documented shape.  acum and dtq hold
        one row per kernel head: with bf16 and a head dim of 64 r, head h
        runs as the r kernel heads h r .. h r + r - 1 (the same values)."""
        d, L, Q = self.dims, self.layout, self.chunk_len
        nc, H, P, N = L.nc_max, d.nheads, d.headdim, d.dstate
        Hk = (L.dtq_offset - L.acum_offset) // (nc * Q * 4) if nc else H  # kernel heads
        ws = self.workspace
        io = torch.bfloat16 if d.io_dtype == SSD_BF16 else torch.float32  # states and hprev

        def sl(off, n, dtype):
            nbytes = n * torch.tensor([], dtype=dtype).element_size()
            return ws[off:off + nbytes].view(dtype)

        if name == "acum":
            return sl(L.acum_offset, nc * Hk * Q, torch.float32).view(nc, Hk, Q)
        if name == "dtq":
            return sl(L.dtq_offset, nc * Hk * Q, torch.float32).view(nc, Hk, Q)
        if name == "states":
            return sl(L.states_offset, nc * H * P * N, io).view(nc, H, P, N)
        if name == "hprev":
            return sl(L.hprev_offset, nc * H * P * N, io).view(nc, H, P, N)
        if name == "chunk_table":
            return sl(L.chunk_table_offset, nc * 4, torch.int32).view(nc, 4)
        if name == "chunk_dir":
            return sl(L.chunk_dir_offset, d.nseq + 2, torch.int32)
        raise KeyError(name)


class SSDTrainForward:
    """The chunk-parallel forward for training: y and the final state from the
    four stages at chunk length 256 (head-batched kernels), and the state
    entering every 64-token chunk -- what fused_bwd takes as chunk_states --
    from the first three stages at chunk length 64 (the same kernels, bit for
    bit the hprev a chunk-64 forward leaves).  For few long sequences, where
    the one-pass forward has too few (sequence, head) blocks.  bf16 io."""

    def __init__(self, dims, device="cuda"):
        self.p256 = SSDForward(dims, 256, device=device)
        self.p64 = SSDForward(dims, 64, device=device)

    def __call__(self, x, dt, A, B, C, D=None, init_state=None, cu_seqlens=None, y=None,
                 final_state=None, want_final: bool = True, stream=None):
        """y, final_state, chunk_states (a view of this plan's workspace, valid
        until the next call)."""
        y, final_state = self.p256(x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state,
                                   want_final, stream)
        self.p64.cumsum(dt, A, cu_seqlens, stream)
        self.p64.state(x, B, stream)
        self.p64.passing(init_state, None, stream)
        return y, final_state, self.p64.saved_states()


def chunk_scan_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                   C: torch.Tensor, D: Optional[torch.Tensor] = None, chunk_len: int = 256,
                   init_state: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """y, final_state = SSD forward (allocates outputs and a workspace)."""
    dims = dims_for(x, B, cu_seqlens)
    plan = SSDForward(dims, chunk_len, device=x.device)
    return plan(x, dt, A, B, C, D, init_state, cu_seqlens)


def fused_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
              C: torch.Tensor, D: Optional[torch.Tensor] = None,
              init_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None, want_final: bool = True,
              chunk_states: Optional[torch.Tensor] = None,
              stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """y, final_state = SSD forward in one pass per (sequence, head) (ssd_fused_fwd:
    bf16, head dim 64 / 128 / 192 / 256, dstate 64 / 128 / 256; no workspace).  Same arguments and
    results as chunk_scan_fwd.  With chunk_states (a uint8 device buffer of
    fused_states_bytes(...) bytes, see make_fused_states) it also saves the
    state entering every 64-token chunk for fused_bwd (ssd_fused_fwd_train)."""
    dims = dims_for(x, B, cu_seqlens)
    if cu_seqlens is not None:
        validate_cu_seqlens(cu_seqlens, dims.seqlen)
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and want_final:
        nrows = dims.nseq if dims.nseq > 0 else dims.batch
        final_state = torch.empty((nrows, dims.nheads, dims.headdim, dims.dstate),
                                  dtype=torch.float32, device=x.device)
    if chunk_states is None:
        libssd.ssd_fused_fwd(x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state, dims,
                             stream)
    else:
        libssd.ssd_fused_fwd_train(x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state,
                                   chunk_states, chunk_states.numel() * chunk_states.element_size(),
                                   dims, stream)
    return y, final_state


def fused_split_seg_len(x: torch.Tensor, B: torch.Tensor) -> int:
    """The library's segment length for fused_fwd_split on this device (the
    sequence length rounded up to 32, i.e. no split, when sequences x heads
    already fill the GPU)."""
    return libssd.ssd_fused_split_seg_len(dims_for(x, B, None))


def fused_fwd_split(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                    C: torch.Tensor, D: Optional[torch.Tensor] = None,
                    init_state: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                    final_state: Optional[torch.Tensor] = None, want_final: bool = True,
                    seg_len: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                    chunk_states: Optional[torch.Tensor] = None,
                    stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """y, final_state = the one-pass forward over segments of seg_len tokens
    (ssd_fused_fwd_split: fixed-length batches; a state-only pass, the
    hand-off between segments, then every segment from its entering state).
    Same arguments and results as fused_fwd without cu_seqlens.  seg_len
    defaults to fused_split_seg_len; workspace (uint8, device) is allocated
    when not given.  chunk_states (from make_fused_states; seg_len a multiple
    of 64): also save the state entering every 64-token pair for fused_bwd
    (ssd_fused_fwd_split_train)."""
    dims = dims_for(x, B, None)
    if seg_len is None:
        seg_len = libssd.ssd_fused_split_seg_len(dims)
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and want_final:
        final_state = torch.empty((dims.batch, dims.nheads, dims.headdim, dims.dstate),
                                  dtype=torch.float32, device=x.device)
    need = libssd.ssd_fused_split_workspace_size(dims, seg_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if chunk_states is not None:
        libssd.ssd_fused_fwd_split_train(x, dt, A, B, C, D, init_state, y, final_state,
                                         chunk_states, chunk_states.numel(), seg_len, dims,
                                         workspace, stream)
    else:
        libssd.ssd_fused_fwd_split(x, dt, A, B, C, D, init_state, y, final_state, seg_len, dims,
                                   workspace, stream)
    return y, final_state


def make_fused_states(x: torch.Tensor, B: torch.Tensor,
                      cu_seqlens: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A device byte buffer for fused_fwd's saved chunk states."""
    dims = dims_for(x, B, cu_seqlens)
    n = libssd.ssd_fused_states_size(dims)
    if n == 0:
        raise SSDUnsupported(libssd.SSD_ERR_UNSUPPORTED, "shape outside the one-pass forward")
    return torch.empty(n, dtype=torch.uint8, device=x.device)


def fused_bwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
              C: torch.Tensor, D: Optional[torch.Tensor], chunk_states: torch.Tensor,
              dy: torch.Tensor, dfinal: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, want_dinit: bool = True,
              workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of fused_fwd (ssd_fused_bwd) for the loss
    sum <dy, y> + sum <dfinal, final_state>, given the chunk states fused_fwd
    saved for the same inputs.  Returns a dict with dx (like x, bf16), ddt
    (like dt, float32), dA [H], dB and dC (float32, shaped like B and C),
    dD [H] (None when D is None) and dinit [rows, H, P, N] (None unless
    want_dinit)."""
    dims = dims_for(x, B, cu_seqlens)
    if cu_seqlens is not None:
        validate_cu_seqlens(cu_seqlens, dims.seqlen)
    dev = x.device
    nrows = dims.nseq if dims.nseq > 0 else dims.batch
    if workspace is None:
        n = libssd.ssd_fused_bwd_workspace_size(dims)
        if n == 0:
            raise SSDUnsupported(libssd.SSD_ERR_UNSUPPORTED,
                                 "shape outside the backward's (bf16, head dim 64, N 64, 128 or 256, "
                                 "an even number of heads per group)")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    out = dict(dx=torch.empty_like(x), ddt=torch.empty(dt.shape, dtype=torch.float32, device=dev),
               dA=torch.empty(dims.nheads, dtype=torch.float32, device=dev),
               dB=torch.empty(B.shape, dtype=torch.float32, device=dev),
               dC=torch.empty(C.shape, dtype=torch.float32, device=dev),
               dD=torch.empty(dims.nheads, dtype=torch.float32, device=dev) if D is not None else None,
               dinit=torch.empty((nrows, dims.nheads, dims.headdim, dims.dstate),
                                 dtype=torch.float32, device=dev) if want_dinit else None)
    libssd.ssd_fused_bwd(x, dt, A, B, C, D, cu_seqlens, chunk_states,
                         chunk_states.numel() * chunk_states.element_size(), dy, dfinal,
                         out["dx"], out["ddt"], out["dA"], out["dB"], out["dC"], out["dD"],
                         out["dinit"], dims, workspace, workspace.numel(), stream)
    return out


def chunk_scan_bwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                   C: torch.Tensor, D: Optional[torch.Tensor], dy: torch.Tensor,
                   dfinal: Optional[torch.Tensor] = None,
                   init_state: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, want_dinit: bool = True,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of chunk_scan_fwd (ssd_chunk_scan_bwd: every shape the
    forward takes, fp32 or bf16; no saved states, the chunk states are formed
    again) for the loss sum <dy, y> + sum <dfinal, final_state>.  Returns the
    same dict as fused_bwd (dx like x)."""
    dims = dims_for(x, B, cu_seqlens)
    if cu_seqlens is not None:
        validate_cu_seqlens(cu_seqlens, dims.seqlen)
    dev = x.device
    nrows = dims.nseq if dims.nseq > 0 else dims.batch
    if workspace is None:
        n = libssd.ssd_chunk_scan_bwd_workspace_size(dims)
        if n == 0:
            raise SSDUnsupported(libssd.SSD_ERR_UNSUPPORTED, "shape outside the forward's")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    out = dict(dx=torch.empty_like(x), ddt=torch.empty(dt.shape, dtype=torch.float32, device=dev),
               dA=torch.empty(dims.nheads, dtype=torch.float32, device=dev),
               dB=torch.empty(B.shape, dtype=torch.float32, device=dev),
               dC=torch.empty(C.shape, dtype=torch.float32, device=dev),
               dD=torch.empty(dims.nheads, dtype=torch.float32, device=dev) if D is not None else None,
               dinit=torch.empty((nrows, dims.nheads, dims.headdim, dims.dstate),
                                 dtype=torch.float32, device=dev) if want_dinit else None)
    libssd.ssd_chunk_scan_bwd(x, dt, A, B, C, D, init_state, cu_seqlens, dy, dfinal, out["dx"],
                              out["ddt"], out["dA"], out["dB"], out["dC"], out["dD"],
                              out["dinit"], dims, workspace, workspace.numel(), stream)
    return out


def step(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
         state: torch.Tensor, D: Optional[torch.Tensor] = None,
         y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step (ssd_step): x [S, H, P], dt [S, H], B/C [S, G, N],
    state [S, H, P, N] float32 (updated in place).  Returns y [S, H, P]."""
    if x.dim() != 3 or B.dim() != 3 or state.dim() != 4:
        raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG,
                                 "x [S,H,P], B/C [S,G,N], state [S,H,P,N] expected")
    S, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dims = make_dims(S, 1, H, P, N, G, 0, _io_dtype(x))
    if y is None:
        y = torch.empty_like(x)
    libssd.ssd_step(x, dt, A, B, C, D, state, y, dims, stream)
    return y


def conv1d_silu(inp: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                cu_seqlens: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Causal depthwise conv1d (width weight.shape[1] <= 4) + SiLU over the token
    axis.  inp: [B, L, C] or (packed, with cu_seqlens) [T, C]; its last dim must
    be contiguous, and it may be a column slice of wider rows (x, B or C of a
    packed projection).  weight [C, K] float32, bias [C] float32 or None.
    Returns out (contiguous, same shape) unless given."""
    if inp.stride(-1) != 1:
        raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG, "channels must be contiguous")
    C = inp.shape[-1]
    if cu_seqlens is not None:
        if inp.dim() != 2:
            raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG, "packed inp must be [T, C]")
        T = inp.shape[0]
        batch, seqlen, nseq = 1, T, cu_seqlens.numel() - 1
        validate_cu_seqlens(cu_seqlens, T)
    else:
        if inp.dim() != 3:
            raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG, "inp must be [B, L, C]")
        batch, seqlen, nseq = inp.shape[0], inp.shape[1], 0
        if batch > 1 and inp.stride(0) != seqlen * inp.stride(1):
            raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG, "rows must be evenly strided")
    in_stride = inp.stride(-2)
    if out is None:
        out = torch.empty(inp.shape, dtype=inp.dtype, device=inp.device)
    libssd.ssd_conv1d_silu(inp, in_stride, weight, bias, weight.shape[1], out, out.stride(-2),
                           batch, seqlen, nseq, cu_seqlens, C, _io_dtype(inp), stream)
    return out


def gate_rmsnorm(y: torch.Tensor, z: torch.Tensor, weight: Optional[torch.Tensor] = None,
                 eps: float = 1e-5, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y * SiLU(z), then (with a weight) RMS norm over the last dim(s) of width
    `weight.numel()`: y and z [..., H, P] or [..., W], contiguous."""
    W = weight.numel() if weight is not None else y.shape[-1] * (y.shape[-2] if y.dim() >= 3 else 1)
    if y.numel() % W:
        raise SSDInvalidArgument(libssd.SSD_ERR_INVALID_ARG, "width does not divide the tensor")
    if out is None:
        out = torch.empty_like(y)
    libssd.ssd_gate_rmsnorm(y, z, weight, eps, out, y.numel() // W, W, _io_dtype(y), stream)
    return out
