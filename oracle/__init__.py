"""TEST INFRASTRUCTURE ONLY: the CPU oracle of the Mamba-2 SSD forward.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library (``mamba_ssd_layer_amd``)
never imports it, and it never imports the GPU library: the two share no code.
The only shared module is ``workloads`` (seeded random inputs, no SSD math).

Contents
  recurrence(...)   fp64 token-by-token recurrence, C + OpenMP (ssd_recurrence.c).
                    This is the oracle the GPU path is checked against.
  quadratic(...)    the attention-like dual Y = (L o C B^T) X, numpy fp64.
  chunked(...)      the blockwise algorithm (intra-chunk masked product, chunk
                    states, state hand-off, inter-chunk output), numpy fp64; it
                    also returns the per-chunk intermediates.
  recurrence_py(...) the same recurrence as plain numpy loops (tiny inputs).
  recurrence_bwd(...) fp64 gradients of the forward (dx, ddt, dA, dB, dC, dD,
                    dh0) by the chain rule through the recurrence, tokens in
                    reverse (C + OpenMP, ssd_recurrence_bwd.c).
  conv1d_silu(...), gate_rmsnorm(...), silu(...)
                    the core's neighbours in the Mamba-2 block (block.py): the
                    causal depthwise convolution + SiLU before it, the SiLU gate
                    and RMS normalisation after it, numpy fp64.

Nothing here is "parity unpinned": tests/test_oracle.py pins recurrence() to
hand-computed values, closed forms, the quadratic dual, the A = 0 linear
attention special case, chunk/split invariance, linearity, the rank bound and
brute force on tiny inputs; tests/test_oracle_block.py pins the block
neighbours to torch's own conv1d / silu / rms_norm in fp64 on the CPU (library
routines), to closed forms (width-1 kernel, shift kernels, zero gate) and to
the scale invariance of the normalisation; tests/test_oracle_bwd.py pins
recurrence_bwd() to the adjoint identity of the forward (exact for x, B, C, D,
h0 and the final-state seed, in which the forward is linear) and to central
finite differences of the forward for dt and A.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

from .reference import quadratic, chunked, recurrence_py  # noqa: F401
from .block import conv1d_silu, gate_rmsnorm, silu  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.ssd_oracle_recurrence.restype = ctypes.c_int
        lib.ssd_oracle_recurrence.argtypes = [i64, p, i64, i64, i64, i64, p, p, p, p, p, p,
                                              p, i64, p, p, p, ctypes.c_int]
        lib.ssd_oracle_recurrence_bwd.restype = ctypes.c_int
        lib.ssd_oracle_recurrence_bwd.argtypes = [i64, p, i64, i64, i64, i64, p, p, p, p, p, p,
                                                  p, p, p, i64, p, p, p, p, p, p, p, p,
                                                  ctypes.c_int]
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        lib.ssd_oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def recurrence(x: np.ndarray, dt: np.ndarray, A: np.ndarray, B: np.ndarray,
               C: np.ndarray, D: Optional[np.ndarray], h0: Optional[np.ndarray],
               seq_off: np.ndarray, pairs: Optional[Sequence[Tuple[int, int]]] = None,
               nthreads: int = 0):
    """fp64 recurrence over packed sequences.

    x [T,H,P], dt [T,H], A [H], B/C [T,G,N], D [H]|None, h0 [nseq,H,P,N]|None,
    seq_off [nseq+1] token offsets.  All float inputs float32 (upcast exactly).

    pairs=None: returns (y [T,H,P] float64, final [nseq,H,P,N] float64).
    pairs=[(s,h),...]: returns (list of y blocks [len_s, P], final [npairs,P,N]).
    """
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    dt = np.ascontiguousarray(dt, dtype=np.float32)
    A = np.ascontiguousarray(A, dtype=np.float32)
    B = np.ascontiguousarray(B, dtype=np.float32)
    C = np.ascontiguousarray(C, dtype=np.float32)
    D = None if D is None else np.ascontiguousarray(D, dtype=np.float32)
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float32)
    seq_off = np.ascontiguousarray(seq_off, dtype=np.int64)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    nseq = len(seq_off) - 1
    if int(seq_off[-1]) != T:
        raise ValueError("seq_off[-1] must equal the token count")
    lens = np.diff(seq_off)
    if pairs is None:
        pr = None
        np_ = nseq * H
        ytot = T * H * P
    else:
        pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        np_ = pr.shape[0]
        ytot = int(sum(lens[s] for s, _ in pr)) * P
    y = np.empty(ytot, dtype=np.float64)
    hf = np.empty((np_, P, N), dtype=np.float64)
    rc = lib.ssd_oracle_recurrence(nseq, _ptr(seq_off), H, P, N, G, _ptr(x), _ptr(dt),
                                   _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), np_,
                                   _ptr(pr), _ptr(y), _ptr(hf), int(nthreads))
    if rc != 0:
        raise ValueError("ssd_oracle_recurrence rejected its arguments")
    if pairs is None:
        # compact blocks are (s, h)-major [len_s, P]; scatter to [T, H, P]
        yfull = np.empty((T, H, P), dtype=np.float64)
        off = 0
        for s in range(nseq):
            n = int(lens[s])
            blk = y[off:off + n * H * P].reshape(H, n, P)
            yfull[seq_off[s]:seq_off[s + 1]] = blk.transpose(1, 0, 2)
            off += n * H * P
        return yfull, hf.reshape(nseq, H, P, N)
    out = []
    off = 0
    for s, _ in pr:
        n = int(lens[s])
        out.append(y[off:off + n * P].reshape(n, P))
        off += n * P
    return out, hf


def recurrence_bwd(x, dt, A, B, C, D, h0, seq_off, dy, dfinal=None, pairs=None,
                   nthreads: int = 0):
    """fp64 gradients of L = sum <dy_t, y_t> + <dfinal, final> through the
    recurrence (ssd_recurrence_bwd.c: the chain rule, tokens in reverse).

    Inputs as recurrence() plus dy [T,H,P] and dfinal [nseq,H,P,N] or None
    (all float32, upcast exactly).  Returns a dict of float64 arrays:
      dx [T,H,P], ddt [T,H], dB [T,G,N], dC [T,G,N] (summed over the heads of
      each group), dA [H], dD [H] (summed over sequences), dh0 [nseq,H,P,N].
    With pairs=[(s,h),...] only those pairs are computed: dx, ddt, dh0 hold
    them (zeros elsewhere), dB/dC hold only their heads' shares, and dA/dD
    become per-pair arrays [npairs].
    """
    lib = _load()
    f32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    x, dt, A, B, C, D, h0, dy, dfinal = (f32(a) for a in (x, dt, A, B, C, D, h0, dy, dfinal))
    seq_off = np.ascontiguousarray(seq_off, dtype=np.int64)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    nseq = len(seq_off) - 1
    if int(seq_off[-1]) != T or dy.shape != x.shape:
        raise ValueError("shapes")
    pr = None if pairs is None else np.ascontiguousarray(
        np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
    np_ = nseq * H if pr is None else pr.shape[0]
    dx = np.zeros((T, H, P))
    ddt = np.zeros((T, H))
    dBh = np.zeros((T, H, N))
    dCh = np.zeros((T, H, N))
    dA_p = np.zeros(np_)
    dD_p = np.zeros(np_)
    dh0_p = np.zeros((np_, P, N))
    rc = lib.ssd_oracle_recurrence_bwd(nseq, _ptr(seq_off), H, P, N, G, _ptr(x), _ptr(dt),
                                       _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(dy),
                                       _ptr(dfinal), np_, _ptr(pr), _ptr(dx), _ptr(ddt),
                                       _ptr(dBh), _ptr(dCh), _ptr(dA_p), _ptr(dD_p),
                                       _ptr(dh0_p), int(nthreads))
    if rc != 0:
        raise ValueError("ssd_oracle_recurrence_bwd rejected its arguments")
    grp = (np.arange(H) * G) // H
    dB = np.zeros((T, G, N))
    dC = np.zeros((T, G, N))
    for h in range(H):
        dB[:, grp[h]] += dBh[:, h]
        dC[:, grp[h]] += dCh[:, h]
    out = {"dx": dx, "ddt": ddt, "dB": dB, "dC": dC}
    if pr is None:
        out["dA"] = dA_p.reshape(nseq, H).sum(0)
        out["dD"] = dD_p.reshape(nseq, H).sum(0)
        out["dh0"] = dh0_p.reshape(nseq, H, P, N)
    else:
        out["dA"], out["dD"] = dA_p, dD_p
        dh0 = np.zeros((nseq, H, P, N))
        for k, (s, h) in enumerate(pr):
            dh0[s, h] = dh0_p[k]
        out["dh0"] = dh0
    return out


def recurrence_workload(w, pairs=None, nthreads: int = 0):
    """recurrence() on a workloads.Workload."""
    return recurrence(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off, pairs=pairs,
                      nthreads=nthreads)
