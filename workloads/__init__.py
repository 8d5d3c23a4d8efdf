"""Seeded synthetic inputs for the SSD chunked-scan forward.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It only draws random numbers and lays them out; it holds none of the
SSD arithmetic (no decay, no scan, no contraction).  Both sides receive the
exact same values: for bf16 workloads every x, B, C element is rounded to a
bf16-representable float32 here (round-to-nearest-even), so the oracle's fp64
upcast and the GPU's bf16 tensors hold identical numbers.

Canonical host layout (all C-contiguous, token-major):
  x  [T, H, P]   float32 (bf16-exact for bf16 workloads)
  dt [T, H]      float32, already positive (the op takes dt as given)
  A  [H]         float32
  B  [T, G, N]   float32 (bf16-exact for bf16 workloads)
  C  [T, G, N]   float32 (bf16-exact for bf16 workloads)
  D  [H]         float32
  h0 [nseq, H, P, N] float32 or None
  seq_off [nseq + 1] int64 token offsets (fixed-length batches: b * L)
T is the total token count (batch * L for fixed-length batches).

Distributions (Mamba-2 style parameterisation; the pages put softplus on dt and
a negative exponential on A, "Mamba-2 Architecture: State Space Duality
Explained", Step 2):
  x ~ N(0, 1); dt = softplus(z - shift), z ~ N(0, 1), shift 2 (3 for the long
  context workloads); A = -exp(U(0, ln 16)); B, C ~ N(0, 1) / sqrt(N);
  D ~ N(0, 1); h0 = 0, except the packed variable-length workload, where
  h0 ~ N(0, 0.1^2).  Draw order: [lengths] -> x -> z -> A -> B -> C -> D -> [h0].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "make_workload", "make_custom", "make_output_grads", "bf16_round_",
    "bf16_bits", "describe",
]

_SLAB = 1 << 24  # elements per generation / rounding slab (bounds temporaries)


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str            # "f32" or "bf16"
    seed: int
    dt_shift: float = 2.0
    nseq: int = 0         # > 0: packed variable-length batch with this many sequences
    max_len: int = 0      # varlen: lengths ~ U[1, max_len]
    init_std: float = 0.0  # > 0: nonzero initial state ~ N(0, init_std^2)
    description: str = ""


# The seeded workloads.  Names say what they are; sizes are in the fields.
WORKLOADS = {
    s.name: s for s in [
        Spec("tiny_f32", 1, 256, 4, 16, 16, 1, 64, "f32", 0,
             description="tiny fp32 SSD forward, B1 L256 H4 P16 N16 G1 Q64"),
        Spec("small_bf16", 4, 2048, 24, 64, 128, 1, 256, "bf16", 1000,
             description="small Mamba-2 layer, B4 L2048 H24 P64 N128 G1 Q256, bf16"),
        Spec("large_bf16", 8, 4096, 80, 64, 128, 1, 256, "bf16", 2000,
             description="large Mamba-2 layer, B8 L4096 H80 P64 N128 G1 Q256, bf16"),
        Spec("long_n64", 1, 65536, 80, 64, 64, 1, 256, "bf16", 3000, dt_shift=3.0,
             description="long context, B1 L65536 H80 P64 N64 G1 Q256, bf16"),
        Spec("long_n128", 1, 65536, 80, 64, 128, 1, 256, "bf16", 3001, dt_shift=3.0,
             description="long context, B1 L65536 H80 P64 N128 G1 Q256, bf16"),
        Spec("long_n256", 1, 65536, 80, 64, 256, 1, 256, "bf16", 3002, dt_shift=3.0,
             description="long context, B1 L65536 H80 P64 N256 G1 Q256, bf16"),
        Spec("varlen_bf16", 1, 0, 64, 64, 128, 8, 256, "bf16", 4000, nseq=64,
             max_len=8192, init_std=0.1,
             description="packed varlen, 64 seqs len U[1,8192], H64 P64 N128 G8 Q256, "
                         "h0 ~ N(0, 0.1^2), bf16"),
    ]
}


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    chunk: int
    batch: int            # fixed-length rows (1 for varlen)
    seqlen: int           # L for fixed-length; total tokens T for varlen
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    nseq: int             # 0 for fixed-length batches
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: Optional[np.ndarray]
    h0: Optional[np.ndarray]
    seq_off: np.ndarray   # int64 [nseq_or_batch + 1]
    cu_seqlens: Optional[np.ndarray]  # int32 [nseq + 1] for varlen, else None

    @property
    def tokens(self) -> int:
        return int(self.seq_off[-1])

    @property
    def nsequences(self) -> int:
        return len(self.seq_off) - 1


def bf16_round_(a: np.ndarray) -> np.ndarray:
    """Round a float32 array in place to the nearest bf16 value (ties to even).

    Works on the bit pattern: add 0x7FFF plus the lowest kept bit, clear the low
    16 bits.  Inputs here are finite, so no NaN/Inf handling is needed.
    """
    assert a.dtype == np.float32 and a.flags.c_contiguous
    u = a.reshape(-1).view(np.uint32)
    for lo in range(0, u.size, _SLAB):
        s = u[lo:lo + _SLAB]
        s += np.uint32(0x7FFF) + ((s >> np.uint32(16)) & np.uint32(1))
        s &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of a bf16-exact float32 array."""
    assert a.dtype == np.float32
    u = np.ascontiguousarray(a).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal32(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for lo in range(0, n, _SLAB):
        hi = min(n, lo + _SLAB)
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)
    return out.reshape(shape)


def _softplus64(z: np.ndarray) -> np.ndarray:
    # log(1 + e^z), written to stay finite for large |z|
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def make_custom(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                ngroups: int, chunk: int, dtype: str, seed: int, *,
                dt_shift: float = 2.0, lens=None, init_std: float = 0.0,
                with_D: bool = True, name: str = "custom",
                a_log_range=(0.0, math.log(16.0)), dt_const: Optional[float] = None,
                a_zero: bool = False) -> Workload:
    """Draw one seeded workload.

    lens: if given, a packed variable-length batch with these sequence lengths
    (batch must be 1 and seqlen is ignored).  a_log_range: A = -exp(U(lo, hi)).
    dt_const / a_zero: overrides for long-memory stress inputs.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    if lens is not None:
        lens = np.asarray(lens, dtype=np.int64)
        if batch != 1:
            raise ValueError("packed variable-length batches have batch == 1")
        seq_off = np.zeros(len(lens) + 1, dtype=np.int64)
        np.cumsum(lens, out=seq_off[1:])
        T = int(seq_off[-1])
        nseq = len(lens)
        L = T
    else:
        T = batch * seqlen
        seq_off = np.arange(batch + 1, dtype=np.int64) * seqlen
        nseq = 0
        L = seqlen
    H, P, N, G = nheads, headdim, dstate, ngroups
    x = _normal32(rng, (T, H, P))
    z = rng.standard_normal((T, H))
    if dt_const is not None:
        dt = np.full((T, H), dt_const, dtype=np.float32)
    else:
        dt = _softplus64(z - dt_shift).astype(np.float32)
    A = (-np.exp(rng.uniform(a_log_range[0], a_log_range[1], H))).astype(np.float32)
    if a_zero:
        A[:] = 0.0
    Bm = _normal32(rng, (T, G, N))
    Cm = _normal32(rng, (T, G, N))
    scale = np.float32(1.0 / math.sqrt(N))
    Bm *= scale
    Cm *= scale
    D = rng.standard_normal(H).astype(np.float32)
    if not with_D:
        D = None
    h0 = None
    nrows = nseq if nseq else batch
    if init_std > 0.0:
        h0 = (_normal32(rng, (nrows, H, P, N)) * np.float32(init_std)).astype(np.float32)
    if dtype == "bf16":
        bf16_round_(x)
        bf16_round_(Bm)
        bf16_round_(Cm)
    cu = seq_off.astype(np.int32) if nseq else None
    return Workload(name=name, dtype=dtype, chunk=chunk, batch=batch if not nseq else 1,
                    seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G, nseq=nseq,
                    x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, h0=h0, seq_off=seq_off,
                    cu_seqlens=cu)


def make_output_grads(w: Workload, seed: int, dfinal_std: float = 1.0):
    """Seeded upstream gradients for a backward pass over w: dy [T, H, P] ~
    N(0, 1) (bf16-exact for bf16 workloads) and dfinal [rows, H, P, N] ~
    N(0, dfinal_std^2) float32 (None when dfinal_std is 0).  Draw order: dy ->
    dfinal."""
    rng = np.random.default_rng(seed)
    dy = _normal32(rng, (w.tokens, w.nheads, w.headdim))
    if w.dtype == "bf16":
        bf16_round_(dy)
    dfinal = None
    if dfinal_std > 0.0:
        dfinal = (_normal32(rng, (w.nsequences, w.nheads, w.headdim, w.dstate)) *
                  np.float32(dfinal_std)).astype(np.float32)
    return dy, dfinal


def make_workload(name: str) -> Workload:
    """The seeded workload of that name (see WORKLOADS)."""
    s = WORKLOADS[name]
    if s.nseq:
        return _make_varlen(s)
    return make_custom(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups,
                       s.chunk, s.dtype, s.seed, dt_shift=s.dt_shift,
                       init_std=s.init_std, name=s.name)


def _make_varlen(s: Spec) -> Workload:
    # One stream: lengths first, then the tensors in the documented order.
    rng = np.random.default_rng(s.seed)
    lens2 = rng.integers(1, s.max_len + 1, s.nseq)
    seq_off = np.zeros(s.nseq + 1, dtype=np.int64)
    np.cumsum(lens2, out=seq_off[1:])
    T = int(seq_off[-1])
    H, P, N, G = s.nheads, s.headdim, s.dstate, s.ngroups
    x = _normal32(rng, (T, H, P))
    z = rng.standard_normal((T, H))
    dt = _softplus64(z - s.dt_shift).astype(np.float32)
    A = (-np.exp(rng.uniform(0.0, math.log(16.0), H))).astype(np.float32)
    Bm = _normal32(rng, (T, G, N))
    Cm = _normal32(rng, (T, G, N))
    scale = np.float32(1.0 / math.sqrt(N))
    Bm *= scale
    Cm *= scale
    D = rng.standard_normal(H).astype(np.float32)
    h0 = (_normal32(rng, (s.nseq, H, P, N)) * np.float32(s.init_std)).astype(np.float32)
    bf16_round_(x)
    bf16_round_(Bm)
    bf16_round_(Cm)
    return Workload(name=s.name, dtype=s.dtype, chunk=s.chunk, batch=1, seqlen=T,
                    nheads=H, headdim=P, dstate=N, ngroups=G, nseq=s.nseq, x=x, dt=dt,
                    A=A, B=Bm, C=Cm, D=D, h0=h0, seq_off=seq_off,
                    cu_seqlens=seq_off.astype(np.int32))


def describe(w: Workload) -> dict:
    return {"workload": w.name, "tokens": w.tokens, "batch": w.batch,
            "seqlen": w.seqlen if not w.nseq else None, "nseq": w.nseq or None,
            "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate,
            "ngroups": w.ngroups, "chunk": w.chunk, "dtype": w.dtype}
