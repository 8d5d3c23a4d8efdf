"""libssd C ABI on the host (no GPU): the library loads, exports every entry
point declared in include/ssd.h, computes the documented workspace layout, and
rejects bad arguments with the documented status before touching the GPU.

Only invalid calls are made here, so nothing reaches a kernel launch.
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

libssd = pytest.importorskip("mamba_ssd_layer_amd.libssd")
from mamba_ssd_layer_amd.libssd import (SSD_BF16, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED,  # noqa: E402
                                        SSD_ERR_WORKSPACE, SSD_F32, SSD_OK, make_dims)

L = libssd.lib()
FAKE = 0x7f0000000000  # aligned, never dereferenced: validation fails first


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = header_functions()
    assert "ssd_chunk_scan_fwd" in names and len(names) >= 9
    for n in names:
        assert hasattr(L, n), f"libssd.so does not export {n}"
    assert set(names) == set(libssd.EXPORTS)


def test_version_and_status_strings():
    text = open(HEADER).read()
    ver = int(re.search(r"#define SSD_VERSION (\d+)", text).group(1))
    assert libssd.ssd_version() == ver
    for s in range(5):
        assert libssd.ssd_status_string(s)
    assert libssd.ssd_status_string(SSD_OK) == "ok"
    assert libssd.ssd_status_string(99) == "unknown status"


def _ws_expected(batch, L_, H, P, N, G, Q, nseq=0, io=2):
    al = lambda v: (v + 255) // 256 * 256
    if nseq:
        nc = math.ceil(L_ / Q) + nseq
    else:
        nc = batch * math.ceil(L_ / Q)
    off = al(nc * H * Q * 4)
    off = al(off + nc * H * Q * 4)
    off = al(off + nc * H * P * N * io)  # chunk states, io precision
    off = al(off + nc * H * P * N * io)  # hprev
    if nseq:
        off = al(off + nc * 16)
        off = al(off + (nseq + 2) * 4)
    return nc, max(off, 256)


@pytest.mark.parametrize("case", [
    (8, 4096, 80, 64, 128, 1, 256, 0, SSD_BF16),
    (4, 2048, 24, 64, 128, 1, 256, 0, SSD_BF16),
    (1, 65536, 80, 64, 256, 1, 256, 0, SSD_BF16),
    (1, 275772, 64, 64, 128, 8, 256, 64, SSD_BF16),
    (1, 256, 4, 16, 16, 1, 64, 0, SSD_F32),
    (3, 1000, 2, 64, 64, 2, 128, 0, SSD_BF16),
    (2, 300, 4, 32, 48, 2, 64, 0, SSD_BF16),      # bf16 on the vector-ALU kernels
])
def test_workspace_layout(case):
    b, L_, H, P, N, G, Q, nseq, io = case
    d = make_dims(b, L_, H, P, N, G, nseq, io)
    lay = libssd.ssd_get_workspace_layout(d, Q)
    nc, total = _ws_expected(b, L_, H, P, N, G, Q, nseq, 2 if io == SSD_BF16 else 4)
    assert lay.nc_max == nc
    assert lay.total_bytes == total == libssd.ssd_workspace_size(d, Q)
    offs = [lay.acum_offset, lay.dtq_offset, lay.states_offset, lay.hprev_offset]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    if nseq:
        assert lay.hprev_offset < lay.chunk_table_offset < lay.chunk_dir_offset < lay.total_bytes


def test_varlen_chunk_bound_covers_every_split():
    # sum over sequences of ceil(len/Q) never exceeds ceil(T/Q) + nseq
    import numpy as np
    r = np.random.default_rng(0)
    for _ in range(200):
        nseq = int(r.integers(1, 50))
        lens = r.integers(0, 700, nseq)
        Q = int(r.choice([64, 128, 256]))
        T = int(lens.sum())
        assert sum(math.ceil(l / Q) for l in lens) <= math.ceil(T / Q) + nseq


def fwd(dims, Q=256, x=FAKE, dt=FAKE, A=FAKE, B=FAKE + (1 << 30), C=FAKE + (2 << 30), D=None,
        init=None, cu=None, y=FAKE + (3 << 30), fin=None, ws=FAKE + (4 << 30), wsb=None):
    if wsb is None:
        wsb = L.ssd_workspace_size(ctypes.byref(dims), Q)
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.ssd_chunk_scan_fwd(v(x), v(dt), v(A), v(B), v(C), v(D), Q, v(init), v(cu), v(y),
                                v(fin), ctypes.byref(dims), v(ws), wsb, None)


def good():
    return make_dims(2, 512, 4, 64, 64, 1, 0, SSD_BF16)


@pytest.mark.parametrize("mut,expect", [
    (dict(batch=0), SSD_ERR_INVALID_ARG),
    (dict(seqlen=-1), SSD_ERR_INVALID_ARG),
    (dict(nheads=0), SSD_ERR_INVALID_ARG),
    (dict(ngroups=3), SSD_ERR_UNSUPPORTED),          # 4 % 3 != 0
    (dict(nseq=2), SSD_ERR_INVALID_ARG),             # packed needs batch == 1
    (dict(io_dtype=7), SSD_ERR_INVALID_ARG),
    (dict(reserved=1), SSD_ERR_INVALID_ARG),
    (dict(headdim=72), SSD_ERR_UNSUPPORTED),          # not a multiple of 16
    (dict(headdim=272), SSD_ERR_UNSUPPORTED),         # above 256
    (dict(dstate=40), SSD_ERR_UNSUPPORTED),
    (dict(dstate=512), SSD_ERR_UNSUPPORTED),
    (dict(nheads=70000, ngroups=1), SSD_ERR_UNSUPPORTED),
])
def test_bad_dims(mut, expect):
    d = good()
    for k, v in mut.items():
        setattr(d, k, v)
    wsb = 1 << 40
    assert fwd(d, wsb=wsb) == expect


@pytest.mark.parametrize("P,N", [(16, 16), (32, 64), (48, 128), (96, 32), (112, 256), (64, 48),
                                 (128, 16), (240, 80)])
def test_bf16_vector_path_shapes_are_accepted(P, N):
    # bf16 head dims and state sizes outside the MFMA kernels' set (P a
    # multiple of 64 with N in {64, 128, 256}) run on the vector-ALU stage
    # kernels: every multiple of 16 up to 256 is a valid shape
    d = make_dims(2, 300, 4, P, N, 2, 0, SSD_BF16)
    for Q in (64, 128, 256):
        assert L.ssd_workspace_size(ctypes.byref(d), Q) > 0


@pytest.mark.parametrize("Q,expect", [(32, SSD_ERR_UNSUPPORTED), (100, SSD_ERR_UNSUPPORTED),
                                      (512, SSD_ERR_UNSUPPORTED), (0, SSD_ERR_INVALID_ARG),
                                      (-64, SSD_ERR_INVALID_ARG)])
def test_bad_chunk_len(Q, expect):
    assert fwd(good(), Q=Q, wsb=1 << 40) == expect


def test_null_and_misaligned_pointers():
    d = good()
    assert fwd(d, x=None) == SSD_ERR_INVALID_ARG
    assert fwd(d, dt=None) == SSD_ERR_INVALID_ARG
    assert fwd(d, A=None) == SSD_ERR_INVALID_ARG
    assert fwd(d, B=None) == SSD_ERR_INVALID_ARG
    assert fwd(d, C=None) == SSD_ERR_INVALID_ARG
    assert fwd(d, y=None) == SSD_ERR_INVALID_ARG
    assert fwd(d, x=FAKE + 8) == SSD_ERR_INVALID_ARG       # x needs 16-byte alignment
    assert fwd(d, dt=FAKE + 2) == SSD_ERR_INVALID_ARG
    assert fwd(d, init=FAKE + (5 << 30) + 4) == SSD_ERR_INVALID_ARG
    assert fwd(d, ws=FAKE + (4 << 30) + 16) == SSD_ERR_INVALID_ARG  # workspace: 256 bytes


def test_workspace_checks():
    d = good()
    need = L.ssd_workspace_size(ctypes.byref(d), 256)
    assert need > 0
    assert fwd(d, wsb=need - 1) == SSD_ERR_WORKSPACE
    assert fwd(d, ws=None) == SSD_ERR_WORKSPACE


def test_overlaps_rejected():
    d = good()
    xbytes = 2 * 512 * 4 * 64 * 2
    assert fwd(d, y=FAKE) == SSD_ERR_INVALID_ARG                 # y == x
    assert fwd(d, y=FAKE + xbytes - 16) == SSD_ERR_INVALID_ARG   # y tail overlaps x
    sb = 2 * 4 * 64 * 64 * 4
    base = FAKE + (6 << 30)
    assert fwd(d, init=base, fin=base + 256) == SSD_ERR_INVALID_ARG   # partial overlap
    # final_state == init_state is allowed; with a too-small workspace the call
    # still stops before any launch, proving the aliasing check passed
    assert fwd(d, init=base, fin=base, wsb=16) == SSD_ERR_WORKSPACE
    assert fwd(d, init=base, fin=base + sb, wsb=16) == SSD_ERR_WORKSPACE


def test_packed_needs_cu_seqlens():
    d = make_dims(1, 1000, 4, 64, 64, 2, 3, SSD_BF16)
    assert fwd(d, cu=None, wsb=1 << 40) == SSD_ERR_INVALID_ARG
    assert fwd(d, cu=FAKE + (7 << 30), wsb=16) == SSD_ERR_WORKSPACE


def test_per_stage_entry_points_validate():
    d = good()
    v = ctypes.c_void_p
    dp = ctypes.byref(d)
    assert L.ssd_chunk_cumsum(None, v(FAKE), 256, None, dp, v(FAKE), 1 << 40, None) == SSD_ERR_INVALID_ARG
    assert L.ssd_chunk_state(v(FAKE), None, 256, dp, v(FAKE), 1 << 40, None) == SSD_ERR_INVALID_ARG
    assert L.ssd_state_passing(v(FAKE + 4), None, 256, dp, v(FAKE), 1 << 40, None) == SSD_ERR_INVALID_ARG
    assert L.ssd_chunk_scan(v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 256, dp, v(FAKE), 1 << 40,
                            None) == SSD_ERR_INVALID_ARG   # y == x
    assert L.ssd_chunk_scan(v(FAKE), v(FAKE), v(FAKE), None, v(FAKE + (3 << 30)), 256, dp,
                            v(FAKE), 16, None) == SSD_ERR_WORKSPACE


def test_layout_rejects_like_fwd():
    d = good()
    d.headdim = 56  # not a multiple of 16
    with pytest.raises(libssd.SSDUnsupported):
        libssd.ssd_get_workspace_layout(d, 256)
    assert libssd.ssd_workspace_size(d, 256) == 0
    d = good()
    with pytest.raises(libssd.SSDUnsupported):
        libssd.ssd_get_workspace_layout(d, 96)


# ---------------------------------------------------------------- ssd_step
def step(d, **kw):
    """ssd_step with distinct, aligned fake pointers 1 GiB apart (overridable)."""
    v = ctypes.c_void_p
    args = dict(x=FAKE, dt=FAKE + (1 << 30), A=FAKE + (2 << 30), B=FAKE + (3 << 30),
                C=FAKE + (4 << 30), D=None, state=FAKE + (5 << 30), y=FAKE + (7 << 30))
    args.update(kw)
    return L.ssd_step(*(None if args[k] is None else v(args[k])
                        for k in ("x", "dt", "A", "B", "C", "D", "state", "y")),
                      ctypes.byref(d), None)


def good_step():
    return make_dims(4, 1, 8, 64, 128, 2, 0, SSD_BF16)


def test_step_dims():
    d = good_step(); d.seqlen = 2
    assert step(d) == SSD_ERR_INVALID_ARG          # one token per sequence
    d = good_step(); d.nseq = 3
    assert step(d) == SSD_ERR_INVALID_ARG
    d = good_step(); d.ngroups = 3
    assert step(d) == SSD_ERR_UNSUPPORTED          # G must divide H
    d = good_step(); d.dstate = 96
    assert step(d) == SSD_ERR_UNSUPPORTED
    d = good_step(); d.io_dtype = 7
    assert step(d) == SSD_ERR_INVALID_ARG
    d = good_step(); d.batch = 0
    assert step(d, x=None, dt=None, B=None, C=None, state=None, y=None) == SSD_OK  # nothing to do


def test_step_pointers():
    d = good_step()
    for k in ("x", "dt", "A", "B", "C", "state", "y"):
        assert step(d, **{k: None}) == SSD_ERR_INVALID_ARG, k
    assert step(d, x=FAKE + 8) == SSD_ERR_INVALID_ARG
    assert step(d, state=FAKE + (5 << 30) + 4) == SSD_ERR_INVALID_ARG
    assert step(d, D=FAKE + (6 << 30) + 2) == SSD_ERR_INVALID_ARG


def test_step_overlaps():
    d = good_step()
    sb = 4 * 8 * 64 * 128 * 4
    assert step(d, y=FAKE) == SSD_ERR_INVALID_ARG                      # y == x
    assert step(d, state=FAKE + (3 << 30)) == SSD_ERR_INVALID_ARG      # state == B
    assert step(d, y=FAKE + (5 << 30) + sb - 16) == SSD_ERR_INVALID_ARG  # y inside the state
    assert step(d, A=FAKE + (5 << 30) + 64) == SSD_ERR_INVALID_ARG     # A inside the state


# ---------------------------------------------------------------- block neighbours
def conv(**kw):
    v = ctypes.c_void_p
    a = dict(inp=FAKE, in_stride=64, weight=FAKE + (1 << 30), bias=None, K=4, out=FAKE + (2 << 30),
             out_stride=64, batch=2, seqlen=100, nseq=0, cu=None, channels=64, io=SSD_BF16)
    a.update(kw)
    pv = lambda x: None if x is None else v(x)
    return L.ssd_conv1d_silu(pv(a["inp"]), a["in_stride"], pv(a["weight"]), pv(a["bias"]), a["K"],
                             pv(a["out"]), a["out_stride"], a["batch"], a["seqlen"], a["nseq"],
                             pv(a["cu"]), a["channels"], a["io"], None)


def test_conv1d_validation():
    assert conv(K=0) == SSD_ERR_INVALID_ARG
    assert conv(K=5) == SSD_ERR_UNSUPPORTED
    assert conv(channels=60) == SSD_ERR_INVALID_ARG           # bf16: multiple of 8
    assert conv(in_stride=32) == SSD_ERR_INVALID_ARG          # stride < channels
    assert conv(out_stride=68) == SSD_ERR_INVALID_ARG         # not a multiple of 8
    assert conv(weight=None) == SSD_ERR_INVALID_ARG
    assert conv(inp=FAKE + 8) == SSD_ERR_INVALID_ARG          # 16-byte alignment
    assert conv(out=FAKE + 64) == SSD_ERR_INVALID_ARG         # out overlaps in
    assert conv(nseq=3, batch=2) == SSD_ERR_INVALID_ARG       # packed needs batch 1
    assert conv(nseq=3, batch=1, cu=None) == SSD_ERR_INVALID_ARG
    assert conv(io=5) == SSD_ERR_INVALID_ARG
    assert conv(seqlen=0, inp=None, out=None) == SSD_OK       # nothing to do
    assert conv(io=SSD_F32, channels=36, in_stride=36, out_stride=36, seqlen=0) == SSD_OK


def test_gate_rmsnorm_validation():
    v = ctypes.c_void_p
    g = lambda y=FAKE, z=FAKE + (1 << 30), w=None, eps=1e-5, out=FAKE + (2 << 30), T=10, W=64, io=SSD_BF16: \
        L.ssd_gate_rmsnorm(None if y is None else v(y), None if z is None else v(z),
                           None if w is None else v(w), eps, None if out is None else v(out), T, W, io, None)
    assert g(W=60) == SSD_ERR_INVALID_ARG
    assert g(eps=-1.0) == SSD_ERR_INVALID_ARG
    assert g(eps=float("nan")) == SSD_ERR_INVALID_ARG
    assert g(y=None) == SSD_ERR_INVALID_ARG
    assert g(out=FAKE + 16) == SSD_ERR_INVALID_ARG     # partial overlap with y
    assert g(w=FAKE + (3 << 30) + 2) == SSD_ERR_INVALID_ARG
    assert g(T=0, y=None, z=None, out=None) == SSD_OK


# ---------------------------------------------------------------- ssd_fused_fwd
def fused(d, **kw):
    """ssd_fused_fwd with distinct, aligned fake pointers 1 GiB apart (overridable)."""
    v = ctypes.c_void_p
    args = dict(x=FAKE, dt=FAKE + (1 << 30), A=FAKE + (2 << 30), B=FAKE + (3 << 30),
                C=FAKE + (4 << 30), D=None, init=None, cu=None, y=FAKE + (7 << 30),
                fin=FAKE + (5 << 30))
    args.update(kw)
    return L.ssd_fused_fwd(*(None if args[k] is None else v(args[k])
                             for k in ("x", "dt", "A", "B", "C", "D", "init", "cu", "y", "fin")),
                           ctypes.byref(d), None)


@pytest.mark.parametrize("mut,expect", [
    (dict(io_dtype=SSD_F32), SSD_ERR_UNSUPPORTED),    # bf16 only
    (dict(headdim=32), SSD_ERR_UNSUPPORTED),          # head dim a multiple of 64
    (dict(headdim=96), SSD_ERR_UNSUPPORTED),
    (dict(headdim=320), SSD_ERR_UNSUPPORTED),         # at most 256
    (dict(dstate=32), SSD_ERR_UNSUPPORTED),           # N in {64, 128, 256}
    (dict(ngroups=3), SSD_ERR_UNSUPPORTED),           # 4 % 3 != 0
    (dict(reserved=1), SSD_ERR_INVALID_ARG),
    (dict(batch=-1), SSD_ERR_INVALID_ARG),
])
def test_fused_dims(mut, expect):
    d = good()
    for k, val in mut.items():
        setattr(d, k, val)
    assert fused(d) == expect
    assert L.ssd_fused_states_size(ctypes.byref(d)) == 0


@pytest.mark.parametrize("mut", [
    dict(),
    dict(headdim=128), dict(headdim=192), dict(headdim=256),   # heads split into 64-row halves
    dict(dstate=128), dict(dstate=256),
    dict(ngroups=4),                                          # one head per group
    dict(nheads=6, ngroups=2),                                # three heads per group
])
def test_fused_supported_shapes(mut):
    # host-only: a supported shape has a nonzero saved-state size (no launch here)
    d = good()
    for k, val in mut.items():
        setattr(d, k, val)
    n = L.ssd_fused_states_size(ctypes.byref(d))
    pairs = d.batch * -(-d.seqlen // 64)
    assert n == -(-(pairs * d.nheads * d.headdim * d.dstate * 2) // 256) * 256
    # the chunked forward takes the same shapes
    assert L.ssd_workspace_size(ctypes.byref(d), 256) > 0


@pytest.mark.parametrize("mut,ok", [
    (dict(), True), (dict(dstate=128), True),
    (dict(dstate=256), True), (dict(dstate=32), False), (dict(headdim=128), False),
    (dict(ngroups=4), False), (dict(nheads=6, ngroups=2), False),
])
def test_backward_shapes(mut, ok):
    d = good()
    for k, val in mut.items():
        setattr(d, k, val)
    assert (L.ssd_fused_bwd_workspace_size(ctypes.byref(d)) > 0) == ok


def test_fused_pointers_and_overlaps():
    d = good()
    for k in ("x", "dt", "A", "B", "C", "y"):
        assert fused(d, **{k: None}) == SSD_ERR_INVALID_ARG, k
    assert fused(d, x=FAKE + 8) == SSD_ERR_INVALID_ARG               # 16-byte alignment
    assert fused(d, init=FAKE + (6 << 30) + 4) == SSD_ERR_INVALID_ARG
    assert fused(d, y=FAKE) == SSD_ERR_INVALID_ARG                   # y == x
    assert fused(d, y=FAKE + (3 << 30) + 64) == SSD_ERR_INVALID_ARG  # y over B
    base = FAKE + (6 << 30)
    assert fused(d, init=base, fin=base + 256) == SSD_ERR_INVALID_ARG  # partial state overlap
    dp = make_dims(1, 1000, 4, 64, 64, 2, 3, SSD_BF16)
    assert fused(dp, cu=None) == SSD_ERR_INVALID_ARG                 # packed needs cu_seqlens


# ------------------------------------------- ssd_fused_fwd_train, ssd_fused_bwd
def test_fused_states_size():
    # bf16 [npairs][H][P][N], npairs = batch * ceil(L / 64), rounded up to 256 bytes
    d = good()  # 2 x 512 tokens, H 4, P 64, N 64
    assert L.ssd_fused_states_size(ctypes.byref(d)) == 2 * 8 * 4 * 64 * 64 * 2
    d = make_dims(3, 1000, 4, 64, 128, 2, 0, SSD_BF16)
    assert L.ssd_fused_states_size(ctypes.byref(d)) == 3 * 16 * 4 * 64 * 128 * 2
    dp = make_dims(1, 1000, 4, 64, 64, 2, 3, SSD_BF16)  # packed: ceil(T / 64) + nseq
    assert L.ssd_fused_states_size(ctypes.byref(dp)) == (16 + 3) * 4 * 64 * 64 * 2
    # the backward's workspace: the state gradients like the states; with few
    # (sequence, head pair) blocks (here 3 x 2) also two fp32 tiles and a decay
    # per 256-token segment and head (ceil(1000 / 256) + 3 segments)
    nseg = 4 + 3
    ws = (16 + 3) * 4 * 64 * 64 * 2 + 2 * nseg * 4 * 64 * 64 * 4 + 256
    assert L.ssd_fused_bwd_workspace_size(ctypes.byref(dp)) == ws
    big = make_dims(8, 4096, 80, 64, 128, 1, 0, SSD_BF16)  # 8 x 40 blocks: one pass per sequence
    assert L.ssd_fused_bwd_workspace_size(ctypes.byref(big)) == 8 * 64 * 80 * 64 * 128 * 2
    # one 65,536-token sequence, 80 heads (40 head pairs): segments of 2048
    # tokens, the longest power of two giving at least 1024 (segment, head pair)
    # blocks (4096 would give 640); packed, ceil(T / 2048) + nseq segments
    per = lambda nseg, N: 2 * nseg * 80 * 64 * N * 4 + -(-(nseg * 80 * 4) // 256) * 256
    ln = make_dims(1, 65536, 80, 64, 128, 1, 0, SSD_BF16)
    assert L.ssd_fused_bwd_workspace_size(ctypes.byref(ln)) == 1024 * 80 * 64 * 128 * 2 + per(32, 128)
    lp = make_dims(1, 65536, 80, 64, 64, 1, 2, SSD_BF16)
    assert L.ssd_fused_bwd_workspace_size(ctypes.byref(lp)) == \
        (1024 + 2) * 80 * 64 * 64 * 2 + per(32 + 2, 64)
    # N 256: the workspace of an N 128 backward (two halves run in turn), then
    # one half's B, C, d(final), ddt, dB, dC, d(init) (the second half adds its
    # dx into the first's as it writes it)
    d = good()  # 2 x 512 tokens, H 4, P 64, G 1
    d.dstate = 256
    T, H, P, rows = 1024, 4, 64, 2
    nseg = 2 * 2
    half = 2 * 8 * H * P * 128 * 2 + 2 * nseg * H * P * 128 * 4 + 256
    extra = (2 * T * 128 * 2 + rows * H * P * 128 * 4
             + T * H * 4 + 2 * T * 128 * 4 + rows * H * P * 128 * 4)
    assert L.ssd_fused_bwd_workspace_size(ctypes.byref(d)) == half + extra
    for mut, fwd_ok in ((dict(io_dtype=SSD_F32), False), (dict(headdim=128), True),
                        (dict(ngroups=4), True)):
        d = good()
        for k, val in mut.items():
            setattr(d, k, val)
        assert (L.ssd_fused_states_size(ctypes.byref(d)) > 0) == fwd_ok
        assert L.ssd_fused_bwd_workspace_size(ctypes.byref(d)) == 0  # outside the backward's shapes


def fused_train(d, states=FAKE + (8 << 30), nbytes=None, **kw):
    v = ctypes.c_void_p
    args = dict(x=FAKE, dt=FAKE + (1 << 30), A=FAKE + (2 << 30), B=FAKE + (3 << 30),
                C=FAKE + (4 << 30), D=None, init=None, cu=None, y=FAKE + (7 << 30),
                fin=FAKE + (5 << 30))
    args.update(kw)
    if nbytes is None:
        nbytes = L.ssd_fused_states_size(ctypes.byref(d))
    return L.ssd_fused_fwd_train(*(None if args[k] is None else v(args[k])
                                   for k in ("x", "dt", "A", "B", "C", "D", "init", "cu", "y",
                                             "fin")),
                                 None if states is None else v(states), ctypes.c_size_t(nbytes),
                                 ctypes.byref(d), None)


def test_fused_train_validation():
    d = good()
    need = L.ssd_fused_states_size(ctypes.byref(d))
    assert fused_train(d, nbytes=need - 1) == SSD_ERR_WORKSPACE
    assert fused_train(d, states=FAKE + (8 << 30) + 8) == SSD_ERR_INVALID_ARG  # alignment
    assert fused_train(d, states=FAKE + (7 << 30)) == SSD_ERR_INVALID_ARG      # over y
    assert fused_train(d, states=FAKE + 4096) == SSD_ERR_INVALID_ARG           # over x
    assert fused_train(d, x=None) == SSD_ERR_INVALID_ARG
    d.dstate = 32
    assert fused_train(d) == SSD_ERR_UNSUPPORTED


BWD_ARGS = ("x", "dt", "A", "B", "C", "D", "cu", "states", "dy", "dfinal", "dx", "ddt", "dA",
            "dB", "dC", "dD", "dinit")


def fused_bwd(d, sbytes=None, ws=FAKE + (20 << 30), wbytes=None, **kw):
    v = ctypes.c_void_p
    args = {k: FAKE + (i << 30) for i, k in enumerate(BWD_ARGS)}
    args.update(D=None, dD=None, cu=None, dfinal=None, dinit=None)
    args.update(kw)
    sbytes = L.ssd_fused_states_size(ctypes.byref(d)) if sbytes is None else sbytes
    wbytes = L.ssd_fused_bwd_workspace_size(ctypes.byref(d)) if wbytes is None else wbytes
    ptrs = [None if args[k] is None else v(args[k]) for k in BWD_ARGS]
    return L.ssd_fused_bwd(*ptrs[:8], ctypes.c_size_t(sbytes), *ptrs[8:], ctypes.byref(d),
                           None if ws is None else v(ws), ctypes.c_size_t(wbytes), None)


def test_fused_bwd_validation():
    d = good()
    sneed = L.ssd_fused_states_size(ctypes.byref(d))
    wneed = L.ssd_fused_bwd_workspace_size(ctypes.byref(d))
    for k in ("x", "dt", "A", "B", "C", "dy", "dx", "ddt", "dA", "dB", "dC", "states"):
        assert fused_bwd(d, **{k: None}) == SSD_ERR_INVALID_ARG, k
    assert fused_bwd(d, sbytes=sneed - 1) == SSD_ERR_WORKSPACE
    assert fused_bwd(d, wbytes=wneed - 1) == SSD_ERR_WORKSPACE
    assert fused_bwd(d, ws=None) == SSD_ERR_WORKSPACE
    assert fused_bwd(d, dD=FAKE + (21 << 30)) == SSD_ERR_INVALID_ARG         # dD without D
    assert fused_bwd(d, D=FAKE + (21 << 30)) == SSD_ERR_INVALID_ARG          # D without dD
    assert fused_bwd(d, dx=FAKE + 64) == SSD_ERR_INVALID_ARG                 # dx over x
    assert fused_bwd(d, dB=FAKE + (10 << 30)) == SSD_ERR_INVALID_ARG         # dB over dx
    assert fused_bwd(d, dinit=FAKE + (20 << 30)) == SSD_ERR_INVALID_ARG      # over workspace
    assert fused_bwd(d, dB=FAKE + (13 << 30) + 8) == SSD_ERR_INVALID_ARG     # alignment
    dp = make_dims(1, 1000, 4, 64, 64, 2, 3, SSD_BF16)
    assert fused_bwd(dp) == SSD_ERR_INVALID_ARG                              # packed needs cu
    d.io_dtype = SSD_F32
    assert fused_bwd(d) == SSD_ERR_UNSUPPORTED


# ---------------------------------------------------------------- ssd_chunk_scan_fwd_noalloc
def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define SSD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == libssd.NOALLOC_SCRATCH_BYTES


def noalloc(d, Q=256, **kw):
    v = ctypes.c_void_p
    args = dict(x=FAKE, dt=FAKE + (1 << 30), A=FAKE + (2 << 30), B=FAKE + (3 << 30),
                C=FAKE + (4 << 30), D=None, init=None, cu=None, y=FAKE + (7 << 30), fin=None)
    args.update(kw)
    a = [None if args[k] is None else v(args[k]) for k in ("x", "dt", "A", "B", "C", "D")]
    b = [None if args[k] is None else v(args[k]) for k in ("init", "cu", "y", "fin")]
    return L.ssd_chunk_scan_fwd_noalloc(*a, Q, *b, ctypes.byref(d), None)


def test_noalloc_validates_before_any_hip_call():
    # beyond the scratch array: refused (the large layer's ~350 MB workspace)
    big = make_dims(8, 4096, 80, 64, 128, 1, 0, SSD_BF16)
    assert L.ssd_workspace_size(ctypes.byref(big), 256) > libssd.NOALLOC_SCRATCH_BYTES
    assert noalloc(big) == SSD_ERR_WORKSPACE
    # the same argument checks as the workspace forward
    d = good()
    assert noalloc(d, x=None) == SSD_ERR_INVALID_ARG
    assert noalloc(d, y=FAKE) == SSD_ERR_INVALID_ARG               # y == x
    assert noalloc(d, Q=100) == SSD_ERR_UNSUPPORTED
    d.ngroups = 3
    assert noalloc(d) == SSD_ERR_UNSUPPORTED


def _split_ws(b, L, H, P, N, S):
    al = lambda v: (v + 255) // 256 * 256
    nseg = -(-L // S)
    if nseg <= 1:
        return 0
    hr = P // 64 if P % 64 == 0 else 1
    Hk, Pk = H * hr, P // hr
    return al(b * nseg * Hk * Pk * N * 4) + al(b * (nseg - 1) * Hk * 4)


@pytest.mark.parametrize("case", [(1, 65536, 80, 64, 128, 1024), (8, 4096, 80, 64, 128, 1024),
                                  (2, 1000, 4, 128, 64, 256), (3, 100, 2, 64, 256, 32),
                                  (2, 500, 4, 64, 64, 512)])
def test_split_workspace_size(case):
    b, L_, H, P, N, S = case
    d = make_dims(b, L_, H, P, N, 1, 0, SSD_BF16)
    assert L.ssd_fused_split_workspace_size(ctypes.byref(d), S) == _split_ws(b, L_, H, P, N, S)


def test_split_validates_before_any_hip_call():
    v = ctypes.c_void_p
    d = make_dims(2, 1000, 4, 64, 64, 1, 0, SSD_BF16)
    dp = ctypes.byref(d)
    need = L.ssd_fused_split_workspace_size(dp, 256)
    args = lambda S, ws, wsb, y=FAKE + (3 << 30): L.ssd_fused_fwd_split(
        v(FAKE), v(FAKE + (5 << 30)), v(FAKE + (6 << 30)), v(FAKE + (1 << 30)),
        v(FAKE + (2 << 30)), None, None, v(y), None, S, dp, v(ws), wsb, None)
    assert args(0, FAKE + (4 << 30), need) == SSD_ERR_INVALID_ARG      # seg_len 0
    assert args(100, FAKE + (4 << 30), need) == SSD_ERR_INVALID_ARG    # not a multiple of 32
    assert args(256, FAKE + (4 << 30), need - 1) == SSD_ERR_WORKSPACE  # too small
    assert args(256, 0, need) == SSD_ERR_WORKSPACE                    # missing
    assert args(256, FAKE + (4 << 30) + 16, need) == SSD_ERR_INVALID_ARG  # misaligned
    assert args(256, FAKE + (4 << 30), need, y=FAKE) == SSD_ERR_INVALID_ARG  # y == x
    assert args(256, FAKE, need) == SSD_ERR_INVALID_ARG                # workspace over x
    # packed sequences are not split; f32 io and P 32 are outside the one-pass shapes
    dpk = make_dims(1, 1000, 4, 64, 64, 1, 3, SSD_BF16)
    assert L.ssd_fused_fwd_split(v(FAKE), v(FAKE + (5 << 30)), v(FAKE + (6 << 30)),
                                 v(FAKE + (1 << 30)), v(FAKE + (2 << 30)), None, None,
                                 v(FAKE + (3 << 30)), None, 256, ctypes.byref(dpk),
                                 v(FAKE + (4 << 30)), 1 << 40, None) == SSD_ERR_UNSUPPORTED
    for dd in (make_dims(2, 1000, 4, 64, 64, 1, 0, SSD_F32), make_dims(2, 1000, 4, 32, 64, 1, 0,
                                                                       SSD_BF16)):
        assert L.ssd_fused_fwd_split(v(FAKE), v(FAKE + (5 << 30)), v(FAKE + (6 << 30)),
                                     v(FAKE + (1 << 30)), v(FAKE + (2 << 30)), None, None,
                                     v(FAKE + (3 << 30)), None, 256, ctypes.byref(dd),
                                     v(FAKE + (4 << 30)), 1 << 40, None) == SSD_ERR_UNSUPPORTED


def test_split_train_validates_before_any_hip_call():
    v = ctypes.c_void_p
    d = make_dims(2, 1000, 4, 64, 64, 1, 0, SSD_BF16)
    dp = ctypes.byref(d)
    need = L.ssd_fused_split_workspace_size(dp, 256)
    hb = L.ssd_fused_states_size(dp)
    ST = FAKE + (8 << 30)
    args = lambda S=256, st=ST, stb=hb, wsb=need: L.ssd_fused_fwd_split_train(
        v(FAKE), v(FAKE + (5 << 30)), v(FAKE + (6 << 30)), v(FAKE + (1 << 30)),
        v(FAKE + (2 << 30)), None, None, v(FAKE + (3 << 30)), None, v(st), stb, S, dp,
        v(FAKE + (4 << 30)), wsb, None)
    assert args(st=0) == SSD_ERR_INVALID_ARG              # the states are required
    assert args(S=96, wsb=1 << 30) == SSD_ERR_INVALID_ARG  # a multiple of 32, not of 64
    assert args(stb=hb - 1) == SSD_ERR_WORKSPACE           # states buffer too small
    assert args(st=ST + 8) == SSD_ERR_INVALID_ARG          # misaligned
    assert args(st=FAKE + (4 << 30)) == SSD_ERR_INVALID_ARG  # over the workspace
    assert args(st=FAKE + (3 << 30)) == SSD_ERR_INVALID_ARG  # over y


def _gbwd_ws(b, L_, H, P, N, G, nseq, io):
    al = lambda v: (v + 255) // 256 * 256
    nc, fwd_total = _ws_expected(b, L_, H, P, N, G, 64, nseq, io)
    tile = al(nc * H * P * N * 4)
    return al(fwd_total) + 2 * tile


@pytest.mark.parametrize("case", [(1, 256, 4, 16, 16, 1, 0, SSD_F32), (2, 1000, 4, 64, 256, 2, 0, SSD_BF16),
                                  (1, 700, 4, 32, 64, 2, 6, SSD_BF16), (8, 4096, 80, 64, 128, 1, 0, SSD_BF16)])
def test_general_bwd_workspace_size(case):
    b, L_, H, P, N, G, nseq, io = case
    d = make_dims(b, L_, H, P, N, G, nseq, io)
    got = L.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(d))
    assert got == _gbwd_ws(b, L_, H, P, N, G, nseq, 2 if io == SSD_BF16 else 4)


def test_general_bwd_validates_before_any_hip_call():
    v = ctypes.c_void_p
    d = make_dims(2, 300, 4, 32, 48, 2, 0, SSD_BF16)
    dp = ctypes.byref(d)
    need = L.ssd_chunk_scan_bwd_workspace_size(dp)
    assert need > 0
    F = lambda k: v(FAKE + (k << 30))
    base = dict(x=F(0), dt=F(1), A=F(2), B=F(3), C=F(4), D=None, init=None, cu=None, dy=F(5),
                dfinal=None, dx=F(6), ddt=F(7), dA=F(8), dB=F(9), dC=F(10), dD=None, dinit=None,
                ws=F(11), wsb=need)

    def call(**kw):
        a = dict(base, **kw)
        return L.ssd_chunk_scan_bwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"],
                                    a["cu"], a["dy"], a["dfinal"], a["dx"], a["ddt"], a["dA"],
                                    a["dB"], a["dC"], a["dD"], a["dinit"], dp, a["ws"], a["wsb"],
                                    None)
    assert call(wsb=need - 1) == SSD_ERR_WORKSPACE
    assert call(ws=None) == SSD_ERR_WORKSPACE
    assert call(ws=v(FAKE + (11 << 30) + 64)) == SSD_ERR_INVALID_ARG   # misaligned
    assert call(dx=None) == SSD_ERR_INVALID_ARG
    assert call(dA=None) == SSD_ERR_INVALID_ARG
    assert call(dD=F(12)) == SSD_ERR_INVALID_ARG                       # dD without D
    assert call(dx=F(0)) == SSD_ERR_INVALID_ARG                        # dx over x
    assert call(dB=F(10)) == SSD_ERR_INVALID_ARG                       # dB over dC
    assert call(ws=F(6)) == SSD_ERR_INVALID_ARG                        # workspace over dx
    bad = make_dims(2, 300, 4, 40, 48, 2, 0, SSD_BF16)                 # head dim 40
    assert L.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(bad)) == 0
