"""The Python binding's own checks, on the CPU (no GPU, no kernel launch).

The C entry points see only pointers, so the binding checks every tensor's
dtype and element count against the dims before it passes a pointer on: a
bf16 dt or an int64 cu_seqlens would otherwise make the kernels read past a
buffer or split the sequences wrongly.  These checks run before the
tensor's device is looked at, so CPU tensors exercise them here; a tensor
that passes them is then refused for not being on the GPU.
"""
import pytest
import torch

import mamba_ssd_layer_amd as ssd
from mamba_ssd_layer_amd import libssd

T_, H_, P_, N_, G_ = 6, 4, 16, 16, 2


def dims(nseq=0, io=libssd.SSD_F32):
    if nseq:
        return libssd.make_dims(1, T_, H_, P_, N_, G_, nseq, io)
    return libssd.make_dims(2, T_ // 2, H_, P_, N_, G_, 0, io)


def good(io=torch.float32, nseq=0):
    f = torch.float32
    t = dict(x=torch.zeros(T_, H_, P_, dtype=io), dt=torch.zeros(T_, H_, dtype=f),
             A=torch.zeros(H_, dtype=f), B=torch.zeros(T_, G_, N_, dtype=io),
             C=torch.zeros(T_, G_, N_, dtype=io), D=torch.zeros(H_, dtype=f),
             y=torch.zeros(T_, H_, P_, dtype=io),
             init=torch.zeros(max(nseq, 2), H_, P_, N_, dtype=f),
             fin=torch.zeros(max(nseq, 2), H_, P_, N_, dtype=f),
             cu=torch.tensor([0, 2, 6], dtype=torch.int32) if nseq else None,
             ws=torch.zeros(256, dtype=torch.uint8))
    return t


def call_fwd(t, d):
    libssd.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 64, t["init"],
                              t["cu"], t["y"], t["fin"], d, t["ws"])


def expect(msg, fn):
    with pytest.raises(libssd.SSDInvalidArgument, match=msg):
        fn()


def test_well_formed_arguments_reach_the_device_check():
    # everything right: the only complaint is that the tensors live on the CPU
    expect("not on the GPU", lambda: call_fwd(good(), dims()))
    expect("not on the GPU", lambda: call_fwd(good(nseq=2), dims(nseq=2)))


@pytest.mark.parametrize("name,bad,msg", [
    ("dt", torch.zeros(T_, H_, dtype=torch.bfloat16), "dt must be torch.float32"),
    ("dt", torch.zeros(T_ - 1, H_), "dt must hold"),
    ("A", torch.zeros(H_ + 1), "A must hold"),
    ("A", torch.zeros(H_, dtype=torch.float64), "A must be torch.float32"),
    ("D", torch.zeros(H_ - 1), "D must hold"),
    ("x", torch.zeros(T_, H_, P_, dtype=torch.bfloat16), "x must be torch.float32"),
    ("x", torch.zeros(T_, H_, P_ // 2), "x must hold"),
    ("B", torch.zeros(T_, G_, N_ + 16), "B must hold"),
    ("C", torch.zeros(T_, G_ + 1, N_), "C must hold"),
    ("C", None, "C is required"),
    ("y", torch.zeros(T_, H_, P_ - 1), "y must hold"),
    ("y", torch.zeros(T_, H_, P_, dtype=torch.float16), "y must be torch.float32"),
    ("init", torch.zeros(1, H_, P_, N_), "init_state must hold"),
    ("fin", torch.zeros(2, H_, P_, N_, dtype=torch.bfloat16), "final_state must be"),
])
def test_forward_rejects_wrong_dtype_or_size(name, bad, msg):
    t = good()
    t[name] = bad
    expect(msg, lambda: call_fwd(t, dims()))


def test_cu_seqlens_dtype_count_and_presence():
    t = good(nseq=2)
    t["cu"] = torch.tensor([0, 2, 6], dtype=torch.int64)  # what torch.cumsum returns
    expect("cu_seqlens must be torch.int32", lambda: call_fwd(t, dims(nseq=2)))
    t["cu"] = torch.tensor([0, 6], dtype=torch.int32)
    expect("cu_seqlens must hold 3", lambda: call_fwd(t, dims(nseq=2)))
    t["cu"] = None
    expect("cu_seqlens is required", lambda: call_fwd(t, dims(nseq=2)))
    t = good()
    t["cu"] = torch.tensor([0, 3, 6], dtype=torch.int32)
    expect("fixed-length", lambda: call_fwd(t, dims()))


@pytest.mark.parametrize("cu,ok", [
    ([0, 2, 6], True), ([0, 0, 6], True), ([0, 6, 6], True),
    ([1, 2, 6], False),   # does not start at 0
    ([0, 4, 3], False),   # ends below T, decreases
    ([0, 4, 2, 6], False),  # decreases in the middle
    ([0, 2, 7], False),   # ends past T
])
def test_cu_seqlens_values_checked_on_the_host(cu, ok):
    c = torch.tensor(cu, dtype=torch.int32)
    if ok:
        ssd.validate_cu_seqlens(c, 6)
        libssd.check_cu_seqlens(cu, 6)
    else:
        expect("cu_seqlens must start at 0", lambda: ssd.validate_cu_seqlens(c, 6))


def test_cu_seqlens_rechecked_after_an_in_place_write():
    c = torch.tensor([0, 2, 6], dtype=torch.int32)
    ssd.validate_cu_seqlens(c, 6)
    c[1] = 9  # bumps the tensor's version
    expect("cu_seqlens must start at 0", lambda: ssd.validate_cu_seqlens(c, 6))


def test_step_and_backward_check_their_tensors():
    f = torch.float32
    d = libssd.make_dims(3, 1, H_, P_, N_, G_, 0, libssd.SSD_F32)
    x = torch.zeros(3, H_, P_)
    st = torch.zeros(3, H_, P_, N_, dtype=torch.bfloat16)
    expect("state must be torch.float32",
           lambda: libssd.ssd_step(x, torch.zeros(3, H_), torch.zeros(H_), torch.zeros(3, G_, N_),
                                   torch.zeros(3, G_, N_), None, st, torch.zeros_like(x), d))
    t = good(io=torch.bfloat16)
    db = dims(io=libssd.SSD_BF16)
    ws = torch.zeros(64, dtype=torch.uint8)
    expect("dB must hold",
           lambda: libssd.ssd_fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None, ws,
                                        64, t["x"], None, t["x"].clone(), torch.zeros(T_, H_, dtype=f),
                                        torch.zeros(H_), torch.zeros(T_, G_, N_ - 1),
                                        torch.zeros(T_, G_, N_), torch.zeros(H_), None, db, ws, 64))
    expect("exceeds its buffer",
           lambda: libssd.ssd_fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None, ws,
                                        65, t["x"], None, t["x"].clone(), torch.zeros(T_, H_, dtype=f),
                                        torch.zeros(H_), torch.zeros(T_, G_, N_),
                                        torch.zeros(T_, G_, N_), torch.zeros(H_), None, db, ws, 64))


def test_block_neighbours_check_their_tensors():
    x = torch.zeros(2, 5, 16, dtype=torch.bfloat16)
    expect("weight must hold",
           lambda: libssd.ssd_conv1d_silu(x, 16, torch.zeros(16, 3), None, 4, torch.zeros_like(x),
                                          16, 2, 5, 0, None, 16, libssd.SSD_BF16))
    expect("out must be torch.bfloat16",
           lambda: libssd.ssd_conv1d_silu(x, 16, torch.zeros(16, 4), None, 4,
                                          torch.zeros(2, 5, 16), 16, 2, 5, 0, None, 16,
                                          libssd.SSD_BF16))
    expect("inp is smaller",
           lambda: libssd.ssd_conv1d_silu(x, 32, torch.zeros(16, 4), None, 4, torch.zeros_like(x),
                                          16, 2, 5, 0, None, 16, libssd.SSD_BF16))
    y = torch.zeros(4, 64, dtype=torch.bfloat16)
    expect("z must be torch.bfloat16",
           lambda: libssd.ssd_gate_rmsnorm(y, torch.zeros(4, 64), None, 1e-5, y.clone(), 4, 64,
                                           libssd.SSD_BF16))
    expect("weight must hold",
           lambda: libssd.ssd_gate_rmsnorm(y, y.clone(), torch.zeros(32), 1e-5, y.clone(), 4, 64,
                                           libssd.SSD_BF16))
