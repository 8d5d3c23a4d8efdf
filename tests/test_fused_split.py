"""ssd_fused_fwd_split (the one-pass forward over segments of a sequence: a
state-only pass, the hand-off between segments, every segment from its
entering state) on the GPU against the fp64 oracle, at the forward's
tolerance: the long single-sequence workloads it is for (every output, with
the error on the first tokens after each segment boundary reported too),
ragged last segments, split head dims, N 256, one-chunk segments, and the
aliasing and no-split cases against ssd_fused_fwd.
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mamba_ssd_layer_amd as ssd  # noqa: E402
from gpu_helpers import check_full, check_whole, say, upload  # noqa: E402


def run_split(w, seg_len=None, t=None, init="h0", final_state=None):
    if t is None:
        t = upload(w)
    h0 = t["h0"] if init == "h0" else init
    y, fin = ssd.fused_fwd_split(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], h0,
                                 final_state=final_state, seg_len=seg_len)
    torch.cuda.synchronize()
    return y, fin, t


@pytest.mark.parametrize("name", ["long_n64", "long_n128", "long_n256"])
def test_long_context_whole(name):
    # one 65,536-token sequence, cut at the library's segment length
    w = workloads.make_workload(name)
    t = upload(w)
    S = ssd.fused_split_seg_len(t["x"], t["B"])
    say(f"  {name}: segment length {S}")
    assert 0 < S < w.seqlen and S % 32 == 0
    y, fin, _ = run_split(w, S, t)
    check_whole(w, y, fin, label=f"split {name} S{S}", head_tokens=8, chunk=S)


@pytest.mark.parametrize("N", [64, 128])
def test_ragged_last_segment(N):
    # 1000 tokens in segments of 256 (the last 232), two groups, initial state
    w = workloads.make_custom(3, 1000, 4, 64, N, 2, 256, "bf16", seed=1400 + N, init_std=0.2)
    y, fin, _ = run_split(w, 256)
    check_full(w, y, fin, label=f"split ragged N{N}")


@pytest.mark.parametrize("P,N,S", [(128, 128, 192), (64, 256, 160), (256, 64, 96)])
def test_head_dims_and_state_sizes(P, N, S):
    w = workloads.make_custom(2, 777, 4, P, N, 2, 256, "bf16", seed=1450 + P + N, init_std=0.2)
    y, fin, _ = run_split(w, S)
    check_full(w, y, fin, label=f"split P{P} N{N} S{S}")


def test_one_chunk_segments():
    # segments of 32 tokens: every chunk hands its state on through the workspace
    w = workloads.make_custom(2, 300, 4, 64, 64, 1, 64, "bf16", seed=1490, init_std=0.3)
    y, fin, _ = run_split(w, 32)
    check_full(w, y, fin, label="split S32")


def test_no_split_is_the_one_pass_forward():
    # seg_len >= seqlen: no workspace, the same kernel launch as ssd_fused_fwd
    w = workloads.make_custom(2, 500, 4, 64, 128, 2, 256, "bf16", seed=1500, init_std=0.2)
    t = upload(w)
    assert ssd.libssd.ssd_fused_split_workspace_size(ssd.dims_for(t["x"], t["B"]), 512) == 0
    y1, f1, _ = run_split(w, 512, t)
    y2, f2 = ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_final_state_may_alias_init_state():
    # the hand-off reads init_state before the last segments write final_state
    w = workloads.make_custom(2, 700, 4, 64, 64, 2, 256, "bf16", seed=1510, init_std=0.3)
    t = upload(w)
    y1, f1, _ = run_split(w, 128, t)
    st = t["h0"].clone()
    y2, f2, _ = run_split(w, 128, t, init=st, final_state=st)
    assert f2.data_ptr() == st.data_ptr()
    assert torch.equal(y1, y2) and torch.equal(f1, st)


def test_no_D_no_init():
    w = workloads.make_custom(2, 600, 4, 64, 128, 1, 256, "bf16", seed=1520, with_D=False)
    assert w.D is None and w.h0 is None
    y, fin, _ = run_split(w, 256)
    check_full(w, y, fin, label="split no D no init")


def test_large_bf16_split_whole():
    # the headline shape cut into 1024-token segments: four per sequence
    w = workloads.make_workload("large_bf16")
    y, fin, _ = run_split(w, 1024)
    check_whole(w, y, fin, label="split large_bf16 S1024", head_tokens=8, chunk=1024)


def test_seg_len_rule():
    # few long sequences are cut; a batch whose (sequence, head) rows fill the
    # GPU is not; packed batches have no split
    x = torch.empty(1, 65536, 80, 64, dtype=torch.bfloat16, device="cuda")
    B = torch.empty(1, 65536, 1, 128, dtype=torch.bfloat16, device="cuda")
    S = ssd.fused_split_seg_len(x, B)
    assert 512 <= S < 65536 and S & (S - 1) == 0
    x2 = torch.empty(64, 1000, 80, 64, dtype=torch.bfloat16, device="cuda")
    B2 = torch.empty(64, 1000, 1, 128, dtype=torch.bfloat16, device="cuda")
    assert ssd.fused_split_seg_len(x2, B2) == 1024  # 1000 rounded up to 32
    say(f"  segment length for 1 x 65536 x 80 heads: {S}")
