"""ssd_fused_fwd (the one-pass forward, state kept on chip) on the GPU against
the fp64 oracle, at the forward's tolerance (max |err| / max |ref| <= 2e-2 for
bf16): every output compared, the full-size workloads by streaming the
oracle over blocks of (sequence, head) pairs, and the edge cases of the chunked forward's tests
(ragged tails, empty and one-token sequences, slow decay, aliased states).
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mamba_ssd_layer_amd as ssd  # noqa: E402
from gpu_helpers import (TOL, check_full, check_whole, rel, run, say, upload,  # noqa: E402
                         y_host)

FUSED_CHUNK = 32  # the one-pass forward walks 32-token chunks


def run_fused(w, t=None, init="h0", final_state=None):
    if t is None:
        t = upload(w)
    h0 = t["h0"] if init == "h0" else init
    y, fin = ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], h0, t["cu"],
                           final_state=final_state)
    torch.cuda.synchronize()
    return y, fin, t


def test_small_bf16_full():
    w = workloads.make_workload("small_bf16")
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label="fused small_bf16")


def test_large_bf16_whole():
    # the headline shape: 8 x 4096 tokens, 80 heads, P 64, N 128
    w = workloads.make_workload("large_bf16")
    y, fin, _ = run_fused(w)
    check_whole(w, y, fin, label="fused large_bf16", head_tokens=8, chunk=FUSED_CHUNK)


def test_varlen_whole():
    # 64 packed sequences of mixed length, 8 groups, nonzero initial states
    w = workloads.make_workload("varlen_bf16")
    y, fin, _ = run_fused(w)
    check_whole(w, y, fin, label="fused varlen_bf16", head_tokens=8, chunk=FUSED_CHUNK)


@pytest.mark.parametrize("name", ["long_n64", "long_n128", "long_n256"])
def test_long_context_whole(name):
    # one 65,536-token sequence: the state is carried (with its running
    # power-of-two scale) across 2,048 chunks
    w = workloads.make_workload(name)
    y, fin, _ = run_fused(w)
    check_whole(w, y, fin, label=f"fused {name}", head_tokens=8, chunk=FUSED_CHUNK)


@pytest.mark.parametrize("N", [64, 128])
def test_ragged_tail(N):
    # 1000 tokens: 31 full 32-token chunks and a tail of 8; G = 2
    w = workloads.make_custom(3, 1000, 4, 64, N, 2, 256, "bf16", seed=1100 + N, init_std=0.2)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label=f"fused ragged N{N}")


@pytest.mark.parametrize("P,N", [(64, 256), (128, 64), (128, 128), (128, 256), (256, 128)])
def test_head_dims_and_state_sizes(P, N):
    # head dim 64 r as r kernel heads of 64 rows; N 256 in four wavefronts of
    # 16 state rows; ragged tail, two groups, nonzero initial state
    w = workloads.make_custom(2, 1000, 4, P, N, 2, 256, "bf16", seed=1250 + P + N, init_std=0.2)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label=f"fused P{P} N{N}")


@pytest.mark.parametrize("H,G", [(6, 2), (5, 5), (3, 1)])
def test_odd_heads_per_group(H, G):
    # one head a block where the heads of a group do not pair up
    w = workloads.make_custom(2, 500, H, 64, 128, G, 256, "bf16", seed=1260 + H, init_std=0.2)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label=f"fused H{H} G{G}")


@pytest.mark.parametrize("N", [64, 128, 256])
def test_head_pairs_path(N):
    # enough (sequence, head pair) blocks to fill the GPU: the two-heads-a-block
    # instance at N 64 and 128 (the small problems above take the one-head
    # instance); N 256 takes one head a block at any size
    w = workloads.make_custom(4, 300, 128, 64, N, 8, 256, "bf16", seed=1270 + N, init_std=0.2)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label=f"fused head pairs N{N}")


@pytest.mark.parametrize("N", [64, 128])
def test_head_triples_path(N):
    # three heads a block (one block a CU): 4 rows x 192 heads (G 2, 96 heads a
    # group) make 256 head-triple blocks
    w = workloads.make_custom(4, 300, 192, 64, N, 2, 256, "bf16", seed=1275 + N, init_std=0.2)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label=f"fused head triples N{N}")


@pytest.mark.parametrize("kind", ["A_zero", "dt_small"])
def test_long_memory_n256(kind):
    kw = {"A_zero": dict(a_zero=True), "dt_small": dict(dt_const=1e-3)}[kind]
    w = workloads.make_custom(2, 900, 4, 64, 256, 1, 256, "bf16", seed=1280, init_std=0.5, **kw)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label=f"fused N256 {kind}")


@pytest.mark.parametrize("G", [1, 4])
def test_groups(G):
    w = workloads.make_custom(2, 600, 8, 64, 64, G, 256, "bf16", seed=1200 + G)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label=f"fused G{G}")


@pytest.mark.parametrize("kind", ["A_zero", "A_tiny", "dt_small"])
def test_long_memory(kind):
    # slow or no decay: the state carried across chunks dominates y
    kw = {"A_zero": dict(a_zero=True),
          "A_tiny": dict(a_log_range=(np.log(1e-4), np.log(1e-2))),
          "dt_small": dict(dt_const=1e-3)}[kind]
    w = workloads.make_custom(2, 1500, 4, 64, 128, 1, 256, "bf16", seed=1300, init_std=0.5, **kw)
    y, fin, _ = run_fused(w)
    _, _, y_ref, _ = check_full(w, y, fin, label=f"fused {kind}")
    # first 8 tokens of each 32-token chunk, where the state handed in dominates
    yg = y_host(y, w)
    sel = np.tile((np.arange(w.seqlen) % FUSED_CHUNK) < 8, w.batch)
    e = np.max(np.abs(yg[sel] - y_ref[sel])) / np.max(np.abs(y_ref[sel]))
    say(f"    first 8 tokens of each chunk: rel err {e:.3e}")
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("dt_shift", [-1.0, 0.5])
def test_fast_decay(dt_shift):
    # large dt: chunks whose own decay exceeds 2^-40 (handled in the exact
    # per-chunk form) next to chunks whose decay is folded into the state's
    # running scale, which is renormalised every few chunks
    w = workloads.make_custom(2, 1200, 8, 64, 128, 2, 256, "bf16", seed=1350, init_std=0.5,
                              dt_shift=dt_shift)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label=f"fused fast decay {dt_shift}")


def test_varlen_edge_lengths():
    # empty, one-token, exactly one and two chunks, one token either side of
    # a chunk boundary, and a long sequence; nonzero initial states
    lens = [1, 0, 32, 31, 33, 64, 0, 700, 3, 1024, 1]
    w = workloads.make_custom(1, 0, 4, 64, 64, 2, 256, "bf16", seed=1400, lens=lens, init_std=0.3)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label="fused varlen edges")
    f = fin.cpu().numpy()
    for s, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(f[s], w.h0[s])


def test_empty_input_returns_init_state():
    w = workloads.make_custom(2, 0, 4, 64, 128, 1, 256, "bf16", seed=1500, init_std=0.5)
    y, fin, t = run_fused(w)
    assert y.numel() == 0
    assert torch.equal(fin, t["h0"])


def test_final_state_may_alias_init_state():
    w = workloads.make_custom(2, 777, 4, 64, 64, 2, 256, "bf16", seed=1600, init_std=0.5)
    t = upload(w)
    st = t["h0"].clone()
    y, fin, _ = run_fused(w, t, init=st, final_state=st)
    assert fin.data_ptr() == st.data_ptr()
    check_full(w, y, fin, label="fused aliased state")


def test_no_D_no_init():
    w = workloads.make_custom(2, 500, 4, 64, 128, 1, 256, "bf16", seed=1700, with_D=False)
    y, fin, _ = run_fused(w)
    check_full(w, y, fin, label="fused D=None")


def test_agrees_with_chunked_forward():
    # the two forwards round differently (bf16 operands at different points),
    # so they agree to the bf16 tolerance, not bit for bit
    w = workloads.make_custom(4, 2048, 16, 64, 128, 2, 256, "bf16", seed=1800, init_std=0.2)
    yc, fc, _, t = run(w)
    yf, ff, _ = run_fused(w, t)
    ey = rel(y_host(yf, w), y_host(yc, w).astype(np.float64))
    ef = rel(ff.cpu().numpy(), fc.cpu().numpy().astype(np.float64))
    say(f"  fused vs chunked: y rel diff {ey:.3e}, final rel diff {ef:.3e}")
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


def test_unsupported_shapes_raise():
    w = workloads.make_custom(1, 64, 4, 32, 64, 1, 256, "bf16", seed=1900)  # head dim 32
    t = upload(w)
    with pytest.raises(ssd.SSDUnsupported):
        ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"])
    w = workloads.make_custom(1, 64, 4, 64, 64, 1, 256, "f32", seed=1901)
    t = upload(w)
    with pytest.raises(ssd.SSDUnsupported):
        ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"])
