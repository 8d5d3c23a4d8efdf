"""ssd_chunk_scan_bwd (the general backward: every shape the forward takes,
fp32 or bf16, on the vector ALU, no saved states) on the GPU against the fp64
backward oracle (oracle.recurrence_bwd, pinned to the adjoint identity and to
finite differences of the forward oracle).

Tolerance: max |gpu - oracle| / max |oracle| per gradient.  fp32 inputs: 1e-4
(every step in fp32; the sums of up to 64 x 256 terms and the exp
approximation stay near 1e-6).  bf16 inputs: 2e-2, the forward's bound (the
chunk-start states are kept in bf16 like the forward's hprev, dx is rounded
to bf16).
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mamba_ssd_layer_amd as ssd  # noqa: E402
import oracle  # noqa: E402
from gpu_helpers import DEV, rel, say, upload  # noqa: E402

TOL = {"f32": 1e-4, "bf16": 2e-2}


def run_bwd(w, seed, dfinal_std=1.0):
    dy, dfinal = workloads.make_output_grads(w, seed, dfinal_std)
    t = upload(w)
    io = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dyd = torch.from_numpy(dy).to(DEV).to(io).view(t["x"].shape)
    dfd = None if dfinal is None else torch.from_numpy(dfinal).to(DEV)
    g = ssd.chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dyd, dfd,
                           init_state=t["h0"], cu_seqlens=t["cu"])
    torch.cuda.synchronize()
    return g, dy, dfinal


def host(g, w):
    T, H, P, G, N = w.tokens, w.nheads, w.headdim, w.ngroups, w.dstate
    out = {"dx": g["dx"].float().cpu().numpy().reshape(T, H, P),
           "ddt": g["ddt"].cpu().numpy().reshape(T, H),
           "dB": g["dB"].cpu().numpy().reshape(T, G, N),
           "dC": g["dC"].cpu().numpy().reshape(T, G, N),
           "dA": g["dA"].cpu().numpy(),
           "dh0": g["dinit"].cpu().numpy()}
    if g["dD"] is not None:
        out["dD"] = g["dD"].cpu().numpy()
    return out


def check(w, seed, label, dfinal_std=1.0):
    g, dy, dfinal = run_bwd(w, seed, dfinal_std)
    ref = oracle.recurrence_bwd(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off, dy, dfinal)
    got = host(g, w)
    tol = TOL[w.dtype]
    errs = {k: rel(got[k], ref[k]) for k in got}
    say(f"  {label}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f" (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{label}: {k} rel err {v:.3e} > {tol}"


def test_tiny_f32_workload():
    # the fp32 workload: B1 L256 H4 P16 N16
    check(workloads.make_workload("tiny_f32"), 1, "general bwd tiny_f32")


@pytest.mark.parametrize("P,N,G", [(16, 16, 1), (48, 32, 2), (64, 256, 2), (32, 64, 4)])
def test_f32_shapes(P, N, G):
    # ragged tail (1000 = 15 x 64 + 40), initial state, two sequences
    w = workloads.make_custom(2, 1000, 4, P, N, G, 64, "f32", seed=3000 + P + N + G, init_std=0.3)
    check(w, 2, f"general bwd f32 P{P} N{N} G{G}")


@pytest.mark.parametrize("P,N", [(64, 256), (32, 64), (128, 128), (96, 48)])
def test_bf16_shapes(P, N):
    w = workloads.make_custom(2, 700, 4, P, N, 2, 64, "bf16", seed=3100 + P + N, init_std=0.3)
    check(w, 3, f"general bwd bf16 P{P} N{N}")


def test_packed_edge_lengths():
    # packed sequences of lengths 0, 1, 63, 64, 65 and 300: empty sequences pass
    # d(final_state) through to d(init_state)
    lens = [0, 1, 63, 64, 65, 300]
    w = workloads.make_custom(1, 0, 4, 32, 64, 2, 64, "bf16", seed=3200, lens=lens, init_std=0.3)
    check(w, 4, "general bwd packed edge lengths")


def test_no_D_no_init_no_dfinal():
    w = workloads.make_custom(2, 300, 4, 64, 64, 1, 64, "f32", seed=3300, with_D=False)
    check(w, 5, "general bwd no D, no init, no dfinal", dfinal_std=0.0)


def test_slow_and_fast_decay():
    for k, rng in enumerate([(-9.0, -6.0), (2.0, 3.5)]):
        w = workloads.make_custom(1, 500, 4, 32, 32, 1, 64, "f32", seed=3400 + k,
                                  a_log_range=rng, init_std=0.3)
        check(w, 6 + k, f"general bwd A range {rng}")


@pytest.mark.parametrize("N", [128, 256])
def test_agrees_with_the_fast_backward(N):
    # a shape both backward paths take: the same gradients to the bf16 bound
    w = workloads.make_custom(2, 640, 4, 64, N, 2, 64, "bf16", seed=3500 + N, init_std=0.3)
    g, dy, dfinal = run_bwd(w, 7)
    t = upload(w)
    st = ssd.make_fused_states(t["x"], t["B"], t["cu"])
    ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"],
                  chunk_states=st)
    dyd = torch.from_numpy(dy).to(DEV).to(torch.bfloat16).view(t["x"].shape)
    g2 = ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], st, dyd,
                       torch.from_numpy(dfinal).to(DEV), t["cu"])
    torch.cuda.synchronize()
    a, b = host(g, w), host(g2, w)
    errs = {k: rel(a[k], b[k]) for k in a}
    say("  general vs fast backward: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= 2e-2 for v in errs.values())


def test_long_n256_whole():
    # one 65,536-token sequence, 80 heads, N 256: every gradient against the
    # oracle
    w = workloads.make_workload("long_n256")
    check(w, 8, "general bwd long_n256")
