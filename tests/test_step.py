"""ssd_step (single-token recurrent decode) on the GPU against the fp64 oracle.

The oracle is the same sequential recurrence the forward is checked against:
a run of K decode steps from a state h0 must give the oracle's y for those K
tokens and its final state.  Tolerances are the forward's (max |err| / max |ref|
over the whole tensor: 1e-4 fp32, 2e-2 bf16).
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
from gpu_helpers import TOL, say, upload  # noqa: E402


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def decode_run(w, t, steps, t0=0, state=None):
    """Run `steps` decode steps over tokens t0.. of every sequence; returns
    y [S, steps, H, P] (float64) and the state after the last step."""
    S, H, P = w.batch, w.nheads, w.headdim
    if state is None:
        state = t["h0"].clone() if t["h0"] is not None else torch.zeros(
            S, H, P, w.dstate, dtype=torch.float32, device=t["x"].device)
    ys = []
    for k in range(t0, t0 + steps):
        x = t["x"][:, k].contiguous()
        y = ssd.step(x, t["dt"][:, k].contiguous(), t["A"], t["B"][:, k].contiguous(),
                     t["C"][:, k].contiguous(), state, D=t["D"])
        ys.append(y.float())
    torch.cuda.synchronize()
    return torch.stack(ys, 1).cpu().numpy().astype(np.float64), state


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
def test_step_matches_recurrence(dtype, N):
    # a few steps from a nonzero state; G = 2 groups, P not a power of two
    w = workloads.make_custom(3, 5, 4, 24, N, 2, 64, dtype, seed=700 + N, init_std=0.5)
    t = upload(w)
    y, state = decode_run(w, t, steps=5)
    y_ref, f_ref = oracle.recurrence_workload(w)
    y_ref = y_ref.reshape(w.batch, w.seqlen, w.nheads, w.headdim)
    ey, ef = rel(y, y_ref), rel(state.cpu().numpy(), f_ref)
    say(f"  step {dtype} N{N}: y rel err {ey:.3e}, state rel err {ef:.3e}")
    assert ey <= TOL[dtype] and ef <= TOL[dtype]


def test_step_without_D_and_one_head_dim():
    w = workloads.make_custom(2, 3, 2, 1, 64, 1, 64, "f32", seed=710, init_std=1.0, with_D=False)
    t = upload(w)
    y, state = decode_run(w, t, steps=3)
    y_ref, f_ref = oracle.recurrence_workload(w)
    assert rel(y, y_ref.reshape(y.shape)) <= TOL["f32"]
    assert rel(state.cpu().numpy(), f_ref) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_continues_the_chunked_forward(dtype):
    # prefill 600 tokens with the chunked forward, then decode 6 more: the same
    # y and final state as the recurrence over all 606 tokens
    L0, K = 600, 6
    P = 64 if dtype == "bf16" else 32
    w = workloads.make_custom(2, L0 + K, 8, P, 128, 2, 256, dtype, seed=720, init_std=0.3,
                              dt_shift=3.0)
    t = upload(w)
    pre = {k: (v[:, :L0].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in t.items()}
    _, fin = ssd.chunk_scan_fwd(pre["x"], pre["dt"], pre["A"], pre["B"], pre["C"], pre["D"], 256,
                                pre["h0"])
    y, state = decode_run(w, t, steps=K, t0=L0, state=fin)
    y_ref, f_ref = oracle.recurrence_workload(w)
    y_ref = y_ref.reshape(w.batch, w.seqlen, w.nheads, w.headdim)[:, L0:]
    ey, ef = rel(y, y_ref), rel(state.cpu().numpy(), f_ref)
    say(f"  prefill {L0} + decode {K} ({dtype}): y rel err {ey:.3e}, state rel err {ef:.3e}")
    assert ey <= TOL[dtype] and ef <= TOL[dtype]


def test_step_large_batch():
    # a serving-sized step: 64 sequences, 64 heads, N = 128 (one token each)
    w = workloads.make_custom(64, 1, 64, 64, 128, 8, 64, "bf16", seed=730, init_std=0.1)
    t = upload(w)
    y, state = decode_run(w, t, steps=1)
    y_ref, f_ref = oracle.recurrence_workload(w)
    ey, ef = rel(y, y_ref.reshape(y.shape)), rel(state.cpu().numpy(), f_ref)
    say(f"  step S64 H64 N128: y rel err {ey:.3e}, state rel err {ef:.3e}")
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


def test_step_zero_dt_keeps_state_and_gives_Cx_readout():
    # dt = 0: the state is unchanged bit for bit (decay 1, no input) and
    # y = C . state + D x
    w = workloads.make_custom(2, 1, 4, 64, 64, 1, 64, "f32", seed=740, init_std=1.0)
    t = upload(w)
    t["dt"].zero_()
    state = t["h0"].clone()
    y = ssd.step(t["x"][:, 0].contiguous(), t["dt"][:, 0].contiguous(), t["A"],
                 t["B"][:, 0].contiguous(), t["C"][:, 0].contiguous(), state, D=t["D"])
    torch.cuda.synchronize()
    assert torch.equal(state, t["h0"])
    h0 = w.h0.astype(np.float64)
    C = w.C.reshape(2, 1, 64).astype(np.float64)
    x = w.x.reshape(2, 4, 64).astype(np.float64)
    ref = np.einsum("sn,shpn->shp", C[:, 0], h0) + w.D.astype(np.float64)[None, :, None] * x
    assert rel(y.cpu().numpy().astype(np.float64), ref) <= TOL["f32"]
