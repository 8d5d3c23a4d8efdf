"""GPU parity of each stage (chunk_cumsum, chunk_state, state_passing,
chunk_scan) through its own C entry point, against the intermediates of the
numpy fp64 blockwise reference (oracle.chunked), on problems with several
chunks, a ragged last chunk and (for packed batches) sequences that restart.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mamba_ssd_layer_amd as ssd  # noqa: E402
from gpu_helpers import plan_for, rel, say, upload, y_host  # noqa: E402

CASES = {
    # name: (builder kwargs)
    "fixed_bf16": dict(batch=2, seqlen=700, nheads=4, headdim=64, dstate=128, ngroups=2,
                       chunk=256, dtype="bf16", seed=1, init_std=0.3),
    "fixed_f32": dict(batch=2, seqlen=300, nheads=3, headdim=16, dstate=32, ngroups=1,
                      chunk=64, dtype="f32", seed=2, init_std=0.3),
    "packed_bf16": dict(batch=1, seqlen=0, nheads=4, headdim=64, dstate=64, ngroups=4,
                        chunk=128, dtype="bf16", seed=3, init_std=0.3,
                        lens=[5, 300, 0, 128, 129, 1]),
    # bf16 on the vector-ALU stage kernels (head dim 32, state 48)
    "vector_bf16": dict(batch=2, seqlen=300, nheads=4, headdim=32, dstate=48, ngroups=2,
                        chunk=128, dtype="bf16", seed=6, init_std=0.3),
    # head dim 128: each head runs as two kernel heads of 64 state rows
    "split_bf16": dict(batch=2, seqlen=333, nheads=2, headdim=128, dstate=64, ngroups=1,
                       chunk=64, dtype="bf16", seed=5, init_std=0.3),
}
# per-stage tolerances (relative to the max of the reference)
TOL_STAGE = {"f32": 1e-5, "bf16": 1e-2}


def build(name):
    kw = dict(CASES[name])
    lens = kw.pop("lens", None)
    b, L, H, P, N, G = (kw.pop(k) for k in ("batch", "seqlen", "nheads", "headdim", "dstate",
                                            "ngroups"))
    return workloads.make_custom(b, L, H, P, N, G, kw.pop("chunk"), kw.pop("dtype"),
                                 kw.pop("seed"), lens=lens, **kw)


def chunk_index(w, it):
    """Map reference chunks (sequence-major) to workspace chunk indices."""
    Q = w.chunk
    if not w.nseq:
        ncr = -(-w.seqlen // Q)
        return [s * ncr + (st - w.seq_off[s]) // Q for s, st in zip(it["chunk_seq"], it["chunk_start"])]
    return list(range(len(it["chunk_len"])))


@pytest.mark.parametrize("name", list(CASES))
def test_stages(name):
    w = build(name)
    t = upload(w)
    plan = plan_for(w, t)
    tol = TOL_STAGE[w.dtype]
    y_ref, f_ref, it = oracle.chunked(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off, w.chunk,
                                      return_intermediates=True)
    cidx = chunk_index(w, it)
    lens = it["chunk_len"]

    # stage 1: cumulative log-decay and transposed dt
    plan.cumsum(t["dt"], t["A"], t["cu"])
    torch.cuda.synchronize()
    acum = plan.view("acum").cpu().numpy()
    dtq = plan.view("dtq").cpu().numpy()
    # kernel heads: a head of 64 r rows is r kernel heads with its dt and A
    hr = acum.shape[1] // w.nheads
    num = den = 0.0
    for k, c in enumerate(cidx):
        n = lens[k]
        ref = np.repeat(it["Acum"][k, :, :n], hr, axis=0)
        num = max(num, float(np.max(np.abs(acum[c, :, :n] - ref))))
        den = max(den, float(np.max(np.abs(ref))))
        # padding past a partial chunk repeats the last value; dt is zero there
        assert np.array_equal(acum[c, :, n:], np.repeat(acum[c, :, n - 1:n], w.chunk - n, axis=1))
        assert np.all(dtq[c, :, n:] == 0)
        t0 = it["chunk_start"][k]
        assert np.array_equal(dtq[c, :, :n], np.repeat(w.dt[t0:t0 + n].T, hr, axis=0))
    say(f"  {name}: acum rel err {num / den:.3e}")
    assert num / den <= 1e-5

    # stage 2: chunk states
    plan.state(t["x"], t["B"])
    torch.cuda.synchronize()
    S = plan.view("states").float().cpu().numpy()
    e = rel(S[cidx], it["S"])
    say(f"  {name}: chunk states rel err {e:.3e}")
    assert e <= tol

    # stage 3: state passing
    fin = torch.empty_like(t["h0"]) if t["h0"] is not None else None
    plan.passing(t["h0"], fin)
    torch.cuda.synchronize()
    Hp = plan.view("hprev").float().cpu().numpy()
    e = rel(Hp[cidx], it["Hprev"])
    ef = rel(fin.cpu().numpy(), f_ref)
    say(f"  {name}: hprev rel err {e:.3e}, final rel err {ef:.3e}")
    assert e <= tol and ef <= tol

    # stage 4: chunk scan
    y = torch.empty_like(t["x"])
    plan.scan(t["x"], t["B"], t["C"], t["D"], y)
    torch.cuda.synchronize()
    ey = rel(y_host(y, w), y_ref)
    say(f"  {name}: y rel err {ey:.3e}")
    assert ey <= (1e-4 if w.dtype == "f32" else 2e-2)


def test_chunk_table_rejects_bad_cu_seqlens_without_faulting():
    # cu_seqlens decreasing in the middle: lengths are clamped, the error word
    # is set, and every access stays inside the workspace
    w = workloads.make_custom(1, 0, 2, 64, 64, 1, 64, "bf16", seed=4, lens=[100, 50, 80])
    t = upload(w)
    t["cu"] = torch.tensor([0, 100, 60, 230], dtype=torch.int32, device=t["x"].device)
    plan = plan_for(w, t)
    # the Python plan refuses such offsets on the host ...
    with pytest.raises(ssd.SSDInvalidArgument):
        plan.cumsum(t["dt"], t["A"], t["cu"])
    # ... the C entry point takes them and the device side contains them
    ssd.libssd.ssd_chunk_cumsum(t["dt"], t["A"], plan.chunk_len, t["cu"], plan.dims,
                                plan.workspace)
    torch.cuda.synchronize()
    d = plan.view("chunk_dir").cpu().numpy()
    assert d[-1] != 0
    assert 0 <= d[w.nseq] <= plan.layout.nc_max
