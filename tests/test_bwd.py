"""ssd_fused_bwd (the gradients of the one-pass forward) on the GPU against the
fp64 oracle of the backward pass (oracle.recurrence_bwd, itself pinned to the
adjoint identity and to finite differences of the forward oracle).

Tolerance: each gradient's max |gpu - oracle| / max |oracle| <= 2e-2, the
forward's bf16 bound.  The path rounds to bf16 where the forward does (the
operands of every MFMA: dy and C, the decay-weighted products of a chunk) and
in three more places, each a relative 2^-9: the saved chunk-start states, the
saved state gradients and the dx output.  Each output is a sum of O(P N) such
terms with independent rounding, so the normalised error stays near 1e-3;
2e-2 leaves room for the cancellation in ddt's and dA's sums of signed terms.
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

TOLB = 2e-2


def fwd_bwd(w, t, dy, dfinal):
    st = ssd.make_fused_states(t["x"], t["B"], t["cu"])
    y, fin = ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"],
                           chunk_states=st)
    dyd = torch.from_numpy(dy).to(DEV).to(torch.bfloat16).view(t["x"].shape)
    dfd = None if dfinal is None else torch.from_numpy(dfinal).to(DEV)
    g = ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], st, dyd, dfd, t["cu"])
    torch.cuda.synchronize()
    return y, fin, st, g


def host(g, w):
    T, H, P, G, N = w.tokens, w.nheads, w.headdim, w.ngroups, w.dstate
    out = {"dx": g["dx"].float().cpu().numpy().reshape(T, H, P),
           "ddt": g["ddt"].cpu().numpy().reshape(T, H),
           "dB": g["dB"].cpu().numpy().reshape(T, G, N),
           "dC": g["dC"].cpu().numpy().reshape(T, G, N),
           "dA": g["dA"].cpu().numpy()}
    if g["dD"] is not None:
        out["dD"] = g["dD"].cpu().numpy()
    if g["dinit"] is not None:
        out["dh0"] = g["dinit"].cpu().numpy()
    return out


def check_grads(w, g, ref, label, names=None, tol=TOLB):
    got = host(g, w)
    names = names or [k for k in ("dx", "ddt", "dB", "dC", "dA", "dD", "dh0") if k in got]
    errs = {k: rel(got[k], ref[k]) for k in names}
    say(f"  {label}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f" (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{label}: {k} rel err {v:.3e} > {tol}"
    return errs


def full_case(w, seed, dfinal_std=1.0, label=""):
    dy, dfinal = workloads.make_output_grads(w, seed, dfinal_std)
    t = upload(w)
    _, _, _, g = fwd_bwd(w, t, dy, dfinal)
    ref = oracle.recurrence_bwd(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off, dy, dfinal)
    return check_grads(w, g, ref, label or w.name)


def test_small_full():
    w = workloads.make_custom(2, 300, 4, 64, 64, 2, 256, "bf16", seed=2100, init_std=0.3)
    full_case(w, 1, label="bwd small N64 G2")


@pytest.mark.parametrize("N", [64, 128, 256])
def test_ragged_tail(N):
    # 1000 tokens a row: 31 full 32-token chunks and a tail of 8
    w = workloads.make_custom(3, 1000, 4, 64, N, 2, 256, "bf16", seed=2200 + N, init_std=0.2)
    full_case(w, 2, label=f"bwd ragged N{N}")


@pytest.mark.parametrize("G", [1, 4])
def test_groups(G):
    # 8 heads: 8 heads share B, C (G 1) or 2 do (G 4); dB, dC sum over them
    w = workloads.make_custom(2, 600, 8, 64, 128, G, 256, "bf16", seed=2300 + G, init_std=0.1)
    full_case(w, 3, label=f"bwd G{G}")


def test_n256_full():
    # N 256 runs as two halves of 128 state columns: dB, dC, d(init) of each
    # half in its own columns, dx, ddt, dA summed over the halves
    w = workloads.make_custom(2, 640, 4, 64, 256, 2, 256, "bf16", seed=2150, init_std=0.3)
    full_case(w, 21, label="bwd N256 G2")


def test_n256_many_heads():
    # 4 rows x 128 heads in 8 groups: 256 (row, head pair) blocks in the reverse
    # sweep (one pass per block, not segmented), 16 heads walked per chunk block
    w = workloads.make_custom(4, 300, 128, 64, 256, 8, 256, "bf16", seed=2170, init_std=0.2)
    full_case(w, 23, label="bwd N256 many heads")


def test_n256_packed_no_dfinal():
    lens = [1, 0, 33, 64, 65, 500]
    w = workloads.make_custom(1, 0, 4, 64, 256, 1, 256, "bf16", seed=2160, lens=lens,
                              init_std=0.3)
    full_case(w, 22, dfinal_std=0.0, label="bwd N256 packed, no dfinal")


def test_varlen_edge_lengths():
    lens = [1, 0, 32, 31, 33, 64, 0, 700, 3, 1024, 1]
    w = workloads.make_custom(1, 0, 4, 64, 64, 2, 256, "bf16", seed=2400, lens=lens, init_std=0.3)
    full_case(w, 4, label="bwd varlen edges")


def test_no_D_no_init_no_dfinal():
    w = workloads.make_custom(2, 500, 4, 64, 128, 1, 256, "bf16", seed=2500, with_D=False)
    dy, _ = workloads.make_output_grads(w, 5, 0.0)
    t = upload(w)
    _, _, _, g = fwd_bwd(w, t, dy, None)
    assert g["dD"] is None
    ref = oracle.recurrence_bwd(w.x, w.dt, w.A, w.B, w.C, None, None, w.seq_off, dy, None)
    check_grads(w, g, ref, "bwd no D / h0 / dfinal")


@pytest.mark.parametrize("dt_shift", [-1.0, 0.5])
def test_fast_decay(dt_shift):
    w = workloads.make_custom(2, 700, 4, 64, 128, 2, 256, "bf16", seed=2600, init_std=0.5,
                              dt_shift=dt_shift)
    full_case(w, 6, label=f"bwd fast decay {dt_shift}")


@pytest.mark.parametrize("kind", ["A_zero", "dt_small"])
def test_long_memory(kind):
    kw = {"A_zero": dict(a_zero=True), "dt_small": dict(dt_const=1e-3)}[kind]
    w = workloads.make_custom(2, 900, 4, 64, 64, 1, 256, "bf16", seed=2700, init_std=0.5, **kw)
    full_case(w, 7, label=f"bwd {kind}")


@pytest.mark.parametrize("P,N", [(64, 64), (128, 128), (64, 256)])
def test_saved_states_are_prefix_final_states(P, N):
    # the state entering 64-token pair b of a row is the oracle's final state
    # of the row's first 64 b tokens (from the same initial state); the saving
    # forward also serves head dims above 64 (the backward does not)
    w = workloads.make_custom(2, 200, 4, P, N, 2, 256, "bf16", seed=2800 + P + N, init_std=0.3)
    t = upload(w)
    st = ssd.make_fused_states(t["x"], t["B"], t["cu"])
    ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"],
                  chunk_states=st)
    torch.cuda.synchronize()
    H, P, N, L = w.nheads, w.headdim, w.dstate, w.seqlen
    npair = (L + 63) // 64
    hs = st.view(torch.bfloat16)[: w.batch * npair * H * P * N].float().cpu().numpy()
    hs = hs.reshape(w.batch, npair, H, P, N)
    worst = 0.0
    for b in range(w.batch):
        sl = slice(b * L, (b + 1) * L)
        for k in range(npair):
            n = 64 * k
            if n == 0:
                ref = w.h0[b].astype(np.float64)
            else:
                _, f = oracle.recurrence(w.x[sl][:n], w.dt[sl][:n], w.A, w.B[sl][:n],
                                         w.C[sl][:n], w.D, w.h0[b:b + 1], np.array([0, n]))
                ref = f[0]
            worst = max(worst, rel(hs[b, k], ref))
    say(f"  saved states: rel err {worst:.3e}")
    assert worst <= 1e-2


def test_train_forward_matches_plain_forward():
    # saving the states changes nothing in y or the final state, bit for bit
    w = workloads.make_custom(2, 777, 4, 64, 128, 2, 256, "bf16", seed=2900, init_std=0.2)
    t = upload(w)
    y1, f1 = ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"])
    st = ssd.make_fused_states(t["x"], t["B"], t["cu"])
    y2, f2 = ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"],
                           chunk_states=st)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_large_sampled():
    # the headline shape, 8 x 4096 tokens, 80 heads, P 64, N 128, G 1: dx,
    # ddt and dinit on sampled (sequence, head) pairs; dB and dC of one whole
    # sequence (all 80 heads of its group)
    w = workloads.make_workload("large_bf16")
    dy, dfinal = workloads.make_output_grads(w, 8)
    t = upload(w)
    _, _, _, g = fwd_bwd(w, t, dy, dfinal)
    got = host(g, w)
    r = np.random.default_rng(0)
    pairs = sorted({(0, 0), (7, 79), (3, 40)} | {(int(r.integers(8)), int(r.integers(80)))
                                                 for _ in range(5)})
    ref = oracle.recurrence_bwd(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off, dy, dfinal,
                                pairs=pairs)
    so = w.seq_off
    num = {k: 0.0 for k in ("dx", "ddt", "dh0")}
    den = dict(num)
    for k, (s, h) in enumerate(pairs):
        a, b = so[s], so[s + 1]
        for name, gv, rv in (("dx", got["dx"][a:b, h], ref["dx"][a:b, h]),
                             ("ddt", got["ddt"][a:b, h], ref["ddt"][a:b, h]),
                             ("dh0", got["dh0"][s, h], ref["dh0"][s, h])):
            num[name] = max(num[name], float(np.max(np.abs(gv - rv))))
            den[name] = max(den[name], float(np.max(np.abs(rv))))
    errs = {k: num[k] / den[k] for k in num}
    # one sequence, every head: its rows of dB and dC are complete
    s = 5
    a, b = so[s], so[s + 1]
    ref1 = oracle.recurrence_bwd(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off, dy, dfinal,
                                 pairs=[(s, h) for h in range(w.nheads)])
    errs["dB"] = rel(got["dB"][a:b], ref1["dB"][a:b])
    errs["dC"] = rel(got["dC"][a:b], ref1["dC"][a:b])
    say("  bwd large sampled: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOLB, f"{k} rel err {v:.3e}"


def test_unsupported_and_invalid():
    w = workloads.make_custom(1, 64, 4, 32, 64, 1, 256, "bf16", seed=3000)
    t = upload(w)
    with pytest.raises(ssd.SSDUnsupported):
        ssd.make_fused_states(t["x"], t["B"])
    # forward-only shapes: head dim 128, odd heads per group
    for P, N, H, G in ((128, 64, 4, 1), (64, 64, 3, 1)):
        w = workloads.make_custom(1, 64, H, P, N, G, 256, "bf16", seed=3002)
        t = upload(w)
        st = ssd.make_fused_states(t["x"], t["B"])
        with pytest.raises(ssd.SSDUnsupported):
            ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], st,
                          torch.zeros_like(t["x"]))
    w = workloads.make_custom(1, 64, 4, 64, 64, 1, 256, "bf16", seed=3001)
    t = upload(w)
    st = ssd.make_fused_states(t["x"], t["B"])
    dy = torch.zeros_like(t["x"])
    with pytest.raises(ssd.SSDWorkspaceError):  # saved states too small
        ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], st[:16], dy)
    with pytest.raises(ssd.SSDInvalidArgument):  # dD without D is refused
        ssd.libssd.ssd_fused_bwd(
            t["x"], t["dt"], t["A"], t["B"], t["C"], None, None, st, st.numel(), dy, None,
            torch.empty_like(dy), torch.empty_like(t["dt"]), torch.empty(4, device=DEV),
            torch.empty(t["B"].shape, device=DEV), torch.empty(t["C"].shape, device=DEV),
            torch.empty(4, device=DEV), None, ssd.dims_for(t["x"], t["B"], None),
            torch.empty_like(st), st.numel())


def seq_oracle(w, s, heads, dy, dfinal):
    """The backward oracle on sequence s alone (its rows of every input), for
    the given heads: the oracle's outputs are full-size arrays, so slicing keeps
    them small at the packed workload's 275k tokens."""
    a, b = int(w.seq_off[s]), int(w.seq_off[s + 1])
    one = lambda arr: None if arr is None else arr[s:s + 1]
    return oracle.recurrence_bwd(w.x[a:b], w.dt[a:b], w.A, w.B[a:b], w.C[a:b], w.D, one(w.h0),
                                 np.array([0, b - a]), dy[a:b], one(dfinal),
                                 pairs=[(0, h) for h in heads])


def sampled_check(w, g, pairs, label, dy, dfinal, group_seq=None):
    """dx, ddt, dinit on sampled (sequence, head) pairs; dB and dC on the rows
    of sequence group_seq[0] for group group_seq[1] (all its heads)."""
    got = host(g, w)
    so = w.seq_off
    num = {k: 0.0 for k in ("dx", "ddt", "dh0")}
    den = dict(num)
    for s in sorted({s for s, _ in pairs}):
        heads = [h for s2, h in pairs if s2 == s]
        ref = seq_oracle(w, s, heads, dy, dfinal)
        a, b = so[s], so[s + 1]
        for h in heads:
            for name, gv, rv in (("dx", got["dx"][a:b, h], ref["dx"][:, h]),
                                 ("ddt", got["ddt"][a:b, h], ref["ddt"][:, h]),
                                 ("dh0", got["dh0"][s, h], ref["dh0"][0, h])):
                if rv.size:
                    num[name] = max(num[name], float(np.max(np.abs(gv - rv))))
                    den[name] = max(den[name], float(np.max(np.abs(rv))))
    errs = {k: num[k] / den[k] for k in num if den[k] > 0}
    if group_seq is not None:
        s, gr = group_seq
        hpg = w.nheads // w.ngroups
        ref1 = seq_oracle(w, s, range(gr * hpg, (gr + 1) * hpg), dy, dfinal)
        a, b = so[s], so[s + 1]
        errs["dB"] = rel(got["dB"][a:b, gr], ref1["dB"][:, gr])
        errs["dC"] = rel(got["dC"][a:b, gr], ref1["dC"][:, gr])
    say(f"  {label}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOLB, f"{label}: {k} rel err {v:.3e}"


def test_varlen_workload_sampled():
    # 64 packed sequences of lengths U[1, 8192] (275,772 tokens), H 64, G 8,
    # nonzero initial states: sampled pairs, and dB / dC of one (sequence, group)
    w = workloads.make_workload("varlen_bf16")
    dy, dfinal = workloads.make_output_grads(w, 9)
    t = upload(w)
    _, _, _, g = fwd_bwd(w, t, dy, dfinal)
    lens = np.diff(w.seq_off)
    s_long = int(np.argmax(lens))
    pairs = sorted({(0, 0), (63, 63), (s_long, 17), (int(np.argmin(lens)), 40), (20, 5), (41, 62)})
    sampled_check(w, g, pairs, "bwd varlen_bf16 sampled", dy, dfinal, group_seq=(s_long, 3))


def test_long_n64_sampled():
    # one 65,536-token sequence, 80 heads, N 64: 2048 chunks swept backwards
    w = workloads.make_workload("long_n64")
    dy, dfinal = workloads.make_output_grads(w, 10)
    t = upload(w)
    _, _, _, g = fwd_bwd(w, t, dy, dfinal)
    pairs = [(0, 0), (0, 33), (0, 79)]
    sampled_check(w, g, pairs, "bwd long_n64 sampled", dy, dfinal)


def test_long_n256_sampled():
    # one 65,536-token sequence, 80 heads, N 256: the two-half backward over
    # 1024 pairs of chunks, sampled heads
    w = workloads.make_workload("long_n256")
    dy, dfinal = workloads.make_output_grads(w, 14)
    t = upload(w)
    _, _, _, g = fwd_bwd(w, t, dy, dfinal)
    sampled_check(w, g, [(0, 0), (0, 41), (0, 79)], "bwd long_n256 sampled", dy, dfinal)


@pytest.mark.parametrize("N", [64, 256])
def test_split_one_pass_saving_states(N):
    # ssd_fused_fwd_split_train: 2000 tokens a row in segments of 512 (the
    # last 464), initial states.  y and the final state bit for bit those of
    # the split forward without saving; the saved states those of the oracle's
    # prefixes (segment starts included); the backward from them the oracle's
    w = workloads.make_custom(2, 2000, 4, 64, N, 2, 256, "bf16", seed=3300 + N, init_std=0.3)
    dy, dfinal = workloads.make_output_grads(w, 15)
    t = upload(w)
    y1, f1 = ssd.fused_fwd_split(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"],
                                 seg_len=512)
    st = ssd.make_fused_states(t["x"], t["B"])
    y2, f2 = ssd.fused_fwd_split(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"],
                                 seg_len=512, chunk_states=st)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    H, P, L = w.nheads, w.headdim, w.seqlen
    npair = (L + 63) // 64
    hs = st.view(torch.bfloat16)[: w.batch * npair * H * P * N].float().cpu().numpy()
    hs = hs.reshape(w.batch, npair, H, P, N)
    worst = 0.0
    for b in range(w.batch):
        sl = slice(b * L, (b + 1) * L)
        for k in (0, 1, 7, 8, 9, 16, 24, npair - 1):  # pairs 8, 16, 24 start segments
            n = 64 * k
            if n == 0:
                ref = w.h0[b].astype(np.float64)
            else:
                _, f = oracle.recurrence(w.x[sl][:n], w.dt[sl][:n], w.A, w.B[sl][:n],
                                         w.C[sl][:n], w.D, w.h0[b:b + 1], np.array([0, n]))
                ref = f[0]
            worst = max(worst, rel(hs[b, k], ref))
    say(f"  split saving N{N}: saved states rel err {worst:.3e}")
    assert worst <= 1e-2
    dyd = torch.from_numpy(dy).to(DEV).to(torch.bfloat16).view(t["x"].shape)
    g = ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], st, dyd,
                      torch.from_numpy(dfinal).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.recurrence_bwd(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off, dy, dfinal)
    check_grads(w, g, ref, f"bwd from the split one-pass forward's states N{N}")


def test_long_n128_split_one_pass_saving_sampled():
    # the 65,536-token sequence at the library's segment length: the backward
    # from the split one-pass forward's saved states, sampled heads
    w = workloads.make_workload("long_n128")
    dy, dfinal = workloads.make_output_grads(w, 16)
    t = upload(w)
    S = ssd.fused_split_seg_len(t["x"], t["B"])
    st = ssd.make_fused_states(t["x"], t["B"])
    ssd.fused_fwd_split(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], seg_len=S,
                        chunk_states=st)
    dyd = torch.from_numpy(dy).to(DEV).to(torch.bfloat16).view(t["x"].shape)
    g = ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], st, dyd,
                      torch.from_numpy(dfinal).to(DEV))
    torch.cuda.synchronize()
    sampled_check(w, g, [(0, 3), (0, 50)], f"bwd long_n128 from the split one-pass forward S{S}",
                  dy, dfinal)


def test_packed_long_sequences_sampled():
    # two packed sequences of 40,000 and 25,536 tokens, 80 heads: 80 (sequence,
    # head pair) blocks, so the reverse sweep runs in 2048-token segments over
    # packed sequences (a segment may end at a sequence's end); sampled heads
    # of both sequences (the state gradient the segments hand on enters dx,
    # ddt and d(init_state))
    w = workloads.make_custom(1, 0, 80, 64, 128, 1, 256, "bf16", seed=3400, lens=[40000, 25536],
                              init_std=0.3)
    dy, dfinal = workloads.make_output_grads(w, 17)
    t = upload(w)
    _, _, _, g = fwd_bwd(w, t, dy, dfinal)
    pairs = [(0, 0), (0, 47), (1, 13), (1, 79)]
    sampled_check(w, g, pairs, "bwd two long packed sequences, sampled", dy, dfinal)


def test_long_n64_split_training_forward_sampled():
    # the training step's forward at this shape (SSDTrainForward: chunk 256 for
    # y, chunk 64 for the states), then the segmented backward from its states
    w = workloads.make_workload("long_n64")
    dy, dfinal = workloads.make_output_grads(w, 11)
    t = upload(w)
    tplan = ssd.SSDTrainForward(ssd.dims_for(t["x"], t["B"], t["cu"]), device=DEV)
    _, _, states = tplan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"])
    dyd = torch.from_numpy(dy).to(DEV).to(torch.bfloat16).view(t["x"].shape)
    g = ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], states, dyd,
                      torch.from_numpy(dfinal).to(DEV), t["cu"])
    torch.cuda.synchronize()
    sampled_check(w, g, [(0, 5), (0, 46)], "bwd long_n64 from the split forward, sampled", dy,
                  dfinal)


@pytest.mark.parametrize("packed", [False, True])
def test_states_from_chunked_forward(packed):
    # the four-stage forward with chunk length 64 leaves the same states in its
    # workspace (hprev): the backward from them matches the oracle
    if packed:
        w = workloads.make_custom(1, 0, 4, 64, 128, 2, 64, "bf16", seed=3100, init_std=0.3,
                                  lens=[300, 0, 65, 1000, 1])
    else:
        w = workloads.make_custom(2, 700, 4, 64, 64, 1, 64, "bf16", seed=3101, init_std=0.3)
    dy, dfinal = workloads.make_output_grads(w, 12)
    t = upload(w)
    plan = ssd.SSDForward(ssd.dims_for(t["x"], t["B"], t["cu"]), 64, device=DEV)
    plan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"])
    states = plan.saved_states()
    dyd = torch.from_numpy(dy).to(DEV).to(torch.bfloat16).view(t["x"].shape)
    g = ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], states, dyd,
                      torch.from_numpy(dfinal).to(DEV), t["cu"])
    torch.cuda.synchronize()
    ref = oracle.recurrence_bwd(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off, dy, dfinal)
    check_grads(w, g, ref, f"bwd from chunked-forward states ({'packed' if packed else 'fixed'})")


@pytest.mark.parametrize("packed", [False, True])
def test_split_training_forward(packed):
    # SSDTrainForward: y and the final state from chunk length 256, the states
    # from the first three stages at chunk length 64 -- bit for bit the hprev of
    # the chunk-64 forward; y within the forward's tolerance of the oracle; the
    # backward from those states matches the oracle
    if packed:
        w = workloads.make_custom(1, 0, 4, 64, 128, 2, 64, "bf16", seed=3200, init_std=0.3,
                                  lens=[300, 0, 65, 1000, 1])
    else:
        w = workloads.make_custom(2, 700, 4, 64, 64, 1, 64, "bf16", seed=3201, init_std=0.3)
    dy, dfinal = workloads.make_output_grads(w, 13)
    t = upload(w)
    dims = ssd.dims_for(t["x"], t["B"], t["cu"])
    tplan = ssd.SSDTrainForward(dims, device=DEV)
    y, fin, states = tplan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"])
    plan = ssd.SSDForward(dims, 64, device=DEV)
    plan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"])
    torch.cuda.synchronize()
    # the pairs the sequences use (a packed batch's buffer is sized by a bound)
    lens = np.diff(w.seq_off)
    nb = int(sum(-(-int(n) // 64) for n in lens)) * w.nheads * w.headdim * w.dstate * 2
    assert torch.equal(states[:nb], plan.saved_states()[:nb])
    y_ref, f_ref = oracle.recurrence(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off)
    yg = y.float().cpu().numpy().reshape(y_ref.shape)
    ey = float(np.max(np.abs(yg - y_ref)) / np.max(np.abs(y_ref)))
    ef = float(np.max(np.abs(fin.cpu().numpy() - f_ref)) / np.max(np.abs(f_ref)))
    say(f"  split training forward ({'packed' if packed else 'fixed'}): y {ey:.3e}, final {ef:.3e}")
    assert ey <= 2e-2 and ef <= 2e-2
    dyd = torch.from_numpy(dy).to(DEV).to(torch.bfloat16).view(t["x"].shape)
    g = ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], states, dyd,
                      torch.from_numpy(dfinal).to(DEV), t["cu"])
    torch.cuda.synchronize()
    ref = oracle.recurrence_bwd(w.x, w.dt, w.A, w.B, w.C, w.D, w.h0, w.seq_off, dy, dfinal)
    check_grads(w, g, ref, f"bwd from split-forward states ({'packed' if packed else 'fixed'})")
