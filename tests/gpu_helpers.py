"""Helpers for the GPU tests: upload a seeded workload, run libssd, compare with
the fp64 oracle.  Not collected by pytest (no test_ prefix)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mamba_ssd_layer_amd as ssd
import oracle

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def upload(w):
    """Device tensors of a workloads.Workload in the API shapes."""
    io = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T, H, P, G, N = w.tokens, w.nheads, w.headdim, w.ngroups, w.dstate
    lead = (1, T) if w.nseq else (w.batch, w.seqlen)

    def dev(a, shape, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        if dtype is not None:
            t = t.to(dtype)
        return t.view(*shape).contiguous()

    t = {
        "x": dev(w.x, (*lead, H, P), io),
        "dt": dev(w.dt, (*lead, H)),
        "A": dev(w.A, (H,)),
        "B": dev(w.B, (*lead, G, N), io),
        "C": dev(w.C, (*lead, G, N), io),
        "D": None if w.D is None else dev(w.D, (H,)),
        "h0": None if w.h0 is None else dev(w.h0, w.h0.shape),
        "cu": None if not w.nseq else dev(w.cu_seqlens, (w.nseq + 1,)),
    }
    return t


def plan_for(w, t, chunk=None):
    dims = ssd.dims_for(t["x"], t["B"], t["cu"])
    return ssd.SSDForward(dims, chunk or w.chunk, device=DEV)


def run(w, chunk=None, t=None, plan=None):
    if t is None:
        t = upload(w)
    if plan is None:
        plan = plan_for(w, t, chunk)
    y, fin = plan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"])
    torch.cuda.synchronize()
    return y, fin, plan, t


def y_host(y, w) -> np.ndarray:
    return y.float().cpu().numpy().reshape(w.tokens, w.nheads, w.headdim)


def rel(got, ref) -> float:
    den = float(np.max(np.abs(ref)))
    if den == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / den


def check_full(w, y, fin, tol=None, label=""):
    """Whole-tensor comparison with the oracle (small problems)."""
    tol = TOL[w.dtype] if tol is None else tol
    y_ref, f_ref = oracle.recurrence_workload(w)
    ey = rel(y_host(y, w), y_ref)
    ef = rel(fin.cpu().numpy(), f_ref)
    say(f"  {label or w.name}: y rel err {ey:.3e}, final rel err {ef:.3e} (tol {tol:g})")
    assert ey <= tol, f"y rel err {ey} > {tol}"
    assert ef <= tol, f"final rel err {ef} > {tol}"
    return ey, ef, y_ref, f_ref


def _pair_blocks(w, budget_bytes=1 << 29):
    """(sequence, head range) blocks covering every pair, each small enough
    that its fp64 oracle output stays under budget_bytes."""
    lens = np.diff(w.seq_off)
    per_head = lambda s: max(1, int(lens[s])) * w.headdim * 8
    for s in range(w.nsequences):
        hc = int(max(16, min(w.nheads, budget_bytes // per_head(s))))
        for h0 in range(0, w.nheads, hc):
            yield s, h0, min(w.nheads, h0 + hc)


def check_whole(w, y, fin, tol=None, label="", head_tokens=None, chunk=None):
    """Whole-tensor comparison with the oracle on workloads too large to hold
    the fp64 reference at once: every (sequence, head) pair is computed by the
    oracle in blocks (one sequence, a run of heads) and compared with the
    matching slice of y and final_state; the bound is applied to the maxima
    over the whole tensors, max|y - y_ref| / max|y_ref|.  head_tokens: also
    bound the error on the first k tokens of each chunk (chunk length
    `chunk`, default the workload's), where the state handed in dominates."""
    tol = TOL[w.dtype] if tol is None else tol
    chunk = chunk or w.chunk
    so = w.seq_off
    num = den = fnum = fden = hnum = hden = 0.0
    fg_all = fin.cpu().numpy()
    npairs = 0
    for s, ha, hb in _pair_blocks(w):
        pairs = [(s, h) for h in range(ha, hb)]
        ys, fs = oracle.recurrence_workload(w, pairs=pairs)
        t0, t1 = int(so[s]), int(so[s + 1])
        if t1 > t0:
            yg = y.view(w.tokens, w.nheads, w.headdim)[t0:t1, ha:hb].float().cpu().numpy()
        for k, h in enumerate(range(ha, hb)):
            ref = ys[k]
            if ref.size:
                got = yg[:, k]
                d = np.abs(got - ref)
                num = max(num, float(d.max()))
                den = max(den, float(np.abs(ref).max()))
                if head_tokens:
                    sel = (np.arange(ref.shape[0]) % chunk) < head_tokens
                    hnum = max(hnum, float(d[sel].max()))
                    hden = max(hden, float(np.abs(ref[sel]).max()))
            fnum = max(fnum, float(np.max(np.abs(fg_all[s, h] - fs[k]))))
            fden = max(fden, float(np.max(np.abs(fs[k]))))
            npairs += 1
    assert npairs == w.nsequences * w.nheads
    ey = num / den if den else num
    ef = fnum / fden if fden else fnum
    msg = (f"  {label or w.name}: all {npairs} (sequence, head) pairs, y rel err {ey:.3e}, "
           f"final rel err {ef:.3e}")
    if head_tokens:
        eh = hnum / hden if hden else hnum
        msg += f", first-{head_tokens}-tokens-of-chunk{chunk} rel err {eh:.3e}"
    say(msg + f" (tol {tol:g})")
    assert ey <= tol, f"y rel err {ey} > {tol}"
    assert ef <= tol, f"final rel err {ef} > {tol}"
    if head_tokens:
        assert eh <= tol, f"chunk-head rel err {eh} > {tol}"
    return ey, ef


def sample_pairs(w, n, seed=0):
    """A spread of (sequence, head) pairs: first/last sequence and head, the
    longest and shortest sequence, plus random ones."""
    r = np.random.default_rng(seed)
    ns, H = w.nsequences, w.nheads
    lens = np.diff(w.seq_off)
    cand = {(0, 0), (ns - 1, H - 1), (int(np.argmax(lens)), H // 2),
            (int(np.argmin(lens)), H - 1)}
    while len(cand) < n:
        cand.add((int(r.integers(ns)), int(r.integers(H))))
    return sorted(cand)[:max(n, 4)]


def check_sampled(w, y, fin, pairs, tol=None, label="", head_tokens=None):
    """Compare sampled (sequence, head) outputs with the oracle, one pair at a
    time.  head_tokens: also report the error on the first k tokens of each
    chunk (where the state handed in dominates)."""
    tol = TOL[w.dtype] if tol is None else tol
    ys, fs = oracle.recurrence_workload(w, pairs=pairs)
    yg = y_host(y, w)
    fg = fin.cpu().numpy()
    so = w.seq_off
    num = den = 0.0
    fnum = fden = 0.0
    hnum = hden = 0.0
    for k, (s, h) in enumerate(pairs):
        ref = ys[k]
        got = yg[so[s]:so[s + 1], h]
        num = max(num, float(np.max(np.abs(got - ref))) if ref.size else 0.0)
        den = max(den, float(np.max(np.abs(ref))) if ref.size else 0.0)
        fnum = max(fnum, float(np.max(np.abs(fg[s, h] - fs[k]))))
        fden = max(fden, float(np.max(np.abs(fs[k]))))
        if head_tokens and ref.size:
            idx = np.arange(ref.shape[0])
            sel = (idx % w.chunk) < head_tokens
            if np.any(sel):
                hnum = max(hnum, float(np.max(np.abs(got[sel] - ref[sel]))))
                hden = max(hden, float(np.max(np.abs(ref[sel]))))
    ey = num / den if den else num
    ef = fnum / fden if fden else fnum
    msg = f"  {label or w.name}: {len(pairs)} pairs, y rel err {ey:.3e}, final rel err {ef:.3e}"
    if head_tokens:
        eh = hnum / hden if hden else hnum
        msg += f", first-{head_tokens}-tokens-of-chunk rel err {eh:.3e}"
    say(msg + f" (tol {tol:g})")
    assert ey <= tol, f"y rel err {ey} > {tol}"
    assert ef <= tol, f"final rel err {ef} > {tol}"
    if head_tokens:
        assert eh <= tol, f"chunk-head rel err {eh} > {tol}"
    return ey, ef
