#!/usr/bin/env python3
"""Benchmark of the Mamba-2 SSD chunked-scan forward (libssd) on one MI355X.

A step is one full forward over one batch of seeded synthetic input already
resident in HBM, timed up to three ways: the chunked forward
(ssd_chunk_scan_fwd: chunk_cumsum, chunk_state, state_passing, chunk_scan);
where its shape is supported, the one-pass forward (ssd_fused_fwd: the same
steps per 32-token chunk with the state kept on chip); and, for few long
fixed-length sequences, the one-pass forward over segments
(ssd_fused_fwd_split).  `value` is the fastest (named in config.path); all are
reported.  Prints one JSON line with whole-job tokens/s, the roofline position
of that path's dominant kernel (the whole path for the split forward; timed
with HIP events on the launch stream), per-kernel figures of the chunked
stages (each
kernel's bandwidth against the published peak and against a plain copy
measured in the same run, and its algorithmic MFMA flops against the peak),
and the CPU oracle timed on a bounded sample of the same workload on the host
cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/sec per layer + % of MFMA/HBM roofline (H=80,P=64,N=128)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector
STAGES = ["chunk_cumsum", "chunk_state", "state_passing", "chunk_scan"]
KERNEL_SOURCES = {
    "chunk_cumsum": "k_scan_prep.hip", "state_passing": "k_scan_prep.hip",
    "chunk_state": "k_chunk_state.hip", "chunk_scan": "k_chunk_scan.hip",
    "fused_fwd": "k_fused.hip", "fused_fwd_split": "k_fused.hip",
}
FUSED_CHUNK = 32  # the one-pass forward's chunk length
FLUSH_BYTES = 1 << 30  # written between timed steps: four times the 256 MB MALL


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def algorithmic(w, stage: str):
    """Compulsory HBM bytes and MFMA flops of one launch of a stage.

    Per token (T tokens, nc chunks, S sequences, s = element bytes of x/B/C/y,
    h = element bytes of the hprev buffer):
      chunk_cumsum   bytes 8 H                      (dt in, cumulative decay out)
      chunk_state    bytes s H P + s G N + 8 H, plus h H P N per chunk (S out, in
                     the io precision like hprev)
                     flops 2 H P N
      state_passing  bytes 2 h H P N per chunk (S in, hprev out), plus 4 H P N per sequence for
                     the final state (and 4 H P N more when an initial state is read)
      chunk_scan     bytes 2 s H P + 2 s G N + 8 H, plus h H P N per chunk
                     flops H (2 P N + (Q + 1) P) + G (Q + 1) N  (causal pairs only,
                     C.B^T once per group)
      fused_fwd      bytes 2 s H P + 2 s G N + 4 H, plus 4 H P N per sequence for
                     the final state (and the initial state when read)
                     flops H (4 P N + 33 P) + 33 G N  (Q = 32: inter, state, intra)
      fused_fwd_split  the forward's, as fused_fwd (its state-only pass re-reads
                     x, B and dt of all segments but the last, and the segment
                     states cross HBM: work of the split, not of the forward)
    """
    T, H, P, N, G, Q = w.tokens, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nseq = w.nsequences
    lens = [int(w.seq_off[i + 1] - w.seq_off[i]) for i in range(nseq)]
    nc = sum(-(-L // Q) for L in lens)
    s = 2 if w.dtype == "bf16" else 4
    hsz = s
    if stage == "chunk_cumsum":
        return 8 * T * H, 0
    if stage == "chunk_state":
        return s * T * H * P + s * T * G * N + 8 * T * H + hsz * nc * H * P * N, 2 * T * H * P * N
    if stage == "state_passing":
        init = 4 * nseq * H * P * N if w.h0 is not None else 0
        return 2 * hsz * nc * H * P * N + 4 * nseq * H * P * N + init, 0
    if stage == "chunk_scan":
        b = 2 * s * T * H * P + 2 * s * T * G * N + 8 * T * H + hsz * nc * H * P * N
        f = T * (H * (2 * P * N + (Q + 1) * P) + G * (Q + 1) * N)
        return b, f
    if stage in ("fused_fwd", "fused_fwd_split"):
        q = FUSED_CHUNK
        init = 4 * nseq * H * P * N if w.h0 is not None else 0
        b = 2 * s * T * H * P + 2 * s * T * G * N + 4 * T * H + 4 * nseq * H * P * N + init
        f = T * (H * (4 * P * N + (q + 1) * P) + G * (q + 1) * N)
        return b, f
    raise KeyError(stage)


def kernel_hash(stage: str) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[stage], "ssd_device.hpp"):
        with open(os.path.join(ROOT, "mamba_ssd_layer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(stage: str, workload: str):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != kernel_hash(stage):
        return None
    return rec.get("traffic_bytes")


def cpu_baseline(w, target_cpu_seconds: float = 20.0):
    """The fp64 oracle, as it stands, on a bounded sample of (sequence, head)
    pairs of the same workload, scaled to tokens/s of the whole workload."""
    import numpy as np
    import oracle
    threads = oracle.max_threads()
    nseq, H = w.nsequences, w.nheads
    total_pairs = nseq * H
    r = np.random.default_rng(1)
    order = [(int(p // H), int(p % H)) for p in r.permutation(total_pairs)]
    # calibrate on one pair, single-threaded
    t0 = time.perf_counter()
    oracle.recurrence_workload(w, pairs=order[:1], nthreads=1)
    per_pair = time.perf_counter() - t0
    n = int(max(1, min(total_pairs, target_cpu_seconds / max(per_pair, 1e-6))))
    n = max(min(threads, total_pairs), (n // threads) * threads)
    n = min(n, total_pairs)
    pairs = order[:n]
    lens = np.diff(w.seq_off)
    sample_tokens = int(sum(lens[s] for s, _ in pairs))  # token-heads in the sample
    t0 = time.perf_counter()
    oracle.recurrence_workload(w, pairs=pairs, nthreads=threads)
    el = time.perf_counter() - t0
    used = min(threads, n)
    # the workload is T tokens x H heads of work; the sample covered sample_tokens token-heads
    value = (sample_tokens / H) / el
    return {"value": value, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{n} of {total_pairs} (sequence, head) pairs of {w.name}, "
                      f"{sample_tokens} token-heads, fp64 recurrence, {el:.2f} s wall on {used} "
                      f"threads ({per_pair:.2f} s for one pair on one thread)"}


def copy_bandwidth(torch, dev, mib: int = 1024, reps: int = 5) -> float:
    """GB/s of a plain elementwise copy (dst = -src, fp32, one read and one
    write per element) of mib MiB: the bandwidth a streaming kernel can reach
    on this GPU, next to the published 8 TB/s."""
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        torch.neg(src, out=dst)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return 2 * n * 4 / t / 1e9


def decode_step(torch, ssd, workloads, dev, steps: int, warmup: int):
    """ssd_step on a serving-sized batch: 128 sequences, the large layer's heads
    and state (H80 P64 N128, bf16 io), one token each.  The fp32 state (671 MB)
    exceeds the 256 MB MALL, so every step streams it from HBM; the step is
    bound by reading and writing it once."""
    import numpy as np
    w = workloads.make_custom(128, 1, 80, 64, 128, 1, 64, "bf16", seed=5000, init_std=0.1)
    S, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups

    def up(a, shape, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return (t.to(dtype) if dtype is not None else t).view(*shape).contiguous()

    x = up(w.x, (S, H, P), torch.bfloat16)
    dt = up(w.dt, (S, H))
    A = up(w.A, (H,))
    Bm = up(w.B, (S, G, N), torch.bfloat16)
    Cm = up(w.C, (S, G, N), torch.bfloat16)
    D = up(w.D, (H,))
    state = up(w.h0, (S, H, P, N))
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        ssd.step(x, dt, A, Bm, Cm, state, D=D, y=y)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        ssd.step(x, dt, A, Bm, Cm, state, D=D, y=y)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    nbytes = 2 * S * H * P * N * 4 + 2 * S * H * P * 2 + 2 * S * G * N * 2 + S * H * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"bench: decode step S{S} H{H} P{P} N{N}: {us:.1f} us, {gbs:.0f} GB/s")
    return {"workload": f"decode_s{S}_h{H}_p{P}_n{N}_g{G}_bf16", "sequences": S, "us": round(us, 2),
            "tokens_per_s": round(S / (us * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": nbytes}}


def block_neighbours(torch, ssd, dev, w, steps: int, warmup: int):
    """The core's neighbours at the workload's widths: the causal conv1d + SiLU
    over x|B|C (H*P + 2*G*N channels) and the SiLU gate + RMS norm over y
    (H*P channels), on seeded synthetic bf16 inputs generated on the device.
    Both are HBM-bound; bytes = one read of each input and one write."""
    gen = torch.Generator(device=dev).manual_seed(6000)
    T, HP, GN = w.tokens, w.nheads * w.headdim, w.ngroups * w.dstate
    lead = (w.batch, w.seqlen) if not w.nseq else (1, T)
    C = HP + 2 * GN
    xbc = torch.randn(*lead, C, generator=gen, device=dev).to(torch.bfloat16)
    cw = torch.randn(C, 4, generator=gen, device=dev) * 0.5
    cb = torch.randn(C, generator=gen, device=dev) * 0.1
    y = torch.randn(T, HP, generator=gen, device=dev).to(torch.bfloat16)
    z = torch.randn(T, HP, generator=gen, device=dev).to(torch.bfloat16)
    nw = 1.0 + 0.1 * torch.randn(HP, generator=gen, device=dev)
    cout = torch.empty_like(xbc)
    gout = torch.empty_like(y)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    res = {}
    for name, fn, nbytes in (
            ("conv1d_silu", lambda: ssd.conv1d_silu(xbc, cw, cb, out=cout), 2 * xbc.numel() * 2),
            ("gate_rmsnorm", lambda: ssd.gate_rmsnorm(y, z, nw, 1e-5, out=gout), 3 * y.numel() * 2)):
        us = timed(fn)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "bytes": nbytes, "GBs": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"bench: {name}: {us:.1f} us, {gbs:.0f} GB/s")
    res["widths"] = {"conv_channels": C, "gate_channels": HP, "tokens": T}
    return res


def backward_bytes(w):
    """Compulsory HBM bytes of the two backward kernels (bf16 io, s = 2; S
    sequences; states kept per 64-token pair, p = the batch's pairs, one
    s P N tile per pair and head):
      k_bwd_reverse  dy, C, dt in; the state gradient leaving every pair out;
                     dfinal in and dinit out per sequence:
                     s T H P + s T G N + 4 T H + s p H P N + 8 S H P N
      k_bwd_chunk    x, dy, B, C, dt, every pair's saved state and state
                     gradient in; dx, ddt, dB, dC (float) out:
                     3 s T H P + 2 s T G N + 8 T H + 8 T G N + 2 s p H P N
    (the neighbour-chunk rows a block also reads, and the second read of a
    pair's tiles, are re-reads the kernel arranges to hit L2)"""
    T, H, P, N, G = w.tokens, w.nheads, w.headdim, w.dstate, w.ngroups
    S = w.nsequences
    lens = [int(w.seq_off[i + 1] - w.seq_off[i]) for i in range(S)]
    pr = sum(-(-L // 64) for L in lens)
    s = 2
    rev = s * T * H * P + s * T * G * N + 4 * T * H + s * pr * H * P * N + 8 * S * H * P * N
    chk = 3 * s * T * H * P + 2 * s * T * G * N + 8 * T * H + 8 * T * G * N + 2 * s * pr * H * P * N
    return rev, chk


def training_step(torch, ssd, workloads, w, t, steps: int, warmup: int):
    """A forward that leaves the state entering every 64-token chunk, then the
    backward (ssd_fused_bwd) for seeded upstream gradients dy, dfinal; each
    timed with HIP events on the launch stream. Three or four forwards leave
    those states: the one-pass forward saving them (ssd_fused_fwd_train), the
    four-stage forward with chunk length 64 (its hprev), SSDTrainForward (y
    from the four stages at chunk length 256, the states from the first three
    at chunk length 64) and, where the library cuts the sequences, the split
    one-pass forward saving them (ssd_fused_fwd_split_train); the fastest is
    the step's forward (fwd_train_path), the others are reported beside it."""
    dev = t["x"].device
    dy, dfinal = workloads.make_output_grads(w, 6100)
    dyd = torch.from_numpy(dy).to(dev).to(torch.bfloat16).view(t["x"].shape)
    dfd = torch.from_numpy(dfinal).to(dev)
    states = ssd.make_fused_states(t["x"], t["B"], t["cu"])
    ws = torch.empty(ssd.libssd.ssd_fused_bwd_workspace_size(ssd.dims_for(t["x"], t["B"], t["cu"])),
                     dtype=torch.uint8, device=dev)
    y = torch.empty_like(t["x"])
    fin = torch.empty_like(dfd)
    stream = torch.cuda.current_stream()

    def fwd():
        ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"], y=y,
                      final_state=fin, chunk_states=states)

    plan64 = ssd.SSDForward(ssd.dims_for(t["x"], t["B"], t["cu"]), 64, device=dev)

    def fwd64():
        plan64(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"], y=y,
               final_state=fin)

    tplan = ssd.SSDTrainForward(ssd.dims_for(t["x"], t["B"], t["cu"]), device=dev)

    def fwd_split():
        tplan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"], y=y,
              final_state=fin)

    # the split one-pass forward saving the states, where the library cuts the
    # sequences (fixed-length batches; segments a multiple of 64 tokens)
    dims = ssd.dims_for(t["x"], t["B"], t["cu"])
    seg = ssd.libssd.ssd_fused_split_seg_len(dims) if not w.nseq else 0
    fwd_seg = None
    if 0 < seg < w.seqlen and seg % 64 == 0:
        wseg = torch.empty(max(1, ssd.libssd.ssd_fused_split_workspace_size(dims, seg)),
                           dtype=torch.uint8, device=dev)

        def fwd_seg():
            ssd.fused_fwd_split(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], y=y,
                                final_state=fin, seg_len=seg, workspace=wseg,
                                chunk_states=states)

    def bwd():
        ssd.fused_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], states, dyd, dfd, t["cu"],
                      workspace=ws)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    by_path = {"ssd_fused_fwd_train": timed(fwd), "ssd_chunk_scan_fwd_q64": timed(fwd64),
               "SSDTrainForward": timed(fwd_split)}
    if fwd_seg is not None:
        by_path["ssd_fused_fwd_split_train"] = timed(fwd_seg)
    bus = timed(bwd)
    path = min(by_path, key=by_path.get)
    fus = by_path[path]
    rev, chk = backward_bytes(w)
    T = w.tokens
    res = {"fwd_train_us": round(fus, 2), "fwd_train_path": path,
           "fwd_train_us_by_path": {k: round(v, 2) for k, v in by_path.items()},
           "bwd_us": round(bus, 2),
           "tokens_per_s": round(T / ((fus + bus) * 1e-6), 1),
           "bwd_tokens_per_s": round(T / (bus * 1e-6), 1),
           "bwd_bytes": {"k_bwd_reverse": rev, "k_bwd_chunk": chk},
           "bwd_GBs": round((rev + chk) / (bus * 1e-6) / 1e9, 1),
           "bwd_hbm_frac": round((rev + chk) / (bus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"bench: training step: forward saving states {by_path['ssd_fused_fwd_train']:.1f} us "
        f"(one-pass), {by_path['ssd_chunk_scan_fwd_q64']:.1f} us (four-stage, chunk 64), "
        f"{by_path['SSDTrainForward']:.1f} us (chunk 256 + chunk-64 states), "
        + (f"{by_path['ssd_fused_fwd_split_train']:.1f} us (split one-pass), "
           if "ssd_fused_fwd_split_train" in by_path else "")
        + f"backward {bus:.1f} us, "
        f"{res['tokens_per_s'] / 1e6:.1f} M tokens/s")
    return res


def training_step_general(torch, ssd, workloads, w, t, plan, steps: int, warmup: int):
    """The training step where the fast backward does not take the shape (fp32
    io, N = 256, head dims other than 64): the four-stage forward, then the
    general backward (ssd_chunk_scan_bwd: the chunk states formed again, every
    gradient on the vector ALU), each timed with HIP events on the launch
    stream."""
    dev = t["x"].device
    dy, dfinal = workloads.make_output_grads(w, 6100)
    dyd = torch.from_numpy(dy).to(dev).to(t["x"].dtype).view(t["x"].shape)
    dfd = torch.from_numpy(dfinal).to(dev)
    dims = ssd.dims_for(t["x"], t["B"], t["cu"])
    ws = torch.empty(ssd.libssd.ssd_chunk_scan_bwd_workspace_size(dims), dtype=torch.uint8,
                     device=dev)
    y = torch.empty_like(t["x"])
    fin = torch.empty_like(dfd)
    stream = torch.cuda.current_stream()

    def fwd():
        plan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"], y=y,
             final_state=fin)

    def bwd():
        ssd.chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dyd, dfd,
                           init_state=t["h0"], cu_seqlens=t["cu"], workspace=ws)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    fus, bus = timed(fwd), timed(bwd)
    T = w.tokens
    res = {"fwd_train_us": round(fus, 2), "fwd_train_path": "ssd_chunk_scan_fwd",
           "bwd_path": "ssd_chunk_scan_bwd", "bwd_us": round(bus, 2),
           "tokens_per_s": round(T / ((fus + bus) * 1e-6), 1),
           "bwd_tokens_per_s": round(T / (bus * 1e-6), 1)}
    log(f"bench: training step (general backward): forward {fus:.1f} us, backward {bus:.1f} us, "
        f"{res['tokens_per_s'] / 1e6:.2f} M tokens/s")
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stage-timing", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the single-token decode (ssd_step) measurement")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the forward-with-saved-states + backward timing")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the conv1d+SiLU and gate+RMS-norm measurements")
    ap.add_argument("--settle-ms", type=float, default=2500.0,
                    help="untimed forward steps for this long before the first timed region, so "
                         "every path is timed at the GPU's sustained clock")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run 3 elementwise copies (dst = -src, one read and one write per "
                         "element) of MIB MiB: a known-size reference for the hardware byte "
                         "counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: libssd has no multi-GPU path (the SSD forward "
              "shards over (sequence, head) with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mamba_ssd_layer_amd as ssd
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"bench: copy calibration, 3 copies of {n} bytes ({args.calibrate_copy} MiB read + "
            f"{args.calibrate_copy} MiB written each)")
        del src, dst
    log(f"bench: generating workload {args.workload}")
    w = workloads.make_workload(args.workload)
    io = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T, H, P, G, N = w.tokens, w.nheads, w.headdim, w.ngroups, w.dstate
    lead = (1, T) if w.nseq else (w.batch, w.seqlen)

    def up(a, shape, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return (t.to(dtype) if dtype is not None else t).view(*shape).contiguous()

    x = up(w.x, (*lead, H, P), io)
    dt = up(w.dt, (*lead, H))
    A = up(w.A, (H,))
    Bm = up(w.B, (*lead, G, N), io)
    Cm = up(w.C, (*lead, G, N), io)
    D = up(w.D, (H,))
    h0 = up(w.h0, w.h0.shape) if w.h0 is not None else None
    cu = up(w.cu_seqlens, (w.nseq + 1,)) if w.nseq else None
    dims = ssd.dims_for(x, Bm, cu)
    plan = ssd.SSDForward(dims, w.chunk, device=dev)
    y = torch.empty_like(x)
    fin = torch.empty((w.nsequences, H, P, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"bench: {T} tokens, workspace {plan.layout.total_bytes / 2**20:.1f} MiB; "
        f"{args.warmup} warmup + {args.steps} timed steps")

    def step():
        plan(x, dt, A, Bm, Cm, D, h0, cu, y=y, final_state=fin)

    # between timed steps, a buffer four times the 256 MB MALL is written and
    # then read, so no step starts with its inputs or intermediates in the
    # memory-side cache; the read leaves the MALL holding clean lines (after
    # the write alone it holds 256 MB of dirty ones, which the next timed
    # kernel would pay to write back: chunk_state 111 -> 170 us at the large
    # layer)
    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sum = torch.empty((), dtype=torch.float32, device=dev)

    def flush(i: int = 0) -> None:
        flush_buf.fill_(float(i))
        torch.sum(flush_buf, dim=0, out=flush_sum)

    # clock settling before anything is timed: the GPU starts from idle clocks
    # and takes over a second of sustained work to reach its steady clock, so
    # the first timed path would otherwise run partly below it (untimed; the
    # timed regions below are exactly `steps` steps each)
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_ms * 1e-3:
        flush()
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed_steps(fn):
        """Per-launch durations (us) of `steps` launches of fn, each bracketed
        by HIP events on the launch stream with a MALL flush before it; plus
        the wall time of the whole region."""
        evs = []
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i in range(args.steps):
            flush(i)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in evs], time.perf_counter() - w0

    def back_to_back(fn):
        """Mean duration (us) of `steps` launches issued back to back (no flush)."""
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e3

    def summary(per, wall):
        return {"us": round(float(np.median(per)), 2), "mean_us": round(float(np.mean(per)), 2),
                "min_us": round(float(np.min(per)), 2), "max_us": round(float(np.max(per)), 2),
                "wall_s": round(wall, 3)}

    per, wall = timed_steps(step)
    chunked_t = summary(per, wall)
    chunked_t["back_to_back_us"] = round(back_to_back(step), 2)
    ms = chunked_t["us"] / 1e3
    value = T / (ms / 1e3)
    log(f"bench: chunked forward median {chunked_t['us']:.1f} us/step (flushed; mean "
        f"{chunked_t['mean_us']:.1f}, back to back {chunked_t['back_to_back_us']:.1f}), "
        f"{value / 1e6:.1f} M tokens/s")

    # the one-pass forward on the same inputs, where its shape is supported
    fused = None
    if w.dtype == "bf16" and ssd.libssd.ssd_fused_states_size(dims) > 0:
        yf = torch.empty_like(x)
        ff = torch.empty_like(fin)

        def fstep():
            ssd.fused_fwd(x, dt, A, Bm, Cm, D, h0, cu, y=yf, final_state=ff)

        for _ in range(args.warmup):
            fstep()
        fper, fwall = timed_steps(fstep)
        fsum = summary(fper, fwall)
        fsum["back_to_back_us"] = round(back_to_back(fstep), 2)
        fb, ff_ = algorithmic(w, "fused_fwd")
        ft = fsum["us"] * 1e-6
        fused = {**fsum, "tokens_per_s": round(T / ft, 1), "bytes": fb, "flops": ff_,
                 "GBs": round(fb / ft / 1e9, 1), "TFLOPs": round(ff_ / ft / 1e12, 2),
                 "hbm_frac": round(fb / ft / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"bench: one-pass forward median {fsum['us']:.1f} us/step (flushed; mean "
            f"{fsum['mean_us']:.1f}, back to back {fsum['back_to_back_us']:.1f}), "
            f"{T / ft / 1e6:.1f} M tokens/s")

    # the split one-pass forward, where the library cuts the sequences into
    # segments (few long fixed-length sequences)
    split = None
    seg_len = ssd.libssd.ssd_fused_split_seg_len(dims) if fused is not None and not w.nseq else 0
    if 0 < seg_len < w.seqlen:
        ys_ = torch.empty_like(x)
        fs_ = torch.empty_like(fin)
        wsp = torch.empty(ssd.libssd.ssd_fused_split_workspace_size(dims, seg_len),
                          dtype=torch.uint8, device=dev)

        def sstep():
            ssd.fused_fwd_split(x, dt, A, Bm, Cm, D, h0, y=ys_, final_state=fs_, seg_len=seg_len,
                                workspace=wsp)

        for _ in range(args.warmup):
            sstep()
        sper, swall = timed_steps(sstep)
        ssum = summary(sper, swall)
        ssum["back_to_back_us"] = round(back_to_back(sstep), 2)
        sb, sf = algorithmic(w, "fused_fwd_split")
        st_ = ssum["us"] * 1e-6
        split = {**ssum, "seg_len": seg_len, "tokens_per_s": round(T / st_, 1), "bytes": sb,
                 "flops": sf, "GBs": round(sb / st_ / 1e9, 1),
                 "TFLOPs": round(sf / st_ / 1e12, 2),
                 "hbm_frac": round(sb / st_ / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"bench: split one-pass forward (segments of {seg_len}) median {ssum['us']:.1f} "
            f"us/step (flushed; mean {ssum['mean_us']:.1f}, back to back "
            f"{ssum['back_to_back_us']:.1f}), {T / st_ / 1e6:.1f} M tokens/s")

    # per-stage times: the same stages launched one by one, each after a
    # MALL flush, HIP events around each launch (median over steps)
    stage_us, stage_mean_us = {}, {}
    if not args.no_stage_timing:
        calls = {
            "chunk_cumsum": lambda: plan.cumsum(dt, A, cu),
            "chunk_state": lambda: plan.state(x, Bm),
            "state_passing": lambda: plan.passing(h0, fin),
            "chunk_scan": lambda: plan.scan(x, Bm, Cm, D, y),
        }
        evs = {s_: [] for s_ in STAGES}
        for i in range(args.steps):
            for s_ in STAGES:
                flush(i)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                calls[s_]()
                e1.record(stream)
                evs[s_].append((e0, e1))
        torch.cuda.synchronize()
        for s_ in STAGES:
            d_ = [a_.elapsed_time(b_) * 1e3 for a_, b_ in evs[s_]]
            stage_us[s_] = float(np.median(d_))
            stage_mean_us[s_] = float(np.mean(d_))
    del flush_buf
    copy_gbs = copy_bandwidth(torch, dev)
    log(f"bench: plain copy {copy_gbs:.0f} GB/s")

    def fracs(b, f, t):
        """achieved bandwidth as a fraction of the measured copy's, and
        algorithmic flops as a fraction of the MFMA peak"""
        mfma_peak = BF16_MFMA_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
        return {"copy_frac": round(b / t / 1e9 / copy_gbs, 4),
                "mfma_frac": round(f / t / 1e12 / mfma_peak, 4)}

    if fused is not None:
        fused.update(fracs(fused["bytes"], fused["flops"], fused["us"] * 1e-6))
    if split is not None:
        split.update(fracs(split["bytes"], split["flops"], split["us"] * 1e-6))
    kernels = {}
    for s in STAGES:
        b, f = algorithmic(w, s)
        entry = {"bytes": b, "flops": f}
        if s in stage_us:
            t = stage_us[s] * 1e-6
            entry.update(us=round(stage_us[s], 2), mean_us=round(stage_mean_us[s], 2), GBs=round(b / t / 1e9, 1),
                         TFLOPs=round(f / t / 1e12, 2) if f else 0.0,
                         hbm_frac=round(b / t / 1e9 / HBM_PEAK_GBS, 4), **fracs(b, f, t))
        kernels[s] = entry
    def roofline_of(kernel: str, us: float):
        b, f = algorithmic(w, kernel)
        t = us * 1e-6
        mfma_peak = BF16_MFMA_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
        t_hbm = b / (HBM_PEAK_GBS * 1e9)
        t_mfma = f / (mfma_peak * 1e12)
        if t_hbm >= t_mfma:
            r = {"bound": "hbm", "achieved": round(b / t / 1e9, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s"}
        else:
            r = {"bound": "mfma" if w.dtype == "bf16" else "alu",
                 "achieved": round(f / t / 1e12, 2), "peak": mfma_peak, "unit": "TFLOP/s"}
        r["frac"] = round(r["achieved"] / r["peak"], 4)
        r["traffic"] = load_traffic(kernel, w.name)
        r.update(fracs(b, f, t))
        r["kernel"] = kernel
        r["kernel_us"] = round(us, 2)
        r["algorithmic_bytes"] = b
        r["algorithmic_flops"] = f
        return r

    chunked_roofline = None
    if stage_us:
        dom = max(stage_us, key=stage_us.get)
        chunked_roofline = roofline_of(dom, stage_mean_us[dom])
    chunked = {**chunked_t, "tokens_per_s": round(value, 1), "roofline": chunked_roofline}
    path, roofline, ms_step = "ssd_chunk_scan_fwd", chunked_roofline, ms
    if fused is not None:
        fused["roofline"] = roofline_of("fused_fwd", fused["mean_us"])
        if fused["us"] < ms_step * 1e3:
            path, roofline, ms_step, value = ("ssd_fused_fwd", fused["roofline"], fused["us"] / 1e3,
                                              fused["tokens_per_s"])
    if split is not None:
        # three launches (state-only pass, hand-off, forward): the roofline of
        # the whole path, its algorithmic bytes over its mean time
        split["roofline"] = roofline_of("fused_fwd_split", split["mean_us"])
        if split["us"] < ms_step * 1e3:
            path, roofline, ms_step, value = ("ssd_fused_fwd_split", split["roofline"],
                                              split["us"] / 1e3, split["tokens_per_s"])

    decode = None
    if not args.no_decode:
        decode = decode_step(torch, ssd, workloads, dev, args.steps, args.warmup)

    train = None
    tens = {"x": x, "dt": dt, "A": A, "B": Bm, "C": Cm, "D": D, "h0": h0, "cu": cu}
    if fused is not None and not args.no_train and ssd.libssd.ssd_fused_bwd_workspace_size(dims) > 0:
        train = training_step(torch, ssd, workloads, w, tens, args.steps, args.warmup)
    elif not args.no_train and ssd.libssd.ssd_chunk_scan_bwd_workspace_size(dims) > 0:
        train = training_step_general(torch, ssd, workloads, w, tens, plan, args.steps,
                                      args.warmup)

    block = None
    if not args.no_block:
        block = block_neighbours(torch, ssd, dev, w, args.steps, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample")
        cpu = cpu_baseline(w)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "timing": (f"value: the median of {args.steps} launches, each after a "
                   f"{FLUSH_BYTES >> 20} MiB write and read that flush the 256 MB MALL, HIP events "
                   "on the launch stream; roofline.achieved: algorithmic bytes / the mean of the "
                   "same launches"),
        "config": {**workloads.describe(w), "path": path,
                   "chunk": FUSED_CHUNK if path.startswith("ssd_fused_fwd") else w.chunk,
                   **({"seg_len": split["seg_len"]} if path == "ssd_fused_fwd_split" else {}),
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline, "cpu_baseline": cpu,
        "forwards": {"ssd_chunk_scan_fwd": chunked, "ssd_fused_fwd": fused,
                     "ssd_fused_fwd_split": split},
        "kernels": kernels, "copy_GBs": round(copy_gbs, 1), "decode_step": decode,
        "block_neighbours": block,
        "training_step": train,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
