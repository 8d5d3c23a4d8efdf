"""The algorithmic byte and flop counts bench.py divides measured times by,
recomputed here term by term from the tensor sizes of the large layer
(B 8, L 4096, H 80, P 64, N 128, G 1, bf16; chunk 256 for the four stages, 32
for the one-pass forward), so a slip in the accounting (a missing tensor, a
wrong element size, a per-group term counted per head) shows up on the CPU."""
import importlib.util
import os
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)

B, L, H, P, N, G = 8, 4096, 80, 64, 128, 1
T = B * L
NC = B * (L // 256)   # chunks of 256 tokens
S2 = 2                # bf16 element bytes (x, B, C, y, chunk states, hprev)


def large():
    # the sizes the accounting reads, without drawing the tensors
    return SimpleNamespace(tokens=T, nheads=H, headdim=P, dstate=N, ngroups=G, chunk=256,
                           dtype="bf16", h0=None, nsequences=B,
                           seq_off=np.arange(B + 1, dtype=np.int64) * L)


def test_stage_bytes_and_flops():
    w = large()
    x = T * H * P * S2          # x (or y) once
    bc = T * G * N * S2         # B (or C) once
    dt = T * H * 4
    states = NC * H * P * N * S2
    final = B * H * P * N * 4
    assert bench.algorithmic(w, "chunk_cumsum") == (2 * dt, 0)          # dt in, acum out
    assert bench.algorithmic(w, "chunk_state") == (x + bc + 2 * dt + states, 2 * T * H * P * N)
    # S in, hprev out, the final state out (no initial state in this workload)
    assert bench.algorithmic(w, "state_passing") == (2 * states + final, 0)
    Q = 256
    flops_scan = T * (H * (2 * P * N + (Q + 1) * P) + G * (Q + 1) * N)
    assert bench.algorithmic(w, "chunk_scan") == (2 * x + 2 * bc + 2 * dt + states, flops_scan)


def test_fused_forward_accounting():
    w = large()
    b, f = bench.algorithmic(w, "fused_fwd")
    x = T * H * P * S2
    bc = T * G * N * S2
    # x in, y out, B and C in, dt in (4 bytes), the final state out
    assert b == 2 * x + 2 * bc + T * H * 4 + B * H * P * N * 4
    assert f == T * (H * (4 * P * N + 33 * P) + 33 * G * N)


def test_backward_accounting():
    w = large()
    rev, chk = bench.backward_bytes(w)
    pairs = B * (L // 64)
    tile = H * P * N * S2
    x = T * H * P * S2
    bc = T * G * N * S2
    assert rev == x + bc + 4 * T * H + pairs * tile + 8 * B * H * P * N
    assert chk == 3 * x + 2 * bc + 8 * T * H + 8 * T * G * N + 2 * pairs * tile
