"""Failure containment on the GPU: a NaN or Inf in the inputs of one
(sequence, head) of a packed batch stays inside that pair.  Every recurrence
h_t = exp(dt_t A_h) h_{t-1} + dt_t x_t B_t^T of one (sequence, head) is
independent of every other (page "State Space Duality and Mamba-2: Unifying
Transformers and Semiseparable Matrices", "Mathematical Foundations"; heads of
a group share only B and C), so a poisoned x or dt of one pair must leave the
y and final state of every other pair finite and bit-identical to a clean run
-- for both forwards.  Poison sits at a sequence's first token (next to the
previous sequence's partial last chunk), at a sequence's last token and in the
middle of a sequence."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mamba_ssd_layer_amd as ssd  # noqa: E402
from gpu_helpers import plan_for, say, upload  # noqa: E402

LENS = [300, 0, 257, 64, 1000, 33, 512, 95]


def _case():
    w = workloads.make_custom(1, 0, 8, 64, 64, 2, 64, "bf16", seed=2100, lens=LENS,
                              init_std=0.3)
    so = w.seq_off
    # (sequence, head, tensor, token) of each poisoned entry
    poison = [(2, 3, "x", int(so[2])),          # first token of sequence 2
              (4, 6, "dt", int(so[5]) - 1),     # last token of sequence 4
              (6, 0, "x", int(so[6]) + 200)]    # middle of sequence 6
    return w, poison


def _poisoned(t, poison):
    p = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    x = p["x"].view(-1, p["x"].shape[-2], p["x"].shape[-1])
    dt = p["dt"].view(-1, p["dt"].shape[-1])
    for _, h, what, tok in poison:
        if what == "x":
            x[tok, h, 5] = float("nan")
        else:
            dt[tok, h] = float("inf")
    return p


def _check(w, poison, y_c, f_c, y_p, f_p, label):
    so = w.seq_off
    bad = {(s, h) for s, h, _, _ in poison}
    H = w.nheads
    yc = y_c.view(w.tokens, H, -1)
    yp = y_p.view(w.tokens, H, -1)
    n = 0
    for s in range(w.nsequences):
        for h in range(H):
            if (s, h) in bad:
                continue
            a, b = yc[so[s]:so[s + 1], h], yp[so[s]:so[s + 1], h]
            assert torch.isfinite(b.float()).all(), f"{label}: y of ({s},{h}) not finite"
            assert torch.equal(a, b), f"{label}: y of ({s},{h}) changed"
            assert torch.isfinite(f_p[s, h]).all(), f"{label}: final of ({s},{h}) not finite"
            assert torch.equal(f_c[s, h], f_p[s, h]), f"{label}: final of ({s},{h}) changed"
            n += 1
    # the poison did reach its own pairs, in y or in the final state (the test
    # is not vacuous).  An infinite dt at a sequence's last token zeroes the
    # decay of everything before it and leaves that token's y to the
    # infinite diagonal term, which the one-pass kernel's clamped exponent
    # keeps finite; the final state is not.
    hit = 0
    for s, h, _, _ in poison:
        hit += int(not (torch.isfinite(yp[so[s]:so[s + 1], h].float()).all()
                        and torch.isfinite(f_p[s, h]).all()))
    say(f"  {label}: {n} clean pairs bit-identical, {hit} of {len(poison)} poisoned pairs "
        "non-finite")
    assert hit == len(poison)


def test_chunked_forward_contains_nonfinite():
    w, poison = _case()
    t = upload(w)
    plan = plan_for(w, t)
    y_c, f_c = plan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"])
    y_c, f_c = y_c.clone(), f_c.clone()
    p = _poisoned(t, poison)
    y_p, f_p = plan(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"], p["cu"])
    torch.cuda.synchronize()
    _check(w, poison, y_c, f_c, y_p, f_p, "four-stage")


def test_fused_forward_contains_nonfinite():
    w, poison = _case()
    t = upload(w)
    y_c, f_c = ssd.fused_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"])
    torch.cuda.synchronize()
    p = _poisoned(t, poison)
    y_p, f_p = ssd.fused_fwd(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"], p["cu"])
    torch.cuda.synchronize()
    _check(w, poison, y_c, f_c, y_p, f_p, "one-pass")
