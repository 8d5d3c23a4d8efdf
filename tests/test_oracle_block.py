"""Pins of the block-neighbour oracle (oracle/block.py) on the CPU: library
routines (torch's conv1d, silu and rms_norm in fp64), closed forms and
invariants -- chosen so that a dropped term, an off-by-one in the causal
window or a missing reset at a sequence start fails one of them."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import block as ob

RNG = np.random.default_rng(11)


def seqs(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def torch_conv_silu(inp, w, b, seq_off):
    """Per sequence: depthwise conv1d with left padding K-1, truncated."""
    K = w.shape[1]
    outs = []
    for s in range(len(seq_off) - 1):
        seg = torch.from_numpy(inp[seq_off[s]:seq_off[s + 1]].T[None])  # [1, C, L]
        L = seg.shape[-1]
        o = F.conv1d(seg, torch.from_numpy(w)[:, None, :], None if b is None else torch.from_numpy(b),
                     padding=K - 1, groups=w.shape[0])[..., :L]
        outs.append(F.silu(o)[0].T.numpy())
    return np.concatenate(outs, 0)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_matches_torch(K):
    lens = [7, 1, 12, 5]
    inp = RNG.standard_normal((sum(lens), 6))
    w = RNG.standard_normal((6, K))
    b = RNG.standard_normal(6)
    off = seqs(lens)
    np.testing.assert_allclose(ob.conv1d_silu(inp, w, b, off), torch_conv_silu(inp, w, b, off),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ob.conv1d_silu(inp, w, None, off), torch_conv_silu(inp, w, None, off),
                               rtol=1e-12, atol=1e-12)


def test_conv_width_one_is_pointwise():
    inp = RNG.standard_normal((9, 4))
    w = RNG.standard_normal((4, 1))
    b = RNG.standard_normal(4)
    got = ob.conv1d_silu(inp, w, b, seqs([9]))
    v = inp * w[:, 0] + b
    np.testing.assert_allclose(got, v / (1 + np.exp(-v)), rtol=1e-13)


@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_conv_shift_kernels_and_reset(k):
    # weight e_k on a width-4 kernel: out[t] = silu(inp[t - 3 + k]) inside a
    # sequence, silu(0) = 0 where that position precedes the sequence start
    lens = [5, 2, 6]
    off = seqs(lens)
    inp = RNG.standard_normal((sum(lens), 3))
    w = np.zeros((3, 4))
    w[:, k] = 1.0
    got = ob.conv1d_silu(inp, w, None, off)
    want = np.zeros_like(inp)
    for s in range(len(lens)):
        for t in range(off[s], off[s + 1]):
            src = t - 3 + k
            if src >= off[s]:
                want[t] = inp[src] / (1 + np.exp(-inp[src]))
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)


def test_silu_values():
    v = np.array([-800.0, -3.0, 0.0, 2.5, 800.0])
    np.testing.assert_allclose(ob.silu(v), F.silu(torch.from_numpy(v)).numpy(), rtol=1e-14, atol=1e-300)
    assert ob.silu(np.array([0.0]))[0] == 0.0
    assert ob.silu(np.array([800.0]))[0] == 800.0


def test_gate_alone():
    y = RNG.standard_normal((4, 10))
    z = RNG.standard_normal((4, 10))
    np.testing.assert_allclose(ob.gate_rmsnorm(y, z, None, 1e-5), y * z / (1 + np.exp(-z)), rtol=1e-13)
    assert np.all(ob.gate_rmsnorm(y, np.zeros_like(z), None, 1e-5) == 0)


@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_rmsnorm_matches_torch(eps):
    y = RNG.standard_normal((5, 16))
    z = RNG.standard_normal((5, 16))
    w = RNG.standard_normal(16)
    g = torch.from_numpy(y) * F.silu(torch.from_numpy(z))
    want = F.rms_norm(g, (16,), torch.from_numpy(w), eps).numpy()
    np.testing.assert_allclose(ob.gate_rmsnorm(y, z, w, eps), want, rtol=1e-12, atol=1e-12)


def test_rmsnorm_scale_invariance():
    # with eps = 0, scaling y by a > 0 leaves the normalised output unchanged
    y = RNG.standard_normal((3, 32))
    z = RNG.standard_normal((3, 32))
    w = RNG.standard_normal(32)
    np.testing.assert_allclose(ob.gate_rmsnorm(7.5 * y, z, w, 0.0), ob.gate_rmsnorm(y, z, w, 0.0),
                               rtol=1e-12)


def test_mutants_are_caught():
    # planted mistakes in copies of the oracle are caught by the pins above
    lens = [6, 3]
    off = seqs(lens)
    inp = RNG.standard_normal((9, 2))
    w = RNG.standard_normal((2, 4))
    ref = torch_conv_silu(inp, w, None, off)

    def no_reset(inp, w, b, seq_off):  # window reaches across sequence starts
        return ob.conv1d_silu(inp, w, b, np.array([0, seq_off[-1]]))

    def off_by_one(inp, w, b, seq_off):  # window shifted one token late
        K = w.shape[1]
        w2 = np.concatenate([np.zeros((w.shape[0], 1)), w[:, :K - 1]], 1)
        return ob.conv1d_silu(inp, w2, b, seq_off)

    for mut in (no_reset, off_by_one):
        assert not np.allclose(mut(inp, w, None, off), ref, rtol=1e-9, atol=1e-9), mut.__name__
