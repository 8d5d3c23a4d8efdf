"""Pins of the backward oracle (oracle.recurrence_bwd) to things other than
itself, on the CPU.

L = sum_t <dy_t, y_t> + <dfinal, final>, evaluated by the plain-numpy forward
recurrence (oracle.recurrence_py, fp64 throughout):
  * x, B, C, D, h0 enter the forward linearly (each with the others fixed), so
    for any direction V:  L(theta + V) - L(theta) = <dL/dtheta, V>  exactly, up
    to rounding;
  * dt and A enter through exp(dt A) and the input weight: central finite
    differences of L along random directions;
  * dh0 of an empty sequence is dfinal itself; dD is sum_t <dy_t, x_t>.
A dropped term, a wrong sign, a transposed operand or a missed group sum in the
chain rule breaks one of these.
"""
import numpy as np
import pytest

import oracle



def problem(seed=3, lens=(5, 0, 7), H=4, P=3, N=5, G=2):
    r = np.random.default_rng(seed)
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    T = int(sum(lens))
    seq_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    p = dict(x=f(T, H, P), dt=(np.log1p(np.exp(f(T, H))) * 0.7).astype(np.float32),
             A=(-np.exp(r.uniform(-1, 1.5, H))).astype(np.float32),
             B=f(T, G, N), C=f(T, G, N), D=f(H), h0=f(len(lens), H, P, N) * np.float32(0.5))
    dy = f(T, H, P)
    dfin = f(len(lens), H, P, N)
    return p, seq_off, dy, dfin


def loss(p, seq_off, dy, dfin):
    y, fin = oracle.recurrence_py(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"],
                                  seq_off)
    return float(np.sum(dy.astype(np.float64) * y) + np.sum(dfin.astype(np.float64) * fin))


def grads(p, seq_off, dy, dfin):
    return oracle.recurrence_bwd(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"],
                                 seq_off, dy, dfin)


@pytest.mark.parametrize("name,gname", [("x", "dx"), ("B", "dB"), ("C", "dC"), ("D", "dD"),
                                        ("h0", "dh0")])
def test_adjoint_identity_for_linear_inputs(name, gname):
    p, so, dy, dfin = problem()
    g = grads(p, so, dy, dfin)
    r = np.random.default_rng(11)
    L0 = loss(p, so, dy, dfin)
    for _ in range(3):
        V = r.standard_normal(p[name].shape)
        q = dict(p)
        q[name] = p[name].astype(np.float64) + V
        lhs = loss(q, so, dy, dfin) - L0
        rhs = float(np.sum(g[gname] * V))
        assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(rhs)), (name, lhs, rhs)


@pytest.mark.parametrize("name,gname", [("dt", "ddt"), ("A", "dA")])
def test_finite_differences_for_decay_inputs(name, gname):
    p, so, dy, dfin = problem(seed=5)
    g = grads(p, so, dy, dfin)
    r = np.random.default_rng(13)
    for _ in range(3):
        V = r.standard_normal(p[name].shape)
        eps = 1e-6
        qp, qm = dict(p), dict(p)
        qp[name] = p[name].astype(np.float64) + eps * V
        qm[name] = p[name].astype(np.float64) - eps * V
        fd = (loss(qp, so, dy, dfin) - loss(qm, so, dy, dfin)) / (2 * eps)
        an = float(np.sum(g[gname] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_closed_forms():
    p, so, dy, dfin = problem(seed=7)
    g = grads(p, so, dy, dfin)
    # the empty sequence passes dfinal straight through to dh0
    assert np.array_equal(g["dh0"][1], dfin[1].astype(np.float64))
    # dD = sum_t <dy_t, x_t> per head
    ref = np.einsum("thp,thp->h", dy.astype(np.float64), p["x"].astype(np.float64))
    assert np.allclose(g["dD"], ref, rtol=1e-12, atol=1e-12)


def test_pairs_match_full_run():
    p, so, dy, dfin = problem(seed=9)
    full = grads(p, so, dy, dfin)
    pairs = [(0, 1), (2, 3)]
    part = oracle.recurrence_bwd(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"], so,
                                 dy, dfin, pairs=pairs)
    for s, h in pairs:
        t0, t1 = so[s], so[s + 1]
        assert np.array_equal(part["dx"][t0:t1, h], full["dx"][t0:t1, h])
        assert np.array_equal(part["ddt"][t0:t1, h], full["ddt"][t0:t1, h])
        assert np.array_equal(part["dh0"][s, h], full["dh0"][s, h])


def test_long_sequence_across_checkpoints():
    # 150 tokens: the reverse sweep recomputes the states from checkpoints
    # taken every 64 tokens
    p, so, dy, dfin = problem(seed=21, lens=(150, 3), H=2, P=2, N=3, G=1)
    g = grads(p, so, dy, dfin)
    r = np.random.default_rng(23)
    L0 = loss(p, so, dy, dfin)
    V = r.standard_normal(p["x"].shape)
    q = dict(p)
    q["x"] = p["x"].astype(np.float64) + V
    rhs = float(np.sum(g["dx"] * V))
    assert abs(loss(q, so, dy, dfin) - L0 - rhs) <= 1e-9 * max(1.0, abs(rhs))
    V = r.standard_normal(p["dt"].shape)
    eps = 1e-6
    qp, qm = dict(p), dict(p)
    qp["dt"] = p["dt"].astype(np.float64) + eps * V
    qm["dt"] = p["dt"].astype(np.float64) - eps * V
    fd = (loss(qp, so, dy, dfin) - loss(qm, so, dy, dfin)) / (2 * eps)
    an = float(np.sum(g["ddt"] * V))
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))
