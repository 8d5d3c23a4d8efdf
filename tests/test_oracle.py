"""Pins for the CPU oracle (no GPU).

The oracle (oracle.recurrence, fp64 C) is checked against things other than
itself: hand-computed values from the printed 3x3 semiseparable matrix, closed
forms, the quadratic (attention-like) dual, the A = 0 reduction to causal
linear attention, chunk and split invariance, linearity, the rank bound of the
off-diagonal blocks, brute force on tiny inputs and the head-to-group map.
A mutation section plants plausible mistakes in copies of the recurrence and
checks that at least one pin catches each.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import chunked, quadratic, recurrence_py
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- helpers
def rnd_case(seed, T=37, H=4, P=3, N=5, G=2, nseq=None, with_h0=True, with_D=True,
             a_scale=1.0):
    """Small random packed batch.  nseq: lengths split of T (None = one sequence)."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, H, P)).astype(np.float32)
    dt = (0.05 + 0.5 * r.random((T, H))).astype(np.float32)
    A = (-a_scale * np.exp(r.uniform(0, math.log(8), H))).astype(np.float32)
    B = (r.standard_normal((T, G, N)) / math.sqrt(N)).astype(np.float32)
    C = (r.standard_normal((T, G, N)) / math.sqrt(N)).astype(np.float32)
    D = r.standard_normal(H).astype(np.float32) if with_D else None
    if nseq is None:
        seq_off = np.array([0, T], np.int64)
    else:
        cuts = np.sort(r.choice(np.arange(0, T + 1), nseq - 1, replace=True))
        seq_off = np.concatenate([[0], cuts, [T]]).astype(np.int64)
    ns = len(seq_off) - 1
    h0 = (0.3 * r.standard_normal((ns, H, P, N))).astype(np.float32) if with_h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, h0=h0, seq_off=seq_off)


def c_oracle(x, dt, A, B, C, D, h0, seq_off):
    return oracle.recurrence(x, dt, A, B, C, D, h0, seq_off)


def relerr(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) / den


def load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            vals[k.strip()] = [float(t) for t in v.split()]
    return vals


def golden_case(name):
    g = load_golden(name)
    H, P, N, G = (int(g[k][0]) for k in ("H", "P", "N", "G"))
    T = len(g["dt"]) // H
    case = dict(
        x=np.array(g["x"], np.float32).reshape(T, H, P),
        dt=np.array(g["dt"], np.float32).reshape(T, H),
        A=np.array(g["A"], np.float32).reshape(H),
        B=np.array(g["B"], np.float32).reshape(T, G, N),
        C=np.array(g["C"], np.float32).reshape(T, G, N),
        D=np.array(g["D"], np.float32).reshape(H) if "D" in g else None,
        h0=np.array(g["h0"], np.float32).reshape(1, H, P, N) if "h0" in g else None,
        seq_off=np.array([0, T], np.int64),
    )
    y = np.array(g["y"]).reshape(T, H, P)
    fin = np.array(g["final"]).reshape(1, H, P, N)
    return case, y, fin


# --------------------------------------------------------------------------- pins
# Each pin takes an implementation fn(x, dt, A, B, C, D, h0, seq_off) -> (y, final)
# and raises AssertionError when it does not hold.

def pin_golden_matrix(fn):
    case, y, fin = golden_case("matrix3x3_scalar.txt")
    yo, fo = fn(**case)
    assert relerr(yo, y) < 1e-7 and relerr(fo, fin) < 1e-7, (yo.ravel(), fo.ravel())


def pin_golden_dt_skip_init(fn):
    case, y, fin = golden_case("dt_skip_init_2x2.txt")
    yo, fo = fn(**case)
    assert relerr(yo, y) < 1e-7 and relerr(fo, fin) < 1e-7, (yo.ravel(), fo.ravel())


def pin_quadratic_dual(fn, seed=1, **kw):
    case = rnd_case(seed, **kw)
    yo, fo = fn(**case)
    yq, fq = quadratic(**case)
    assert relerr(yo, yq) < 1e-12 and relerr(fo, fq) < 1e-12


def pin_linear_attention(fn, seed=2):
    """A = 0: every decay is 1, the SSD is causal linear attention with
    V = dt*x, K = B, Q = C plus the initial state and the skip."""
    case = rnd_case(seed, T=29, H=2, P=3, N=4, G=1)
    case["A"][:] = 0.0
    yo, fo = fn(**case)
    x, dt, B, C, D, h0 = (case[k] for k in ("x", "dt", "B", "C", "D", "h0"))
    T, H, P = x.shape
    for h in range(H):
        kv = np.einsum("tp,tn->tpn", dt[:, h, None].astype(np.float64) * x[:, h], B[:, 0].astype(np.float64))
        hs = np.cumsum(kv, axis=0) + h0[0, h][None]
        y = np.einsum("tpn,tn->tp", hs, C[:, 0].astype(np.float64)) + float(D[h]) * x[:, h].astype(np.float64)
        assert relerr(yo[:, h], y) < 1e-12
        assert relerr(fo[0, h], hs[-1]) < 1e-12


def pin_chunk_invariance(fn, seed=3):
    case = rnd_case(seed, T=41, H=2, P=2, N=3, G=1, nseq=3)
    yo, fo = fn(**case)
    for Q in (1, 2, 3, 7, 16, 41):
        yc, fc = chunked(**case, Q=Q)
        assert relerr(yo, yc) < 1e-12 and relerr(fo, fc) < 1e-12, Q


def pin_geometric(fn):
    """Constant x, B, C, dt = delta, h0 = 0: y_t = delta (C.B) x (1 - a^{t+1})/(1 - a) + D x."""
    T, P, N = 50, 3, 4
    delta, Aval = 0.3, -0.7
    r = np.random.default_rng(4)
    xv = r.standard_normal(P).astype(np.float32)
    bv = r.standard_normal(N).astype(np.float32)
    cv = r.standard_normal(N).astype(np.float32)
    case = dict(x=np.tile(xv, (T, 1, 1)), dt=np.full((T, 1), delta, np.float32),
                A=np.array([Aval], np.float32), B=np.tile(bv, (T, 1, 1)),
                C=np.tile(cv, (T, 1, 1)), D=np.array([0.25], np.float32), h0=None,
                seq_off=np.array([0, T], np.int64))
    yo, fo = fn(**case)
    a = math.exp(float(np.float32(delta)) * float(np.float32(Aval)))
    d = float(np.float32(delta))
    t = np.arange(T)
    geo = (1 - a ** (t + 1)) / (1 - a)
    cb = float(np.dot(cv.astype(np.float64), bv.astype(np.float64)))
    y = d * cb * geo[:, None] * xv[None].astype(np.float64) + 0.25 * xv[None].astype(np.float64)
    assert relerr(yo[:, 0], y) < 1e-12
    fin = d * geo[-1] * np.outer(xv.astype(np.float64), bv.astype(np.float64))
    assert relerr(fo[0, 0], fin) < 1e-12


def pin_zero_input(fn, seed=5):
    """x = 0: y_t = exp(s_t) C_t h0^T, final = exp(s_end) h0."""
    case = rnd_case(seed, T=23, H=3, P=2, N=3, G=3)
    case["x"][:] = 0.0
    yo, fo = fn(**case)
    dt, A, C, h0 = (case[k] for k in ("dt", "A", "C", "h0"))
    for h in range(3):
        s = np.cumsum(dt[:, h].astype(np.float64) * float(A[h]))
        y = np.exp(s)[:, None] * (C[:, h].astype(np.float64) @ h0[0, h].astype(np.float64).T)
        assert relerr(yo[:, h], y) < 1e-12
        assert relerr(fo[0, h], math.exp(s[-1]) * h0[0, h].astype(np.float64)) < 1e-12


def pin_skip_only(fn, seed=6):
    """B = 0 and h0 = 0, or C = 0: nothing reaches the readout, y = D x."""
    for which in ("B", "C"):
        case = rnd_case(seed, T=19, H=2, P=3, N=2, G=1, with_h0=(which == "C"))
        case[which][:] = 0.0
        yo, _ = fn(**case)
        y = case["D"][None, :, None].astype(np.float64) * case["x"]
        assert relerr(yo, y) < 1e-14, which


def pin_split(fn, seed=7):
    """Running [0,L1) then [L1,L) from the first final state equals one run."""
    case = rnd_case(seed, T=40, H=2, P=2, N=3, G=1)
    yo, fo = fn(**case)
    L1 = 17
    first = {k: (v[:L1] if k in ("x", "dt", "B", "C") else v) for k, v in case.items()}
    first["seq_off"] = np.array([0, L1], np.int64)
    y1, f1 = fn(**first)
    second = {k: (v[L1:] if k in ("x", "dt", "B", "C") else v) for k, v in case.items()}
    second["seq_off"] = np.array([0, 40 - L1], np.int64)
    second["h0"] = f1.astype(np.float32)
    y2, f2 = fn(**second)
    # f1 is rounded to float32 to be fed back, so compare loosely
    assert relerr(np.concatenate([y1, y2]), yo) < 1e-6 and relerr(f2, fo) < 1e-6


def pin_varlen_independent(fn, seed=8):
    case = rnd_case(seed, T=45, H=2, P=2, N=3, G=1, nseq=4)
    yo, fo = fn(**case)
    so = case["seq_off"]
    for s in range(len(so) - 1):
        a, b = int(so[s]), int(so[s + 1])
        one = {k: (v[a:b] if k in ("x", "dt", "B", "C") else v) for k, v in case.items()}
        one["h0"] = case["h0"][s:s + 1]
        one["seq_off"] = np.array([0, b - a], np.int64)
        y1, f1 = fn(**one)
        assert relerr(y1, yo[a:b]) < 1e-14 if b > a else True
        assert np.allclose(f1[0], fo[s], rtol=1e-14, atol=1e-14)


def pin_linearity(fn, seed=9):
    c1 = rnd_case(seed, T=21, H=2, P=2, N=3, G=1)
    c2 = rnd_case(seed + 100, T=21, H=2, P=2, N=3, G=1)
    for k in ("dt", "A", "B", "C", "D"):
        c2[k] = c1[k]
    alpha, beta = 0.5, -2.0  # exact in float32
    c3 = dict(c1)
    c3["x"] = (alpha * c1["x"] + beta * c2["x"]).astype(np.float32)
    c3["h0"] = (alpha * c1["h0"] + beta * c2["h0"]).astype(np.float32)
    y1, f1 = fn(**c1)
    y2, f2 = fn(**c2)
    y3, f3 = fn(**c3)
    # x and h0 combos are rounded to float32, hence the loose bound
    assert relerr(y3, alpha * y1 + beta * y2) < 1e-6
    assert relerr(f3, alpha * f1 + beta * f2) < 1e-6


def pin_rank(fn, seed=10):
    """The input-to-output matrix M (probed column by column with unit inputs)
    is lower triangular and its blocks strictly below the diagonal have rank
    at most N (the semiseparable structure)."""
    T, N = 24, 3
    r = np.random.default_rng(seed)
    base = dict(dt=(0.1 + 0.3 * r.random((T, 1))).astype(np.float32),
                A=np.array([-0.4], np.float32),
                B=r.standard_normal((T, 1, N)).astype(np.float32),
                C=r.standard_normal((T, 1, N)).astype(np.float32), D=None, h0=None,
                seq_off=np.array([0, T], np.int64))
    M = np.zeros((T, T))
    for i in range(T):
        x = np.zeros((T, 1, 1), np.float32)
        x[i] = 1.0
        y, _ = fn(x=x, **base)
        M[:, i] = y[:, 0, 0]
    assert np.max(np.abs(np.triu(M, 1))) == 0.0
    for k in (5, 12, 19):
        sv = np.linalg.svd(M[k:, :k], compute_uv=False)
        assert sv[N] < 1e-12 * sv[0] and sv[N - 1] > 1e-8 * sv[0], sv[:N + 1]
    # brute force: the literal product formula M[j,i] = C_j (prod_{k=i+1..j} a_k) B_i dt_i
    a = np.exp(base["dt"][:, 0].astype(np.float64) * float(base["A"][0]))
    for j in range(T):
        for i in range(j + 1):
            prod = 1.0
            for k in range(i + 1, j + 1):
                prod *= a[k]
            ref = float(np.dot(base["C"][j, 0].astype(np.float64), base["B"][i, 0].astype(np.float64))) \
                * prod * float(base["dt"][i, 0])
            assert abs(M[j, i] - ref) <= 1e-12 * max(1.0, abs(ref))


def pin_groups(fn, seed=11):
    """H = 4, G = 2: heads 0,1 read group 0 and heads 2,3 read group 1."""
    case = rnd_case(seed, T=15, H=4, P=2, N=3, G=2)
    yo, fo = fn(**case)
    for h in range(4):
        g = h * 2 // 4
        one = dict(x=case["x"][:, h:h + 1], dt=case["dt"][:, h:h + 1], A=case["A"][h:h + 1],
                   B=np.ascontiguousarray(case["B"][:, g:g + 1]),
                   C=np.ascontiguousarray(case["C"][:, g:g + 1]),
                   D=case["D"][h:h + 1], h0=case["h0"][:, h:h + 1], seq_off=case["seq_off"])
        y1, f1 = fn(**one)
        assert relerr(y1[:, 0], yo[:, h]) < 1e-14 and relerr(f1[0, 0], fo[0, h]) < 1e-14


def pin_empty_sequence(fn, seed=12):
    """A zero-length sequence emits nothing and returns its initial state."""
    case = rnd_case(seed, T=10, H=2, P=2, N=2, G=1)
    case["seq_off"] = np.array([0, 4, 4, 10], np.int64)
    case["h0"] = (0.5 * np.random.default_rng(1).standard_normal((3, 2, 2, 2))).astype(np.float32)
    _, fo = fn(**case)
    assert np.array_equal(fo[1], case["h0"][1].astype(np.float64))


PINS = [pin_golden_matrix, pin_golden_dt_skip_init, pin_quadratic_dual, pin_linear_attention,
        pin_chunk_invariance, pin_geometric, pin_zero_input, pin_skip_only, pin_split,
        pin_varlen_independent, pin_linearity, pin_rank, pin_groups, pin_empty_sequence]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(c_oracle)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_numpy_recurrence_pin(pin):
    pin(recurrence_py)


def test_quadratic_dual_varlen_groups():
    pin_quadratic_dual(c_oracle, seed=21, T=60, H=6, P=4, N=6, G=3, nseq=5)
    pin_quadratic_dual(c_oracle, seed=22, T=33, H=2, P=8, N=16, G=1, with_h0=False, with_D=False)


def test_quadratic_dual_long_memory():
    # small |A|: the state carries far, so cross-chunk terms matter
    pin_quadratic_dual(c_oracle, seed=23, T=80, H=2, P=3, N=4, G=1, a_scale=1e-3)


# --------------------------------------------------------------------------- host logic
def test_pairs_subset_matches_full():
    case = rnd_case(30, T=50, H=3, P=4, N=5, G=1, nseq=3)
    y, f = c_oracle(**case)
    pairs = [(2, 1), (0, 0), (1, 2)]
    ys, fs = oracle.recurrence(**case, pairs=pairs)
    so = case["seq_off"]
    for k, (s, h) in enumerate(pairs):
        assert np.array_equal(ys[k], y[so[s]:so[s + 1], h])
        assert np.array_equal(fs[k], f[s, h])


def test_thread_count_does_not_change_result():
    case = rnd_case(31, T=64, H=8, P=4, N=8, G=2, nseq=2)
    y1, f1 = oracle.recurrence(**case, nthreads=1)
    y4, f4 = oracle.recurrence(**case, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(f1, f4)


def test_oracle_rejects_bad_args():
    case = rnd_case(32, T=10, H=2, P=2, N=2, G=1)
    case["seq_off"] = np.array([0, 6, 4, 10], np.int64)
    case["h0"] = None
    with pytest.raises(ValueError):
        oracle.recurrence(**case)


def test_chunked_intermediates_consistent():
    case = rnd_case(33, T=70, H=2, P=3, N=4, G=1, nseq=2)
    y, f, it = chunked(**case, Q=16, return_intermediates=True)
    # the hand-off identity: Hprev of the next chunk = exp(Acum_last) Hprev + S
    for k in range(len(it["chunk_len"]) - 1):
        if it["chunk_seq"][k] != it["chunk_seq"][k + 1]:
            continue
        n = it["chunk_len"][k]
        for h in range(2):
            nxt = math.exp(it["Acum"][k, h, n - 1]) * it["Hprev"][k, h] + it["S"][k, h]
            assert np.allclose(nxt, it["Hprev"][k + 1, h], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------- workloads
def test_workload_shapes_and_determinism():
    w = workloads.make_workload("tiny_f32")
    assert w.x.shape == (256, 4, 16) and w.B.shape == (256, 1, 16) and w.tokens == 256
    w2 = workloads.make_workload("tiny_f32")
    assert np.array_equal(w.x, w2.x) and np.array_equal(w.dt, w2.dt)
    assert np.all(w.dt > 0) and np.all(w.A < 0) and np.all(w.A >= -16)


def test_varlen_workload_lengths():
    s = workloads.WORKLOADS["varlen_bf16"]
    lens = np.random.default_rng(s.seed).integers(1, s.max_len + 1, s.nseq)
    assert int(lens.sum()) == 275772 and lens.min() >= 1 and lens.max() <= 8192


def test_bf16_rounding_is_nearest_even():
    # bf16 keeps 7 mantissa bits: one ulp at 1.0 is 2^-7
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -9, 1.0 + 3 * 2 ** -8,
                  -3.14159], np.float32)
    b = workloads.bf16_round_(a.copy())
    assert b[0] == 1.0
    assert b[1] == 1.0                       # half an ulp, tie -> even (down)
    assert b[2] == 1.0 + 2 ** -7             # 0.75 ulp -> up
    assert b[3] == 1.0                       # 0.25 ulp -> down
    assert b[4] == 1.0 + 2 ** -6             # 1.5 ulp, tie -> even (up)
    assert b[5] == np.float32(-3.140625)
    bits = workloads.bf16_bits(b)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), b)


# --------------------------------------------------------------------------- mutations
# Copies of the recurrence with one planted mistake each.  Every one must fail
# at least one pin above; otherwise the pins would let that mistake through.

def _mutant(kind):
    def fn(x, dt, A, B, C, D, h0, seq_off):
        x = np.asarray(x, np.float64)
        T, H, P = x.shape
        G, N = B.shape[1], B.shape[2]
        nseq = len(seq_off) - 1
        y = np.zeros((T, H, P))
        fin = np.zeros((nseq, H, P, N))
        for s in range(nseq):
            for h in range(H):
                g = (h % G) if kind == "group_map" else (h * G) // H
                st = np.zeros((P, N)) if (h0 is None or kind == "drop_h0") else np.array(h0[s, h], np.float64)
                prev_dt = 0.0
                for t in range(int(seq_off[s]), int(seq_off[s + 1])):
                    d = float(dt[t, h])
                    dd = prev_dt if kind == "decay_index" else d
                    sign = -1.0 if kind == "decay_sign" else 1.0
                    a = math.exp(sign * dd * float(A[h]))
                    w = 1.0 if kind == "no_dt_weight" else d
                    Bt, Ct = np.asarray(B[t, g], np.float64), np.asarray(C[t, g], np.float64)
                    if kind == "swap_BC":
                        Bt, Ct = Ct, Bt
                    old = st
                    st = a * st + w * np.outer(x[t, h], Bt)
                    y[t, h] = (old if kind == "read_before_update" else st) @ Ct
                    if D is not None and kind != "drop_D":
                        y[t, h] += float(D[h]) * x[t, h]
                    prev_dt = d
                fin[s, h] = st
        return y, fin
    return fn


MUTANTS = ["drop_D", "decay_sign", "no_dt_weight", "read_before_update", "swap_BC",
           "decay_index", "group_map", "drop_h0"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_mutant(kind):
    fn = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {kind!r}"
