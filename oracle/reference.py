"""TEST INFRASTRUCTURE ONLY: numpy fp64 forms of the SSD forward.

All functions take one packed batch in the canonical layout
  x [T,H,P], dt [T,H], A [H], B/C [T,G,N], D [H]|None, h0 [nseq,H,P,N]|None,
  seq_off [nseq+1]
and return fp64 results.  Head h reads group g = floor(h*G/H).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _group(h: int, H: int, G: int) -> int:
    return (h * G) // H


def recurrence_py(x, dt, A, B, C, D, h0, seq_off):
    """Token-by-token recurrence in plain numpy (small inputs only).

    h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t^T ; y_t = C_t h_t + D x_t.
    Page "State Space Duality and Mamba-2 ...", "Mathematical Foundations"
    (recurrence) and "The Scalar-Identity Structural Constraint" (A_t = a_t I).
    """
    x = np.asarray(x, np.float64)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    nseq = len(seq_off) - 1
    y = np.zeros((T, H, P))
    fin = np.zeros((nseq, H, P, N))
    for s in range(nseq):
        for h in range(H):
            g = _group(h, H, G)
            st = np.zeros((P, N)) if h0 is None else np.array(h0[s, h], np.float64)
            for t in range(int(seq_off[s]), int(seq_off[s + 1])):
                d = float(dt[t, h])
                st = np.exp(d * float(A[h])) * st + d * np.outer(x[t, h], np.asarray(B[t, g], np.float64))
                y[t, h] = st @ np.asarray(C[t, g], np.float64)
                if D is not None:
                    y[t, h] += float(D[h]) * x[t, h]
            fin[s, h] = st
    return y, fin


def quadratic(x, dt, A, B, C, D, h0, seq_off):
    """The attention-like (matrix) dual of the recurrence, per sequence and head.

    y = M x + exp(s) (C h0^T) + D x with the lower-triangular (diagonal
    included) matrix M[j,i] = (C_j . B_i) exp(s_j - s_i) dt_i, i <= j, and
    s = cumsum(dt * A) the log of the cumulative decay:
      - page "State Space Duality and Mamba-2 ...", "Mathematical Foundations"
        (M_{j,i} = C_j^T (prod_{k=i+1}^{j} A_k) B_i and the printed 3x3 matrix,
        whose diagonal holds C_j B_j) and "The Scalar-Identity Structural
        Constraint" (the product of scalar decays is exp(s_j - s_i));
      - page "Mamba-2 Architecture: State Space Duality Explained", "1. The
        Core Duality" (y_t as the sum over s <= t).
    The final state is the same sum read at the last token:
      h_end = exp(s_end) h0 + sum_i exp(s_end - s_i) dt_i x_i B_i^T.
    """
    x = np.asarray(x, np.float64)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    nseq = len(seq_off) - 1
    y = np.zeros((T, H, P))
    fin = np.zeros((nseq, H, P, N))
    for s in range(nseq):
        a, b = int(seq_off[s]), int(seq_off[s + 1])
        L = b - a
        for h in range(H):
            g = _group(h, H, G)
            hin = np.zeros((P, N)) if h0 is None else np.asarray(h0[s, h], np.float64)
            if L == 0:
                fin[s, h] = hin
                continue
            d = np.asarray(dt[a:b, h], np.float64)
            sc = np.cumsum(d * float(A[h]))
            Cm = np.asarray(C[a:b, g], np.float64)
            Bm = np.asarray(B[a:b, g], np.float64)
            lower = np.tril(np.ones((L, L), dtype=bool))
            diff = np.where(lower, sc[:, None] - sc[None, :], -np.inf)
            M = (Cm @ Bm.T) * np.exp(diff) * d[None, :]
            xs = x[a:b, h]
            y[a:b, h] = M @ xs + np.exp(sc)[:, None] * (Cm @ hin.T)
            if D is not None:
                y[a:b, h] += float(D[h]) * xs
            w = np.exp(sc[-1] - sc) * d
            fin[s, h] = np.exp(sc[-1]) * hin + (xs * w[:, None]).T @ Bm
    return y, fin


def chunked(x, dt, A, B, C, D, h0, seq_off, Q: int, return_intermediates: bool = False):
    """The blockwise (chunked) evaluation, per sequence and head.

    Page "Mamba-2 Architecture: State Space Duality Explained", "2. The
    Chunked SSD Algorithm": the sequence is cut into chunks of Q tokens (the
    last one partial); inside a chunk the output is the masked product
    (C B^T o L) X; each chunk leaves a state contribution; the states are
    handed from chunk to chunk by a scalar recurrence; the state entering a
    chunk adds its contribution C h_prev to that chunk's outputs.  The page's
    listing leaves out the decay weights of the chunk state and of the
    inter-chunk output; they are the ones the recurrence implies:
      Acum_l     = sum_{k<=l} dt_k A        (log-decay from chunk start, inclusive)
      intra  y_l = sum_{s<=l} (C_l . B_s) exp(Acum_l - Acum_s) dt_s x_s
      inter  y_l = exp(Acum_l) C_l h_prev^T
      state  S   = sum_l exp(Acum_last - Acum_l) dt_l x_l B_l^T
      hand-off h_next = exp(Acum_last) h_prev + S
    Chunks restart at every sequence start.

    With return_intermediates, also returns a dict of per-chunk arrays, chunks
    numbered sequence-major: 'Acum' [nc,H,Q] (positions past a partial chunk's
    end are NaN), 'S' [nc,H,P,N], 'Hprev' [nc,H,P,N], 'chunk_seq', 'chunk_start',
    'chunk_len' [nc].
    """
    x = np.asarray(x, np.float64)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    nseq = len(seq_off) - 1
    y = np.zeros((T, H, P))
    fin = np.zeros((nseq, H, P, N))
    starts, lens, seqs = [], [], []
    for s in range(nseq):
        a, b = int(seq_off[s]), int(seq_off[s + 1])
        for c0 in range(a, b, Q):
            starts.append(c0)
            lens.append(min(Q, b - c0))
            seqs.append(s)
    nc = len(starts)
    inter = None
    if return_intermediates:
        inter = {"Acum": np.full((nc, H, Q), np.nan), "S": np.zeros((nc, H, P, N)),
                 "Hprev": np.zeros((nc, H, P, N)), "chunk_seq": np.array(seqs, np.int64),
                 "chunk_start": np.array(starts, np.int64),
                 "chunk_len": np.array(lens, np.int64)}
    for h in range(H):
        g = _group(h, H, G)
        Ah = float(A[h])
        state = None
        cur_seq = -1
        for k in range(nc):
            s = seqs[k]
            if s != cur_seq:
                if cur_seq >= 0:
                    fin[cur_seq, h] = state
                cur_seq = s
                state = np.zeros((P, N)) if h0 is None else np.array(h0[s, h], np.float64)
            c0, n = starts[k], lens[k]
            sl = slice(c0, c0 + n)
            d = np.asarray(dt[sl, h], np.float64)
            acum = np.cumsum(d * Ah)
            Cm = np.asarray(C[sl, g], np.float64)
            Bm = np.asarray(B[sl, g], np.float64)
            xs = x[sl, h]
            lower = np.tril(np.ones((n, n), dtype=bool))
            Lmask = np.exp(np.where(lower, acum[:, None] - acum[None, :], -np.inf)) * d[None, :]
            y_intra = ((Cm @ Bm.T) * Lmask) @ xs
            y_inter = np.exp(acum)[:, None] * (Cm @ state.T)
            y[sl, h] = y_intra + y_inter
            if D is not None:
                y[sl, h] += float(D[h]) * xs
            w = np.exp(acum[-1] - acum) * d
            S = (xs * w[:, None]).T @ Bm
            if inter is not None:
                inter["Acum"][k, h, :n] = acum
                inter["S"][k, h] = S
                inter["Hprev"][k, h] = state
            state = np.exp(acum[-1]) * state + S
        if cur_seq >= 0:
            fin[cur_seq, h] = state
        # sequences without any chunk (length 0) keep their initial state
        for s in range(nseq):
            if seq_off[s + 1] == seq_off[s]:
                fin[s, h] = 0.0 if h0 is None else np.asarray(h0[s, h], np.float64)
    if return_intermediates:
        return y, fin, inter
    return y, fin
