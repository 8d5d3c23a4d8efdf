"""TEST INFRASTRUCTURE ONLY: numpy fp64 forms of the SSD core's neighbours in
the Mamba-2 block (page "Mamba-2 Architecture: State Space Duality Explained",
"Step 2: Full Mamba-2 Block with Gated Projections", and the block diagram of
page "State Space Duality and Mamba-2: Unifying Transformers and
Semiseparable Matrices", section on the Mamba-2 architecture block):

  before the core: a causal depthwise 1-D convolution over the token axis of
    each channel (kernel width K, bias), then SiLU;
  after the core:  the output gated by SiLU of the gate branch z, then an
    RMS normalisation over the full channel width with a learned weight.

Plain loops and vector ops in the order the pages state them; no blocking or
fusion.  Token tensors are packed [T, channels]; seq_off [nseq + 1] gives the
sequence starts (the convolution window never reaches across one).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def silu(v):
    """v * sigmoid(v), with sigmoid(v) = exp(-log(1 + exp(-v))) (no overflow)."""
    v = np.asarray(v, np.float64)
    return v * np.exp(-np.logaddexp(0.0, -v))


def conv1d_silu(inp, weight, bias: Optional[np.ndarray], seq_off):
    """out[t, c] = silu(bias[c] + sum_{k<K} weight[c, k] * inp[t - (K-1) + k, c]),
    where positions before the sequence's first token read zero (a causal
    convolution: left padding of K-1, outputs truncated to the sequence)."""
    inp = np.asarray(inp, np.float64)
    w = np.asarray(weight, np.float64)
    T, Cch = inp.shape
    K = w.shape[1]
    out = np.zeros((T, Cch))
    for s in range(len(seq_off) - 1):
        t0, t1 = int(seq_off[s]), int(seq_off[s + 1])
        for t in range(t0, t1):
            acc = np.zeros(Cch) if bias is None else np.asarray(bias, np.float64).copy()
            for k in range(K):
                src = t - (K - 1) + k
                if src >= t0:
                    acc += w[:, k] * inp[src]
            out[t] = silu(acc)
    return out


def gate_rmsnorm(y, z, weight: Optional[np.ndarray], eps: float):
    """g = y * silu(z); with a weight, g / sqrt(mean over channels of g^2 + eps)
    * weight per token row; without one, g alone."""
    g = np.asarray(y, np.float64) * silu(z)
    if weight is None:
        return g
    ms = np.mean(g * g, axis=-1, keepdims=True)
    return g / np.sqrt(ms + eps) * np.asarray(weight, np.float64)
