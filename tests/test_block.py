"""The core's block neighbours on the GPU against the fp64 oracle
(oracle/block.py): ssd_conv1d_silu (causal depthwise conv1d + SiLU) and
ssd_gate_rmsnorm (y * SiLU(z), RMS norm).  Inputs are seeded normals; the
bound is max |err| / max |ref| over the whole output, 1e-5 for fp32 and 1e-2
for bf16 (one bf16 rounding of the output, plus bf16 inputs)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mamba_ssd_layer_amd as ssd  # noqa: E402
import oracle  # noqa: E402
from gpu_helpers import DEV, say  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 1e-2}
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def draw(shape, dtype, rng):
    a = rng.standard_normal(shape).astype(np.float32)
    t = torch.from_numpy(a).to(DEV).to(DT[dtype])
    return t, t.float().cpu().numpy().astype(np.float64)  # the values the GPU sees


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_fixed_batch(dtype, K):
    rng = np.random.default_rng(800 + K)
    Bn, L, C = 3, 77, 48
    x, xh = draw((Bn, L, C), dtype, rng)
    w = rng.standard_normal((C, K)).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    out = ssd.conv1d_silu(x, torch.from_numpy(w).to(DEV), torch.from_numpy(b).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.conv1d_silu(xh.reshape(-1, C), w, b, np.arange(0, Bn * L + 1, L))
    e = rel(out.float().cpu().numpy().reshape(-1, C), ref)
    say(f"  conv {dtype} K{K}: rel err {e:.3e}")
    assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_packed_sequences(dtype):
    # empty, length-1 and longer sequences; thread runs of 32 tokens cross
    # sequence starts; no bias
    rng = np.random.default_rng(810)
    lens = [1, 0, 5, 33, 0, 2, 70, 31, 1]
    T, C = sum(lens), 40
    x, xh = draw((T, C), dtype, rng)
    w = rng.standard_normal((C, 4)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out = ssd.conv1d_silu(x, torch.from_numpy(w).to(DEV), None, torch.from_numpy(cu).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.conv1d_silu(xh, w, None, cu)
    e = rel(out.float().cpu().numpy(), ref)
    say(f"  conv packed {dtype}: rel err {e:.3e}")
    assert e <= TOL[dtype]


def test_conv_reads_slices_of_a_packed_projection():
    # x, B and C are column slices of one [B, L, Cx + 2 Cb] projection; each is
    # convolved in place of its slice with its own weights
    rng = np.random.default_rng(820)
    Bn, L, Cx, Cb = 2, 300, 128, 32
    xbc, xbch = draw((Bn, L, Cx + 2 * Cb), "bf16", rng)
    w = rng.standard_normal((Cx + 2 * Cb, 4)).astype(np.float32)
    b = rng.standard_normal(Cx + 2 * Cb).astype(np.float32)
    off = np.arange(0, Bn * L + 1, L)
    for lo, hi in ((0, Cx), (Cx, Cx + Cb), (Cx + Cb, Cx + 2 * Cb)):
        out = ssd.conv1d_silu(xbc[..., lo:hi], torch.from_numpy(w[lo:hi]).to(DEV),
                              torch.from_numpy(b[lo:hi]).to(DEV))
        torch.cuda.synchronize()
        assert out.is_contiguous()
        ref = oracle.conv1d_silu(xbch.reshape(-1, Cx + 2 * Cb)[:, lo:hi], w[lo:hi], b[lo:hi], off)
        assert rel(out.float().cpu().numpy().reshape(-1, hi - lo), ref) <= TOL["bf16"]


def test_conv_large_layer():
    # the large layer's x/B/C width (80 heads x 64 + 2 x 128) over 8 x 4096 tokens
    rng = np.random.default_rng(830)
    Bn, L, C = 8, 4096, 80 * 64 + 2 * 128
    x, xh = draw((Bn, L, C), "bf16", rng)
    w = rng.standard_normal((C, 4)).astype(np.float32) * 0.5
    b = rng.standard_normal(C).astype(np.float32) * 0.1
    out = ssd.conv1d_silu(x, torch.from_numpy(w).to(DEV), torch.from_numpy(b).to(DEV))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().reshape(-1, C)
    # every row against the oracle (each batch row is its own sequence)
    ref = oracle.conv1d_silu(xh.reshape(-1, C), w, b, np.arange(0, Bn * L + 1, L))
    e = rel(got, ref)
    say(f"  conv large layer: rel err {e:.3e}")
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_norm", [False, True])
def test_gate_rmsnorm(dtype, with_norm):
    rng = np.random.default_rng(840)
    T, H, P = 50, 6, 64
    y, yh = draw((T, H, P), dtype, rng)
    z, zh = draw((T, H, P), dtype, rng)
    w = rng.standard_normal(H * P).astype(np.float32) if with_norm else None
    out = ssd.gate_rmsnorm(y, z, None if w is None else torch.from_numpy(w).to(DEV), eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.gate_rmsnorm(yh.reshape(T, -1), zh.reshape(T, -1), w, 1e-5)
    e = rel(out.float().cpu().numpy().reshape(T, -1), ref)
    say(f"  gate{'+norm' if with_norm else ''} {dtype}: rel err {e:.3e}")
    assert e <= TOL[dtype]


def test_gate_rmsnorm_in_place():
    rng = np.random.default_rng(850)
    y, yh = draw((64, 5120), "bf16", rng)
    z, zh = draw((64, 5120), "bf16", rng)
    w = rng.standard_normal(5120).astype(np.float32)
    out = ssd.gate_rmsnorm(y, z, torch.from_numpy(w).to(DEV), eps=1e-6, out=y)
    torch.cuda.synchronize()
    assert out.data_ptr() == y.data_ptr()
    assert rel(y.float().cpu().numpy(), oracle.gate_rmsnorm(yh, zh, w, 1e-6)) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_silu_saturation(dtype):
    # pre-activations far into both tails and around 0: with weight 1, no bias
    # and width 1 the convolution is silu(x) itself, and the gate with z = x
    # and y = 1 is silu(x) too; SiLU goes to 0 on the left (1 + e^{-v}
    # overflows) and to v on the right, with no inf or NaN on the way
    v = np.concatenate([-np.logspace(3, -30, 60), [0.0], np.logspace(-30, 3, 60),
                        [-89.0, -88.0, -87.0, -20.0, -1.0, 1.0, 20.0, 87.0, 88.0, 89.0]])
    v = np.concatenate([v, np.zeros(-len(v) % 8)])  # 8 channels a token row
    x = torch.from_numpy(v.astype(np.float32)).to(DEV).to(DT[dtype]).view(-1, 8)
    xh = x.float().cpu().numpy().astype(np.float64)
    out = ssd.conv1d_silu(x.view(1, -1, 8), torch.ones(8, 1, device=DEV), None)
    gout = ssd.gate_rmsnorm(torch.ones_like(x), x, None, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.conv1d_silu(xh, np.ones((8, 1)), None, np.array([0, xh.shape[0]]))
    for name, got in (("conv", out.float().cpu().numpy().reshape(-1, 8)),
                      ("gate", gout.float().cpu().numpy().reshape(-1, 8))):
        assert np.all(np.isfinite(got)), name
        err = np.abs(got - ref) / np.maximum(np.abs(ref), 1.0)
        say(f"  silu tails {name} {dtype}: max err / max(1, |ref|) {err.max():.3e}")
        assert err.max() <= TOL[dtype]
