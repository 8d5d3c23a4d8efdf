"""ssd_chunk_scan_fwd_noalloc (the forward whose workspace is the library's
fixed per-device scratch array) on the GPU, through the C ABI, against
ssd_chunk_scan_fwd with a workspace of its own: the same kernels on the same
inputs, so the results must agree bit for bit, and both must meet the oracle's
bf16 bound.  Two calls in a row, the second on a smaller (packed) input, so
the second call runs over the first call's leftovers in the scratch array.
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mamba_ssd_layer_amd as ssd  # noqa: E402
from gpu_helpers import check_full, plan_for, say, upload  # noqa: E402

L = ssd.libssd


def both(w, chunk):
    t = upload(w)
    plan = plan_for(w, t, chunk)
    y_ref, f_ref = plan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], t["cu"])
    y = torch.empty_like(t["x"])
    f = torch.empty_like(f_ref)
    L.ssd_chunk_scan_fwd_noalloc(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk, t["h0"],
                                 t["cu"], y, f, plan.dims)
    torch.cuda.synchronize()
    return y, f, y_ref, f_ref, plan


def test_noalloc_matches_workspace_forward_twice():
    # first call: the small Mamba-2 layer (4 x 2048 tokens, 24 heads, N 128),
    # about 26 MB of workspace
    w1 = workloads.make_workload("small_bf16")
    y, f, y_ref, f_ref, plan = both(w1, 256)
    assert plan.layout.total_bytes <= L.NOALLOC_SCRATCH_BYTES
    assert torch.equal(y, y_ref) and torch.equal(f, f_ref)
    check_full(w1, y, f, label="no-alloc call 1 (small_bf16)")
    # second call, smaller: packed sequences with initial states, 8 groups,
    # chunk 64 -- its chunk table lands where the first call left states
    lens = [1, 0, 300, 64, 65, 511, 7]
    w2 = workloads.make_custom(1, 0, 16, 64, 64, 8, 64, "bf16", seed=7100, lens=lens,
                               init_std=0.3)
    y, f, y_ref, f_ref, plan2 = both(w2, 64)
    assert plan2.layout.total_bytes < plan.layout.total_bytes
    assert torch.equal(y, y_ref) and torch.equal(f, f_ref)
    check_full(w2, y, f, label="no-alloc call 2 (packed, smaller)")
    say("  no-alloc forward bit-identical to the workspace forward on both calls")


def test_noalloc_rejects_problems_beyond_the_scratch():
    # the large layer needs ~350 MB of workspace: refused before any launch
    w = workloads.make_custom(8, 4096, 80, 64, 128, 1, 256, "bf16", seed=7200)
    dims = ssd.make_dims(8, 4096, 80, 64, 128, 1)
    assert L.ssd_workspace_size(dims, 256) > L.NOALLOC_SCRATCH_BYTES
    t = upload(w)
    y = torch.empty_like(t["x"])
    with pytest.raises(ssd.SSDWorkspaceError):
        L.ssd_chunk_scan_fwd_noalloc(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 256, None,
                                     None, y, None, dims)
