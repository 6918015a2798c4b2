"""The allocation-free dispatch layout (moe_dispatch_layout_noalloc) against the entry point
with a caller's workspace (moe_dispatch_layout), bit for bit, and against the oracle.

Two calls in a row on the library's shared scratch, the second smaller than the first, so
the second reads a count table that still holds the first call's larger contents.
"""
import numpy as np
import pytest
import torch

import combine_grouped_gemm_amd as moe
import workload as w
from oracle import moe_oracle as oracle
from tests.gpu_util import say, sync

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _compare(N, E, k, kind, seed):
    idx = w.fixed_route(N, E, k, kind, seed=seed)
    if kind == "random":   # a few ids out of range: skipped (send_pos -1) by both entry points
        idx = idx.clone()
        idx[::97, 0] = E
    d = idx.to(DEV)
    ref = moe.moe_dispatch_layout(d, E)
    got = moe.moe_dispatch_layout_noalloc(d, E)
    sync()
    for g, r in zip(got[:3], ref[:3]):
        assert torch.equal(g, r)
    # src_slot is defined on the rows of valid pairs only (rows >= offsets[E] stay untouched)
    nv = int(ref[1][E].item())
    assert torch.equal(got[3][:nv], ref[3][:nv])
    rn, ro, rs, rss = oracle.dispatch_layout(np.where(idx.numpy() < E, idx.numpy(), 0), E)
    n_e = got[0].cpu().numpy()
    valid = idx.numpy().reshape(-1) < E
    if valid.all():
        assert np.array_equal(n_e, rn)
        assert np.array_equal(got[1].cpu().numpy(), ro)
        assert np.array_equal(got[2].cpu().numpy(), rs)
        assert np.array_equal(got[3].cpu().numpy(), rss)
    else:
        assert np.array_equal(got[2].cpu().numpy()[~valid], np.full((~valid).sum(), -1))
        assert int(n_e.sum()) == int(valid.sum())
    say(f"  noalloc layout N={N} E={E} k={k} {kind}: equal to the workspace entry point")


def test_noalloc_layout_two_calls_second_smaller():
    _compare(8192, 256, 8, "random", seed=1)      # 64 chunks x 256 experts of counts
    _compare(300, 64, 4, "random", seed=2)        # a smaller table over the stale one


def test_noalloc_layout_largest_tables():
    # the most chunks (4096) times 256 experts fills the 4 MiB exactly; E = 1024 with 1024 chunks
    _compare(1 << 19, 256, 8, "round_robin", seed=3)
    _compare(1 << 17, 1024, 8, "round_robin", seed=4)
    _compare(1, 8, 2, "hot", seed=5)


def test_noalloc_layout_rejects_tables_beyond_the_scratch():
    nk = (1 << 20) + 1024           # 1025 chunks of 1024 slots ...
    N, k, E = nk // 8, 8, 1024      # ... times 1024 experts > 4 MiB
    assert moe.moe_workspace_bytes(moe.MOE_OP_DISPATCH_LAYOUT, N, 0, 0, E, k, 0) > moe.MOE_LAYOUT_SCRATCH_BYTES
    st = moe.lib().moe_dispatch_layout_noalloc(4096, N, k, E, 4096, 4096, 4096, 4096, None)
    assert st == moe.MOE_ERR_WORKSPACE
