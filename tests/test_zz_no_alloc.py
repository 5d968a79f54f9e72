"""vsa2_route_noalloc: the router with its scratch in the library's fixed
device array instead of a caller workspace.  Its block scores must equal
vsa2_route's bit for bit (same kernels, same inputs), on two calls in a row
with the second on a smaller problem, and on a padded grid (whose key-
existence words also live in the scratch).  Problems beyond the fixed array
are refused before anything is enqueued."""

import ctypes

import pytest
import torch

from video_dit_trainable_amd import vsa2
from video_dit_trainable_amd.configs import Workload
from video_dit_trainable_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu


def _routed_both(w):
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(w, device=dev)
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype)
    pooled = torch.empty(vsa2.pooled_size(p), dtype=torch.uint8, device=dev)
    vsa2.vsa2_pool(p, q, k, v, pooled)
    ws = torch.empty(vsa2.workspace_size(p, vsa2.OP_ROUTE), dtype=torch.uint8, device=dev)
    want = torch.full((w.batch, w.heads, w.nb, w.nb), float("nan"), device=dev)
    got = torch.full_like(want, float("nan"))
    vsa2.vsa2_route(p, pooled, want, ws)
    vsa2.vsa2_route_noalloc(p, pooled, got)
    torch.cuda.synchronize()
    return want, got


def test_noalloc_router_matches_the_workspace_router():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert vsa2.route_noalloc_limit() == 8 << 20
    # the 480p training grid (28x32x52, 728 cubes, 20 heads: 466 KB of LSE),
    # then a smaller problem (the short grid at 4 heads), then a padded grid
    cases = [Workload("nalloc480", 3, (28, 32, 52), 1, 20, 128, "bf16", 64, "lowrank"),
             Workload("nalloc_small", 2, (16, 32, 64), 1, 4, 128, "bf16", 64, "lowrank"),
             Workload("nalloc_pad", 6, (15, 31, 62), 1, 3, 64, "bf16", 64, "lowrank")]
    for w in cases:
        print(f"no-alloc router case {w.name} grid {w.grid} heads {w.heads}", flush=True)
        want, got = _routed_both(w)
        assert not torch.isnan(want).any()
        assert torch.equal(got, want), f"{w.name}: the no-allocation router differs from vsa2_route"


def test_noalloc_router_refuses_problems_beyond_its_scratch():
    L = vsa2.lib()
    # 720p with 80 heads needs 80 x 27,456 x 4 B = 8.8 MB of LSE, beyond 8 MiB
    big = vsa2.problem(1, 80, 128, (44, 48, 104), "bf16")
    assert L.vsa2_route_noalloc(ctypes.byref(big), 0x10000, 0x20000, None) == vsa2.VSA2_E_SCRATCH
    ok = vsa2.problem(1, 20, 128, (44, 48, 104), "bf16")
    assert L.vsa2_route_noalloc(ctypes.byref(ok), None, 0x20000, None) == vsa2.VSA2_E_ARG
