"""GPU parity of the VSA router baseline: coarse scores P_c (Eq.(1)-(2) of
"Improving Video Sparse Attention with Fine-grained Router and Sparse
Rebasing", the router of its Figure 1 left) and the TopK per query block.

P_c must match the oracle within 1e-4 relative (rows sum to 1); the per-row
selection must equal the exact top k of each row of the GPU's own scores
(ties to the lower column), and match the oracle's selection outside a
relative 1e-3 band around each row's cut-off.
"""

import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import vsa2_oracle as orc
from video_dit_trainable_amd import vsa2
from video_dit_trainable_amd.configs import WORKLOADS, Workload
from video_dit_trainable_amd.inputs import make_gate_inputs, make_qkv

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny"]
MID = Workload("mid", 12, (8, 16, 32), 1, 4, 128, "bf16", 8, "lowrank", train=True)               # nb = 64
RAGGED = Workload("ragged", 13, (4, 8, 20), 1, 3, 64, "bf16", 3, "lowrank", train=True)           # nb = 10
B128 = Workload("b128-bf16", 32, (8, 16, 32), 1, 3, 128, "bf16", 4, "lowrank", skew=True, train=True, block=128)
PAD = Workload("pad-b64", 23, (9, 6, 21), 1, 2, 64, "bf16", 5, "lowrank", train=True)
BIG = Workload("coarse3", 17, (8, 20, 64), 1, 2, 64, "bf16", 12, "lowrank", train=True)           # nb = 160
CASES = [TINY, MID, RAGGED, B128, PAD, BIG]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vsa2.lib()


def _dev():
    return torch.device("cuda:0")


def _route(w):
    q, k, v = make_qkv(w)
    x, w_g = make_gate_inputs(w)
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype, block=w.block)
    layer = vsa2.Layer(p, w.topk, w.d_model, device=_dev())
    qd, kd, vd, xd, wd = (t.to(_dev()) for t in (q, k, v, x, w_g))
    o = layer.forward(qd, kd, vd, xd, wd, router="vsa")
    torch.cuda.synchronize()
    return q, k, v, layer, o


def _oracle_scores(w, q, k, h):
    return orc.coarse_scores(gu.f64(q[0, h]), gu.f64(k[0, h]), w.grid, bf16_pooled=w.dtype == "bf16", block=w.block)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_coarse_scores_and_row_topk(w):
    q, k, v, layer, _ = _route(w)
    got = gu.f64(layer.scores[0])
    np.testing.assert_allclose(got.sum(axis=2), 1.0, rtol=2e-5)
    kr = min(w.topk, w.nblk)
    gu.check_csr_csc(layer.row_ptr[0], layer.col_idx[0], layer.col_ptr[0], layer.row_idx[0], w.nblk, w.nblk * kr)
    sel = gu.masks_from_csr(layer.row_ptr[0], layer.col_idx[0], w.nblk)
    for h in range(w.heads):
        want = _oracle_scores(w, q, k, h)
        np.testing.assert_allclose(got[h], want, rtol=1e-4, atol=1e-4 * want.mean())
        # exactly the per-row top k of the GPU's own scores
        mine = orc.topk_per_row(layer.scores[0, h].double().cpu().numpy(), w.topk)[0]
        assert np.array_equal(sel[h], mine), f"head {h}: not the per-row top k of the GPU scores"
        # and the oracle's selection outside each row's 1e-3 band
        ref = orc.topk_per_row(want, w.topk)[0]
        for i in range(w.nblk):
            tau = np.sort(want[i])[::-1][kr - 1]
            band = np.abs(want[i] - tau) <= 1e-3 * tau
            assert np.array_equal(sel[h, i, ~band], ref[i, ~band]), f"head {h} row {i}"


@pytest.mark.parametrize("nb,topk,levels", [(32, 8, 5), (10, 4, 2), (200, 17, 7), (15, 15, 4), (33, 40, 3),
                                           (130, 1, 1000), (300, 64, 3)])
def test_row_topk_exact_with_ties(nb, topk, levels):
    rng = np.random.default_rng(nb * 77 + topk)
    H = 3
    scores = rng.integers(0, levels, size=(H, nb, nb)).astype(np.float32) / np.float32(levels)
    scores[0, :, :3] = 0.0
    p = vsa2.problem(1, H, 64, (4, 4, 4 * nb), "f32")
    k = vsa2.budget(p, topk)
    dev = _dev()
    s = torch.tensor(scores, device=dev)[None].contiguous()
    rp = torch.empty((1, H, nb + 1), dtype=torch.int32, device=dev)
    ci = torch.empty((1, H, k), dtype=torch.int32, device=dev)
    cp = torch.empty_like(rp)
    ri = torch.empty_like(ci)
    ws = torch.empty(vsa2.workspace_size(p, vsa2.OP_TOPK_ROW), dtype=torch.uint8, device=dev)
    vsa2.vsa2_topk_per_row(p, s, topk, rp, ci, cp, ri, ws)
    torch.cuda.synchronize()
    assert k == nb * min(topk, nb)
    gu.check_csr_csc(rp[0], ci[0], cp[0], ri[0], nb, k)
    got = gu.masks_from_csr(rp[0], ci[0], nb)
    for h in range(H):
        want = orc.topk_per_row(scores[h].astype(np.float64), topk)[0]
        assert np.array_equal(got[h], want), f"head {h}: {np.sum(got[h] != want)} mismatches"


def test_vsa_router_drives_the_fine_branch():
    w = MID
    q, k, v, layer, o = _route(w)
    sel = gu.masks_from_csr(layer.row_ptr[0], layer.col_idx[0], w.nblk)
    for h in range(w.heads):
        want, _ = orc.fine_forward(gu.f64(q[0, h]), gu.f64(k[0, h]), gu.f64(v[0, h]), sel[h])
        gu.assert_close_bf16(gu.f64(layer.o_f[0, h]), want, f"O_f head {h}")
    assert np.all(sel.sum(axis=2) == w.topk)           # every query block keeps exactly K blocks
