"""The work schedule of the fine branch on the GPU.

For each (batch, head) the schedule orders the cubes by a min-hash of their
lists (query cubes by their CSR rows for the forward and dQ, KV cubes by their
CSC columns for dK/dV), cuts the order into 8 contiguous ranges of equal work,
one per XCD, puts the long lists of each range first, and appends the range
to that XCD's queue.  Checked here:
  * the queues against a recomputation from the CSR / CSC the schedule was
    built from: the min-hash keys, the (key, id) order, the equal-work cut,
    the long-first order inside each range and the queue layout, item for
    item; every cube appears exactly once;
  * that the fine branch run through the schedule gives the per-cube launch's
    results bit for bit (an item is computed the same way whoever takes it)
    and the oracle's;
  * that building it and running through it is bitwise reproducible;
  * odd cube counts, empty lists and padded grids;
  * that a buffer no build wrote (zeros, random bytes) and a schedule built
    for another selection still give the per-cube results bit for bit;
  * MMDiT text rows: each text cube is one more item, its list every cube;
    every queue opens with its text items, head by head, text cubes 2u and
    2u + 1 of head h side by side in queue (h ceil(ntc / 2) + u) mod 8.
"""

import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import vsa2_oracle as orc
from video_dit_trainable_amd import vsa2
from video_dit_trainable_amd.configs import WORKLOADS, Workload
from video_dit_trainable_amd.inputs import make_grad_out, make_qkv, make_selection

pytestmark = pytest.mark.gpu

MID = Workload("mid", 12, (8, 16, 32), 1, 4, 128, "bf16", 8, "lowrank", train=True)          # nb = 64
ODD = Workload("odd", 14, (4, 12, 20), 1, 2, 128, "f32", 5, "lowrank", skew=True, train=True)  # nb = 15
PAD = Workload("pad", 18, (7, 15, 30), 1, 3, 64, "bf16", 6, "lowrank", skew=True, train=True)  # padded, nb = 64
SHORT = WORKLOADS["short"]                                                                    # nb = 512, 20 heads
CASES = [MID, ODD, PAD]
OVH = 4   # the schedule's fixed cost of an item, in list entries
MAGIC = 0x53434844  # header word 17 of a built side, beside the item count in word 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vsa2.lib()


def _dev():
    return torch.device("cuda:0")


def _up(x):
    return (x + 255) // 256 * 256


def decode(layer):
    """The schedule buffer as numpy: per side (query cubes, KV cubes) the
    header (queue starts [8], queue lengths [8], item count, marker) and the
    item array."""
    n_items = layer.bh * (layer.nb + layer.ntc)
    raw = layer.sched.cpu().numpy()
    side = 256 + _up(n_items * 4)
    assert layer.sched.numel() >= 2 * side
    out = []
    for off in (0, side):
        hdr = raw[off:off + 72].view(np.int32)
        assert hdr[16] == n_items and hdr[17] == MAGIC, "header count / marker"
        items = raw[off + 256:off + 256 + n_items * 4].view(np.int32)
        out.append((hdr[:8].copy(), hdr[8:16].copy(), items.copy()))
    return out


def _mh1(j):
    return (j * 40503 + 12345) & 0xFFFF


def _mh2(j):
    return ((j ^ 0x5A5A) * 52429 + 777) & 0xFFFF


def expected_queues(ptr, idx, nb, ntc=0):
    """The queues, recomputed from the lists of every head (ptr [bh, nb+1],
    idx [bh, k]) by the rules the schedule states; ntc text cubes per head
    are items nb .. nb + ntc - 1 of it."""
    queues = [[] for _ in range(8)]
    n = nb + ntc
    for h in range(ptr.shape[0]):
        for t in range(ntc):
            queues[(h * ((ntc + 1) // 2) + t // 2) % 8].append(h * n + nb + t)
    for h in range(ptr.shape[0]):
        lists = [idx[h, ptr[h, c]:ptr[h, c + 1]] for c in range(nb)]
        keys = [((int(min(_mh1(l))) << 16) | int(min(_mh2(l)))) if len(l) else 0xFFFFFFFF for l in lists]
        order = sorted(range(nb), key=lambda c: (keys[c], c))
        w = np.array([len(lists[c]) + OVH for c in order], dtype=np.int64)
        before = np.concatenate([[0], np.cumsum(w)[:-1]])
        xcd = np.minimum(7, (8 * (2 * before + w)) // (2 * w.sum()))
        cls = [int(np.floor(np.log2(len(lists[c]) + 1))) for c in order]
        for x in range(8):
            pos = [p for p in range(nb) if xcd[p] == x]
            pos.sort(key=lambda p: (-cls[p], p))
            queues[x] += [h * n + order[p] for p in pos]
    return queues


def check_side(hdr_start, hdr_len, items, ptr, idx, nb, ntc=0):
    want = expected_queues(ptr, idx, nb, ntc)
    assert list(hdr_len) == [len(q) for q in want]
    assert list(hdr_start) == list(np.concatenate([[0], np.cumsum(hdr_len)[:-1]]))
    for x in range(8):
        got = items[hdr_start[x]:hdr_start[x] + hdr_len[x]]
        assert got.tolist() == want[x], f"queue {x} differs"
    assert sorted(items.tolist()) == list(range(ptr.shape[0] * (nb + ntc))), "every cube exactly once"


def _layer(w, dev):
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype)
    layer = vsa2.Layer(p, w.topk, w.d_model, device=dev)
    assert layer.sched is not None
    return p, layer


@pytest.mark.parametrize("w", CASES + [SHORT], ids=lambda w: w.name)
def test_schedule_queues_from_router_selection(w):
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    p, layer = _layer(w, dev)
    vsa2.vsa2_pool(p, q, k, v, layer.pooled)
    vsa2.vsa2_route(p, layer.pooled, layer.scores, layer.ws)
    layer.sched.zero_()      # padding between the parts is never written: start both builds from zero
    vsa2.vsa2_topk_per_seq(p, layer.scores, w.topk, layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx,
                           layer.ws, sched=layer.sched)
    torch.cuda.synchronize()
    first = layer.sched.clone()
    (rs, rl, ri), (cs, cl, cidx) = decode(layer)
    rp, ci, cp, rix = (t[0].cpu().numpy() for t in (layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx))
    check_side(rs, rl, ri, rp, ci, w.nb)
    check_side(cs, cl, cidx, cp, rix, w.nb)
    # the same selection gives the same schedule (built again through the CSR)
    layer.sched.zero_()
    vsa2.vsa2_plan_from_csr(p, w.topk, layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx, layer.ws,
                            sched=layer.sched)
    torch.cuda.synchronize()
    assert torch.equal(layer.sched, first)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_scheduled_fine_branch_matches_per_cube_and_oracle(w):
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    d_o = make_grad_out(w, device=dev)
    p, layer = _layer(w, dev)
    rp, ci = make_selection(w, device=dev)     # heavy-tailed rows, some empty
    layer.set_selection(rp, ci)
    args = (layer.row_ptr, layer.col_idx)
    lists = (layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx)
    out = {}
    for mode, sched in (("per-cube", None), ("scheduled", layer.sched)):
        o_f, lse = torch.empty_like(layer.o_f), torch.empty_like(layer.lse)
        vsa2.vsa2_sparse_attn_fwd(p, w.topk, q, k, v, *args, o_f, lse, layer.ws, sched=sched)
        g = [torch.full_like(q, float("nan")) for _ in range(3)]
        vsa2.vsa2_sparse_attn_bwd(p, w.topk, q, k, v, o_f, lse, d_o, *lists, None, *g, layer.ws, sched=sched)
        torch.cuda.synchronize()
        out[mode] = (o_f, lse, g)
    (o1, l1, g1), (o2, l2, g2) = out["per-cube"], out["scheduled"]
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "the scheduled forward differs from the per-cube one"
    for name, a, b in zip(("dQ", "dK", "dV"), g1, g2):
        assert torch.equal(a, b), f"{name}: the scheduled backward differs from the per-cube one"
    real = orc.token_valid(w.grid)
    for h in range(w.heads):
        mask = orc.csr_to_mask(rp[0, h].cpu().numpy(), ci[0, h].cpu().numpy(), w.nb)
        qh, kh, vh, dh = (gu.f64(t[0, h]) for t in (q, k, v, d_o))
        o, lse = orc.fine_forward(qh, kh, vh, mask, valid=real)
        if w.dtype == "f32":
            gu.assert_close_f32(gu.f64(o2[0, h]), o, f"O_f head {h}")
        else:
            gu.assert_close_bf16(gu.f64(o2[0, h]), o, f"O_f head {h}")
        dq, dk, dv = orc.fine_backward(qh, kh, vh, mask, dh, valid=real)
        for name, got, want in zip(("dQ", "dK", "dV"), g2, (dq, dk, dv)):
            rr = gu.rel_l2(gu.f64(got[0, h]), want)
            assert rr <= (1e-4 if w.dtype == "f32" else 2e-2), f"{name} head {h}: rel-L2 {rr:.3g}"


def test_scheduled_backward_is_deterministic():
    w = MID
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    d_o = make_grad_out(w, device=dev)
    p, layer = _layer(w, dev)
    layer.set_selection(*make_selection(w, device=dev))
    lists = (layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx)
    vsa2.vsa2_sparse_attn_fwd(p, w.topk, q, k, v, layer.row_ptr, layer.col_idx, layer.o_f, layer.lse, layer.ws,
                              sched=layer.sched)
    runs = []
    for _ in range(2):
        g = [torch.empty_like(q) for _ in range(3)]
        vsa2.vsa2_sparse_attn_bwd(p, w.topk, q, k, v, layer.o_f, layer.lse, d_o, *lists, None, *g, layer.ws,
                                  sched=layer.sched)
        torch.cuda.synchronize()
        runs.append(g)
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def _fine(p, w, layer, q, k, v, d_o, sched):
    o_f, lse = torch.empty_like(layer.o_f), torch.empty_like(layer.lse)
    vsa2.vsa2_sparse_attn_fwd(p, w.topk, q, k, v, layer.row_ptr, layer.col_idx, o_f, lse, layer.ws, sched=sched)
    g = [torch.full_like(q, float("nan")) for _ in range(3)]
    vsa2.vsa2_sparse_attn_bwd(p, w.topk, q, k, v, o_f, lse, d_o, layer.row_ptr, layer.col_idx, layer.col_ptr,
                              layer.row_idx, None, *g, layer.ws, sched=sched)
    torch.cuda.synchronize()
    return [o_f, lse] + g


@pytest.mark.parametrize("w", [MID, PAD], ids=lambda w: w.name)
def test_unbuilt_or_stale_schedule_gives_the_same_results(w):
    """The fine kernels check the header's item count and marker: a buffer
    that no build wrote makes them take the cubes in plain order, and a
    schedule of another selection still lists every cube once."""
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    d_o = make_grad_out(w, device=dev)
    p, layer = _layer(w, dev)
    names = ("O_f", "LSE", "dQ", "dK", "dV")
    # selection A builds the schedule; selection B (the router's) replaces the
    # lists without touching it
    layer.set_selection(*make_selection(w, device=dev))
    vsa2.vsa2_pool(p, q, k, v, layer.pooled)
    vsa2.vsa2_route(p, layer.pooled, layer.scores, layer.ws)
    vsa2.vsa2_topk_per_seq(p, layer.scores, w.topk, layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx,
                           layer.ws)
    want = _fine(p, w, layer, q, k, v, d_o, None)
    got = _fine(p, w, layer, q, k, v, d_o, layer.sched)
    for nm, a, b in zip(names, want, got):
        assert torch.equal(a, b), f"{nm}: a schedule of another selection changed the result"
    gen = torch.Generator().manual_seed(5)
    for label, fill in (("zeros", torch.zeros(layer.sched.numel(), dtype=torch.uint8)),
                        ("random bytes", torch.randint(0, 256, (layer.sched.numel(),), generator=gen,
                                                       dtype=torch.uint8))):
        layer.sched.copy_(fill.to(dev))
        got = _fine(p, w, layer, q, k, v, d_o, layer.sched)
        for nm, a, b in zip(names, want, got):
            assert torch.equal(a, b), f"{nm}: an unbuilt schedule buffer ({label}) changed the result"


# the schedule build sorts in LDS up to 8192 lists per (batch, head) and counts
# ranks beyond: one case past 4096 (the largest sort) and one past 8192
SORT_MID = Workload("sort-mid", 61, (48, 80, 84), 1, 2, 64, "bf16", 4, "lowrank")     # nb = 5,040
SORT_BIG = Workload("sort-big", 62, (64, 64, 132), 1, 2, 64, "bf16", 4, "lowrank")    # nb = 8,448


@pytest.mark.parametrize("w", [SORT_MID, SORT_BIG], ids=lambda w: w.name)
def test_schedule_queues_on_both_sides_of_the_lds_sort(w):
    dev = _dev()
    p, layer = _layer(w, dev)
    layer.sched.zero_()
    layer.set_selection(*make_selection(w, device=dev))      # the plan call builds the schedule
    torch.cuda.synchronize()
    (rs, rl, ri), (cs, cl, cidx) = decode(layer)
    rp, ci, cp, rix = (t[0].cpu().numpy() for t in (layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx))
    check_side(rs, rl, ri, rp, ci, w.nb)
    check_side(cs, cl, cidx, cp, rix, w.nb)


@pytest.mark.parametrize("w", [MID, SHORT], ids=lambda w: w.name)
def test_forward_only_topk_builds_the_query_side(w):
    """TopK without the CSC (a selection only the forward runs on): the same
    CSR, the same query-cube side of the schedule byte for byte, the KV-cube
    side left alone, and the same forward through it."""
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    p, layer = _layer(w, dev)
    vsa2.vsa2_pool(p, q, k, v, layer.pooled)
    vsa2.vsa2_route(p, layer.pooled, layer.scores, layer.ws)
    layer.sched.zero_()
    vsa2.vsa2_topk_per_seq(p, layer.scores, w.topk, layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx,
                           layer.ws, sched=layer.sched)
    want = [t.clone() for t in (layer.row_ptr, layer.col_idx, layer.sched)]
    o1, l1 = torch.empty_like(layer.o_f), torch.empty_like(layer.lse)
    vsa2.vsa2_sparse_attn_fwd(p, w.topk, q, k, v, layer.row_ptr, layer.col_idx, o1, l1, layer.ws, sched=layer.sched)
    torch.cuda.synchronize()
    layer.row_ptr.fill_(-1)
    layer.col_idx.fill_(-1)
    layer.sched.fill_(7)
    vsa2.vsa2_topk_per_seq(p, layer.scores, w.topk, layer.row_ptr, layer.col_idx, None, None, layer.ws,
                           sched=layer.sched)
    torch.cuda.synchronize()
    assert torch.equal(layer.row_ptr, want[0]) and torch.equal(layer.col_idx, want[1])
    side = 256 + _up(layer.bh * layer.nb * 4)
    raw, ref = layer.sched.cpu().numpy(), want[2].cpu().numpy()
    # the query side: header words and items as with the CSC (the bytes between them are never written)
    assert np.array_equal(raw[:72], ref[:72]) and np.array_equal(raw[256:side], ref[256:side])
    assert np.all(raw[side:2 * side] == 7), "the KV-cube side was written"
    o2, l2 = torch.empty_like(layer.o_f), torch.empty_like(layer.lse)
    vsa2.vsa2_sparse_attn_fwd(p, w.topk, q, k, v, layer.row_ptr, layer.col_idx, o2, l2, layer.ws, sched=layer.sched)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# 128-token blocks: one item per block, run by a whole-block workgroup
B128 = Workload("b128", 32, (8, 16, 32), 1, 3, 128, "bf16", 4, "lowrank", skew=True, train=True, block=128)
B128_PAD = Workload("b128-pad", 33, (5, 6, 9), 1, 2, 64, "bf16", 3, "lowrank", train=True, block=128)


@pytest.mark.parametrize("w", [B128, B128_PAD], ids=lambda w: w.name)
def test_block128_schedule(w):
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    d_o = make_grad_out(w, device=dev)
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype, block=128)
    layer = vsa2.Layer(p, w.topk, w.d_model, device=dev)
    assert layer.sched is not None and layer.nb == w.nblk
    rp, ci = make_selection(w, device=dev)
    layer.sched.zero_()
    layer.set_selection(rp, ci)
    torch.cuda.synchronize()
    (rs, rl, ri), (cs, cl, cidx) = decode(layer)
    rpn, cin, cpn, rin = (t[0].cpu().numpy() for t in (layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx))
    check_side(rs, rl, ri, rpn, cin, w.nblk)
    check_side(cs, cl, cidx, cpn, rin, w.nblk)
    lists = (layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx)
    out = {}
    for mode, sched in (("per-block", None), ("scheduled", layer.sched)):
        o_f, lse = torch.empty_like(layer.o_f), torch.empty_like(layer.lse)
        vsa2.vsa2_sparse_attn_fwd(p, w.topk, q, k, v, layer.row_ptr, layer.col_idx, o_f, lse, layer.ws, sched=sched)
        g = [torch.full_like(q, float("nan")) for _ in range(3)]
        vsa2.vsa2_sparse_attn_bwd(p, w.topk, q, k, v, o_f, lse, d_o, *lists, None, *g, layer.ws, sched=sched)
        torch.cuda.synchronize()
        out[mode] = [o_f, lse] + g
    for name, a, b in zip(("O_f", "LSE", "dQ", "dK", "dV"), out["per-block"], out["scheduled"]):
        assert torch.equal(a, b), f"{name}: the scheduled run differs from the per-block one"
    real = orc.token_valid(w.grid, 128)
    o2, _, dq2, dk2, dv2 = out["scheduled"]
    for h in range(w.heads):
        mask = orc.csr_to_mask(rp[0, h].cpu().numpy(), ci[0, h].cpu().numpy(), w.nblk)
        qh, kh, vh, dh = (gu.f64(t[0, h]) for t in (q, k, v, d_o))
        o, _ = orc.fine_forward(qh, kh, vh, mask, valid=real, block=128)
        gu.assert_close_bf16(gu.f64(o2[0, h]), o, f"O_f head {h}")
        for name, got, want in zip(("dQ", "dK", "dV"), (dq2, dk2, dv2),
                                   orc.fine_backward(qh, kh, vh, mask, dh, valid=real, block=128)):
            rr = gu.rel_l2(gu.f64(got[0, h]), want)
            assert rr <= 2e-2, f"{name} head {h}: rel-L2 {rr:.3g}"


# MMDiT text rows with 64-token blocks: every text cube is one more item
TXT_SCHED = Workload("txt-sched", 45, (8, 16, 32), 1, 3, 128, "bf16", 4, "lowrank", skew=True, train=True,
                     text=600)                                                   # nb = 64, 10 text cubes
TXT_SCHED_PAD = Workload("txt-sched-pad", 46, (7, 13, 15), 1, 2, 64, "f32", 6, "lowrank", train=True, text=150)


@pytest.mark.parametrize("w", [TXT_SCHED, TXT_SCHED_PAD], ids=lambda w: w.name)
def test_text_rows_on_the_schedule(w):
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    d_o = make_grad_out(w, device=dev)
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype, text=w.text)
    layer = vsa2.Layer(p, w.topk, w.d_model, device=dev)
    ntc = -(-w.text // 64)
    assert layer.sched is not None and layer.ntc == ntc
    rp, ci = make_selection(w, device=dev)     # heavy-tailed rows, some empty
    layer.sched.zero_()
    layer.set_selection(rp, ci)
    torch.cuda.synchronize()
    (rs, rl, ri), (cs, cl, cidx) = decode(layer)
    rpn, cin, cpn, rin = (t[0].cpu().numpy() for t in (layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx))
    check_side(rs, rl, ri, rpn, cin, w.nb, ntc)
    check_side(cs, cl, cidx, cpn, rin, w.nb, ntc)
    out = {}
    for mode, sched in (("per-cube", None), ("scheduled", layer.sched)):
        out[mode] = _fine(p, w, layer, q, k, v, d_o, sched)
    for name, a, b in zip(("O_f", "LSE", "dQ", "dK", "dV"), out["per-cube"], out["scheduled"]):
        assert torch.equal(a, b), f"{name}: the scheduled run differs from the per-cube one"
    real = orc.token_valid(w.grid)
    o2, lse2, dq2, dk2, dv2 = out["scheduled"]
    tol = 1e-4 if w.dtype == "f32" else 2e-2
    for h in range(w.heads):
        mask = orc.csr_to_mask(rp[0, h].cpu().numpy(), ci[0, h].cpu().numpy(), w.nb)
        qh, kh, vh, dh = (gu.f64(t[0, h]) for t in (q, k, v, d_o))
        o, _ = orc.fine_forward(qh, kh, vh, mask, valid=real, n_text=w.text)
        if w.dtype == "f32":
            gu.assert_close_f32(gu.f64(o2[0, h]), o, f"O_f head {h}")
        else:
            gu.assert_close_bf16(gu.f64(o2[0, h]), o, f"O_f head {h}")
        for name, got, want in zip(("dQ", "dK", "dV"), (dq2, dk2, dv2),
                                   orc.fine_backward(qh, kh, vh, mask, dh, valid=real, n_text=w.text)):
            rr = gu.rel_l2(gu.f64(got[0, h]), want)
            assert rr <= tol, f"{name} head {h}: rel-L2 {rr:.3g}"


def test_pair_forward_takes_each_list_in_its_own_order():
    """The forward's pairs walk the merge of two lists but give each cube its
    own list's tiles in that list's order: with rows whose columns are out of
    order or repeat a cube (caller errors the header lets stay memory-safe),
    the scheduled forward still equals the one-cube forward bit for bit, and
    with columns merely out of order it still matches the oracle."""
    w = MID
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    p, layer = _layer(w, dev)
    rp, ci = make_selection(w, device=dev)
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy().copy()
    gen = np.random.default_rng(7)
    shuffled = cin.copy()
    for h in range(w.heads):
        for i in range(w.nb):
            a, b = rpn[0, h, i], rpn[0, h, i + 1]
            shuffled[0, h, a:b] = gen.permutation(shuffled[0, h, a:b])
    repeated = shuffled.copy()
    for h in range(w.heads):
        for i in range(0, w.nb, 3):  # every third row repeats its first cube in place of its last
            a, b = rpn[0, h, i], rpn[0, h, i + 1]
            if b - a >= 2:
                repeated[0, h, b - 1] = repeated[0, h, a]
    for label, cols in (("shuffled", shuffled), ("repeated", repeated)):
        layer.set_selection(rp, torch.tensor(cols, dtype=torch.int32, device=dev))
        out = {}
        for mode, sched in (("one cube", None), ("pairs", layer.sched)):
            o_f, lse = torch.empty_like(layer.o_f), torch.empty_like(layer.lse)
            vsa2.vsa2_sparse_attn_fwd(p, w.topk, q, k, v, layer.row_ptr, layer.col_idx, o_f, lse, layer.ws,
                                      sched=sched)
            torch.cuda.synchronize()
            out[mode] = (o_f, lse)
        assert torch.equal(out["one cube"][0], out["pairs"][0]), f"{label}: O_f differs"
        assert torch.equal(out["one cube"][1], out["pairs"][1]), f"{label}: LSE differs"
        if label == "shuffled":
            real = orc.token_valid(w.grid)
            for h in range(w.heads):
                mask = orc.csr_to_mask(rpn[0, h], cin[0, h], w.nb)
                o, _ = orc.fine_forward(*(gu.f64(t[0, h]) for t in (q, k, v)), mask, valid=real)
                gu.assert_close_bf16(gu.f64(out["pairs"][0][0, h]), o, f"O_f head {h}")
