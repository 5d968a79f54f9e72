"""GPU vs CPU-oracle parity at the full 720p sizes, in the launch configuration
the benchmark times (latent 44x48x104 = 219,648 tokens, 20 heads, d = 128,
bf16, per-sequence top64, skewed query-cube scales; the inference shape at
top128).

The oracle cannot redo a whole 720p layer in seconds, so these tests compare
what it can compute one piece at a time -- router rows of sampled query cubes,
one head's full score matrix, the fine outputs and gradients of sampled cubes,
sampled rows of dX and the whole of dW_g (token chunks) -- and check the
properties that hold at any size: every score row sums to 1/8, the selection
is exactly the top k of the GPU's own scores with ties to the lower flat
index, CSR/CSC are each other's transpose with columns ascending.  The same
checks run on the 720p training problem on a grid one short of whole cubes
along every axis (43 x 47 x 103, padded), sampling the border cubes that hold
pad slots; there every pad row of every output must be exactly zero.  And
they run on the 720p training problem with 128-token blocks (4x4x8, two
x-adjacent cubes), where the scores, the selection and the coarse tokens are
per block.

Tolerances as in test_gpu_parity: bf16 outputs max-abs 2e-2 and rel-L2 1e-2,
gradients rel-L2 2e-2, index sets exact outside the relative 1e-3 band.
"""

import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import vsa2_oracle as orc
from video_dit_trainable_amd import vsa2
from video_dit_trainable_amd.configs import WORKLOADS
from video_dit_trainable_amd.inputs import make_gate_inputs, make_grad_out, make_qkv, make_selection

pytestmark = pytest.mark.gpu

TRAIN = WORKLOADS["train720"]
INFER = WORKLOADS["infer720"]
TRAIN_PAD = WORKLOADS["train720pad"]    # 43 x 47 x 103, padded to the same 44 x 48 x 104 slots
TRAIN_B128 = WORKLOADS["train720b128"]  # 128-token blocks (4x4x8), 1716 blocks
TRAIN_TEXT = WORKLOADS["train720text"]  # plus 512 MMDiT text tokens in the fine branch
TRAIN_VSA = WORKLOADS["train720vsa"]    # the VSA router baseline at top128
TRAIN480 = WORKLOADS["train480"]        # 28 x 32 x 52 = 46,592 tokens, 728 cubes


def _dev():
    return torch.device("cuda:0")


def _run(w, topk, train, fine_on="seeded"):
    """The layer on the GPU at full size.  Route + TopK run first and their
    scores and selection are kept for the router/TopK checks; the fine branch,
    coarse branch, gate and backward then run on a seeded selection with the
    exact budget (make_selection, fine_on="seeded"), or, as the benchmark
    runs them, on the router's own selection (fine_on="routed"); the oracle is
    given the same selection.  The fine kernels run through the work schedule
    that TopK (or set_selection) built for that selection, as in the
    benchmark."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    x, w_g = make_gate_inputs(w, device=dev, zero_gate=False)
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype, block=w.block, text=w.text)
    layer = vsa2.Layer(p, topk, w.d_model, device=dev)
    vsa2.vsa2_pool(p, q, k, v, layer.pooled)
    vsa2.vsa2_route(p, layer.pooled, layer.scores, layer.ws)
    vsa2.vsa2_topk_per_seq(p, layer.scores, topk, layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx,
                           layer.ws, sched=layer.sched)
    torch.cuda.synchronize()
    out = dict(w=w, topk=topk, q=q, k=k, v=v, x=x, w_g=w_g, layer=layer,
               routed=[t.clone() for t in (layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx)])
    if fine_on == "seeded":
        sel_rp, sel_ci = make_selection(w, topk=topk)
        out["sel"] = (sel_rp.numpy(), sel_ci.numpy())
        layer.set_selection(sel_rp.to(dev), sel_ci.to(dev))
    else:
        out["sel"] = tuple(t.cpu().numpy() for t in out["routed"][:2])
    layer.forward(q, k, v, x, w_g, route=False)
    if train:
        d_o = make_grad_out(w, device=dev)
        g = layer.grads()
        vsa2.vsa2_coarse_gate_bwd(p, layer.pooled, x, w.d_model, w_g, layer.saved, d_o, g["dqkv_c"], g["dx"],
                                  g["dw_g"], layer.ws)
        # fine-branch gradients alone (no coarse rows added) for the sampled checks
        vsa2.vsa2_sparse_attn_bwd(p, topk, q, k, v, layer.o_f, layer.lse, d_o, layer.row_ptr, layer.col_idx,
                                  layer.col_ptr, layer.row_idx, None, g["dq"], g["dk"], g["dv"], layer.ws,
                                  sched=layer.sched)
        out["d_o"] = d_o
    torch.cuda.synchronize()
    return out


@pytest.fixture(scope="module")
def train720():
    return _run(TRAIN, TRAIN.topk, True)


def _routed(r, h):
    """The GPU router's own selection of head h (CSR)."""
    return r["routed"][0][0, h].cpu().numpy(), r["routed"][1][0, h].cpu().numpy()


def _seeded(r, h):
    """The selection of head h that both sides run the fine branch on (the
    seeded one, or the router's own for a routed run)."""
    return r["sel"][0][0, h], r["sel"][1][0, h]


def _sample_cubes(rp, n_extra=2):
    """Query cubes to check: the longest list, an empty one if any, the first,
    the last and a few spread over the sequence."""
    lens = np.diff(rp)
    nb = len(lens)
    picks = [int(np.argmax(lens)), 0, nb - 1] + [int(i) for i in np.linspace(1, nb - 2, n_extra).round()]
    empty = np.nonzero(lens == 0)[0]
    if len(empty):
        picks.append(int(empty[len(empty) // 2]))
    return sorted(set(picks))


def test_router_rows_and_row_sums(train720):
    r = train720
    w = r["w"]
    scores = r["layer"].scores[0]
    sums = scores.double().sum(dim=2).cpu().numpy()
    np.testing.assert_allclose(sums, 1.0 / 8.0, rtol=1e-4)     # every pooled query's softmax sums to 1
    for h in (0, 13):
        rows = np.array([0, w.nb // 3, w.nb - 1])
        want = orc.router_scores(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), w.grid, bf16_pooled=True, rows=rows)
        got = scores[h].double().cpu().numpy()[rows]
        for n in range(len(rows)):
            assert gu.rel_l2(got[n], want[n]) <= 1e-4, f"head {h} row {rows[n]}"


def test_selection_is_exact_topk_of_gpu_scores(train720):
    r = train720
    w, layer = r["w"], r["layer"]
    k = layer.k
    rp_all, ci_all, cp_all, ri_all = r["routed"]
    gu.check_csr_csc(rp_all[0, [0, 19]], ci_all[0, [0, 19]], cp_all[0, [0, 19]], ri_all[0, [0, 19]], w.nb, k)
    for h in (0, 7, 19):
        s = layer.scores[0, h].cpu().numpy().reshape(-1)         # the GPU's own fp32 scores
        order = np.argsort(-s, kind="stable")                     # score desc, flat index asc
        want = np.zeros(s.size, dtype=bool)
        want[order[:k]] = True
        rp, ci = _routed(r, h)
        got = orc.csr_to_mask(rp, ci, w.nb).reshape(-1)
        assert np.array_equal(got, want), f"head {h}: selection differs from the exact top-k of its scores"


def test_selection_matches_oracle_router_full_head(train720):
    r = train720
    w, layer = r["w"], r["layer"]
    h = 13
    want_scores = orc.router_scores(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), w.grid, bf16_pooled=True)
    rp, ci = _routed(r, h)
    got = orc.csr_to_mask(rp, ci, w.nb)
    outside, band, inside = gu.band_compare(got, want_scores, layer.k)
    assert outside == 0, f"{outside} selection mismatches outside the 1e-3 band ({band} pairs in it)"


@pytest.mark.parametrize("h", [0, 13])
def test_fine_forward_sampled(train720, h):
    r = train720
    w, layer = r["w"], r["layer"]
    rp, ci = _seeded(r, h)
    mask = orc.csr_to_mask(rp, ci, w.nb)
    cubes = _sample_cubes(rp)
    o, lse = orc.fine_forward(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), gu.f64(r["v"][0, h]), mask, rows=cubes)
    toks = orc._tokens_of(cubes)
    got_o = gu.f64(layer.o_f[0, h])[toks]
    got_lse = gu.f64(layer.lse[0, h])[toks]
    gu.assert_close_bf16(got_o, o[toks], f"O_f head {h} cubes {cubes}")
    live = np.isfinite(lse[toks])
    assert np.all(np.isneginf(got_lse[~live])) and np.all(got_o[~live] == 0)
    np.testing.assert_allclose(got_lse[live], lse[toks][live], atol=1e-3)


def test_merged_output_and_gate_sampled(train720):
    _check_merged_output_and_gate(train720, 5)


def _check_merged_output_and_gate(r, h):
    w, layer = r["w"], r["layer"]
    oc_hat, _, g = layer.saved_views()
    rp, ci = _seeded(r, h)
    mask = orc.csr_to_mask(rp, ci, w.nb)
    cubes = _sample_cubes(rp, n_extra=1)
    toks = orc._tokens_of(cubes)
    q, k, v = (gu.f64(t[0, h]) for t in (r["q"], r["k"], r["v"]))
    o_f, _ = orc.fine_forward(q, k, v, mask, rows=cubes)
    want_oc, _, _ = orc.coarse_forward(q, k, v, w.grid)
    gate = orc.gate(gu.f64(r["x"][0][torch.from_numpy(toks).to(_dev())]), gu.f64(r["w_g"]))[:, h]
    gu.assert_close_bf16(gu.f64(oc_hat[0, h]), want_oc, f"O_hat_c head {h}")
    np.testing.assert_allclose(gu.f64(g[0, h])[toks], gate, atol=1e-4, rtol=1e-3)
    want_o = gate[:, None] * want_oc[toks // 64] + o_f[toks]
    gu.assert_close_bf16(gu.f64(layer.o[0, h])[toks], want_o, f"O head {h}", rounding=2.0 ** -8)


@pytest.mark.parametrize("h", [0, 13])
def test_fine_backward_sampled(train720, h):
    r = train720
    w, layer = r["w"], r["layer"]
    g = layer.grads()
    rp, ci = _seeded(r, h)
    mask = orc.csr_to_mask(rp, ci, w.nb)
    q, k, v, d_o = (gu.f64(t[0, h]) for t in (r["q"], r["k"], r["v"], r["d_o"]))
    # dQ of sampled query cubes: their rows alone
    cubes = [c for c in _sample_cubes(rp) if mask[c].any()]
    sub = np.zeros_like(mask)
    sub[cubes] = mask[cubes]
    dq, _, _ = orc.fine_backward(q, k, v, sub, d_o)
    toks = orc._tokens_of(cubes)
    r_dq = gu.rel_l2(gu.f64(g["dq"][0, h])[toks], dq[toks])
    assert r_dq <= 2e-2, f"dQ head {h}: rel-L2 {r_dq:.3g}"
    # dK, dV of two KV cubes: every query row that selected them, whole rows
    lens = mask.sum(axis=0)
    order = np.argsort(lens)
    js = [int(order[len(order) // 2]), int(order[int(len(order) * 0.9)])]
    for j in js:
        rows = np.nonzero(mask[:, j])[0]
        sub = np.zeros_like(mask)
        sub[rows] = mask[rows]
        _, dk, dv = orc.fine_backward(q, k, v, sub, d_o)
        tj = np.arange(64 * j, 64 * j + 64)
        for name, got, want in (("dK", g["dk"], dk), ("dV", g["dv"], dv)):
            rr = gu.rel_l2(gu.f64(got[0, h])[tj], want[tj])
            assert rr <= 2e-2, f"{name} head {h} KV cube {j} ({len(rows)} query cubes): rel-L2 {rr:.3g}"


def test_gate_gradients(train720):
    _check_gate_gradients(train720)


def _check_gate_gradients(r):
    w, layer = r["w"], r["layer"]
    g = layer.grads()
    oc_hat = np.stack([orc.coarse_forward(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), gu.f64(r["v"][0, h]),
                                          w.grid)[0] for h in range(w.heads)])   # [H, nb, d]
    w_g = gu.f64(r["w_g"])
    dw = np.zeros_like(w_g)
    chunk = 16384
    for t0 in range(0, w.L, chunk):
        toks = np.arange(t0, min(w.L, t0 + chunk))
        sl = slice(int(toks[0]), int(toks[-1]) + 1)
        _, dx, part = orc.gate_backward(gu.f64(r["x"][0, sl]), w_g, oc_hat, gu.f64(r["d_o"][0, :, sl]), toks)
        dw += part
        if t0 in (0, 2 * chunk, 8 * chunk):
            rr = gu.rel_l2(gu.f64(g["dx"][0, sl]), dx)
            assert rr <= 2e-2, f"dX tokens {t0}..: rel-L2 {rr:.3g}"
    rr = gu.rel_l2(gu.f64(g["dw_g"]), dw)
    assert rr <= 2e-2, f"dW_g: rel-L2 {rr:.3g}"


# ----------------------------------------------------------------------------- the router's own selection
# The fine branch run on the selection the router and the per-sequence TopK
# made (the benchmark's launch configuration), at the 480p training shape
# (latent 28x32x52 = 46,592 tokens, 728 cubes) and at the 720p training shape.
# Per-sequence TopK (Eq.(8)-(9)) gives the "sink" KV cubes that many query
# cubes select long CSC columns, and the skewed query scales long CSR rows;
# the longest of both are compared with the oracle.
@pytest.fixture(scope="module")
def train480():
    return _run(TRAIN480, TRAIN480.topk, True, fine_on="routed")


@pytest.fixture(scope="module")
def train720_routed():
    return _run(TRAIN, TRAIN.topk, True, fine_on="routed")


ROUTED = ["train480", "train720_routed"]


def test_train480_router_rows_and_selection(train480):
    r = train480
    w, layer = r["w"], r["layer"]
    scores = layer.scores[0]
    np.testing.assert_allclose(scores.double().sum(dim=2).cpu().numpy(), 1.0 / 8.0, rtol=1e-4)
    rp0, _ = _routed(r, 0)
    rows = np.array(sorted({0, int(np.argmax(np.diff(rp0))), w.nb // 2, w.nb - 1}))
    for h in (0, 11):
        want = orc.router_scores(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), w.grid, bf16_pooled=True, rows=rows)
        got = scores[h].double().cpu().numpy()[rows]
        for n in range(len(rows)):
            assert gu.rel_l2(got[n], want[n]) <= 1e-4, f"head {h} row {rows[n]}"
    gu.check_csr_csc(*[t[0, [0, 19]] for t in r["routed"]], w.nb, layer.k)
    for h in (0, 19):
        s = scores[h].cpu().numpy().reshape(-1)
        order = np.argsort(-s, kind="stable")
        want = np.zeros(s.size, dtype=bool)
        want[order[:layer.k]] = True
        rp, ci = _routed(r, h)
        assert np.array_equal(orc.csr_to_mask(rp, ci, w.nb).reshape(-1), want), f"head {h}"
    # one whole head against the oracle router's own top k (exact outside the band)
    h = 7
    want_scores = orc.router_scores(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), w.grid, bf16_pooled=True)
    rp, ci = _routed(r, h)
    outside, band, _ = gu.band_compare(orc.csr_to_mask(rp, ci, w.nb), want_scores, layer.k)
    assert outside == 0, f"{outside} selection mismatches outside the 1e-3 band ({band} pairs in it)"


@pytest.mark.parametrize("name", ROUTED)
@pytest.mark.parametrize("h", [0, 13])
def test_routed_fine_forward_longest_row(request, name, h):
    r = request.getfixturevalue(name)
    w, layer = r["w"], r["layer"]
    rp, ci = _seeded(r, h)
    mask = orc.csr_to_mask(rp, ci, w.nb)
    cubes = _sample_cubes(rp)                             # the longest row and any empty one among them
    o, lse = orc.fine_forward(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), gu.f64(r["v"][0, h]), mask, rows=cubes)
    toks = orc._tokens_of(cubes)
    got_o = gu.f64(layer.o_f[0, h])[toks]
    got_lse = gu.f64(layer.lse[0, h])[toks]
    gu.assert_close_bf16(got_o, o[toks], f"{w.name} O_f head {h} cubes {cubes} (longest list {np.diff(rp).max()})")
    live = np.isfinite(lse[toks])
    assert np.all(np.isneginf(got_lse[~live])) and np.all(got_o[~live] == 0)
    np.testing.assert_allclose(got_lse[live], lse[toks][live], atol=1e-3)


@pytest.mark.parametrize("name", ROUTED)
@pytest.mark.parametrize("h", [0, 13])
def test_routed_fine_backward_long_columns(request, name, h):
    """dK, dV of the longest CSC column of the router's selection and of one
    at the 99th percentile (every query row that selected them, whole rows),
    and dQ of the longest CSR row."""
    r = request.getfixturevalue(name)
    w, layer = r["w"], r["layer"]
    g = layer.grads()
    rp, ci = _seeded(r, h)
    mask = orc.csr_to_mask(rp, ci, w.nb)
    q, k, v, d_o = (gu.f64(t[0, h]) for t in (r["q"], r["k"], r["v"], r["d_o"]))
    lens = mask.sum(axis=0)
    order = np.argsort(lens, kind="stable")
    js = [int(order[-1]), int(order[int(0.99 * (len(order) - 1))])]
    assert lens[js[0]] > 3 * w.topk, f"{w.name} head {h}: no long column ({lens[js[0]]})"
    for j in js:
        rows = np.nonzero(mask[:, j])[0]
        sub = np.zeros_like(mask)
        sub[rows] = mask[rows]
        _, dk, dv = orc.fine_backward(q, k, v, sub, d_o)
        tj = np.arange(64 * j, 64 * j + 64)
        for nm, got, want in (("dK", g["dk"], dk), ("dV", g["dv"], dv)):
            rr = gu.rel_l2(gu.f64(got[0, h])[tj], want[tj])
            assert rr <= 2e-2, f"{w.name} {nm} head {h} KV cube {j} ({len(rows)} query cubes): rel-L2 {rr:.3g}"
    i = int(np.argmax(mask.sum(axis=1)))
    sub = np.zeros_like(mask)
    sub[i] = mask[i]
    dq, _, _ = orc.fine_backward(q, k, v, sub, d_o)
    ti = np.arange(64 * i, 64 * i + 64)
    rr = gu.rel_l2(gu.f64(g["dq"][0, h])[ti], dq[ti])
    assert rr <= 2e-2, f"{w.name} dQ head {h} query cube {i} ({mask[i].sum()} KV cubes): rel-L2 {rr:.3g}"


def test_train480_merged_output_and_gate(train480):
    _check_merged_output_and_gate(train480, 5)


def test_train480_gate_gradients(train480):
    _check_gate_gradients(train480)


def test_inference_top128_sampled():
    r = _run(INFER, 128, False)
    w, layer = r["w"], r["layer"]
    assert layer.k == w.nb * 128
    h = 4
    s = layer.scores[0, h].cpu().numpy().reshape(-1)
    order = np.argsort(-s, kind="stable")
    want = np.zeros(s.size, dtype=bool)
    want[order[:layer.k]] = True
    rp, ci = _routed(r, h)
    assert np.array_equal(orc.csr_to_mask(rp, ci, w.nb).reshape(-1), want)
    rp, ci = _seeded(r, h)
    mask = orc.csr_to_mask(rp, ci, w.nb)
    cubes = _sample_cubes(rp)
    o, _ = orc.fine_forward(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), gu.f64(r["v"][0, h]), mask, rows=cubes)
    toks = orc._tokens_of(cubes)
    gu.assert_close_bf16(gu.f64(layer.o_f[0, h])[toks], o[toks], f"O_f top128 head {h}")


# ----------------------------------------------------------------------------- padded grid
@pytest.fixture(scope="module")
def train720pad():
    return _run(TRAIN_PAD, TRAIN_PAD.topk, True)


def _border_cubes(w):
    """The corner cube (pads along t, y and x), one cube on each border face
    (pads along one axis), and an interior cube."""
    nt, ny, nx = (n // 4 for n in w.pgrid)
    cube = lambda a, b, c: (a * ny + b) * nx + c
    return [cube(nt - 1, ny - 1, nx - 1), cube(nt - 1, ny // 2, nx // 3), cube(nt // 2, ny - 1, nx // 2),
            cube(1, 2, nx - 1), cube(nt // 3, ny // 3, nx // 3)]


def test_padded_router_and_selection(train720pad):
    r = train720pad
    w, layer = r["w"], r["layer"]
    scores = layer.scores[0]
    nq = orc.pool_exists(w.grid, (2, 2, 2)).reshape(-1, 8).sum(axis=1)
    np.testing.assert_allclose(scores.double().sum(dim=2).cpu().numpy(), np.broadcast_to(nq / 64.0, scores.shape[:2]),
                               rtol=1e-4)
    rows = np.array(_border_cubes(w))
    for h in (0, 11):
        want = orc.router_scores(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), w.grid, bf16_pooled=True, rows=rows)
        got = scores[h].double().cpu().numpy()[rows]
        for n in range(len(rows)):
            assert gu.rel_l2(got[n], want[n]) <= 1e-4, f"head {h} row {rows[n]}"
    h = 6
    s = scores[h].cpu().numpy().reshape(-1)
    order = np.argsort(-s, kind="stable")
    want = np.zeros(s.size, dtype=bool)
    want[order[:layer.k]] = True
    rp, ci = _routed(r, h)
    assert np.array_equal(orc.csr_to_mask(rp, ci, w.nb).reshape(-1), want)


def test_padded_outputs_sampled(train720pad):
    r = train720pad
    w, layer = r["w"], r["layer"]
    real = orc.token_valid(w.grid)
    pad = torch.from_numpy(~real).to(_dev())
    g = layer.grads()
    # every pad row of every output, all heads
    assert torch.all(layer.o_f[:, :, pad] == 0) and torch.all(layer.o[:, :, pad] == 0)
    assert torch.all(torch.isneginf(layer.lse[:, :, pad]))
    for name in ("dq", "dk", "dv"):
        assert torch.all(g[name][:, :, pad] == 0), name
    assert torch.all(g["dx"][:, pad] == 0)
    oc_hat, _, gate_saved = layer.saved_views()
    assert torch.all(gate_saved[:, :, pad] == 0)
    # real rows of border cubes against the oracle
    h = 9
    rp, ci = _seeded(r, h)
    mask = orc.csr_to_mask(rp, ci, w.nb)
    cubes = [c for c in _border_cubes(w) if mask[c].any()]
    q, k, v, d_o = (gu.f64(t[0, h]) for t in (r["q"], r["k"], r["v"], r["d_o"]))
    o_f, lse = orc.fine_forward(q, k, v, mask, rows=cubes, valid=real)
    toks = orc._tokens_of(cubes)
    gu.assert_close_bf16(gu.f64(layer.o_f[0, h])[toks], o_f[toks], f"O_f head {h} cubes {cubes}")
    live = np.isfinite(lse[toks])
    np.testing.assert_allclose(gu.f64(layer.lse[0, h])[toks][live], lse[toks][live], atol=1e-3)
    want_oc, _, _ = orc.coarse_forward(q, k, v, w.grid)
    gu.assert_close_bf16(gu.f64(oc_hat[0, h]), want_oc, f"O_hat_c head {h}")
    gate = orc.gate(gu.f64(r["x"][0][torch.from_numpy(toks).to(_dev())]), gu.f64(r["w_g"]), real[toks])[:, h]
    want_o = gate[:, None] * want_oc[toks // 64] + o_f[toks]
    gu.assert_close_bf16(gu.f64(layer.o[0, h])[toks], want_o, f"O head {h}", rounding=2.0 ** -8)
    # dQ of the border query cubes, dK / dV of a border KV cube (fine branch)
    sub = np.zeros_like(mask)
    sub[cubes] = mask[cubes]
    dq, _, _ = orc.fine_backward(q, k, v, sub, d_o, valid=real)
    rr = gu.rel_l2(gu.f64(g["dq"][0, h])[toks], dq[toks])
    assert rr <= 2e-2, f"dQ head {h}: rel-L2 {rr:.3g}"
    j = _border_cubes(w)[0]
    rows = np.nonzero(mask[:, j])[0]
    if len(rows):
        sub = np.zeros_like(mask)
        sub[rows] = mask[rows]
        _, dk, dv = orc.fine_backward(q, k, v, sub, d_o, valid=real)
        tj = np.arange(64 * j, 64 * j + 64)
        for name, got, want in (("dK", g["dk"], dk), ("dV", g["dv"], dv)):
            rr = gu.rel_l2(gu.f64(got[0, h])[tj], want[tj])
            assert rr <= 2e-2, f"{name} head {h} corner KV cube {j}: rel-L2 {rr:.3g}"


# ----------------------------------------------------------------------------- 128-token blocks
@pytest.fixture(scope="module")
def train720b128():
    return _run(TRAIN_B128, TRAIN_B128.topk, True)


def test_block128_router_and_selection(train720b128):
    r = train720b128
    w, layer = r["w"], r["layer"]
    scores = layer.scores[0]
    assert scores.shape == (w.heads, w.nblk, w.nblk)
    np.testing.assert_allclose(scores.double().sum(dim=2).cpu().numpy(), 1.0 / 16.0, rtol=1e-4)   # G = 16
    rows = np.array([0, w.nblk // 3, w.nblk - 1])
    for h in (2, 17):
        want = orc.router_scores(gu.f64(r["q"][0, h]), gu.f64(r["k"][0, h]), w.grid, bf16_pooled=True, rows=rows,
                                 block=128)
        got = scores[h].double().cpu().numpy()[rows]
        for n in range(len(rows)):
            assert gu.rel_l2(got[n], want[n]) <= 1e-4, f"head {h} row {rows[n]}"
    h = 8
    s = scores[h].cpu().numpy().reshape(-1)
    order = np.argsort(-s, kind="stable")
    want = np.zeros(s.size, dtype=bool)
    want[order[:layer.k]] = True
    rp, ci = _routed(r, h)
    assert np.array_equal(orc.csr_to_mask(rp, ci, w.nblk).reshape(-1), want)
    gu.check_csr_csc(*[t[0, [h]] for t in r["routed"]], w.nblk, layer.k)


def test_block128_outputs_sampled(train720b128):
    r = train720b128
    w, layer = r["w"], r["layer"]
    g = layer.grads()
    h = 4
    rp, ci = _seeded(r, h)
    mask = orc.csr_to_mask(rp, ci, w.nblk)
    blocks = [b for b in _sample_cubes(rp) if mask[b].any()]
    q, k, v, d_o = (gu.f64(t[0, h]) for t in (r["q"], r["k"], r["v"], r["d_o"]))
    o_f, lse = orc.fine_forward(q, k, v, mask, rows=blocks, block=128)
    toks = orc._tokens_of(blocks, 128)
    gu.assert_close_bf16(gu.f64(layer.o_f[0, h])[toks], o_f[toks], f"O_f head {h} blocks {blocks}")
    np.testing.assert_allclose(gu.f64(layer.lse[0, h])[toks], lse[toks], atol=1e-3)
    oc_hat, _, gate_saved = layer.saved_views()
    want_oc, _, _ = orc.coarse_forward(q, k, v, w.grid, block=128)
    gu.assert_close_bf16(gu.f64(oc_hat[0, h]), want_oc, f"O_hat_c head {h}")
    gate = orc.gate(gu.f64(r["x"][0][torch.from_numpy(toks).to(_dev())]), gu.f64(r["w_g"]))[:, h]
    want_o = gate[:, None] * want_oc[toks // 128] + o_f[toks]
    gu.assert_close_bf16(gu.f64(layer.o[0, h])[toks], want_o, f"O head {h}", rounding=2.0 ** -8)
    sub = np.zeros_like(mask)
    sub[blocks] = mask[blocks]
    dq, _, _ = orc.fine_backward(q, k, v, sub, d_o, block=128)
    rr = gu.rel_l2(gu.f64(g["dq"][0, h])[toks], dq[toks])
    assert rr <= 2e-2, f"dQ head {h}: rel-L2 {rr:.3g}"
    lens = mask.sum(axis=0)
    j = int(np.argmin(np.where(lens > 0, lens, lens.max() + 1)))  # the shortest column keeps the oracle quick
    rows = np.nonzero(mask[:, j])[0]
    sub = np.zeros_like(mask)
    sub[rows] = mask[rows]
    _, dk, dv = orc.fine_backward(q, k, v, sub, d_o, block=128)
    tj = np.arange(128 * j, 128 * j + 128)
    for name, got, want in (("dK", g["dk"], dk), ("dV", g["dv"], dv)):
        rr = gu.rel_l2(gu.f64(got[0, h])[tj], want[tj])
        assert rr <= 2e-2, f"{name} head {h} KV block {j} ({len(rows)} query blocks): rel-L2 {rr:.3g}"


# ----------------------------------------------------------------------------- MMDiT text tokens
def test_text_rows_at_full_size():
    """720p training with 512 text tokens: the fine outputs of sampled video
    cubes (their keys include every text token) and of all text rows (every
    video and text token) against the oracle; O = O_f on text rows; text
    padding is zero."""
    r = _run(TRAIN_TEXT, TRAIN_TEXT.topk, False)
    w, layer = r["w"], r["layer"]
    h = 3
    rp, ci = _seeded(r, h)
    mask = orc.csr_to_mask(rp, ci, w.nb)
    cubes = _sample_cubes(rp, n_extra=1)                  # includes an empty list: text keys only
    q, k, v = (gu.f64(t[0, h]) for t in (r["q"], r["k"], r["v"]))
    o_f, lse = orc.fine_forward(q, k, v, mask, rows=cubes, n_text=w.text)
    toks = np.concatenate([orc._tokens_of(cubes), w.L + np.arange(w.text)])
    gu.assert_close_bf16(gu.f64(layer.o_f[0, h])[toks], o_f[toks], f"O_f head {h} (video cubes {cubes} + text)")
    np.testing.assert_allclose(gu.f64(layer.lse[0, h])[toks], lse[toks], atol=1e-3)
    assert torch.equal(layer.o[:, :, w.L:], layer.o_f[:, :, w.L:]), "text rows: O must be O_f"
    assert torch.all(layer.o_f[:, :, w.L + w.text:] == 0) and torch.all(torch.isneginf(layer.lse[:, :, w.L + w.text:]))


# ----------------------------------------------------------------------------- VSA router baseline
def test_vsa_router_at_full_size():
    """The VSA router baseline at 720p, top128: P_c rows sum to 1 and match the
    oracle on sampled rows; every row keeps exactly the top 128 of the GPU's
    own scores; the fine forward of sampled cubes on that selection."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = TRAIN_VSA
    dev = _dev()
    q, k, v = make_qkv(w, device=dev)
    x, w_g = make_gate_inputs(w, device=dev, zero_gate=False)
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype, block=w.block)
    layer = vsa2.Layer(p, w.topk, w.d_model, device=dev)
    layer.forward(q, k, v, x, w_g, router="vsa")
    torch.cuda.synchronize()
    scores = layer.scores[0]
    np.testing.assert_allclose(scores.double().sum(dim=2).cpu().numpy(), 1.0, rtol=1e-4)
    for h in (1, 16):
        want = orc.coarse_scores(gu.f64(q[0, h]), gu.f64(k[0, h]), w.grid, bf16_pooled=True)
        got = scores[h].double().cpu().numpy()
        for i in (0, w.nb // 2, w.nb - 1):
            assert gu.rel_l2(got[i], want[i]) <= 1e-4, f"head {h} row {i}"
        sel = orc.csr_to_mask(layer.row_ptr[0, h].cpu().numpy(), layer.col_idx[0, h].cpu().numpy(), w.nb)
        assert np.array_equal(sel, orc.topk_per_row(got, w.topk)[0]), f"head {h}: not the per-row top k"
    h = 16
    sel = orc.csr_to_mask(layer.row_ptr[0, h].cpu().numpy(), layer.col_idx[0, h].cpu().numpy(), w.nb)
    cubes = [0, 1717, w.nb - 1]
    o_f, _ = orc.fine_forward(gu.f64(q[0, h]), gu.f64(k[0, h]), gu.f64(v[0, h]), sel, rows=cubes)
    toks = orc._tokens_of(cubes)
    gu.assert_close_bf16(gu.f64(layer.o_f[0, h])[toks], o_f[toks], f"O_f head {h}")
