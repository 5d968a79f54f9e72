"""GPU parity with 128-token attention blocks (4x4x8: two x-adjacent cubes).

B = 128, R = 8, G = 16 is the blog's inferred setting for the paper's runs
("Improving Video Sparse Attention with Fine-grained Router and Sparse
Rebasing" deep-read, §07); the paper gives no 3D cut, and the cube-tiled
order keeps a pair of x-adjacent cubes contiguous.  The router scores, the
selection and the coarse tokens are per block; the fine kernels tile cubes
and take each selected block as its two cubes.  Grids include padded ones,
one with a cube that holds no token.  Tolerances as in test_gpu_parity.
"""

import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import vsa2_oracle as orc
from video_dit_trainable_amd import vsa2
from video_dit_trainable_amd.configs import Workload
from video_dit_trainable_amd.inputs import make_gate_inputs, make_grad_out, make_qkv

pytestmark = pytest.mark.gpu

B128_F32 = Workload("b128-f32", 31, (8, 8, 16), 1, 2, 64, "f32", 3, "sinusoid", alpha=1.0, train=True,
                    block=128)                                                           # 8 blocks
B128_BF16 = Workload("b128-bf16", 32, (8, 16, 32), 1, 3, 128, "bf16", 4, "lowrank", skew=True, train=True,
                     block=128)                                                          # 32 blocks
B128_PAD = Workload("b128-pad", 33, (5, 6, 9), 1, 2, 64, "bf16", 3, "lowrank", train=True,
                    block=128)                                                           # 8 blocks, an all-pad cube
B128_PAD32 = Workload("b128-pad32", 34, (7, 10, 21), 1, 2, 128, "f32", 5, "lowrank", skew=True, train=True,
                      block=128)                                                         # 18 blocks
CASES = [B128_F32, B128_BF16, B128_PAD, B128_PAD32]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vsa2.lib()


def _dev():
    return torch.device("cuda:0")


def _setup(w, zero_gate=False):
    q, k, v = make_qkv(w)
    x, w_g = make_gate_inputs(w, zero_gate=zero_gate)
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype, block=w.block)
    layer = vsa2.Layer(p, w.topk, w.d_model, device=_dev())
    assert layer.L == w.L and layer.nb == w.nblk
    dev = [t.to(_dev()) for t in (q, k, v, x, w_g)]
    return (q, k, v, x, w_g), dev, layer


def _masks(w, q, k):
    bf = w.dtype == "bf16"
    scores = np.stack([orc.router_scores(gu.f64(q[0, h]), gu.f64(k[0, h]), w.grid, bf16_pooled=bf, block=w.block)
                       for h in range(w.heads)])
    return scores, np.stack([orc.topk_per_sequence(s, w.topk)[0] for s in scores])


def _close(w, got, want, what):
    if w.dtype == "f32":
        gu.assert_close_f32(got, want, what)
    else:
        gu.assert_close_bf16(got, want, what)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_pool_block128(w):
    (q, k, v, x, w_g), (qd, kd, vd, xd, wd), layer = _setup(w)
    vsa2.vsa2_pool(layer.p, qd, kd, vd, layer.pooled)
    torch.cuda.synchronize()
    qr, kr, qc, kc, vc = layer.pooled_views()
    rnd = orc.round_bf16 if w.dtype == "bf16" else (lambda a: a)
    rtol = 8e-3 if w.dtype == "bf16" else 1e-6
    for h in range(w.heads):
        for src, gr, gc in ((q, qr, qc), (k, kr, kc), (v, None, vc)):
            a = gu.f64(src[0, h])
            if gr is not None:
                np.testing.assert_allclose(gu.f64(gr[0, h]), rnd(orc.mean_pool(a, w.grid, (2, 2, 2), w.block)),
                                           rtol=rtol, atol=1e-6)
            got = gu.f64(gc[0, h])
            np.testing.assert_allclose(got[: w.nblk], rnd(orc.block_mean(a, w.grid, w.block)), rtol=rtol, atol=1e-6)
            assert np.all(got[w.nblk:] == 0)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_router_and_topk_block128(w):
    (q, k, v, x, w_g), (qd, kd, vd, xd, wd), layer = _setup(w)
    vsa2.vsa2_pool(layer.p, qd, kd, vd, layer.pooled)
    vsa2.vsa2_route(layer.p, layer.pooled, layer.scores, layer.ws)
    vsa2.vsa2_topk_per_seq(layer.p, layer.scores, w.topk, layer.row_ptr, layer.col_idx, layer.col_ptr,
                           layer.row_idx, layer.ws)
    torch.cuda.synchronize()
    got = gu.f64(layer.scores[0])
    assert got.shape == (w.heads, w.nblk, w.nblk)
    # a query block's row sums to (its 2x2x2 windows holding a real token) / 256
    nq = orc.pool_exists(w.grid, (2, 2, 2), w.block).reshape(-1, 16).sum(axis=1)
    np.testing.assert_allclose(got.sum(axis=2), np.broadcast_to(nq / 256.0, got.shape[:2]), rtol=2e-5)
    scores, _ = _masks(w, q, k)
    for h in range(w.heads):
        np.testing.assert_allclose(got[h], scores[h], rtol=1e-4, atol=1e-4 * scores[h].mean())
    gu.check_csr_csc(layer.row_ptr[0], layer.col_idx[0], layer.col_ptr[0], layer.row_idx[0], w.nblk, layer.k)
    sel = gu.masks_from_csr(layer.row_ptr[0], layer.col_idx[0], w.nblk)
    for h in range(w.heads):
        outside, band, inside = gu.band_compare(sel[h], scores[h], layer.k)
        assert outside == 0, f"head {h}: {outside} selection mismatches outside the band ({band} contested)"


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_fine_forward_block128(w):
    (q, k, v, x, w_g), (qd, kd, vd, xd, wd), layer = _setup(w)
    _, masks = _masks(w, q, k)
    masks[0] = gu.empty_rows(masks[0], [1])                  # an empty query block, budget kept exact
    layer.set_selection(*gu.csr_tensors(masks, _dev()))
    vsa2.vsa2_sparse_attn_fwd(layer.p, w.topk, qd, kd, vd, layer.row_ptr, layer.col_idx, layer.o_f, layer.lse, layer.ws)
    torch.cuda.synchronize()
    real = orc.token_valid(w.grid, w.block)
    for h in range(w.heads):
        o, lse = orc.fine_forward(gu.f64(q[0, h]), gu.f64(k[0, h]), gu.f64(v[0, h]), masks[h], valid=real,
                                  block=w.block)
        got_o, got_lse = gu.f64(layer.o_f[0, h]), gu.f64(layer.lse[0, h])
        _close(w, got_o, o, f"O_f head {h}")
        assert np.all(got_o[~real] == 0) and np.all(np.isneginf(got_lse[~real]))
        live = np.isfinite(lse)
        assert np.array_equal(np.isfinite(got_lse), live)
        np.testing.assert_allclose(got_lse[live], lse[live], atol=1e-4 if w.dtype == "f32" else 1e-3)


@pytest.mark.parametrize("zero_gate", [True, False])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_coarse_gate_block128(w, zero_gate):
    (q, k, v, x, w_g), (qd, kd, vd, xd, wd), layer = _setup(w, zero_gate=zero_gate)
    _, masks = _masks(w, q, k)
    layer.set_selection(*gu.csr_tensors(masks, _dev()))
    o = layer.forward(qd, kd, vd, xd, wd, route=False)
    torch.cuda.synchronize()
    real = orc.token_valid(w.grid, w.block)
    oc_hat, lse_c, g = layer.saved_views()
    gate = orc.gate(gu.f64(x[0]), gu.f64(w_g), real)
    for h in range(w.heads):
        want_oc, want_lse, (qc, kc, _) = orc.coarse_forward(gu.f64(q[0, h]), gu.f64(k[0, h]), gu.f64(v[0, h]),
                                                              w.grid, block=w.block)
        _close(w, gu.f64(oc_hat[0, h]), want_oc, f"O_hat_c head {h}")
        bound = 1e-4 if w.dtype == "f32" else gu.coarse_lse_bound(qc, kc, w.head_dim ** -0.5)
        assert np.all(np.abs(gu.f64(lse_c[0, h]) - want_lse) <= bound), f"lse_c head {h}"
        np.testing.assert_allclose(gu.f64(g[0, h]), gate[:, h], atol=1e-5 if w.dtype == "f32" else 1e-4)
        got_o = gu.f64(o[0, h])
        _close(w, got_o, orc.merge(gate[:, h], want_oc, gu.f64(layer.o_f[0, h]), w.block), f"O head {h}")
        assert np.all(got_o[~real] == 0)
    if zero_gate:
        assert torch.equal(o, layer.o_f), "W_g = 0 must give O = O_f exactly"


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_block128(w):
    (q, k, v, x, w_g), (qd, kd, vd, xd, wd), layer = _setup(w)
    d_o = make_grad_out(w)
    _, masks = _masks(w, q, k)
    layer.set_selection(*gu.csr_tensors(masks, _dev()))
    layer.forward(qd, kd, vd, xd, wd, route=False)
    grads = layer.backward(qd, kd, vd, xd, wd, d_o.to(_dev()))
    torch.cuda.synchronize()
    real = orc.token_valid(w.grid, w.block)
    a = [gu.f64(t[0]) for t in (q, k, v)]
    dq, dk, dv, dx, dw = orc.vsa2_backward(*a, w.grid, masks, gu.f64(x[0]), gu.f64(w_g), gu.f64(d_o[0]),
                                           block=w.block)
    cq, ck, cv = orc.coarse_gate_backward(*a, w.grid, gu.f64(x[0]), gu.f64(w_g), gu.f64(d_o[0]), block=w.block)[:3]
    tol = 1e-4 if w.dtype == "f32" else 2e-2
    for name, want in (("dq", dq), ("dk", dk), ("dv", dv), ("dx", dx), ("dw_g", dw)):
        got = gu.f64(grads[name][0] if name != "dw_g" else grads[name])
        r = gu.rel_l2(got, want.reshape(got.shape))
        assert r <= tol, f"{name}: rel-L2 {r:.3g} > {tol}"
        if name in ("dq", "dk", "dv"):
            assert np.all(got[:, ~real] == 0), f"{name}: nonzero pad rows"
    for i, want in enumerate((cq, ck, cv)):
        r = gu.rel_l2(gu.f64(grads["dqkv_c"][i, 0]), want)
        assert r <= tol, f"dqkv_c[{i}]: rel-L2 {r:.3g}"


def test_block128_pad_values_never_reach_an_output():
    w = B128_PAD
    (q, k, v, x, w_g), (qd, kd, vd, xd, wd), layer = _setup(w, zero_gate=False)
    d_o = make_grad_out(w).to(_dev())
    real = torch.tensor(orc.token_valid(w.grid, w.block), device=_dev())
    gen = torch.Generator(device="cpu").manual_seed(77)
    outs = []
    for trial in range(2):
        if trial:
            for t in (qd, kd, vd, d_o):
                noise = (50.0 * torch.randn(t.shape, generator=gen)).to(t.dtype).to(_dev())
                t[:, :, ~real] = noise[:, :, ~real]
            xd[:, ~real] = (-30.0 * torch.rand(xd[:, ~real].shape, generator=gen)).to(xd.dtype).to(_dev())
        o = layer.forward(qd, kd, vd, xd, wd)
        g = layer.backward(qd, kd, vd, xd, wd, d_o)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (layer.scores, layer.col_idx, layer.o_f, layer.lse, o, g["dq"], g["dk"],
                                         g["dv"], g["dx"], g["dw_g"], g["dqkv_c"])])
    for n, (a, b) in enumerate(zip(*outs)):
        assert torch.equal(a, b), f"output {n} depends on pad values"
