"""Seeded synthetic video-shaped inputs for the VSA2 hot path.

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle consume exactly the
tensors made here (bf16 workloads are rounded once, round-to-nearest-even, and
both sides read the rounded values).

Token order.  The attention layer takes tokens in cube-tiled order (paper
"Improving Video Sparse Attention with Fine-grained Router and Sparse
Rebasing", §2.2 "Permutation"): cube-major over the (T/4, Y/4, X/4) cube grid,
then the eight 2x2x2 sub-cubes of a cube in raster order, then the eight tokens
of a sub-cube in raster order.  Tensors are generated in raster (t, y, x) order
and permuted with :func:`tile_permutation`.  A grid that is not a whole number
of cubes is padded up to one (§2.2 "Kernel Implementation"); the pad slots of
Q, K and V are filled with seeded finite values of a different distribution
(3 + 4 N(0,1)), and those of dO and X are drawn like their real rows, so that
any pad value reaching an output shows.  MMDiT text tokens (workloads with
``text``) follow the video slots as N(0,1) rows, padded to a multiple of 64
with the same pad fill.

Recipes (one torch generator per (workload, batch, tensor, head)):

* ``sinusoid``: N(0,1) + alpha * sin(2*pi*(ft*t/T + fy*y/Y + fx*x/X) + phi) per
  channel, with f in {0,1,2}^3 and phi ~ U[0, 2*pi); Q and K share one draw of
  (f, phi), V has its own.
* ``lowrank``: N(0,1) + alpha * z with z = sum_{r<8} u_r(t,y,x) w_r; u_r is white
  noise smoothed by a Gaussian (sigma = 2 cells per axis) and rescaled to unit
  variance, w_r ~ N(0, I/8).  Q and K share z, V has its own.
* ``skew``: every query cube's 64 rows of Q are multiplied by
  clip(exp(xi), 1/8, 8), xi ~ N(0,1) (heavy-tailed router rows).
* dO ~ N(0,1); X ~ N(0,1) of shape [B, L, H*d]; W_g = 0 (the zero-initialised
  gate) or N(0, 1/(H*d)).
"""

import math

import torch

from .configs import CUBE, Workload

# tensor ids used in the seeds
T_Q, T_K, T_V, T_DO, T_X, T_WG, T_SQK, T_SV, T_SKEW, T_SEL, T_PAD, T_TEXT = range(12)


def seed_of(w: Workload, tensor: int, head: int = 0, batch: int = 0) -> int:
    return 1_000_000 * w.cfg_id + 100_000 * batch + 1000 * tensor + head


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def tile_permutation(grid, device="cpu", block=64) -> torch.Tensor:
    """perm[j] = raster index (t*Y + y)*X + x of the token stored at tiled slot
    j of the grid padded up to whole blocks (x to a multiple of 8 for
    128-token blocks), or -1 where slot j is padding."""
    T, Y, X = grid
    Tp, Yp, Xp = (-(-n // m) * m for n, m in zip(grid, (4, 4, 4 * (block // 64))))
    L = Tp * Yp * Xp
    j = torch.arange(L, device=device, dtype=torch.int64)
    c, s, u = j // 64, (j // 8) % 8, j % 8
    cx = c % (Xp // 4)
    cy = (c // (Xp // 4)) % (Yp // 4)
    ct = c // ((Xp // 4) * (Yp // 4))
    t = 4 * ct + 2 * (s // 4) + u // 4
    y = 4 * cy + 2 * ((s // 2) % 2) + (u // 2) % 2
    x = 4 * cx + 2 * (s % 2) + u % 2
    real = (t < T) & (y < Y) & (x < X)
    return torch.where(real, (t * Y + y) * X + x, torch.full_like(j, -1))


def _to_tiled(x_raster, perm, fill):
    """Raster-order rows [L_real, d] into tiled slots [L, d]; pad slots take
    the rows of ``fill``."""
    real = perm >= 0
    out = fill.clone()
    out[real] = x_raster[perm[real]]
    return out


def _smooth_noise(grid, nfield, sigma, gen, device):
    T, Y, X = grid
    f = torch.randn((nfield, T, Y, X), generator=gen, device=device, dtype=torch.float32)
    rad = int(math.ceil(3 * sigma))
    ker = torch.exp(-0.5 * (torch.arange(-rad, rad + 1, device=device, dtype=torch.float32) / sigma) ** 2)
    ker = (ker / ker.sum()).view(1, 1, -1)
    for axis in (1, 2, 3):
        f = f.movedim(axis, -1)
        shp = f.shape
        f = torch.nn.functional.conv1d(f.reshape(-1, 1, shp[-1]), ker, padding=rad).reshape(shp)
        f = f.movedim(-1, axis)
    f = f - f.mean(dim=(1, 2, 3), keepdim=True)
    f = f / f.std(dim=(1, 2, 3), keepdim=True).clamp_min(1e-12)
    return f.reshape(nfield, -1)  # [nfield, L] raster order


def _structure(w: Workload, tensor: int, head: int, batch: int, device) -> torch.Tensor:
    """Structured component [L, d] in raster order."""
    T, Y, X = w.grid
    d = w.head_dim
    g = _gen(seed_of(w, tensor, head, batch), device)
    if w.gen == "sinusoid":
        f = torch.randint(0, 3, (3, d), generator=g, device=device).to(torch.float32)
        phi = torch.rand((d,), generator=g, device=device) * (2 * math.pi)
        t = torch.arange(T, device=device, dtype=torch.float32).view(T, 1, 1, 1) / T
        y = torch.arange(Y, device=device, dtype=torch.float32).view(1, Y, 1, 1) / Y
        x = torch.arange(X, device=device, dtype=torch.float32).view(1, 1, X, 1) / X
        arg = 2 * math.pi * (f[0] * t + f[1] * y + f[2] * x) + phi
        return torch.sin(arg).reshape(-1, d)
    if w.gen == "lowrank":
        u = _smooth_noise(w.grid, 8, 2.0, g, device)                      # [8, L]
        wr = torch.randn((8, d), generator=g, device=device) / math.sqrt(8.0)
        return u.t().contiguous() @ wr                                   # [L, d]
    raise ValueError(w.gen)


def _storage(t: torch.Tensor, w: Workload) -> torch.Tensor:
    return t.to(torch.bfloat16) if w.dtype == "bf16" else t.to(torch.float32)


def make_qkv(w: Workload, device="cpu", heads=None):
    """Q, K, V as [B, H, rows, d] in storage dtype: the video slots in cube-tiled
    token order, then any MMDiT text rows.

    ``heads`` selects a subset of heads (regenerated exactly as in the full
    tensor); the result then has that many heads.
    """
    heads = list(range(w.heads)) if heads is None else list(heads)
    L, d = w.L, w.head_dim
    perm = tile_permutation(w.grid, device, w.block)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {n: torch.empty((w.batch, len(heads), w.rows, d), dtype=dt, device=device) for n in "qkv"}
    for b in range(w.batch):
        for hi, h in enumerate(heads):
            s_qk = _structure(w, T_SQK, h, b, device)
            s_v = _structure(w, T_SV, h, b, device)
            for ti, (name, tid, s) in enumerate((("q", T_Q, s_qk), ("k", T_K, s_qk), ("v", T_V, s_v))):
                g = _gen(seed_of(w, tid, h, b), device)
                x = torch.randn((w.L_real, d), generator=g, device=device) + w.alpha * s
                if w.padded:
                    # pad slots hold finite garbage (offset, 4x the spread) that
                    # must not reach any output
                    gp = _gen(seed_of(w, T_PAD, 3 * h + ti, b), device)
                    fill = 3.0 + 4.0 * torch.randn((L, d), generator=gp, device=device)
                    x = _to_tiled(x, perm, fill)
                else:
                    x = x[perm]
                if name == "q" and w.skew:
                    gs = _gen(seed_of(w, T_SKEW, h, b), device)
                    xi = torch.randn((w.nb,), generator=gs, device=device)
                    sc = torch.exp(xi).clamp(1.0 / 8.0, 8.0)
                    x = (x.view(w.nb, CUBE, d) * sc.view(w.nb, 1, 1)).view(L, d)
                out[name][b, hi, :L] = _storage(x, w)
                if w.text:
                    # MMDiT text rows: N(0,1) tokens, then padding filled like
                    # the video pad slots
                    gt = _gen(seed_of(w, T_TEXT, 3 * h + ti, b), device)
                    t = torch.randn((w.text, d), generator=gt, device=device)
                    fill = 3.0 + 4.0 * torch.randn((w.rows - L - w.text, d), generator=gt, device=device)
                    out[name][b, hi, L:] = _storage(torch.cat([t, fill]), w)
    return out["q"], out["k"], out["v"]


def make_grad_out(w: Workload, device="cpu", heads=None):
    heads = list(range(w.heads)) if heads is None else list(heads)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = torch.empty((w.batch, len(heads), w.rows, w.head_dim), dtype=dt, device=device)
    for b in range(w.batch):
        for hi, h in enumerate(heads):
            g = _gen(seed_of(w, T_DO, h, b), device)
            out[b, hi] = _storage(torch.randn((w.rows, w.head_dim), generator=g, device=device), w)
    return out


def make_gate_inputs(w: Workload, device="cpu", zero_gate=True, d_model=None):
    """X [B, L, Dm] (storage dtype, tiled order) and W_g [Dm, H] fp32."""
    dm = w.d_model if d_model is None else d_model
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = torch.empty((w.batch, w.L, dm), dtype=dt, device=device)
    for b in range(w.batch):
        g = _gen(seed_of(w, T_X, 0, b), device)
        x[b] = _storage(torch.randn((w.L, dm), generator=g, device=device), w)
    if zero_gate:
        wg = torch.zeros((dm, w.heads), dtype=torch.float32, device=device)
    else:
        g = _gen(seed_of(w, T_WG), device)
        wg = torch.randn((dm, w.heads), generator=g, device=device) / math.sqrt(dm)
    return x, wg


def make_selection(w: Workload, topk=None, device="cpu", seed_offset=0):
    """A seeded block selection with exactly nb*topk pairs per head, as CSR.

    Row counts are heavy-tailed (some rows empty, some long) and the columns of
    a row are a random subset.  Used to drive the sparse attention with a fixed,
    externally chosen mask.  Returns (row_ptr [B,H,nb+1], col_idx [B,H,k]) int32.
    """
    nb = w.nblk
    k = w.budget(topk)
    bh = w.batch * w.heads
    row_ptr = torch.empty((bh, nb + 1), dtype=torch.int32)
    col_idx = torch.empty((bh, k), dtype=torch.int32)
    for i in range(bh):
        g = _gen(seed_of(w, T_SEL, i) + seed_offset, "cpu")
        wgt = torch.exp(1.5 * torch.randn((nb,), generator=g, dtype=torch.float64))
        wgt[torch.rand((nb,), generator=g) < 0.03] = 0.0          # a few empty rows
        cnt = torch.floor(wgt / wgt.sum() * k).to(torch.int64).clamp(max=nb)
        rem = k - int(cnt.sum())
        order = torch.argsort(torch.rand((nb,), generator=g))
        p = 0
        while rem > 0:                                             # hand out the remainder
            r = int(order[p % nb]); p += 1
            if cnt[r] < nb and (wgt[r] > 0 or p > nb):
                cnt[r] += 1; rem -= 1
        keys = torch.rand((nb, nb), generator=g)
        cols = torch.argsort(keys, dim=1)
        rp = torch.zeros(nb + 1, dtype=torch.int64)
        rp[1:] = torch.cumsum(cnt, 0)
        row_ptr[i] = rp.to(torch.int32)
        parts = [torch.sort(cols[r, : int(cnt[r])]).values for r in range(nb)]
        col_idx[i] = torch.cat(parts).to(torch.int32)
    shape = (w.batch, w.heads)
    return row_ptr.view(*shape, nb + 1).to(device), col_idx.view(*shape, k).to(device)
