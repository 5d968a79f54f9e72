"""CPU oracle for the VSA2 attention layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The HIP library never calls it and shares no code with it.

Everything is plain numpy in float64, one (batch, head) at a time, written
from the equations of "Improving Video Sparse Attention with Fine-grained
Router and Sparse Rebasing" (arXiv 2609.32882, §2.1-§2.2, App. B).  Where the
paper leaves a step open, the plain reading is taken and noted at the function.

Conventions shared with the library interface:
  * tokens of one head are in cube-tiled order (§2.2 "Permutation"): the 64
    tokens of a 4x4x4 cube are contiguous, cube-major over the cube grid;
    inside a cube, the eight 2x2x2 sub-cubes in raster order, each holding its
    8 tokens in raster order.  The oracle does not rely on the inner order: it
    rebuilds every token's (t, y, x) from the grid and pools by coordinates.
  * block size B = 64 (one 4x4x4 cube), router pool R = 8 (2x2x2), G = B/R =
    8.  B = 128 is the blog's inferred setting for the paper's own runs (its
    §07; the paper gives no 3D cut): here a 128-token block is two
    x-adjacent cubes, 4x4x8, which the cube-tiled order keeps contiguous
    (cubes 2m and 2m+1), so G = 16 and the grid's x side is padded to a
    multiple of 8.  Blocks are numbered like the cube pairs.
  * softmax scale 1/sqrt(d) unless given.
  * MMDiT text conditioning ([VSA2] §2.2 after Eq.(12): the fine branch
    extends to full video-to-text and text-to-video attention; the blog's
    §06 keeps both dense): n_text text tokens follow the video slots in Q, K,
    V, padded to the tensors' length.  Reading: the joint attention is
    block-sparse only between video blocks; video-text, text-video and
    text-text attention are dense (MMDiT joint attention), one softmax per
    query row.  The router, the coarse branch and the gate see the video
    alone; a text row's O is its O_f.
  * a latent grid whose sides are not multiples of 4 is padded up to the next
    multiple along each axis (§2.2 "Kernel Implementation"); tensors hold the
    padded grid in the order above, and the pad positions are not tokens.
    Readings taken here, where the paper only says that attention to padding
    is masked: a pooling window averages the real tokens it holds, and a
    window holding none does not exist (it is no router key and gives no
    router row; every 4x4x4 cube holds at least one real token); the G x G
    mean of Eq.(7) keeps its denominator, with missing entries counted as
    zero; pad positions are masked as keys, and as queries or gate rows they
    give O_f = 0, LSE = -inf, g = 0, O = 0 and zero gradients; the coarse
    branch's gradient goes back to the n real tokens of a cube as 1/n each.

Parity pins: every function here is checked in tests/test_oracle.py against
closed forms, special cases that reduce to textbook routines (dense softmax
attention, autograd), brute force on tiny inputs and finite differences.
"""

import numpy as np

CUBE_SHAPE = (4, 4, 4)
SUB_SHAPE = (2, 2, 2)


# ----------------------------------------------------------------------------
# layout
# ----------------------------------------------------------------------------
def _check_block(block):
    if block not in (64, 128):
        raise ValueError(f"block size {block} is not 64 or 128")
    return block // 64


def padded_grid(grid, block=64):
    """Each side rounded up to a multiple of the cube side 4 (x to a multiple
    of 8 for 128-token blocks)."""
    mult = (4, 4, 4 * _check_block(block))
    return tuple(-(-int(n) // m) * m for n, m in zip(grid, mult))


def token_coords(grid, block=64):
    """(t, y, x) of every token slot in cube-tiled order, shape [L, 3], L the
    token count of the padded grid.

    Cube-major order over the (T/4, Y/4, X/4) cube grid (§2.2 "Permutation");
    inside a cube the reading taken here is sub-cube-major: slot 64c + 8s + u
    holds sub-cube s (raster over the 2x2x2 sub-cube grid of the cube) and
    position u (raster inside the 2x2x2 sub-cube).  Slots whose coordinates
    reach past ``grid`` are padding.
    """
    T, Y, X = padded_grid(grid, block)
    ct, cy, cx = T // 4, Y // 4, X // 4
    coords = np.empty((T * Y * X, 3), dtype=np.int64)
    slot = 0
    for a in range(ct):
        for b in range(cy):
            for c in range(cx):
                for st in range(2):
                    for sy in range(2):
                        for sx in range(2):
                            for ut in range(2):
                                for uy in range(2):
                                    for ux in range(2):
                                        coords[slot] = (4 * a + 2 * st + ut, 4 * b + 2 * sy + uy, 4 * c + 2 * sx + ux)
                                        slot += 1
    return coords


def token_valid(grid, block=64):
    """True for the slots that hold a token of ``grid`` (not padding), [L]."""
    return np.all(token_coords(grid, block) < np.asarray(grid, dtype=np.int64), axis=1)


def pool_groups(grid, pool, block=64):
    """Token slots of each pooling window, ordered cube-major then window raster
    inside the cube.  Returns int array [L / prod(pool), prod(pool)].

    The windows tile every 4x4x4 cube (pool in {1,2,4}^3), so a pooled token
    index a belongs to cube a // (64 / prod(pool)).
    """
    T, Y, X = padded_grid(grid, block)
    pt, py, px = pool
    coords = token_coords(grid, block)
    slot_of = np.empty((T, Y, X), dtype=np.int64)
    slot_of[coords[:, 0], coords[:, 1], coords[:, 2]] = np.arange(T * Y * X)
    groups = []
    for a in range(T // 4):
        for b in range(Y // 4):
            for c in range(X // 4):
                for wt in range(4 // pt):
                    for wy in range(4 // py):
                        for wx in range(4 // px):
                            t0, y0, x0 = 4 * a + wt * pt, 4 * b + wy * py, 4 * c + wx * px
                            members = slot_of[t0:t0 + pt, y0:y0 + py, x0:x0 + px].reshape(-1)
                            groups.append(members)
    return np.asarray(groups, dtype=np.int64)


def mean_pool(x, grid, pool, block=64):
    """MeanPool over windows of shape ``pool`` (Eq.(1) with the cube, Eq.(5)
    with the router window).  x: [L, d] -> [L / prod(pool), d].  A window
    averages the real tokens it holds; one holding none gives a zero row."""
    grp = pool_groups(grid, pool, block)
    ok = token_valid(grid, block)[grp]                        # [windows, members]
    cnt = ok.sum(axis=1)
    tot = np.where(ok[..., None], np.asarray(x)[grp], 0.0).sum(axis=1)
    return np.where(cnt[:, None] > 0, tot / np.maximum(cnt, 1)[:, None], 0.0)


def pool_exists(grid, pool, block=64):
    """True for the pooling windows that hold at least one real token."""
    return token_valid(grid, block)[pool_groups(grid, pool, block)].any(axis=1)


def block_mean(x, grid, block=64):
    """Eq.(1): the mean of the real tokens of every attention block (a 4x4x4
    cube, or a 4x4x8 pair of cubes).  Cube means come from the coordinates;
    a pair's mean weights its two cubes by their real-token counts."""
    cm = mean_pool(np.asarray(x, np.float64), grid, CUBE_SHAPE, block)
    if block == 64:
        return cm
    n = token_valid(grid, block).reshape(-1, 64).sum(axis=1).astype(np.float64)
    tot = (cm * n[:, None]).reshape(-1, 2, cm.shape[1]).sum(axis=1)
    return tot / n.reshape(-1, 2).sum(axis=1)[:, None]


def round_bf16(x):
    """Round to the nearest bfloat16 (ties to even), returned as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _softmax_rows(s):
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def _scale(d, scale):
    return 1.0 / np.sqrt(d) if not scale else float(scale)


# ----------------------------------------------------------------------------
# router: pool - softmax - pool, Eq.(5)-(7)
# ----------------------------------------------------------------------------
def router_scores(q, k, grid, pool=SUB_SHAPE, scale=None, bf16_pooled=False, rows=None, block=64):
    """Block scores P_r [nb, nb] of one head (Eq.(5)-(7)), nb attention blocks.

    Eq.(5): Q_r, K_r = MeanPool_R(Q, K).  With ``bf16_pooled`` the pooled
    operands are rounded to bf16 before the product (the precision the bf16
    kernels work in; the paper does not state one).
    Eq.(6): P_hat = softmax over all pooled keys of Q_r K_r^T / sqrt(d).
    Eq.(7): P_r[i, j] = mean of the G x G entries of P_hat between block i and
    block j (the paper's MeanPool_{GxG}; the sum would be G^2 times this).
    ``rows`` restricts the output to some query blocks (rows are independent).
    On a padded grid a window with no real token is no key (-inf logit) and
    its query row is left out (zero entries in the mean).
    """
    d = q.shape[1]
    qr = mean_pool(np.asarray(q, np.float64), grid, pool, block)
    kr = mean_pool(np.asarray(k, np.float64), grid, pool, block)
    if bf16_pooled:
        qr, kr = round_bf16(qr), round_bf16(kr)
    ex = pool_exists(grid, pool, block)
    g = block // (pool[0] * pool[1] * pool[2])
    nb = qr.shape[0] // g
    rows = np.arange(nb) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), nb))
    for n, i in enumerate(rows):
        s = qr[i * g:(i + 1) * g] @ kr.T * _scale(d, scale)       # [G, L/R]
        s[:, ~ex] = -np.inf
        p_hat = _softmax_rows(s)
        p_hat[~ex[i * g:(i + 1) * g]] = 0.0
        out[n] = p_hat.reshape(g, nb, g).mean(axis=(0, 2))
    return out


def oracle_block_scores(q, k, grid, scale=None, block=64):
    """P_oracle (Eq.(10)-(11)): token-level softmax, then the mean over each
    (B x B) tile.  Output rows are blocks in block order.  Pad keys are
    masked and pad query rows left out (zero entries in the mean)."""
    d = q.shape[1]
    ok = token_valid(grid, block)
    s = np.asarray(q, np.float64) @ np.asarray(k, np.float64).T * _scale(d, scale)
    s[:, ~ok] = -np.inf
    p = _softmax_rows(s)
    p[~ok] = 0.0
    nb = q.shape[0] // block
    return p.reshape(nb, block, nb, block).mean(axis=(1, 3))


# ----------------------------------------------------------------------------
# per-sequence TopK, Eq.(8)-(9)
# ----------------------------------------------------------------------------
def topk_per_sequence(scores, topk):
    """Keep the nb*topk largest entries of the flattened nb x nb block scores of
    one head (Eq.(8)-(9); the budget is capped at nb^2).  Ties are broken
    toward the lower flat index i*nb + j (the paper leaves ties open).

    Returns (mask [nb, nb] bool, row_ptr [nb+1], col_idx [k], col_ptr [nb+1],
    row_idx [k]) with columns ascending in each row and rows ascending in each
    column.
    """
    scores = np.asarray(scores, np.float64)
    nb = scores.shape[0]
    k = min(nb * topk, nb * nb)
    flat = scores.reshape(-1)
    order = np.lexsort((np.arange(nb * nb), -flat))     # score desc, then index asc
    mask = np.zeros(nb * nb, dtype=bool)
    mask[order[:k]] = True
    mask = mask.reshape(nb, nb)
    return (mask,) + mask_to_csr_csc(mask)


def topk_per_row(scores, topk):
    """The VSA router's selection ([VSA2] §1, Figure 1 left; [blog] §04): every
    query block keeps its own min(topk, nb) largest scores.  Ties go to the
    lower column index.  Returns (mask, row_ptr, col_idx, col_ptr, row_idx)
    as topk_per_sequence does."""
    scores = np.asarray(scores, np.float64)
    nb = scores.shape[0]
    kr = min(topk, nb)
    mask = np.zeros((nb, nb), dtype=bool)
    for i in range(nb):
        order = np.lexsort((np.arange(nb), -scores[i]))     # score desc, then column asc
        mask[i, order[:kr]] = True
    return (mask,) + mask_to_csr_csc(mask)


def coarse_scores(q, k, grid, scale=None, bf16_pooled=False, block=64):
    """The VSA router's block scores: P_c = softmax(Q_c K_c^T / sqrt(d)) over
    the block means (Eq.(1)-(2)), the coarse branch's own attention map.
    With ``bf16_pooled`` the block means are rounded to bf16 first."""
    d = q.shape[1]
    qc, kc = block_mean(q, grid, block), block_mean(k, grid, block)
    if bf16_pooled:
        qc, kc = round_bf16(qc), round_bf16(kc)
    return _softmax_rows(qc @ kc.T * _scale(d, scale))


def mask_to_csr_csc(mask):
    nb = mask.shape[0]
    rows, cols = np.nonzero(mask)                        # row-major: cols ascending per row
    row_ptr = np.zeros(nb + 1, dtype=np.int64)
    np.add.at(row_ptr, rows + 1, 1)
    row_ptr = np.cumsum(row_ptr)
    cols_t, rows_t = np.nonzero(mask.T)                  # column-major: rows ascending per column
    col_ptr = np.zeros(nb + 1, dtype=np.int64)
    np.add.at(col_ptr, cols_t + 1, 1)
    col_ptr = np.cumsum(col_ptr)
    return row_ptr, cols.astype(np.int64), col_ptr, rows_t.astype(np.int64)


def csr_to_mask(row_ptr, col_idx, nb):
    mask = np.zeros((nb, nb), dtype=bool)
    for i in range(nb):
        mask[i, col_idx[row_ptr[i]:row_ptr[i + 1]]] = True
    return mask


# ----------------------------------------------------------------------------
# fine branch, Eq.(12)
# ----------------------------------------------------------------------------
def _tokens_of(blocks, block=64):
    return (np.asarray(blocks)[:, None] * block + np.arange(block)[None, :]).reshape(-1)


def _token_sets(L, mask, valid, block, n_text):
    """Real-token flags of all L rows, the video length and the text tokens.

    Rows [0, Lv) are the video slots (Lv = nb * block), rows [Lv, Lv +
    n_text) the text tokens of MMDiT conditioning ([VSA2] §2.2 after
    Eq.(12)), and any rows after them text padding.
    """
    Lv = mask.shape[0] * block
    ok = np.zeros(L, bool)
    ok[:Lv] = True if valid is None else np.asarray(valid, bool)[:Lv]
    ok[Lv:Lv + n_text] = True
    return ok, Lv, np.arange(Lv, Lv + n_text)


def _query_groups(mask, ok, Lv, text, block, rows):
    """(query rows, key rows) of each softmax group: a video query block sees
    its selected video blocks and every text token; the text queries see every
    video token and every text token (video-text and text-text attention stay
    dense).  Pad rows take part in neither side."""
    nb = mask.shape[0]
    for i in (range(nb) if rows is None else rows):
        qt = _tokens_of([i], block)
        toks = np.concatenate([_tokens_of(np.nonzero(mask[i])[0], block), text])
        yield qt, qt[ok[qt]], toks[ok[toks]]
    if len(text):
        allv = np.arange(Lv)
        yield text, text, np.concatenate([allv[ok[:Lv]], text])


def fine_forward(q, k, v, mask, scale=None, rows=None, valid=None, block=64, n_text=0):
    """Block-sparse attention of one head (Eq.(12), with the -inf mask of §2.1
    outside the selected (B x B) tiles; mask is over the video blocks).

    Returns O_f [L, d] and the natural-log LSE [L].  A query block that sees
    no key has O_f = 0 and LSE = -inf (the paper does not treat empty rows).
    ``rows`` limits the work to some query blocks; other video rows are NaN.
    ``valid`` [Lv] marks the real tokens of a padded video grid: pad keys are
    masked, pad query rows get O_f = 0 and LSE = -inf.  ``n_text`` text tokens
    follow the video rows (MMDiT conditioning; the rows after them are text
    padding): every video query also attends to all of them, and they attend
    to every video and text token.
    """
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    L, d = q.shape
    ok, Lv, text = _token_sets(L, mask, valid, block, n_text)
    sc = _scale(d, scale)
    o = np.full((L, v.shape[1]), np.nan)
    lse = np.full(L, np.nan)
    o[Lv:], lse[Lv:] = 0.0, -np.inf
    for allq, qt, toks in _query_groups(mask, ok, Lv, text, block, rows):
        o[allq], lse[allq] = 0.0, -np.inf
        if len(toks) == 0 or len(qt) == 0:
            continue
        s = q[qt] @ k[toks].T * sc
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        o[qt] = (e / z) @ v[toks]
        lse[qt] = (m + np.log(z))[:, 0]
    return o, lse


def fine_backward(q, k, v, mask, d_o, scale=None, valid=None, block=64, n_text=0):
    """Gradients of Eq.(12) with the mask held fixed (the router takes no
    gradient, §2.1-§2.2).  Returns dQ, dK, dV [L, d]; with ``valid`` and
    ``n_text`` (see fine_forward) pad rows take no part and get zero
    gradients."""
    q, k, v, d_o = (np.asarray(t, np.float64) for t in (q, k, v, d_o))
    L, d = q.shape
    ok, Lv, text = _token_sets(L, mask, valid, block, n_text)
    sc = _scale(d, scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for _, qt, toks in _query_groups(mask, ok, Lv, text, block, None):
        if len(toks) == 0 or len(qt) == 0:
            continue
        s = q[qt] @ k[toks].T * sc
        p = _softmax_rows(s)                       # [rows, keys]
        o = p @ v[toks]
        dp = d_o[qt] @ v[toks].T
        ds = p * (dp - (d_o[qt] * o).sum(axis=1, keepdims=True))
        dq[qt] += ds @ k[toks] * sc
        dk[toks] += ds.T @ q[qt] * sc
        dv[toks] += p.T @ d_o[qt]
    return dq, dk, dv


# ----------------------------------------------------------------------------
# coarse branch, Eq.(1)-(4), and gated merge, Eq.(13)-(14)
# ----------------------------------------------------------------------------
def coarse_forward(q, k, v, grid, scale=None, block=64):
    """Eq.(1)-(3): block mean-pooling, dense softmax attention over the nb
    block tokens.  Returns (O_hat_c [nb, d], lse_c [nb], (q_c, k_c, v_c))."""
    d = q.shape[1]
    qc, kc, vc = (block_mean(t, grid, block) for t in (q, k, v))
    s = qc @ kc.T * _scale(d, scale)
    m = s.max(axis=1, keepdims=True)
    z = np.exp(s - m).sum(axis=1, keepdims=True)
    p = np.exp(s - m) / z
    return p @ vc, (m + np.log(z))[:, 0], (qc, kc, vc)


def repeat_cubes(oc, block=64):
    """Eq.(4): broadcast each block row back to its tokens (cube-tiled order)."""
    return np.repeat(np.asarray(oc, np.float64), block, axis=0)


def gate(x, w_g, valid=None):
    """Eq.(13): G = tanh(X W_g), one gate per token and head.
    x [L, Dm], w_g [Dm, H] -> [L, H]; rows that ``valid`` marks as padding
    are 0."""
    g = np.tanh(np.asarray(x, np.float64) @ np.asarray(w_g, np.float64))
    if valid is not None:
        g[~np.asarray(valid, bool)] = 0.0
    return g


def merge(g_h, oc_hat, o_f, block=64):
    """Eq.(14) for one head: O = G (.) Repeat(O_hat_c) + O_f."""
    return g_h[:, None] * repeat_cubes(oc_hat, block) + np.asarray(o_f, np.float64)


def gate_backward(x, w_g, oc_hat, d_o, tokens, valid=None, block=64):
    """Gate part of the backward of Eq.(13)-(14) for some tokens of one batch
    element: with g = tanh(X W_g) and O_c = Repeat(O_hat_c), dL/dg = dO . O_c
    per token and head, dpre = dL/dg (1 - g^2).

    x [n, Dm] and d_o [H, n, d] hold the rows of ``tokens`` (cube-tiled
    indices); oc_hat [H, nb, d]; w_g [Dm, H].  Returns (dpre [n, H],
    dx [n, Dm] = dpre W_g^T, this slice's share X^T dpre [Dm, H] of dW_g).
    ``valid`` [n] marks real tokens; pad rows get dpre = 0.
    """
    x = np.asarray(x, np.float64)
    w_g = np.asarray(w_g, np.float64)
    g = gate(x, w_g)
    cubes = np.asarray(tokens) // block
    dg = np.stack([(np.asarray(d_o[h], np.float64) * np.asarray(oc_hat[h], np.float64)[cubes]).sum(axis=1)
                   for h in range(w_g.shape[1])], axis=1)
    dpre = dg * (1.0 - g ** 2)
    if valid is not None:
        dpre[~np.asarray(valid, bool)] = 0.0
    return dpre, dpre @ w_g.T, x.T @ dpre


def coarse_gate_backward(q, k, v, grid, x, w_g, d_o, scale=None, block=64):
    """Gradients of Eq.(1)-(4) and (13)-(14) for one batch element.

    q, k, v, d_o: [H, L, d]; x [L, Dm]; w_g [Dm, H].
    Returns (dq_c, dk_c, dv_c [H, nb, d] -- the coarse-branch gradients w.r.t.
    the pooled tensors --, dq, dk, dv [H, L, d] of the coarse branch alone,
    i.e. the pooled gradients spread back with weight 1/n to the n real tokens
    of each block (n = B without padding), dx [L, Dm], dw_g [Dm, H]).
    dO_f = dO because Eq.(14) adds O_f with weight one.
    """
    H, L, d = q.shape
    sc = _scale(d, scale)
    ok = token_valid(grid, block)
    g = gate(x, w_g, ok)                                # [L, H]
    dqc, dkc, dvc, ochat = [], [], [], []
    for h in range(H):
        oc_hat, lse_c, (qc, kc, vc) = coarse_forward(q[h], k[h], v[h], grid, scale, block)
        ochat.append(oc_hat)
        doh = np.asarray(d_o[h], np.float64)
        doc_hat = (g[:, h, None] * doh).reshape(-1, block, d).sum(axis=1)   # Repeat^T
        p = np.exp(qc @ kc.T * sc - lse_c[:, None])
        dvc.append(p.T @ doc_hat)
        dp = doc_hat @ vc.T
        ds = p * (dp - (doc_hat * oc_hat).sum(axis=1, keepdims=True))
        dqc.append(ds @ kc * sc)
        dkc.append(ds.T @ qc * sc)
    dqc, dkc, dvc = np.stack(dqc), np.stack(dkc), np.stack(dvc)
    n = ok.reshape(-1, block).sum(axis=1)                               # real tokens per block
    spread = lambda t: np.repeat(t / n[None, :, None], block, axis=1) * ok[None, :, None]   # MeanPool^T
    _, dx, dw = gate_backward(x, w_g, np.stack(ochat), d_o, np.arange(L), ok, block)
    return dqc, dkc, dvc, spread(dqc), spread(dkc), spread(dvc), dx, dw


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------
def vsa2_forward(q, k, v, grid, topk, x, w_g, scale=None, bf16_pooled=False, mask=None, block=64, n_text=0):
    """One batch element, all heads: router -> TopK -> fine + coarse -> merge.

    q, k, v: [H, L, d] (the video slots, then, with ``n_text``, the text rows of
    MMDiT conditioning padded to the tensor's length); x [Lv, Dm] (video);
    w_g [Dm, H].  ``mask`` [H, nb, nb] skips the router and uses a given
    selection.  The router, the coarse branch and the gate see the video
    alone; a text row's O is its O_f.  Returns a dict of every intermediate.
    """
    H = q.shape[0]
    ok = token_valid(grid, block)
    Lv = len(ok)
    g = gate(x, w_g, ok)
    res = {"scores": [], "mask": [], "o_f": [], "lse": [], "oc_hat": [], "lse_c": [], "o": [], "g": g}
    for h in range(H):
        if mask is None:
            p_r = router_scores(q[h][:Lv], k[h][:Lv], grid, scale=scale, bf16_pooled=bf16_pooled, block=block)
            m = topk_per_sequence(p_r, topk)[0]
            res["scores"].append(p_r)
        else:
            m = mask[h]
        o_f, lse = fine_forward(q[h], k[h], v[h], m, scale, valid=ok, block=block, n_text=n_text)
        oc_hat, lse_c, _ = coarse_forward(q[h][:Lv], k[h][:Lv], v[h][:Lv], grid, scale, block)
        res["mask"].append(m)
        res["o_f"].append(o_f)
        res["lse"].append(lse)
        res["oc_hat"].append(oc_hat)
        res["lse_c"].append(lse_c)
        o = o_f.copy()
        o[:Lv] = merge(g[:, h], oc_hat, o_f[:Lv], block)
        res["o"].append(o)
    return {n: (np.stack(t) if isinstance(t, list) and t else t) for n, t in res.items()}


def vsa2_backward(q, k, v, grid, mask, x, w_g, d_o, scale=None, block=64, n_text=0):
    """Gradients of the whole layer (router excluded) for one batch element.
    Returns dq, dk, dv [H, L, d], dx [Lv, Dm], dw_g [Dm, H]; text rows (see
    vsa2_forward) get their gradients from the fine branch alone."""
    H = q.shape[0]
    ok = token_valid(grid, block)
    Lv = len(ok)
    dq, dk, dv = [], [], []
    for h in range(H):
        a, b, c = fine_backward(q[h], k[h], v[h], mask[h], d_o[h], scale, valid=ok, block=block, n_text=n_text)
        dq.append(a); dk.append(b); dv.append(c)
    dq, dk, dv = np.stack(dq), np.stack(dk), np.stack(dv)
    _, _, _, cq, ck, cv, dx, dw = coarse_gate_backward(q[:, :Lv], k[:, :Lv], v[:, :Lv], grid, x, w_g,
                                                       np.asarray(d_o)[:, :Lv], scale, block)
    dq[:, :Lv] += cq
    dk[:, :Lv] += ck
    dv[:, :Lv] += cv
    return dq, dk, dv, dx, dw


# ----------------------------------------------------------------------------
# cost model, App. B Eq.(15)-(16)
# ----------------------------------------------------------------------------
def sparsity(L, block, pool, topk):
    """Eq.(16): sparsity ~= 1 - (1/R^2 + K*B/L) (router two GEMMs + fine branch;
    coarse branch omitted as in App. B)."""
    return 1.0 - (1.0 / pool ** 2 + topk * block / L)
