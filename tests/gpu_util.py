"""Helpers shared by the GPU parity tests: comparisons and selection plumbing."""

import numpy as np
import torch

from oracle import vsa2_oracle as orc


def f64(t):
    return t.detach().float().cpu().double().numpy()


def rel_l2(got, want):
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def assert_close_bf16(got, want, what, max_abs=2e-2, rel=1e-2, rounding=0.0):
    """bf16 output bound: |got - want| <= max_abs + rounding * |want| elementwise
    and rel-L2 <= rel.  `rounding` is the relative error the storage format
    itself adds: 2^-8 for a value rounded to bf16 twice (the merged output O
    is computed from the bf16-stored O_f and rounded again), 0 otherwise."""
    excess = np.abs(got - want) - rounding * np.abs(want)
    err = float(excess.max()) if got.size else 0.0
    r = rel_l2(got, want)
    assert err <= max_abs and r <= rel, (f"{what}: max-abs beyond storage rounding {err:.3g} (<= {max_abs}), "
                                         f"rel-L2 {r:.3g} (<= {rel})")


def assert_close_f32(got, want, what, tol=1e-4):
    err = float(np.abs(got - want).max()) if got.size else 0.0
    r = rel_l2(got, want)
    assert err <= tol and r <= tol, f"{what}: max-abs {err:.3g}, rel-L2 {r:.3g} (<= {tol})"


def csr_tensors(masks, device):
    """CSR (row_ptr [1,H,nb+1], col_idx [1,H,k]) int32 from oracle masks [H,nb,nb]."""
    rp = np.stack([orc.mask_to_csr_csc(m)[0] for m in masks])
    ci = np.stack([orc.mask_to_csr_csc(m)[1] for m in masks])
    return (torch.tensor(rp, dtype=torch.int32)[None].to(device), torch.tensor(ci, dtype=torch.int32)[None].to(device))


def masks_from_csr(row_ptr, col_idx, nb):
    rp, ci = row_ptr.cpu().numpy(), col_idx.cpu().numpy()
    return np.stack([orc.csr_to_mask(rp[h], ci[h], nb) for h in range(rp.shape[0])])


def check_csr_csc(row_ptr, col_idx, col_ptr, row_idx, nb, k):
    """Structural validity: counts, ascending order in every row and column, and CSC == transpose of CSR."""
    rp, ci, cp, ri = (t.cpu().numpy() for t in (row_ptr, col_idx, col_ptr, row_idx))
    for h in range(rp.shape[0]):
        assert rp[h, 0] == 0 and rp[h, -1] == k and np.all(np.diff(rp[h]) >= 0)
        assert cp[h, 0] == 0 and cp[h, -1] == k and np.all(np.diff(cp[h]) >= 0)
        m = orc.csr_to_mask(rp[h], ci[h], nb)
        assert m.sum() == k, "duplicate columns in a row"
        for i in range(nb):
            row = ci[h, rp[h, i]:rp[h, i + 1]]
            assert np.all(np.diff(row) > 0)
        mt = orc.csr_to_mask(cp[h], ri[h], nb).T
        assert np.array_equal(m, mt), "CSC is not the transpose of CSR"
        for j in range(nb):
            col = ri[h, cp[h, j]:cp[h, j + 1]]
            assert np.all(np.diff(col) > 0), "rows not ascending in a CSC column"


def band_compare(gpu_mask, oracle_scores, k, rel_band=1e-3):
    """Selected sets must agree wherever the oracle score is outside the
    relative band |s - tau| <= rel_band * tau around the oracle's k-th score.
    Returns (mismatches outside the band, band size, mismatches inside)."""
    s = np.asarray(oracle_scores)
    flat = np.sort(s.reshape(-1))[::-1]
    tau = flat[k - 1]
    band = np.abs(s - tau) <= rel_band * tau
    want = orc.topk_per_sequence(s, k // s.shape[0])[0] if k % s.shape[0] == 0 else None
    if want is None:
        raise ValueError("k must be a multiple of nb")
    outside = int(np.sum(gpu_mask[~band] != want[~band]))
    inside = int(np.sum(gpu_mask[band] != want[band]))
    return outside, int(band.sum()), inside


def empty_rows(mask, rows):
    """Clear some query rows of a selection and hand their pairs to the first
    free slots of the other rows, so the per-head budget stays exact."""
    m = mask.copy()
    moved = int(m[rows].sum())
    m[rows] = False
    keep = [r for r in range(m.shape[0]) if r not in rows]
    for r in keep:
        for j in range(m.shape[1]):
            if moved == 0:
                return m
            if not m[r, j]:
                m[r, j] = True
                moved -= 1
    assert moved == 0
    return m


def coarse_lse_bound(qc, kc, scale):
    """Per-row bound on |lse_c(GPU) - lse_c(oracle)| when the pooled coarse
    operands Q_c, K_c are stored in bf16 (each element rounded, relative error
    <= 2^-9) and the oracle keeps them exact.  A logit scale * q . k then moves
    by at most scale * sum_d |q_d k_d| * (2 * 2^-9 + 2^-18), and a log-sum-exp
    moves by at most the largest change of its logits.  1e-4 covers the fp32
    accumulation."""
    a = np.abs(np.asarray(qc)) @ np.abs(np.asarray(kc)).T * scale
    return a.max(axis=1) * (2.0 ** -8 + 2.0 ** -18) + 1e-4
