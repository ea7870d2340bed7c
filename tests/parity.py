"""Comparison rules between the GPU library and the oracle (test helpers).

Rules (identical seeded inputs on both sides):
1. Codes: GPU idx == oracle idx for every coordinate, except where the
   oracle's fp64 rotated coordinate z lies within BAND = 1e-5 of a decision
   threshold; the mismatch fraction must be <= 1e-4.  The near-band fraction
   of the data is reported.
2. QJL bits, conditional: the oracle recomputes p = S r in fp64 from the
   GPU's codes (r = z - c[idx_gpu]); GPU bits == [p >= 0] except where
   |p_i| <= BAND.
3. nu and gamma: relative difference <= 1e-6.
4. Scores and attention outputs: the oracle scores the GPU's codes; per row
   |a - b| / |b| <= 1e-3.  Score and scan rows (one entry per token or
   database row) are also held element-wise: |a_j - b_j| <= 1e-4 max_j |b_j|,
   so that a few wrong tokens in a long row cannot hide under the row norm.
"""

import numpy as np

import oracle

BAND = 1e-5
MAX_MISMATCH = 1e-4
NORM_RTOL = 1e-6
ROW_RTOL = 1e-3
ELEM_RTOL = 1e-4


def to_np(t):
    return t.detach().cpu().numpy()


def gpu_codes(packed, d, code_bits, m=None):
    out = {"idx": oracle.unpack_codes(to_np(packed.idx), d, code_bits),
           "norm": to_np(packed.norm).astype(np.float64)}
    if packed.qjl is not None:
        out["sign"] = oracle.unpack_bits(to_np(packed.qjl), m)
        out["rnorm"] = to_np(packed.rnorm).astype(np.float64)
    return out


def check_codes(gpu_idx, orc_idx, z, thresholds, report=None, chunk=65536):
    """Rule 1; returns (mismatch fraction, near-band fraction)."""
    t = np.asarray(thresholds, dtype=np.float64)
    n = gpu_idx.shape[0]
    mism = 0
    near = 0
    total = gpu_idx.size
    for a in range(0, n, chunk):
        g, o, zz = gpu_idx[a:a + chunk], orc_idx[a:a + chunk], z[a:a + chunk]
        bad = g != o
        if np.any(bad):
            zb = zz[bad]
            dist = np.min(np.abs(zb[:, None] - t[None, :]), axis=1)
            assert np.all(dist <= BAND), "code mismatch outside the boundary band: %g" % dist.max()
            assert np.all(np.abs(g[bad] - o[bad]) == 1)
        mism += int(bad.sum())
        near += int((np.min(np.abs(zz[..., None] - t), axis=-1) <= BAND).sum())
    frac, nfrac = mism / total, near / total
    if report is not None:
        report["code_mismatch_frac"] = frac
        report["near_band_frac"] = nfrac
    assert frac <= MAX_MISMATCH, frac
    return frac, nfrac


def check_qjl(gpu, z, centroids, S, report=None):
    """Rule 2 (and gamma, rule 3)."""
    r = oracle.codec.residual_from_codes(z, gpu["idx"], centroids)
    p = oracle.qjl_projection(r, S)
    want = (p >= 0).astype(np.uint8)
    bad = gpu["sign"] != want
    if np.any(bad):
        assert np.all(np.abs(p[bad]) <= BAND), np.abs(p[bad]).max()
    gamma = np.sqrt(np.sum(r * r, axis=1))
    rel = np.abs(gpu["rnorm"] - gamma) / np.maximum(gamma, 1e-30)
    assert rel.max() <= NORM_RTOL, rel.max()
    if report is not None:
        report["qjl_mismatch_frac"] = float(bad.mean())
    return float(bad.mean())


def check_norm(gpu_norm, orc_norm):
    rel = np.abs(gpu_norm - orc_norm) / np.maximum(orc_norm, 1e-30)
    zero = orc_norm == 0
    assert np.all(gpu_norm[zero] == 0)
    assert rel[~zero].max(initial=0) <= NORM_RTOL, rel[~zero].max(initial=0)


def row_rel_err(a, b):
    a = np.asarray(a, dtype=np.float64).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, np.shape(b)[-1])
    return np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-300)


def check_rows(a, b, tol=ROW_RTOL):
    e = row_rel_err(a, b)
    assert e.max() <= tol, e.max()
    return float(e.max())


def check_scores(a, b, tol=ROW_RTOL, elem=ELEM_RTOL):
    """Rule 4 for score and scan rows: the row rule plus, per row,
    max_j |a_j - b_j| <= elem * max_j |b_j|.  Returns (max row error, max
    element error relative to its row's largest entry)."""
    e = check_rows(a, b, tol)
    a = np.asarray(a, dtype=np.float64).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, np.shape(b)[-1])
    scale = np.maximum(np.max(np.abs(b), axis=1), 1e-300)
    el = np.max(np.abs(a - b), axis=1) / scale
    assert el.max() <= elem, el.max()
    return e, float(el.max())
