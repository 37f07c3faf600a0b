"""Rounding-error bound of the GPU probe's block ratios (test helper).

For query centroid c and permuted key j of key cluster c' the probe needs
the base-2 delta logit D_j = sl2 q-bar_c . (k_j - k-bar_c') (sl2 = scale
log2(e)) and the centroid logit st = sl2 q-bar_c . k-bar_c', formed in double
and rounded once to f32. It forms D_j in one of two ways:
  * bf16 keys: the matrix cores take the raw keys (exact) against
    q' = sl2 q-bar carried as two bf16 parts (a high part and the rounded
    remainder, together within 2^-18 of q'), the accumulator starting at -st;
    2 d/32 MFMAs of 32 exact products each;
  * f32 keys: k_j - k-bar in f32, against q-bar, f32 matrix cores, times sl2.
Per lane it then streams e_j = 2^(D_j - mp) and dd_j = e_j - 2^(-mp) against a
running reference mp >= 0, E = sum dd_j^2 and Z = sum e_j, and a finalize pass
rescales every unit by a = 2^(st + mp - m) and divides:
ratio = sum_units E a^2 / (Z^2 |k_c'|).

Every step's f32 rounding is bounded below (first order, unit roundoff 2^-24,
the hardware exp2 taken to 3 ulp), from the same inputs the kernel received:
  * D_j, bf16 keys: each MFMA's result is taken to carry an error of at most
    33 2^-24 (|accumulator in| + sum |its 32 products|), i.e. the 32 products
    summed one by one in f32 (the worst case, whatever the hardware's internal
    order), which sums to (2 d/32 33 + 2) 2^-24 (|st| + sum_d |q'_d k_jd|)
    with the scale and seed roundings, plus 2^-18 sum_d |q'_d k_jd| for the
    two-part split;
  * D_j, f32 keys: 2 d 2^-24 sl2 sum_d |q-bar_d| |k_jd - k-bar_d|;
  * st in the finalize: 2 2^-24 |st|;
  * exponentials: 3 ulp plus the rounding of their arguments;
  * E: per key 2 |dd| delta(dd) + delta(dd)^2, plus the accumulation chain;
  * Z: the weighted mean of the per-key relative errors (a sum of positive
    terms), plus its summation chain;
  * the finalize rescale, product and division.
With ``mean_tol`` > 0 the bound also covers centroids that differ from the
ones behind the reference values by up to mean_tol (1 + |x|) per coordinate
(the f32 segment means against the oracle's float64 ones).
"""
import math

import numpy as np

LN2 = math.log(2.0)
ULP = 2.0 ** -24


def ratio_error_bound(qbar, kp, kbar, koff, scale, precision, mean_tol=0.0):
    """Absolute bound [Cq, Ck] on |ratio_gpu - ratio_exact| (0 where |k_c'| <= 1
    or the cluster is empty: the kernel writes those exactly)."""
    qbar = np.asarray(qbar, np.float64)
    kp = np.asarray(kp, np.float64)
    kbar = np.asarray(kbar, np.float64)
    koff = np.asarray(koff, np.int64)
    cq, d = qbar.shape
    ck = koff.size - 1
    n = np.diff(koff)
    kappa = np.repeat(np.arange(ck), n)
    sl2 = scale / LN2
    dl = kp - kbar[kappa]                                   # [Nk, d]
    aq, adl = np.abs(qbar), np.abs(dl)
    D = sl2 * (qbar @ dl.T)                                 # [Cq, Nk] base-2 deltas
    st = sl2 * (qbar @ kbar.T)                              # [Cq, Ck]
    if precision == "bf16":
        n_mfma = 2 * (d // 32)
        sqk = sl2 * (aq @ np.abs(kp).T)
        eta = (n_mfma * 33 + 2) * ULP * (np.abs(st)[:, kappa] + sqk) + 2.0 ** -18 * sqk
    else:
        eta = 2 * d * ULP * sl2 * (aq @ adl.T)
    eta = eta + ULP * np.abs(D)
    dst = 2 * ULP * np.abs(st)
    if mean_tol > 0:
        eta = eta + sl2 * mean_tol * ((1 + aq) @ adl.T + aq @ (1 + np.abs(kbar[kappa])).T)
        dst = dst + sl2 * mean_tol * ((1 + aq) @ np.abs(kbar).T + aq @ (1 + np.abs(kbar)).T)

    live = np.nonzero(n > 0)[0]
    starts = koff[live]
    # block-local quantities: the centroid weight of a block is 1
    M = np.maximum(np.maximum.reduceat(D, starts, axis=1), 0.0)   # [Cq, live]
    Mj = np.zeros_like(D)
    Mj[:, :] = np.repeat(M, n[live], axis=1)
    w = np.exp2(D)
    dd = w - 1.0
    e_arg = LN2 * 2 * ULP * (np.abs(D) + Mj)
    dw = w * (LN2 * eta + 3 * 2 * ULP + e_arg)
    d1 = 3 * 2 * ULP + LN2 * 2 * ULP * Mj
    ddd = dw + d1 + ULP * np.abs(dd)
    E = np.add.reduceat(dd * dd, starts, axis=1)
    dE = np.add.reduceat(2 * np.abs(dd) * ddd + ddd * ddd, starts, axis=1)
    dE = dE + E * (n[live] / 4.0 + 16.0) * 2 * ULP

    # absolute base-2 logits and the normaliser, relative to its maximum
    st_j = st[:, kappa]
    s = st_j + D
    m = s.max(axis=1, keepdims=True)
    p = np.exp2(s - m)
    Z = p.sum(axis=1, keepdims=True)
    rel_j = LN2 * (dst[:, kappa] + eta) + 3 * 2 * ULP + e_arg
    maxu = (kp.shape[0] + 255) // 256 + ck
    relZ = (p * rel_j).sum(axis=1, keepdims=True) / Z + (64 + 16 + maxu / 256.0) * ULP
    # finalize: a = 2^(st + mp - m) with rounded arguments, then E a^2 / (Z^2 n)
    stl = st[:, live]
    e_fin = LN2 * 2 * ULP * (np.abs(stl + M) + np.abs(m)) + 3 * 2 * ULP
    scale_blk = np.exp2(2 * (stl - m)) / (Z * Z * n[live])
    rel = 2 * LN2 * dst[:, live] + 2 * e_fin + 2 * relZ + 4 * ULP
    bound = np.zeros((cq, ck))
    bound[:, live] = (dE + E * rel) * scale_blk + 2.0 ** -120
    bound[:, n <= 1] = 0.0
    return bound


def ratio_within_bound(got, want, bound):
    """Boolean mask of ratios within the bound (exact -1 / 0 cases included)."""
    return np.abs(got - want) <= bound


def selection_flips(r_ref, r_gpu, bound, k_off, mask_ref, mask_gpu, q_off=None):
    """Query clusters whose selections differ, and whether every difference
    comes from ratios that the bound cannot separate.

    For each differing query cluster, every pair of live key clusters (x, y)
    that the reference ratios separate by more than bound[x] + bound[y] must
    keep its order in the GPU's greedy order; the first position where the two
    greedy orders part is the fill decision that changed, and its reference
    ratios' relative gap is reported.
    Returns dict(flipped, live, separated_ok, max_rel_gap, max_gap_over_bound).
    """
    k_live = np.nonzero(np.diff(k_off) > 0)[0]
    q_live = np.ones(r_ref.shape[0], bool) if q_off is None else np.diff(q_off) > 0
    diff = np.any(mask_ref != mask_gpu, axis=1) & q_live
    out = dict(flipped=int(diff.sum()), live=int(q_live.sum()), separated_ok=True,
               max_rel_gap=0.0, max_gap_over_bound=0.0)
    for c in np.nonzero(diff)[0]:
        a, g, b = r_ref[c, k_live], r_gpu[c, k_live], bound[c, k_live]
        idx = k_live
        # GPU order: ratio descending, index ascending
        gpu_before = (g[:, None] > g[None, :]) | ((g[:, None] == g[None, :]) &
                                                  (idx[:, None] < idx[None, :]))
        separated = (a[:, None] - a[None, :]) > (b[:, None] + b[None, :])
        if np.any(separated & ~gpu_before):
            out["separated_ok"] = False
        oa = idx[np.lexsort((idx, -a))]
        og = idx[np.lexsort((idx, -g))]
        p = int(np.argmax(oa != og))
        x, y = oa[p], og[p]
        gap = abs(r_ref[c, x] - r_ref[c, y])
        out["max_rel_gap"] = max(out["max_rel_gap"],
                                 gap / max(abs(r_ref[c, x]), abs(r_ref[c, y]), 1e-300))
        out["max_gap_over_bound"] = max(out["max_gap_over_bound"],
                                        gap / max(bound[c, x] + bound[c, y], 1e-300))
    return out
