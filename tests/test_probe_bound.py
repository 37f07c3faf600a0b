"""The probe's rounding-error bound (tests/probe_bound.py) against an f32
emulation of the kernel's arithmetic (CPU only).

The emulation follows the bf16 kernel's steps in float32: q' = sl2 q-bar
split into two bf16 parts, raw bf16 keys, the accumulator seeded with the
centroid logit and the products added in f32, base-2 exponentials against a
running reference, the squared gaps and the normaliser summed in f32, a
rescale to the row maximum and the final division. Its ratios must stay within the
bound of the float64 values, and the bound must stay useful (well below the
ratios themselves) on the blob-structured keys the workloads use.
"""
import math

import numpy as np
import pytest

from oracle import svgear_oracle as O
from probe_bound import ratio_error_bound, ratio_within_bound, selection_flips


def bf16(x):
    """Round float32 values to bfloat16 (nearest, ties to even), as float32."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32)


def emulate_probe_f32(qbar, kp, kbar, koff, scale):
    """The bf16 kernel's arithmetic in float32: q' = sl2 q-bar split into two
    bf16 parts, the accumulator seeded with -sl2 q-bar.k-bar (double, rounded
    once), 32 products per step added in f32, then the streaming sums."""
    f = np.float32
    qbar, kp, kbar = (np.asarray(a, np.float64) for a in (qbar, kp, kbar))
    sl2d = scale * 1.4426950408889634
    sl2 = f(sl2d)
    ck = koff.size - 1
    n = np.diff(koff)
    kappa = np.repeat(np.arange(ck), n)
    qs = (qbar.astype(f) * sl2).astype(f)
    p0 = bf16(qs)
    p1 = bf16((qs - p0).astype(f))
    st = (qbar.astype(f).astype(np.float64) @ kbar.astype(f).astype(np.float64).T * sl2d).astype(f)
    kf = kp.astype(f)
    acc = -st[:, kappa]
    d = kp.shape[1]
    for k in range(0, d, 32):
        for part in (p0, p1):
            acc = (acc + (part[:, k:k + 32] @ kf[:, k:k + 32].T).astype(f)).astype(f)
    D = acc
    cq = qbar.shape[0]
    recs = []  # per block: (reference, Z, E)
    for c2 in range(ck):
        a, b = int(koff[c2]), int(koff[c2 + 1])
        if b == a:
            recs.append(None)
            continue
        Db = D[:, a:b]
        mp = np.maximum(Db.max(axis=1), f(0)).astype(f)
        e = np.exp2((Db - mp[:, None]).astype(f)).astype(f)
        e2 = np.exp2(-mp).astype(f)
        dd = (e - e2[:, None]).astype(f)
        recs.append(((st[:, c2] + mp).astype(f), e.sum(axis=1, dtype=f),
                     (dd * dd).sum(axis=1, dtype=f)))
    ref = np.stack([r[0] for r in recs if r is not None], axis=1)
    m = ref.max(axis=1)
    Z = np.zeros(cq, f)
    for r in recs:
        if r is not None:
            Z = (Z + r[1] * np.exp2((r[0] - m).astype(f))).astype(f)
    ratio = np.full((cq, ck), -1.0, f)
    for c2, r in enumerate(recs):
        if r is None:
            continue
        a = np.exp2((r[0] - m).astype(f)).astype(f)
        ratio[:, c2] = 0.0 if n[c2] == 1 else (r[2] * a * a / (Z * Z) / f(n[c2]))
    return ratio.astype(np.float64)


def blob_head(rng, n, d, ck, sigma=0.25, centres=24):
    cen = rng.standard_normal((centres, d))
    z = rng.integers(0, centres, n)
    k = bf16(cen[z] + sigma * rng.standard_normal((n, d))).astype(np.float64)
    lab = rng.integers(0, ck, n)
    lab[:ck] = np.arange(ck)
    lab[ck] = 0  # one cluster with >= 2 keys for sure
    perm, koff = O.permute(lab, ck)
    kp = k[perm]
    kbar = O.segment_means(kp, koff).astype(np.float32).astype(np.float64)
    return kp, kbar, koff


@pytest.mark.parametrize("seed,d", [(0, 128), (1, 64), (2, 128)])
def test_emulated_kernel_ratios_lie_within_the_bound(seed, d):
    rng = np.random.default_rng(seed)
    kp, kbar, koff = blob_head(rng, 1500, d, 40)
    qbar = (rng.standard_normal((12, d)) * 0.8).astype(np.float32).astype(np.float64)
    scale = 1 / math.sqrt(d)
    want, _ = O.probe(qbar, kp, kbar, koff, scale)
    got = emulate_probe_f32(qbar, kp, kbar, koff, scale)
    bound = ratio_error_bound(qbar, kp, kbar, koff, scale, "bf16")
    ok = ratio_within_bound(got, want, bound)
    assert ok.all(), np.max(np.abs(got - want) / np.maximum(bound, 1e-300))
    live = np.diff(koff) > 1
    rel = bound[:, live] / np.abs(want[:, live])
    # useful: the median relative bound stays well below a percent
    assert np.median(rel) < 2e-3, np.median(rel)


def test_bound_is_zero_where_the_kernel_is_exact_and_catches_a_wrong_ratio():
    rng = np.random.default_rng(5)
    kp, kbar, koff = blob_head(rng, 600, 64, 30)
    # hand cluster 3's keys to cluster 4 and all but one of cluster 5's keys to
    # cluster 6 (an empty cluster, whose ratio the kernel writes as exactly -1,
    # and a one-key cluster, exactly 0)
    koff = koff.copy()
    koff[4] = koff[3]
    koff[6] = koff[5] + 1
    kbar = O.segment_means(kp, koff)
    qbar = rng.standard_normal((5, 64))
    bound = ratio_error_bound(qbar, kp, kbar, koff, 0.125, "bf16")
    n = np.diff(koff)
    assert n[3] == 0 and n[5] == 1
    assert np.all(bound[:, n <= 1] == 0)
    want, _ = O.probe(qbar, kp, kbar, koff, 0.125)
    wrong = want.copy()
    c2 = int(np.argmax(n))
    wrong[:, c2] *= 1.0 + 1e-2   # a one-percent error is never within the bound
    assert not ratio_within_bound(wrong, want, bound)[:, c2].any()


def test_selection_flips_counts_only_unseparated_swaps():
    k_off = np.array([0, 3, 6, 9, 12])
    r_ref = np.array([[0.50, 0.40, 0.399999, 0.1]])
    bound = np.full((1, 4), 1e-5)
    m_ref = np.array([[1, 1, 0, 0]], np.uint8)
    # swapping the two near-equal ratios flips the fill: allowed
    r_gpu = np.array([[0.50, 0.399998, 0.400001, 0.1]])
    m_gpu = np.array([[1, 0, 1, 0]], np.uint8)
    out = selection_flips(r_ref, r_gpu, bound, k_off, m_ref, m_gpu)
    assert out["flipped"] == 1 and out["separated_ok"]
    assert out["max_gap_over_bound"] < 1
    # swapping well-separated ratios is not
    r_bad = np.array([[0.50, 0.1, 0.40, 0.39]])
    out = selection_flips(r_ref, r_bad, bound, k_off, m_ref, np.array([[1, 0, 1, 0]], np.uint8))
    assert out["flipped"] == 1 and not out["separated_ok"]
