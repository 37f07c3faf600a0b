"""Plain CPU oracle of the SVG-EAR routed sparse-attention path.

TEST INFRASTRUCTURE ONLY. This module exists so that tests, the smoke check
and the benchmark's CPU baseline can check the HIP library against an
independent, obviously correct implementation. The product path never
imports it and must not fall back to it.

Source of the method: "SVG-EAR: Parameter-Free Linear Compensation for
Sparse Video Generation via Error-aware Routing" (arXiv 2603.08982), read
from its HTML renderings. Section references below are that paper's:
  * Section 3.1 (Structured Redundancy): cluster, permute, centroid logit.
  * Section 4.1 (Problem Formulation): k-means of Q and K, block-level mask,
    density budget, scale 1/sqrt(d).
  * Section 4.2 (Error-Aware Routing): relaxation to unnormalised weights,
    query-centroid probe (the paper's Equation 5, whose display did not
    survive extraction), error-to-size ratio and greedy fill.
  * Section 4.3 (Linear Compensation): skipped block = |k_c| copies of the
    centroid logit with the mean value.
  * Section 5 "Implementation": routing per query cluster.

Everything here is float64 NumPy, one head at a time, with no blocking,
fusion or reordering beyond what the definitions state. Where the pages are
silent the reading taken is stated at the function (and listed in the
design notes of the repository).

Parity pins: every function below is pinned by tests under ``tests/``
(``test_oracle_*.py``) against closed forms, invariants and special cases;
the one quantity with no pin is the absolute quality of the error estimate
against the true attention error ("parity unpinned": the paper's theorem
statement did not survive extraction).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_operand", "kmeans_assign", "kmeans_update", "kmeans", "permute", "gather",
    "segment_means", "probe", "probe_values", "route", "route_global", "attend", "unpermute",
    "dense_attention", "block_scores", "attention_map_error", "row_spread",
    "routed_attention_head", "RoutedResult",
]


# ----------------------------------------------------------------------------
# operand precision of a floating-point decision
# ----------------------------------------------------------------------------
def round_operand(x, precision: str) -> np.ndarray:
    """Round ``x`` to the precision an operand has when a decision is taken.

    ``"bf16"``: round-to-nearest-even to bfloat16 (8-bit significand);
    ``"f32"``: round to IEEE single; ``"f64"``: unchanged. Returned as float64.
    Used only where floating point decides an integer (the k-means argmin), so
    that the oracle takes that decision from the same operand values as the
    kernel does.
    """
    x = np.asarray(x)
    if precision == "f64":
        return x.astype(np.float64)
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if precision == "f32":
        return x32.astype(np.float64)
    if precision != "bf16":
        raise ValueError(precision)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# cluster (Section 4.1: the rows of Q and of K are each grouped by k-means)
# ----------------------------------------------------------------------------
def kmeans_assign(x, mu, operand: str = "f64") -> np.ndarray:
    """Assignment step of Lloyd's k-means (Section 4.1).

    a_n = argmin_c ||x_n - mu_c||^2. The term ||x_n||^2 is the same for every
    c, so the argmin is taken over ||mu_c||^2 - 2 x_n . mu_c. Ties go to the
    lowest centroid index (numpy's argmin returns the first minimum). The
    centroids enter at ``operand`` precision (see ``round_operand``).
    """
    x = np.asarray(x, dtype=np.float64)
    m = round_operand(mu, operand)
    dist = (m * m).sum(axis=1)[None, :] - 2.0 * (x @ m.T)
    return np.argmin(dist, axis=1).astype(np.int32)


def kmeans_update(x, labels, mu_prev):
    """Update step: each centroid becomes the mean of its members.

    A cluster with no member keeps its previous centroid (the pages do not say;
    this is the usual Lloyd convention). Returns (mu, counts).
    """
    x = np.asarray(x, dtype=np.float64)
    mu_prev = np.asarray(mu_prev, dtype=np.float64)
    c = mu_prev.shape[0]
    counts = np.bincount(labels, minlength=c)
    sums = np.zeros_like(mu_prev)
    np.add.at(sums, labels, x)
    mu = mu_prev.copy()
    nz = counts > 0
    mu[nz] = sums[nz] / counts[nz, None]
    return mu, counts.astype(np.int32)


def kmeans(x, init, iters: int, operand: str = "f64"):
    """Lloyd's k-means from a caller-supplied initial centroid table.

    For t = 1..iters: assign with the current centroids, then replace every
    non-empty centroid by its members' mean. Returns (labels of the last
    assignment, counts, centroids = means of those labels).
    """
    if iters < 1:
        raise ValueError("iters must be >= 1")
    mu = np.asarray(init, dtype=np.float64).copy()
    labels = counts = None
    for _ in range(iters):
        labels = kmeans_assign(x, mu, operand)
        mu, counts = kmeans_update(x, labels, mu)
    return labels, counts, mu


# ----------------------------------------------------------------------------
# permute (Section 3.1: tokens of a cluster are laid out contiguously)
# ----------------------------------------------------------------------------
def permute(labels, c: int):
    """Stable permutation that makes every cluster contiguous.

    perm[p] is the source token placed in slot p; tokens of one cluster keep
    their original order. offsets[c] .. offsets[c+1] is cluster c's slot range.
    """
    labels = np.asarray(labels)
    perm = np.argsort(labels, kind="stable").astype(np.int32)
    counts = np.bincount(labels, minlength=c)
    offsets = np.zeros(c + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return perm, offsets


def gather(x, perm) -> np.ndarray:
    """Rows in permuted order: x_p[p] = x[perm[p]]."""
    return np.asarray(x)[np.asarray(perm)]


def segment_means(xp, offsets) -> np.ndarray:
    """Mean row of every cluster segment of a permuted tensor (Section 4.1/4.3).

    These are the centroids q-bar, k-bar and the mean values v-bar (V follows
    K's clusters, Section 4.3). An empty segment has no mean; it is reported as
    a zero row and is never used downstream.
    """
    xp = np.asarray(xp, dtype=np.float64)
    offsets = np.asarray(offsets)
    c = offsets.shape[0] - 1
    out = np.zeros((c, xp.shape[1]), dtype=np.float64)
    for i in range(c):
        a, b = int(offsets[i]), int(offsets[i + 1])
        if b > a:
            out[i] = xp[a:b].sum(axis=0) / (b - a)
    return out


def unpermute(xp, perm) -> np.ndarray:
    """Inverse of ``gather``: x[perm[p]] = x_p[p]."""
    xp = np.asarray(xp)
    out = np.empty_like(xp)
    out[np.asarray(perm)] = xp
    return out


# ----------------------------------------------------------------------------
# probe (Section 4.2, Equation 5 and "Error estimation")
# ----------------------------------------------------------------------------
def probe(q_centroids, kp, k_centroids, k_offsets, scale: float, mode: str = "weight"):
    """Query-centroid error probe and block error-to-size ratio (Section 4.2).

    Reading of the lost Equation 5 (``mode="weight"``): with query centroid
    q-bar_c standing in for every query of its cluster, and key j in key
    cluster kappa(j),
        s_cj  = scale * q-bar_c . k_j          (logit with the raw key)
        s~_cj = scale * q-bar_c . k-bar_kappa(j)  (logit with the key centroid)
        m_c   = max_j s_cj,   Z_c = sum_j exp(s_cj - m_c)
        eps_cj = (exp(s_cj - m_c) - exp(s~_cj - m_c)) / Z_c,
    i.e. the gap between the attention weights the two logits give, both under
    the centroid query's full softmax normaliser (the relaxed objective compares
    weights, not logits, and the probe kernel subtracts a running maximum
    before exponentiating).

    Block error: every query of cluster c shares the proxy q-bar_c, so the
    block sum is |q_c| * sum_{j in c'} eps_cj^2 and the error-to-size ratio
    divides by |q_c| |k_c'|:
        ratio[c, c'] = (1/|k_c'|) sum_{j in c'} eps_cj^2.
    ratio = -1 marks an empty key cluster.

    ``mode="logit"`` replaces eps by the raw logit gap s_cj - s~_cj (kept only
    for sensitivity studies).

    Returns (ratio [Cq, Ck], log_norm [Cq]) with log_norm = m_c + ln Z_c, the
    log of the centroid query's softmax normaliser over all keys.
    """
    qc = np.asarray(q_centroids, dtype=np.float64)
    kp = np.asarray(kp, dtype=np.float64)
    kc = np.asarray(k_centroids, dtype=np.float64)
    off = np.asarray(k_offsets)
    ck = off.shape[0] - 1
    counts = np.diff(off)
    kappa = np.repeat(np.arange(ck), counts)          # key cluster of each permuted key
    s = scale * (qc @ kp.T)                           # [Cq, Nk]
    s_tilde = (scale * (qc @ kc.T))[:, kappa]         # [Cq, Nk]
    m = s.max(axis=1, keepdims=True)
    z = np.exp(s - m).sum(axis=1, keepdims=True)
    if mode == "weight":
        eps = (np.exp(s - m) - np.exp(s_tilde - m)) / z
    elif mode == "logit":
        eps = s - s_tilde
    else:
        raise ValueError(mode)
    sq = eps * eps
    ratio = np.full((qc.shape[0], ck), -1.0)
    for j in range(ck):
        a, b = int(off[j]), int(off[j + 1])
        if b > a:
            ratio[:, j] = sq[:, a:b].sum(axis=1) / (b - a)
    log_norm = (m + np.log(z))[:, 0]
    return ratio, log_norm


def probe_values(q_centroids, kp, k_centroids, vp, v_centroids, k_offsets, scale: float):
    """Value-aware query-centroid error probe (Section 4.2's value-aware estimate).

    The estimate's display did not survive extraction; the text says it brings
    every v_j and v-bar_j into the error of the compensated output. Reading:
    the compensation replaces key j's contribution p_cj * v_j to the centroid
    query's output by p~_cj * v-bar_kappa(j), where p and p~ are the two weights
    of ``probe`` (exp(s - m)/Z and exp(s~ - m)/Z), and the per-key error is the
    squared norm of that output gap,
        eps_cj = || p_cj v_j - p~_cj v-bar_kappa(j) ||^2,
    aggregated per block as in ``probe``:
        ratio[c, c'] = (1/|k_c'|) sum_{j in c'} eps_cj.
    ``probe``'s per-key term (p - p~)^2 is this with every value a unit scalar.
    ratio = -1 marks an empty key cluster.

    Returns (ratio [Cq, Ck], log_norm [Cq]) as ``probe``.
    """
    qc = np.asarray(q_centroids, dtype=np.float64)
    kp = np.asarray(kp, dtype=np.float64)
    kc = np.asarray(k_centroids, dtype=np.float64)
    vp = np.asarray(vp, dtype=np.float64)
    vc = np.asarray(v_centroids, dtype=np.float64)
    off = np.asarray(k_offsets)
    ck = off.shape[0] - 1
    counts = np.diff(off)
    kappa = np.repeat(np.arange(ck), counts)
    vbar = vc[kappa]                                  # [Nk, d]: each key's mean value
    s = scale * (qc @ kp.T)
    s_tilde = (scale * (qc @ kc.T))[:, kappa]
    m = s.max(axis=1, keepdims=True)
    z = np.exp(s - m).sum(axis=1, keepdims=True)
    p = np.exp(s - m) / z
    pt = np.exp(s_tilde - m) / z
    ratio = np.full((qc.shape[0], ck), -1.0)
    for c in range(qc.shape[0]):
        gap = p[c][:, None] * vp - pt[c][:, None] * vbar
        eps = (gap * gap).sum(axis=1)
        for j in range(ck):
            a, b = int(off[j]), int(off[j + 1])
            if b > a:
                ratio[c, j] = eps[a:b].sum() / (b - a)
    log_norm = (m + np.log(z))[:, 0]
    return ratio, log_norm


# ----------------------------------------------------------------------------
# route (Section 4.2 greedy selection; Section 5 per-query-cluster routing)
# ----------------------------------------------------------------------------
def route(ratio, k_offsets, budget_keys: int, fill: str = "skip", q_offsets=None):
    """Greedy error-to-cost routing, one query cluster at a time.

    For each query cluster (with ``q_offsets`` given, each non-empty one: a
    query cluster without queries has no attention row to route and selects
    nothing): order the non-empty key clusters by ratio,
    highest first (equal ratios: lower key-cluster index first), and walk the
    order once; a key cluster is selected when its keys still fit the
    remaining budget of ``budget_keys`` exact keys (``fill="skip"``: a cluster
    that does not fit is passed over and later, smaller ones may still fit;
    ``fill="stop"``: the walk ends at the first cluster that does not fit).

    Returns (mask [Cq, Ck] uint8, list [Cq, Ck] int32 ascending and padded with
    -1, count [Cq] int32, keys [Cq] int32 = exact keys used).
    """
    ratio = np.asarray(ratio, dtype=np.float64)
    off = np.asarray(k_offsets)
    counts = np.diff(off).astype(np.int64)
    cq, ck = ratio.shape
    mask = np.zeros((cq, ck), dtype=np.uint8)
    lst = np.full((cq, ck), -1, dtype=np.int32)
    cnt = np.zeros(cq, dtype=np.int32)
    used_keys = np.zeros(cq, dtype=np.int32)
    nonempty = np.nonzero(counts > 0)[0]
    q_live = np.ones(cq, dtype=bool) if q_offsets is None else np.diff(np.asarray(q_offsets)) > 0
    for c in range(cq):
        if not q_live[c]:
            continue
        r = ratio[c, nonempty]
        order = nonempty[np.lexsort((nonempty, -r))]
        used = 0
        for j in order:
            if used + counts[j] <= budget_keys:
                mask[c, j] = 1
                used += counts[j]
            elif fill == "stop":
                break
        sel = np.nonzero(mask[c])[0]
        lst[c, : sel.size] = sel
        cnt[c] = sel.size
        used_keys[c] = used
    return mask, lst, cnt, used_keys


def route_global(ratio, q_offsets, k_offsets, budget_entries: int, fill: str = "skip"):
    """Greedy error-to-cost routing over every block of a head at once.

    Section 4.1 bounds the number of exact entries of the block mask by
    rho * N_q * N_k for the whole attention map, and Section 4.2 takes
    blocks in decreasing order of estimated error per entry until that
    budget is spent. Here every block (c, c') with a non-empty query cluster c and a
    non-empty key cluster c' competes for one head-wide budget of
    ``budget_entries`` exact (query, key) entries, and a block costs
    |q_c| * |k_c'| entries (Section 5's split of the budget per query cluster
    is not applied; ``route`` applies it).

    Order: ratio highest first; equal ratios lower query cluster first, then
    lower key cluster. The walk and ``fill`` are those of ``route``.

    Returns (mask [Cq, Ck] uint8, list [Cq, Ck] int32 ascending and padded with
    -1, count [Cq] int32, keys [Cq] int32 = exact keys of each query cluster,
    used = exact entries used, an int).
    """
    ratio = np.asarray(ratio, dtype=np.float64)
    nq = np.diff(np.asarray(q_offsets)).astype(np.int64)
    nk = np.diff(np.asarray(k_offsets)).astype(np.int64)
    cq, ck = ratio.shape
    cs, ks = np.meshgrid(np.arange(cq), np.arange(ck), indexing="ij")
    live = (nq[cs] > 0) & (nk[ks] > 0)
    c_live, k_live = cs[live], ks[live]
    order = np.lexsort((k_live, c_live, -ratio[c_live, k_live]))
    mask = np.zeros((cq, ck), dtype=np.uint8)
    used = 0
    for t in order:
        c, j = int(c_live[t]), int(k_live[t])
        cost = int(nq[c] * nk[j])
        if used + cost <= budget_entries:
            mask[c, j] = 1
            used += cost
        elif fill == "stop":
            break
    lst = np.full((cq, ck), -1, dtype=np.int32)
    cnt = np.zeros(cq, dtype=np.int32)
    keys = np.zeros(cq, dtype=np.int32)
    for c in range(cq):
        sel = np.nonzero(mask[c])[0]
        lst[c, : sel.size] = sel
        cnt[c] = sel.size
        keys[c] = int(nk[sel].sum())
    return mask, lst, cnt, keys, used


# ----------------------------------------------------------------------------
# attend (Section 4.1 mask, Section 4.3 linear compensation)
# ----------------------------------------------------------------------------
def attend(qp, kp, vp, q_offsets, k_offsets, k_centroids, v_centroids, sel_mask, scale: float):
    """Compensated block-sparse attention for permuted Q, K, V (Section 4.3).

    Query i of query cluster c sees one softmax over
      * the exact logits scale * q_i . k_j of every key j in a selected key
        cluster, with values v_j, and
      * for every non-selected, non-empty key cluster c', one logit
        scale * q_i . k-bar_c' counted |k_c'| times (i.e. plus ln |k_c'|), with
        value v-bar_c'.
    The row is formed in full, its maximum subtracted, exponentiated,
    normalised and multiplied by the values.
    """
    qp = np.asarray(qp, dtype=np.float64)
    kp = np.asarray(kp, dtype=np.float64)
    vp = np.asarray(vp, dtype=np.float64)
    kc = np.asarray(k_centroids, dtype=np.float64)
    vc = np.asarray(v_centroids, dtype=np.float64)
    qo = np.asarray(q_offsets)
    ko = np.asarray(k_offsets)
    mask = np.asarray(sel_mask)
    counts = np.diff(ko)
    out = np.zeros((qp.shape[0], vp.shape[1]), dtype=np.float64)
    for c in range(qo.shape[0] - 1):
        a, b = int(qo[c]), int(qo[c + 1])
        if b == a:
            continue
        sel = [j for j in range(counts.size) if mask[c, j] and counts[j] > 0]
        comp = [j for j in range(counts.size) if not mask[c, j] and counts[j] > 0]
        if sel:
            idx = np.concatenate([np.arange(ko[j], ko[j + 1]) for j in sel])
        else:
            idx = np.zeros(0, dtype=np.int64)
        q = qp[a:b]
        logits = np.concatenate(
            [scale * (q @ kp[idx].T), scale * (q @ kc[comp].T) + np.log(counts[comp])[None, :]],
            axis=1)
        values = np.concatenate([vp[idx], vc[comp]], axis=0)
        logits -= logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        w /= w.sum(axis=1, keepdims=True)
        out[a:b] = w @ values
    return out


def dense_attention(q, k, v, scale: float) -> np.ndarray:
    """Full softmax attention softmax(scale Q K^T) V (Section 4.1's A_full)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T)
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return w @ v


# ----------------------------------------------------------------------------
# error analysis (Section 5.3, "Strategy of block selection", Fig. 6a)
# ----------------------------------------------------------------------------
def block_scores(q_centroids, k_centroids, k_offsets, scale: float):
    """Score-based block ranking of the top-p baseline (Section 5.3's first two
    strategies; Sections 1 and 4.2 describe it as selection by approximated
    attention scores).

    Reading: the score of block (c, c') is its share of the centroid query's
    attention mass estimated from the centroids,
        score[c, c'] = |k_c'| exp(scale q-bar_c . k-bar_c') / sum_c'' (same),
    and the baseline selects blocks in decreasing score. Used as the ``ratio``
    of ``route`` it fills the same per-query-cluster budget as the error-aware
    router, which keeps the density of the compared methods equal. Empty key
    clusters score -1.
    """
    qc = np.asarray(q_centroids, dtype=np.float64)
    kc = np.asarray(k_centroids, dtype=np.float64)
    n = np.diff(np.asarray(k_offsets)).astype(np.float64)
    st = scale * (qc @ kc.T)
    live = n > 0
    st_live = np.where(live[None, :], st, -np.inf)
    w = n[None, :] * np.exp(st_live - st_live.max(axis=1, keepdims=True))
    score = w / w.sum(axis=1, keepdims=True)
    return np.where(live[None, :], score, -1.0)


def attention_map_error(qp, kp, q_offsets, k_offsets, k_centroids, sel_mask, scale: float,
                        compensate: bool = True):
    """Distance of a block-sparse attention map from the full one (Section 5.3).

    A_full = softmax(scale Q K^T) row by row. A_sparse keeps the exact weight
    exp(s_ij) of every key in a selected block of the query's cluster; every
    key j of a skipped non-empty key cluster c' gets the centroid weight
    exp(scale q_i . k-bar_c') when ``compensate`` (Section 4.3: the block counts
    |k_c'| copies of the centroid logit) and 0 when not (top-p without
    compensation); each sparse row is normalised by its own sum (a row with
    nothing kept stays 0).

    Returns per query (err [Nq] = sum_j (A_sparse - A_full)_ij^2, z_full [Nq],
    z_sparse [Nq]), both normalisers taken relative to the row maximum of the
    exact logits. Section 5.3's mean squared error is err.sum() / (Nq * Nk).
    """
    qp = np.asarray(qp, dtype=np.float64)
    kp = np.asarray(kp, dtype=np.float64)
    kc = np.asarray(k_centroids, dtype=np.float64)
    qo, ko = np.asarray(q_offsets), np.asarray(k_offsets)
    mask = np.asarray(sel_mask)
    nk = np.diff(ko)
    kappa = np.repeat(np.arange(nk.size), nk)
    err = np.zeros(qp.shape[0])
    zf = np.zeros(qp.shape[0])
    zs = np.zeros(qp.shape[0])
    for c in range(qo.size - 1):
        a, b = int(qo[c]), int(qo[c + 1])
        if b == a:
            continue
        q = qp[a:b]
        s = scale * (q @ kp.T)                                  # [n, Nk]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        full = e / e.sum(axis=1, keepdims=True)
        keep = mask[c][kappa].astype(bool)                      # [Nk]
        w = np.where(keep[None, :], e, 0.0)
        if compensate:
            st = scale * (q @ kc.T)                             # [n, Ck]
            w = np.where(keep[None, :], w, np.exp(st[:, kappa] - m))
        z = w.sum(axis=1, keepdims=True)
        sparse = np.divide(w, z, out=np.zeros_like(w), where=z > 0)
        err[a:b] = ((sparse - full) ** 2).sum(axis=1)
        zf[a:b] = e.sum(axis=1)
        zs[a:b] = z[:, 0]
    return err, zf, zs


def row_spread(xp, offsets, means):
    """Squared distance of every permuted row from its cluster's mean.

    Section 4's bound on the map error carries a residual proportional to the
    clustering error of the queries, delta_q^2 (Section 5.3, Fig. 6b, plots it
    against C_q); its definition did not survive extraction. Reading: the
    per-row spread ||x_i - xbar_c(i)||^2, whose mean over the rows is the
    k-means objective per row (reported as delta_q^2) and whose maximum is
    reported beside it.
    """
    xp = np.asarray(xp, dtype=np.float64)
    mu = np.asarray(means, dtype=np.float64)
    n = np.diff(np.asarray(offsets))
    kappa = np.repeat(np.arange(n.size), n)
    return ((xp - mu[kappa]) ** 2).sum(axis=1)


# ----------------------------------------------------------------------------
# the whole path for one head
# ----------------------------------------------------------------------------
class RoutedResult(dict):
    """Every intermediate of one head's routed path, keyed by name."""

    __getattr__ = dict.__getitem__


def routed_attention_head(q, k, v, cq: int, ck: int, budget_keys: int, iters: int,
                          init_q, init_k, scale: float, operand: str = "f64",
                          labels_q=None, labels_k=None, routing: str = "cluster",
                          value_aware: bool = False) -> RoutedResult:
    """cluster -> permute -> probe -> route -> attend -> unpermute for one head.

    ``labels_q``/``labels_k`` replace the k-means step when given (parity
    "given the same cluster assignment"). ``routing="global"`` takes
    ``budget_keys`` as the head's budget of exact entries (``route_global``);
    ``value_aware=True`` ranks blocks with ``probe_values``.
    """
    if labels_q is None:
        labels_q, _, _ = kmeans(q, init_q, iters, operand)
    if labels_k is None:
        labels_k, _, _ = kmeans(k, init_k, iters, operand)
    perm_q, q_off = permute(labels_q, cq)
    perm_k, k_off = permute(labels_k, ck)
    qp, kp, vp = gather(q, perm_q), gather(k, perm_k), gather(v, perm_k)
    q_bar = segment_means(qp, q_off)
    k_bar = segment_means(kp, k_off)
    v_bar = segment_means(vp, k_off)
    if value_aware:
        ratio, log_norm = probe_values(q_bar, kp, k_bar, vp, v_bar, k_off, scale)
    else:
        ratio, log_norm = probe(q_bar, kp, k_bar, k_off, scale)
    if routing == "global":
        mask, lst, cnt, keys, _ = route_global(ratio, q_off, k_off, budget_keys)
    else:
        mask, lst, cnt, keys = route(ratio, k_off, budget_keys, q_offsets=q_off)
    op = attend(qp, kp, vp, q_off, k_off, k_bar, v_bar, mask, scale)
    o = unpermute(op, perm_q)
    return RoutedResult(labels_q=labels_q, labels_k=labels_k, perm_q=perm_q, perm_k=perm_k,
                        q_off=q_off, k_off=k_off, q_bar=q_bar, k_bar=k_bar, v_bar=v_bar,
                        ratio=ratio, log_norm=log_norm, sel_mask=mask, sel_list=lst,
                        sel_count=cnt, sel_keys=keys, op=op, o=o)
