"""Shared checks of the GPU parity tests (host side: they compare arrays the
GPU produced with the CPU oracle's; nothing here launches work)."""
import math

import numpy as np
import torch

from oracle import svgear_oracle as O
from probe_bound import ratio_error_bound, selection_flips


def f64(t):
    """A tensor as NumPy: integers as they are, floating point as float64."""
    if t.dtype in (torch.int32, torch.uint8, torch.int64):
        return t.detach().cpu().numpy()
    return t.detach().float().cpu().double().numpy()


def tol_out(wl):
    """Output tolerance (relative Frobenius, max-abs): bf16 inputs with f32
    accumulation, or f32 inputs."""
    return (1e-2, 2e-2) if wl.dtype == "bf16" else (1e-4, 1e-4)


def operand(wl):
    return "bf16" if wl.dtype == "bf16" else "f32"


def rel_fro(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def assert_nearest(x, mu, labels, op):
    """Every label is a nearest centroid up to the f32 accumulation bound,
    with the centroids rounded to the kernel's operand precision. Returns the
    number of rows whose label differs from the float64 argmin (near-ties)."""
    m = O.round_operand(mu, op)
    m2 = (m * m).sum(1)
    flips = 0
    step = 8192
    for a in range(0, x.shape[0], step):
        xb = x[a:a + step]
        dist = m2[None, :] - 2.0 * (xb @ m.T)
        best = dist.min(axis=1)
        got = dist[np.arange(xb.shape[0]), labels[a:a + step]]
        scale = m2.max() + 2 * np.linalg.norm(xb, axis=1) * np.sqrt(m2.max())
        slack = 1e-5 * scale
        assert np.all(got - best <= slack), float(np.max(got - best - slack))
        flips += int(np.sum(labels[a:a + step] != np.argmin(dist, axis=1)))
    return flips


def check_whole_head(tag, wl, q, k, v, res, h, max_flip_frac):
    """The oracle's whole path on head h given the GPU's labels against the
    GPU's: selections may differ only through ratios the probe's error bound
    cannot separate (counted and printed), and the output of every query
    cluster that routes like the oracle matches the oracle's output."""
    rt, at = tol_out(wl)
    scale = 1 / math.sqrt(wl.d)
    ref = O.routed_attention_head(
        f64(q[h]), f64(k[h]), f64(v[h]), wl.cq, wl.ck, wl.budget, wl.iters, None, None, scale,
        labels_q=f64(res["labels_q"][h]), labels_k=f64(res["labels_k"][h]))
    gmask = f64(res["sel_mask"][h])
    # the bound covers the GPU's f32 segment means against the oracle's float64 ones
    bound = ratio_error_bound(f64(res["q_bar"][h]), f64(res["kp"][h]), f64(res["k_bar"][h]),
                              ref.k_off, scale, operand(wl), mean_tol=2e-6)
    fl = selection_flips(ref.ratio, f64(res["ratio"][h]), bound, ref.k_off, ref.sel_mask, gmask,
                         ref.q_off)
    qn = np.diff(ref.q_off).astype(np.float64)
    kn = np.diff(ref.k_off).astype(np.float64)
    dens_ref = float((qn[:, None] * ref.sel_mask * kn[None, :]).sum()) / (wl.n * wl.n)
    dens_gpu = float((qn[:, None] * gmask * kn[None, :]).sum()) / (wl.n * wl.n)
    print(f"[parity] whole path {tag} head {h}: {fl['flipped']} of {fl['live']} query clusters "
          f"route differently (first parting gap {fl['max_rel_gap']:.3g} relative, "
          f"{fl['max_gap_over_bound']:.3g} of the bound); exact-entry density "
          f"gpu {dens_gpu:.6f} oracle {dens_ref:.6f}", flush=True)
    assert fl["separated_ok"], "a selection differs where the bound separates the ratios"
    assert fl["flipped"] <= int(max_flip_frac * fl["live"]), fl
    same = np.all(ref.sel_mask == gmask, axis=1)
    got = f64(res["o"][h])
    rows = np.zeros(got.shape[0], dtype=bool)
    for cc in np.nonzero(same)[0]:
        rows[ref.perm_q[ref.q_off[cc]:ref.q_off[cc + 1]]] = True
    assert rel_fro(got[rows], ref.o[rows]) <= rt
    assert np.max(np.abs(got[rows] - ref.o[rows])) <= at
    return fl


