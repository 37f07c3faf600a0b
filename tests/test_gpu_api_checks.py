"""The Python binding refuses a caller's workspace or output tensor that the
kernels would write outside of (wrong dtype, shape or device), before any
launch (needs a GPU: the inputs have to pass their own device checks first).
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def sv():
    from sparse_attention_video_means_amd import svgear
    return svgear


def _inputs(H=2, N=300, d=64, C=5):
    g = torch.Generator().manual_seed(7)
    x = torch.randn(H, N, d, generator=g).to(torch.bfloat16).to(DEV)
    cen = x[:, :C].float().contiguous()
    return x, cen


def test_workspace_of_the_wrong_kind_is_refused():
    S = sv()
    x, cen = _inputs()
    for bad in (torch.empty(1 << 20, dtype=torch.int32, device=DEV),   # not bytes
                torch.empty(1 << 20, dtype=torch.uint8),                # host memory
                torch.empty(2, 1 << 20, dtype=torch.uint8, device=DEV)[:, ::2]):  # strided
        with pytest.raises((TypeError, ValueError), match="ws"):
            S.svgear_cluster(x, cen.clone(), 2, ws=bad)
        with pytest.raises((TypeError, ValueError), match="ws"):
            S.svgear_cluster_permute([x], cen.clone(), 2, ws=bad)


def test_a_good_workspace_is_used_and_a_small_one_replaced():
    S = sv()
    x, cen = _inputs()
    ref_labels, ref_counts = S.svgear_cluster(x, cen.clone(), 2)
    L = S.lib()
    n = L.svgear_cluster_workspace(S.BF16, x.shape[0], x.shape[1], x.shape[2], cen.shape[1])
    for ws in (torch.empty(n, dtype=torch.uint8, device=DEV),
               torch.empty(max(n // 2, 1), dtype=torch.uint8, device=DEV)):
        labels, counts = S.svgear_cluster(x, cen.clone(), 2, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(labels, ref_labels) and torch.equal(counts, ref_counts)


def test_unpermute_output_of_the_wrong_shape_is_refused():
    S = sv()
    x, cen = _inputs()
    labels, _ = S.svgear_cluster(x, cen.clone(), 1)
    perm, _, (xp,), _ = S.svgear_permute(labels, cen.shape[1], [x], with_means=False)
    with pytest.raises(ValueError, match="out"):
        S.svgear_unpermute(xp, perm, out=torch.empty(x.shape[0], x.shape[1] - 1, x.shape[2],
                                                     dtype=x.dtype, device=DEV))
    with pytest.raises(TypeError, match="out"):
        S.svgear_unpermute(xp, perm, out=torch.empty(x.shape, dtype=torch.float32, device=DEV))
    back = S.svgear_unpermute(xp, perm, out=torch.empty_like(x))
    torch.cuda.synchronize()
    assert torch.equal(back, x)


def test_optional_outputs_may_be_null():
    """svgear_route's list, count and keys and svgear_probe's log normalisers
    are optional: with NULL for them the required outputs are bitwise what a
    call that asks for everything writes."""
    import ctypes
    import math

    from sparse_attention_video_means_amd import synth
    S = sv()
    wl = synth.WORKLOADS["tiny"]
    q, k, v = synth.make_qkv(wl)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    scale = 1 / math.sqrt(wl.d)
    res = S.routed_attention(q.to(DEV), k.to(DEV), v.to(DEV), wl.cq, wl.ck, wl.budget, wl.iters,
                             iq.to(DEV), ik.to(DEV), scale)
    L, s, p = S.lib(), S._stream(), S._ptr
    H, Cq, Ck = res["ratio"].shape
    mask = torch.empty_like(res["sel_mask"])
    S._check("svgear_route", L.svgear_route(H, Cq, Ck, p(res["ratio"]), p(res["q_off"]),
                                            p(res["k_off"]), int(wl.budget), p(mask), None,
                                            None, None, None, 0, s))
    kp, Nk = res["kp"], res["kp"].shape[1]
    ratio = torch.empty_like(res["ratio"])
    ws = S._ws(L.svgear_probe_workspace(H, Nk, Cq, Ck), kp.device)
    S._check("svgear_probe", L.svgear_probe(S._dt(kp), H, Nk, wl.d, Cq, Ck, ctypes.c_float(scale),
                                            p(res["q_bar"]), p(kp), p(res["k_bar"]),
                                            p(res["k_off"]), p(ratio), None, p(ws), ws.numel(),
                                            s))
    torch.cuda.synchronize()
    assert torch.equal(mask, res["sel_mask"])
    assert torch.equal(ratio, res["ratio"])
