"""The allocation-free attention entry point against the one that takes a
workspace (needs an MI355X; through the C ABI).

svgear_attend_unpermute_noalloc keeps its scratch in the library's own
device array instead of a caller workspace. On the same inputs it must write
bitwise what svgear_attend_unpermute writes, on two calls in a row (the
second with a smaller problem, so stale contents of the shared array from the
first call would show), for bf16 and f32 inputs.
"""
import ctypes
import math

import pytest
import torch

from sparse_attention_video_means_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    ("bf16 2x3001 Cq=24 Ck=70", synth.WORKLOADS["slice"].with_(name="na_big", heads=2, n=3001,
                                                             cq=24, ck=70, iters=3, centres=48)),
    ("bf16 1x1500 Cq=10 Ck=30", synth.WORKLOADS["slice"].with_(name="na_small", heads=1, n=1500,
                                                             cq=10, ck=30, iters=3, centres=24,
                                                             seed=3)),
    ("f32 1x1200 d=64 Cq=8 Ck=20", synth.WORKLOADS["tiny"].with_(name="na_f32", n=1200, cq=8,
                                                                ck=20, iters=3)),
]


def prepared(wl):
    from sparse_attention_video_means_amd import svgear
    q, k, v = synth.make_qkv(wl)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    return svgear.routed_attention(q.to(DEV), k.to(DEV), v.to(DEV), wl.cq, wl.ck, wl.budget,
                                   wl.iters, iq.to(DEV), ik.to(DEV), 1 / math.sqrt(wl.d))


def call_noalloc(res, scale, out):
    """Through the C ABI: every argument a pointer or a size."""
    from sparse_attention_video_means_amd import svgear
    L = svgear.lib()
    qp = res["qp"]
    H, Nq, d = qp.shape
    Nk = res["kp"].shape[1]
    Cq, Ck = res["q_off"].shape[1] - 1, res["k_off"].shape[1] - 1
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    dt = 1 if qp.dtype == torch.bfloat16 else 0
    return L.svgear_attend_unpermute_noalloc(
        dt, H, Nq, Nk, d, Cq, Ck, float(scale), p(qp), p(res["kp"]), p(res["vp"]),
        p(res["q_off"]), p(res["k_off"]), p(res["k_bar"]), p(res["v_bar"]), p(res["sel_mask"]),
        p(res["perm_q"]), p(out), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    from sparse_attention_video_means_amd import svgear
    runs = []
    for name, wl in CASES:
        print(f"[noalloc] preparing {name}", flush=True)
        res = prepared(wl)
        scale = 1 / math.sqrt(wl.d)
        want = svgear.svgear_attend_unpermute(res["qp"], res["kp"], res["vp"], res["q_off"],
                                              res["k_off"], res["k_bar"], res["v_bar"],
                                              res["sel_mask"], res["perm_q"], scale)
        runs.append((name, res, scale, want))
    torch.cuda.synchronize()
    # consecutive calls, largest first: each must equal its own reference
    for rnd in range(2):
        for name, res, scale, want in runs:
            out = torch.full_like(want, 7.0)
            print(f"[noalloc] call {rnd}: {name}", flush=True)
            assert call_noalloc(res, scale, out) == 0
            torch.cuda.synchronize()
            assert torch.equal(out, want), name


def test_noalloc_rejects_sizes_beyond_its_scratch():
    from sparse_attention_video_means_amd import svgear
    L = svgear.lib()
    fake = ctypes.c_void_p(0x1000)
    other = ctypes.c_void_p(0x2000)
    # bf16, 80 heads x 1024 key clusters x d=128: rounded centroid rows need
    # 2 x 20 MiB, more than the 32 MiB array: refused before any launch
    assert L.svgear_attend_unpermute_noalloc(1, 80, 4096, 4096, 128, 8, 1024, 0.1, fake, fake,
                                             fake, fake, fake, fake, fake, fake, fake, other,
                                             None) == 3
