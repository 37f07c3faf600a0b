"""svgear_cluster_permute against svgear_cluster followed by svgear_permute
(needs an MI355X).

The fused call runs the same kernels in the same order, its last Lloyd pass
writing the permuted copies and means, so every output must be bitwise what
the two separate calls give: labels, counts, centroids, permutation, offsets,
permuted tensors and segment means. Cases: f32 and bf16, d 64 and 128, one
and two tensors, a ragged tail, one cluster, one Lloyd iteration, and as many
clusters as the kernels allow (1024). A second test checks that Lloyd
iterations chain exactly through the centroids.
"""
import pytest
import torch

from sparse_attention_video_means_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    "tiny_f32_one_tensor": (synth.WORKLOADS["tiny"], 1),
    "blobs_bf16_two_tensors": (synth.WORKLOADS["slice"].with_(heads=2, n=3001, cq=24, ck=70,
                                                              iters=5, centres=64), 2),
    "d64_bf16_two_tensors": (synth.WORKLOADS["slice"].with_(heads=1, n=2050, d=64, ck=40,
                                                            iters=4, centres=32), 2),
    "one_cluster": (synth.WORKLOADS["slice"].with_(heads=1, n=1000, ck=1, iters=3), 2),
    "one_iteration": (synth.WORKLOADS["slice"].with_(heads=2, n=1500, ck=30, iters=1), 1),
    "max_clusters": (synth.WORKLOADS["slice"].with_(heads=1, n=5000, ck=1024, iters=2), 2),
}


def sv():
    from sparse_attention_video_means_amd import svgear
    return svgear


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_separate_calls(name):
    wl, nt = CASES[name]
    S = sv()
    q, k, v = synth.make_qkv(wl)
    init = synth.kmeans_init(k, wl.ck, wl.seed, 1).to(DEV)
    tensors = [k.to(DEV), v.to(DEV)][:nt]
    print(f"[cluster_permute] {name}: H={wl.heads} N={wl.n} d={wl.d} C={wl.ck} "
          f"iters={wl.iters} tensors={nt}", flush=True)
    c1 = init.clone()
    labels, counts = S.svgear_cluster(tensors[0], c1, wl.iters)
    perm, off, outs, means = S.svgear_permute(labels, wl.ck, tensors)
    c2 = init.clone()
    labels2, counts2, perm2, off2, outs2, means2 = S.svgear_cluster_permute(tensors, c2, wl.iters)
    torch.cuda.synchronize()
    for a, b in [(labels, labels2), (counts, counts2), (c1, c2), (perm, perm2), (off, off2)] + \
            list(zip(outs, outs2)) + list(zip(means, means2)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["blobs_bf16_two_tensors", "d64_bf16_two_tensors",
                                  "tiny_f32_one_tensor", "max_clusters"])
def test_iterations_chain_exactly(name):
    # Lloyd iteration T of one call equals a fresh one-iteration call started
    # from the centroids that T - 1 iterations left: the centroids, their
    # rounded distance table and the assignment carry nothing else between
    # iterations.
    wl, _ = CASES[name]
    S = sv()
    _, k, _ = synth.make_qkv(wl)
    x = k.to(DEV)
    init = synth.kmeans_init(k, wl.ck, wl.seed, 1).to(DEV)
    iters = max(wl.iters, 3)
    print(f"[cluster_permute] iteration chain {name}: iters={iters}", flush=True)
    c_t = init.clone()
    labels_t, counts_t = S.svgear_cluster(x, c_t, iters)
    c_prev = init.clone()
    S.svgear_cluster(x, c_prev, iters - 1)
    labels_1, counts_1 = S.svgear_cluster(x, c_prev, 1)
    torch.cuda.synchronize()
    assert torch.equal(labels_t, labels_1)
    assert torch.equal(counts_t, counts_1)
    assert torch.equal(c_t, c_prev)
