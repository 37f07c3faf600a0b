"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function include/svgear.h declares, and
reject bad arguments synchronously with the documented status codes before
it touches the device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svgear.h")


@pytest.fixture(scope="module")
def L():
    from sparse_attention_video_means_amd import svgear
    if not os.path.exists(svgear.LIB_PATH):
        from sparse_attention_video_means_amd import build
        build.build()
    return svgear.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svgear_[a-z_]+)\s*\(", text)))


def test_header_declares_the_six_calls():
    names = declared_functions()
    for call in ("cluster", "permute", "probe", "route", "attend", "unpermute"):
        assert f"svgear_{call}" in names


def test_every_declared_symbol_is_exported(L):
    from sparse_attention_video_means_amd import svgear
    names = declared_functions()
    assert set(names) == set(svgear.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.svgear_status_string(0) == b"ok"
    assert L.svgear_status_string(3) == b"workspace too small"
    assert L.svgear_status_string(99) == b"unknown status"


def test_workspace_queries(L):
    a = L.svgear_cluster_workspace(1, 40, 75600, 128, 500)
    b = L.svgear_cluster_workspace(1, 40, 75600, 128, 100)
    assert a > b > 0
    assert L.svgear_cluster_workspace(1, 1, 10, 128, 11) == 0      # C > N
    assert L.svgear_cluster_workspace(1, 1, 2000, 96, 10) == 0     # d not built
    assert L.svgear_cluster_workspace(1, 1, 5000, 128, 1025) == 0  # C > 1024
    assert L.svgear_permute_workspace(1, 8, 16384, 128, 500) > 0
    assert L.svgear_probe_workspace(40, 75600, 100, 500) > 0
    assert L.svgear_probe_workspace(1, 100, 10, 200) == 0          # Ck > Nk


def test_argument_errors_return_before_any_launch(L):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    null = None
    # null input
    assert L.svgear_cluster(1, 1, 100, 64, 4, 1, null, fake, fake, fake, fake, 1 << 30, null) == 1
    # iters < 1
    assert L.svgear_cluster(1, 1, 100, 64, 4, 0, fake, fake, fake, fake, fake, 1 << 30, null) == 1
    # unsupported head dim / dtype
    assert L.svgear_cluster(1, 1, 100, 80, 4, 1, fake, fake, fake, fake, fake, 1 << 30, null) == 2
    assert L.svgear_cluster(7, 1, 100, 64, 4, 1, fake, fake, fake, fake, fake, 1 << 30, null) == 2
    # workspace too small
    assert L.svgear_cluster(1, 1, 100, 64, 4, 1, fake, fake, fake, fake, fake, 16, null) == 3
    # permute: src aliases dst
    arr = (ctypes.c_void_p * 1)(0x1000)
    assert L.svgear_permute(1, 1, 100, 64, 4, fake, fake, fake, 1, arr, arr, None, fake,
                            1 << 30, null) == 1
    assert L.svgear_permute(1, 1, 100, 64, 4, fake, fake, fake, 3, arr, arr, None, fake,
                            1 << 30, null) == 1
    # probe: scale must be positive
    assert L.svgear_probe(1, 1, 100, 64, 4, 4, 0.0, fake, fake, fake, fake, fake, null, fake,
                          1 << 30, null) == 1
    # route: negative budget, Ck too large
    assert L.svgear_route(1, 4, 4, fake, fake, fake, -1, fake, null, null, null, null, 0,
                          null) == 1
    assert L.svgear_route(1, 4, 2000, fake, null, fake, 5, fake, null, null, null, null, 0,
                          null) == 1
    assert L.svgear_route(1, 4, 4, fake, fake, null, 5, fake, null, null, null, null, 0,
                          null) == 1
    assert L.svgear_route_workspace(40, 100, 500) == 0
    # fused cluster + permute: three tensors, aliasing, short workspace
    two = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.svgear_cluster_permute(1, 1, 100, 64, 4, 2, 3, two, two, None, fake, fake, fake,
                                    fake, fake, fake, 1 << 30, null) == 1
    assert L.svgear_cluster_permute(1, 1, 100, 64, 4, 2, 2, two, two, None, fake, fake, fake,
                                    fake, fake, fake, 1 << 30, null) == 1
    out2 = (ctypes.c_void_p * 2)(0x3000, 0x4000)
    assert L.svgear_cluster_permute(1, 1, 100, 64, 4, 2, 2, two, out2, None, fake, fake, fake,
                                    fake, fake, fake, 16, null) == 3
    assert L.svgear_cluster_permute_workspace(1, 40, 75600, 128, 500) > \
        L.svgear_cluster_workspace(1, 40, 75600, 128, 500)
    # value-aware probe: missing values, short workspace
    assert L.svgear_probe_values(1, 1, 100, 64, 4, 4, 0.1, fake, fake, fake, null, fake, fake,
                                 fake, null, fake, 1 << 30, null) == 1
    assert L.svgear_probe_values_workspace(40, 75600, 100, 500) > \
        L.svgear_probe_workspace(40, 75600, 100, 500)
    assert L.svgear_probe_values(1, 1, 100, 64, 4, 4, 0.1, fake, fake, fake, fake, fake, fake,
                                 fake, null, fake, 16, null) == 3
    # clock probe: block and round counts out of range, null output
    assert L.svgear_clock_probe(0, 10, fake, null) == 1
    assert L.svgear_clock_probe(8, 0, fake, null) == 1
    assert L.svgear_clock_probe((1 << 20) + 1, 10, fake, null) == 1
    assert L.svgear_clock_probe(8, 10, null, null) == 1
    assert L.svgear_realtime_khz(null) == 1
    # analysis: bad head dimension, short workspace, null output
    assert L.svgear_row_spread(1, 1, 100, 64, 4, fake, fake, fake, null, null) == 1
    assert L.svgear_block_scores(1, 96, 4, 4, 0.1, fake, fake, fake, fake, null) == 1
    assert L.svgear_map_error_workspace(2, 1000, 50) == 2 * 1000 * 50 * 4
    assert L.svgear_map_error(1, 1, 100, 100, 64, 4, 4, 0.1, fake, fake, fake, fake, fake, fake,
                              1, fake, fake, fake, fake, 16, null) == 3
    # global route: negative budget, Cq too large, short workspace
    assert L.svgear_route_global(1, 4, 4, fake, fake, fake, -1, fake, null, null, null, null,
                                 fake, 1 << 30, null) == 1
    assert L.svgear_route_global(1, 2000, 4, fake, fake, fake, 5, fake, null, null, null, null,
                                 fake, 1 << 30, null) == 1
    assert L.svgear_route_global(1, 4, 4, fake, null, fake, 5, fake, null, null, null, null,
                                 fake, 1 << 30, null) == 1
    # keys and indices, double-buffered, the sorted costs (int64), every
    # block's sorted position, the per-tile digit counts (256 digits x 25 tiles
    # of 2048 blocks) and the per-tile cost sums and minima
    wsg = L.svgear_route_global_workspace(2, 100, 500)
    need = 2 * 100 * 500 * 28 + 2 * 25 * 256 * 4
    assert need <= wsg <= need + 4096
    assert L.svgear_route_global_workspace(2, 100, 1025) == 0
    assert L.svgear_route_global(1, 4, 4, fake, fake, fake, 5, fake, null, null, null, null,
                                 fake, 16, null) == 3
    # attend: C > N on the key side
    assert L.svgear_attend(1, 1, 100, 10, 64, 4, 11, 0.1, fake, fake, fake, fake, fake, fake,
                           fake, fake, fake, fake, 1 << 30, null) == 1
    # attend: bf16 needs a workspace for the rounded centroid rows
    assert L.svgear_attend_workspace(1, 2, 50, 128) > 0
    assert L.svgear_attend_workspace(0, 2, 50, 128) == 0
    assert L.svgear_attend(1, 1, 100, 100, 64, 4, 11, 0.1, fake, fake, fake, fake, fake, fake,
                           fake, fake, fake, null, 0, null) == 3
    # attend with the unpermutation: q_perm required, O must not alias Qp, and the
    # same workspace rule as attend
    other = ctypes.c_void_p(fake.value + 4096)
    assert L.svgear_attend_unpermute(1, 1, 100, 100, 64, 4, 11, 0.1, fake, fake, fake, fake,
                                     fake, fake, fake, fake, null, other, fake, 1 << 30,
                                     null) == 1
    assert L.svgear_attend_unpermute(1, 1, 100, 100, 64, 4, 11, 0.1, fake, fake, fake, fake,
                                     fake, fake, fake, fake, fake, fake, fake, 1 << 30,
                                     null) == 1
    assert L.svgear_attend_unpermute(1, 1, 100, 100, 64, 4, 11, 0.1, fake, fake, fake, fake,
                                     fake, fake, fake, fake, fake, other, null, 0, null) == 3
    # unpermute: aliasing
    assert L.svgear_unpermute(1, 1, 100, 64, fake, fake, fake, null) == 1
    # allocation-free attend: q_perm required, O must not alias Qp, and a
    # problem whose rounded centroid rows exceed the fixed scratch is refused
    assert L.svgear_attend_unpermute_noalloc(1, 1, 100, 100, 64, 4, 11, 0.1, fake, fake, fake,
                                             fake, fake, fake, fake, fake, null, other,
                                             null) == 1
    assert L.svgear_attend_unpermute_noalloc(1, 1, 100, 100, 64, 4, 11, 0.1, fake, fake, fake,
                                             fake, fake, fake, fake, fake, fake, fake,
                                             null) == 1
    assert L.svgear_attend_unpermute_noalloc(1, 80, 4096, 4096, 128, 8, 1024, 0.1, fake, fake,
                                             fake, fake, fake, fake, fake, fake, fake, other,
                                             null) == 3


def _gpu_present():
    import torch
    return torch.cuda.is_available()


def test_valid_calls_without_a_gfx950_device_are_refused(L):
    """With arguments that pass validation, a call on a machine without a
    gfx950 device returns SVGEAR_ERR_UNSUPPORTED instead of launching."""
    if _gpu_present():
        pytest.skip("a GPU is present: these fake pointers must not reach a launch")
    fake = ctypes.c_void_p(0x1000)
    other = ctypes.c_void_p(0x2000)
    null = None
    assert L.svgear_route(1, 4, 4, fake, null, fake, 5, fake, null, null, null, null, 0,
                          null) == 2
    assert L.svgear_unpermute(1, 1, 100, 64, fake, fake, other, null) == 2
    assert L.svgear_block_scores(1, 64, 4, 4, 0.1, fake, fake, fake, fake, null) == 2
    assert L.svgear_status_string(2) == b"unsupported dtype, head dimension or device"


def test_routed_attention_checks_its_inputs_before_any_launch():
    """RoutedAttention passes raw pointers of q, k, v and the initial tables to
    the library, so it must refuse any tensor whose dtype, shape, layout or
    device differs from what it was built for (the kernels would otherwise read
    past the buffers)."""
    import torch

    from sparse_attention_video_means_amd import svgear
    H, N, d, cq, ck = 2, 64, 64, 4, 8
    ra = svgear.RoutedAttention(H, N, d, cq, ck, budget=16, iters=2, dtype=torch.bfloat16,
                                device="cpu")
    good = dict(q=torch.zeros(H, N, d, dtype=torch.bfloat16),
                k=torch.zeros(H, N, d, dtype=torch.bfloat16),
                v=torch.zeros(H, N, d, dtype=torch.bfloat16),
                init_q=torch.zeros(H, cq, d), init_k=torch.zeros(H, ck, d))
    ra.check_inputs(**good)   # matches: no error
    bad = {
        "q": torch.zeros(H, N, d),                                    # f32 for a bf16 object
        "k": torch.zeros(H, N - 1, d, dtype=torch.bfloat16),         # shorter N
        "v": torch.zeros(H, d, N, dtype=torch.bfloat16).transpose(1, 2),  # transposed view
        "init_q": torch.zeros(H, cq + 1, d),                          # wrong cluster count
        "init_k": torch.zeros(H, ck, d, dtype=torch.float64),         # wrong table dtype
    }
    for name, t in bad.items():
        args = dict(good, **{name: t})
        with pytest.raises((TypeError, ValueError), match=name):
            ra(**args)
    if not _gpu_present():
        return
    with pytest.raises(ValueError, match="q"):
        ra.check_inputs(**dict(good, q=good["q"].cuda()))   # another device


def test_header_compiles_as_c_and_the_library_links_from_c(tmp_path):
    """include/svgear.h is a C header: a C99 program (-Wall -Wextra -pedantic
    -Werror) includes it, links libsvgear.so and calls it (host side only)."""
    import shutil
    import subprocess
    from sparse_attention_video_means_amd import svgear
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if os.environ.get("SVGEAR_LIB"):
        # another build of the library (the sanitizer-instrumented one needs
        # its runtime to link a program): this check is about the header
        pytest.skip("SVGEAR_LIB names another build")
    if not os.path.exists(svgear.LIB_PATH):
        from sparse_attention_video_means_amd import build
        build.build()
    exe = str(tmp_path / "abi_from_c")
    libdir = os.path.dirname(svgear.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c_abi", "abi_from_c.c"), "-o", exe,
                        svgear.LIB_PATH, "-Wl,-rpath," + libdir],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0 and "abi from C: ok" in r.stdout, r.stdout
