"""Thin Python binding of libsvgear (ctypes).

Each function takes torch tensors that live on the GPU, checks their dtype,
shape and layout, allocates the outputs and the workspace with torch (torch
is only the allocator and the stream provider here) and calls the C entry
point of the same name on the current HIP stream. All arithmetic happens in
the HIP kernels of libsvgear.so; if the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SVGEAR_LIB names another build of the same library (the host-sanitizer build
# that the ABI tests load); by default the in-tree libsvgear.so.
LIB_PATH = os.environ.get("SVGEAR_LIB") or os.path.join(_HERE, "libsvgear.so")

F32, BF16 = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported dtype, head dimension or device",
          3: "workspace too small", 4: "HIP launch failure"}

_lib = None


class SvgearError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} (status {code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_attention_video_means_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        sig = {
            "svgear_status_string": (ctypes.c_char_p, [i32]),
            "svgear_cluster_workspace": (sz, [i32, i32, i32, i32, i32]),
            "svgear_cluster": (i32, [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "svgear_permute_workspace": (sz, [i32, i32, i32, i32, i32]),
            "svgear_cluster_permute_workspace": (sz, [i32, i32, i32, i32, i32]),
            "svgear_cluster_permute": (i32, [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                             vp, vp, vp, vp, vp, sz, vp]),
            "svgear_permute": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp, sz,
                                     vp]),
            "svgear_probe_workspace": (sz, [i32, i32, i32, i32]),
            "svgear_probe": (i32, [i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp,
                                   sz, vp]),
            "svgear_probe_values_workspace": (sz, [i32, i32, i32, i32]),
            "svgear_probe_values": (i32, [i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, sz, vp]),
            "svgear_route_workspace": (sz, [i32, i32, i32]),
            "svgear_route": (i32, [i32, i32, i32, vp, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp,
                                   sz, vp]),
            "svgear_route_global_workspace": (sz, [i32, i32, i32]),
            "svgear_route_global": (i32, [i32, i32, i32, vp, vp, vp, ctypes.c_int64, vp, vp, vp,
                                          vp, vp, vp, sz, vp]),
            "svgear_attend_workspace": (sz, [i32, i32, i32, i32]),
            "svgear_attend": (i32, [i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp,
                                    vp, vp, vp, vp, sz, vp]),
            "svgear_attend_unpermute": (i32, [i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp,
                                              vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "svgear_attend_unpermute_noalloc": (i32, [i32, i32, i32, i32, i32, i32, i32, f32, vp,
                                                      vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "svgear_unpermute": (i32, [i32, i32, i32, i32, vp, vp, vp, vp]),
            "svgear_block_scores": (i32, [i32, i32, i32, i32, f32, vp, vp, vp, vp, vp]),
            "svgear_map_error_workspace": (sz, [i32, i32, i32]),
            "svgear_row_spread": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
            "svgear_clock_probe": (i32, [i32, i32, vp, vp]),
            "svgear_realtime_khz": (i32, [ctypes.POINTER(i32)]),
            "svgear_map_error": (i32, [i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp,
                                       vp, i32, vp, vp, vp, vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


EXPORTS = ("svgear_status_string", "svgear_cluster_workspace", "svgear_cluster",
           "svgear_permute_workspace", "svgear_permute", "svgear_cluster_permute_workspace",
           "svgear_cluster_permute", "svgear_probe_workspace", "svgear_probe",
           "svgear_probe_values_workspace", "svgear_probe_values",
           "svgear_route_workspace", "svgear_route", "svgear_route_global_workspace",
           "svgear_route_global",
           "svgear_attend_workspace", "svgear_attend", "svgear_attend_unpermute",
           "svgear_attend_unpermute_noalloc", "svgear_unpermute",
           "svgear_block_scores", "svgear_map_error_workspace", "svgear_map_error",
           "svgear_row_spread", "svgear_clock_probe", "svgear_realtime_khz")


def _check(fn: str, code: int):
    if code != 0:
        raise SvgearError(fn, code)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    """Checks a tensor argument before its pointer goes to the library: dtype,
    shape, a dense row-major layout, and the device (``device`` given: that
    device; otherwise any GPU)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None:
        if t.device != torch.device(device):
            raise ValueError(f"{name} must be on {device}, got {t.device}")
    elif not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _user_ws(ws, nbytes: int, device) -> torch.Tensor:
    """The caller's workspace, if one is given (a dense uint8 tensor on the
    call's device; replaced by a new one when smaller than ``nbytes``), else
    a new one."""
    if ws is None:
        return _ws(nbytes, device)
    _need(ws, "ws", torch.uint8, None, device)
    return ws if ws.numel() >= nbytes else _ws(nbytes, device)


# ----------------------------------------------------------------------------
def svgear_cluster(x: torch.Tensor, centroids: torch.Tensor, iters: int, ws=None):
    """k-means of every head's rows; ``centroids`` ([H, C, d] f32) is updated in
    place to the means of the final labels. Returns (labels [H, N], counts [H, C])."""
    _need(x, "x")
    H, N, d = x.shape
    C = centroids.shape[1]
    _need(centroids, "centroids", torch.float32, (H, C, d))
    labels = torch.empty((H, N), dtype=torch.int32, device=x.device)
    counts = torch.empty((H, C), dtype=torch.int32, device=x.device)
    L = lib()
    ws = _user_ws(ws, L.svgear_cluster_workspace(_dt(x), H, N, d, C), x.device)
    _check("svgear_cluster", L.svgear_cluster(_dt(x), H, N, d, C, int(iters), _ptr(x),
                                              _ptr(centroids), _ptr(labels), _ptr(counts),
                                              _ptr(ws), ws.numel(), _stream()))
    return labels, counts


def svgear_permute(labels: torch.Tensor, C: int, tensors, with_means: bool = True, ws=None):
    """Stable cluster-contiguous permutation of one or two tensors sharing
    ``labels``. Returns (perm, offsets, permuted tensors, means or None)."""
    tensors = list(tensors)
    x0 = tensors[0]
    for i, t in enumerate(tensors):
        _need(t, f"tensors[{i}]", x0.dtype, x0.shape)
    H, N, d = x0.shape
    _need(labels, "labels", torch.int32, (H, N))
    dev = x0.device
    perm = torch.empty((H, N), dtype=torch.int32, device=dev)
    offsets = torch.empty((H, C + 1), dtype=torch.int32, device=dev)
    outs = [torch.empty_like(t) for t in tensors]
    means = [torch.empty((H, C, d), dtype=torch.float32, device=dev) for _ in tensors] \
        if with_means else None
    nt = len(tensors)
    src = (ctypes.c_void_p * nt)(*[t.data_ptr() for t in tensors])
    dst = (ctypes.c_void_p * nt)(*[t.data_ptr() for t in outs])
    mp = (ctypes.c_void_p * nt)(*[m.data_ptr() for m in means]) if with_means else None
    L = lib()
    ws = _user_ws(ws, L.svgear_permute_workspace(_dt(x0), H, N, d, C), dev)
    _check("svgear_permute", L.svgear_permute(_dt(x0), H, N, d, C, _ptr(labels), _ptr(perm),
                                              _ptr(offsets), nt, src, dst, mp, _ptr(ws),
                                              ws.numel(), _stream()))
    return perm, offsets, outs, means


def svgear_cluster_permute(tensors, centroids: torch.Tensor, iters: int, with_means: bool = True,
                           ws=None):
    """k-means of ``tensors[0]`` and the stable permutation of every tensor by
    the final labels, in one call. ``centroids`` ([H, C, d] f32) is updated in
    place. Returns (labels, counts, perm, offsets, permuted tensors, means or None),
    bitwise what svgear_cluster followed by svgear_permute returns."""
    tensors = list(tensors)
    x0 = tensors[0]
    for i, t in enumerate(tensors):
        _need(t, f"tensors[{i}]", x0.dtype, x0.shape)
    H, N, d = x0.shape
    C = centroids.shape[1]
    _need(centroids, "centroids", torch.float32, (H, C, d))
    dev = x0.device
    e = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)
    labels, counts, perm, offsets = e(H, N), e(H, C), e(H, N), e(H, C + 1)
    outs = [torch.empty_like(t) for t in tensors]
    means = [torch.empty((H, C, d), dtype=torch.float32, device=dev) for _ in tensors] \
        if with_means else None
    nt = len(tensors)
    src = (ctypes.c_void_p * nt)(*[t.data_ptr() for t in tensors])
    dst = (ctypes.c_void_p * nt)(*[t.data_ptr() for t in outs])
    mp = (ctypes.c_void_p * nt)(*[m.data_ptr() for m in means]) if with_means else None
    L = lib()
    ws = _user_ws(ws, L.svgear_cluster_permute_workspace(_dt(x0), H, N, d, C), dev)
    _check("svgear_cluster_permute", L.svgear_cluster_permute(
        _dt(x0), H, N, d, C, int(iters), nt, src, dst, mp, _ptr(centroids), _ptr(labels),
        _ptr(counts), _ptr(perm), _ptr(offsets), _ptr(ws), ws.numel(), _stream()))
    return labels, counts, perm, offsets, outs, means


def svgear_probe(q_centroids, kp, k_centroids, k_offsets, scale: float, ws=None):
    """Block error-to-size ratios [H, Cq, Ck] and log normalisers [H, Cq]."""
    _need(kp, "kp")
    H, Nk, d = kp.shape
    Cq, Ck = q_centroids.shape[1], k_centroids.shape[1]
    _need(q_centroids, "q_centroids", torch.float32, (H, Cq, d))
    _need(k_centroids, "k_centroids", torch.float32, (H, Ck, d))
    _need(k_offsets, "k_offsets", torch.int32, (H, Ck + 1))
    ratio = torch.empty((H, Cq, Ck), dtype=torch.float32, device=kp.device)
    log_norm = torch.empty((H, Cq), dtype=torch.float32, device=kp.device)
    L = lib()
    ws = _user_ws(ws, L.svgear_probe_workspace(H, Nk, Cq, Ck), kp.device)
    _check("svgear_probe", L.svgear_probe(_dt(kp), H, Nk, d, Cq, Ck, float(scale),
                                          _ptr(q_centroids), _ptr(kp), _ptr(k_centroids),
                                          _ptr(k_offsets), _ptr(ratio), _ptr(log_norm), _ptr(ws),
                                          ws.numel(), _stream()))
    return ratio, log_norm


def svgear_probe_values(q_centroids, kp, k_centroids, vp, v_centroids, k_offsets, scale: float,
                        ws=None):
    """Value-aware block ratios [H, Cq, Ck] and log normalisers [H, Cq]."""
    _need(kp, "kp")
    H, Nk, d = kp.shape
    Cq, Ck = q_centroids.shape[1], k_centroids.shape[1]
    _need(q_centroids, "q_centroids", torch.float32, (H, Cq, d))
    _need(k_centroids, "k_centroids", torch.float32, (H, Ck, d))
    _need(vp, "vp", kp.dtype, (H, Nk, d))
    _need(v_centroids, "v_centroids", torch.float32, (H, Ck, d))
    _need(k_offsets, "k_offsets", torch.int32, (H, Ck + 1))
    ratio = torch.empty((H, Cq, Ck), dtype=torch.float32, device=kp.device)
    log_norm = torch.empty((H, Cq), dtype=torch.float32, device=kp.device)
    L = lib()
    ws = _user_ws(ws, L.svgear_probe_values_workspace(H, Nk, Cq, Ck), kp.device)
    _check("svgear_probe_values", L.svgear_probe_values(
        _dt(kp), H, Nk, d, Cq, Ck, float(scale), _ptr(q_centroids), _ptr(kp), _ptr(k_centroids),
        _ptr(vp), _ptr(v_centroids), _ptr(k_offsets), _ptr(ratio), _ptr(log_norm), _ptr(ws),
        ws.numel(), _stream()))
    return ratio, log_norm


def svgear_route(ratio, k_offsets, budget_keys: int, q_offsets=None):
    """Greedy selection per query cluster; with ``q_offsets`` ([H, Cq+1] int32)
    an empty query cluster selects nothing. Returns (mask u8 [H,Cq,Ck],
    list i32 [H,Cq,Ck], count [H,Cq], keys [H,Cq])."""
    _need(ratio, "ratio", torch.float32)
    H, Cq, Ck = ratio.shape
    _need(k_offsets, "k_offsets", torch.int32, (H, Ck + 1))
    if q_offsets is not None:
        _need(q_offsets, "q_offsets", torch.int32, (H, Cq + 1))
    dev = ratio.device
    mask = torch.empty((H, Cq, Ck), dtype=torch.uint8, device=dev)
    lst = torch.empty((H, Cq, Ck), dtype=torch.int32, device=dev)
    cnt = torch.empty((H, Cq), dtype=torch.int32, device=dev)
    keys = torch.empty((H, Cq), dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.svgear_route_workspace(H, Cq, Ck)
    ws = _ws(nbytes, dev) if nbytes > 0 else None
    _check("svgear_route", L.svgear_route(H, Cq, Ck, _ptr(ratio), _ptr(q_offsets),
                                          _ptr(k_offsets), int(budget_keys), _ptr(mask),
                                          _ptr(lst), _ptr(cnt), _ptr(keys), _ptr(ws),
                                          0 if ws is None else ws.numel(), _stream()))
    return mask, lst, cnt, keys


def svgear_route_global(ratio, q_offsets, k_offsets, budget_entries: int, ws=None):
    """Greedy selection under one budget of exact entries per head.

    Returns (mask u8 [H,Cq,Ck], list i32 [H,Cq,Ck], count [H,Cq], keys [H,Cq],
    used i64 [H])."""
    _need(ratio, "ratio", torch.float32)
    H, Cq, Ck = ratio.shape
    _need(q_offsets, "q_offsets", torch.int32, (H, Cq + 1))
    _need(k_offsets, "k_offsets", torch.int32, (H, Ck + 1))
    dev = ratio.device
    mask = torch.empty((H, Cq, Ck), dtype=torch.uint8, device=dev)
    lst = torch.empty((H, Cq, Ck), dtype=torch.int32, device=dev)
    cnt = torch.empty((H, Cq), dtype=torch.int32, device=dev)
    keys = torch.empty((H, Cq), dtype=torch.int32, device=dev)
    used = torch.empty((H,), dtype=torch.int64, device=dev)
    L = lib()
    ws = _user_ws(ws, L.svgear_route_global_workspace(H, Cq, Ck), dev)
    _check("svgear_route_global", L.svgear_route_global(
        H, Cq, Ck, _ptr(ratio), _ptr(q_offsets), _ptr(k_offsets), int(budget_entries),
        _ptr(mask), _ptr(lst), _ptr(cnt), _ptr(keys), _ptr(used), _ptr(ws), ws.numel(),
        _stream()))
    return mask, lst, cnt, keys, used


def svgear_attend(qp, kp, vp, q_offsets, k_offsets, k_centroids, v_centroids, sel_mask,
                  scale: float, out=None):
    """Compensated block-sparse attention on permuted tensors; returns O_p."""
    _need(qp, "qp")
    H, Nq, d = qp.shape
    Nk = kp.shape[1]
    Cq, Ck = q_offsets.shape[1] - 1, k_offsets.shape[1] - 1
    _need(kp, "kp", qp.dtype, (H, Nk, d))
    _need(vp, "vp", qp.dtype, (H, Nk, d))
    _need(q_offsets, "q_offsets", torch.int32, (H, Cq + 1))
    _need(k_offsets, "k_offsets", torch.int32, (H, Ck + 1))
    _need(k_centroids, "k_centroids", torch.float32, (H, Ck, d))
    _need(v_centroids, "v_centroids", torch.float32, (H, Ck, d))
    _need(sel_mask, "sel_mask", torch.uint8, (H, Cq, Ck))
    op = torch.empty_like(qp) if out is None else out
    _need(op, "out", qp.dtype, qp.shape, qp.device)
    L = lib()
    ws = _ws(L.svgear_attend_workspace(_dt(qp), H, Ck, d), qp.device)
    _check("svgear_attend", L.svgear_attend(_dt(qp), H, Nq, Nk, d, Cq, Ck, float(scale),
                                            _ptr(qp), _ptr(kp), _ptr(vp), _ptr(q_offsets),
                                            _ptr(k_offsets), _ptr(k_centroids),
                                            _ptr(v_centroids), _ptr(sel_mask), _ptr(op),
                                            _ptr(ws), ws.numel(), _stream()))
    return op


def svgear_attend_unpermute(qp, kp, vp, q_offsets, k_offsets, k_centroids, v_centroids,
                            sel_mask, q_perm, scale: float, out=None):
    """svgear_attend with every output row written at its query's original
    position (q_perm [H, Nq] int32, permuted row -> original row); returns O."""
    _need(qp, "qp")
    H, Nq, d = qp.shape
    Nk = kp.shape[1]
    Cq, Ck = q_offsets.shape[1] - 1, k_offsets.shape[1] - 1
    _need(kp, "kp", qp.dtype, (H, Nk, d))
    _need(vp, "vp", qp.dtype, (H, Nk, d))
    _need(q_offsets, "q_offsets", torch.int32, (H, Cq + 1))
    _need(k_offsets, "k_offsets", torch.int32, (H, Ck + 1))
    _need(k_centroids, "k_centroids", torch.float32, (H, Ck, d))
    _need(v_centroids, "v_centroids", torch.float32, (H, Ck, d))
    _need(sel_mask, "sel_mask", torch.uint8, (H, Cq, Ck))
    _need(q_perm, "q_perm", torch.int32, (H, Nq))
    o = torch.empty_like(qp) if out is None else out
    _need(o, "out", qp.dtype, qp.shape, qp.device)
    L = lib()
    ws = _ws(L.svgear_attend_workspace(_dt(qp), H, Ck, d), qp.device)
    _check("svgear_attend_unpermute", L.svgear_attend_unpermute(
        _dt(qp), H, Nq, Nk, d, Cq, Ck, float(scale), _ptr(qp), _ptr(kp), _ptr(vp),
        _ptr(q_offsets), _ptr(k_offsets), _ptr(k_centroids), _ptr(v_centroids), _ptr(sel_mask),
        _ptr(q_perm), _ptr(o), _ptr(ws), ws.numel(), _stream()))
    return o


def svgear_attend_unpermute_noalloc(qp, kp, vp, q_offsets, k_offsets, k_centroids, v_centroids,
                                    sel_mask, q_perm, scale: float, out):
    """svgear_attend_unpermute with the library's own scratch array instead of
    a workspace: nothing is allocated (``out`` is required). Calls that may
    overlap on one GPU race on that array."""
    _need(qp, "qp")
    H, Nq, d = qp.shape
    Nk = kp.shape[1]
    Cq, Ck = q_offsets.shape[1] - 1, k_offsets.shape[1] - 1
    _need(kp, "kp", qp.dtype, (H, Nk, d))
    _need(vp, "vp", qp.dtype, (H, Nk, d))
    _need(q_offsets, "q_offsets", torch.int32, (H, Cq + 1))
    _need(k_offsets, "k_offsets", torch.int32, (H, Ck + 1))
    _need(k_centroids, "k_centroids", torch.float32, (H, Ck, d))
    _need(v_centroids, "v_centroids", torch.float32, (H, Ck, d))
    _need(sel_mask, "sel_mask", torch.uint8, (H, Cq, Ck))
    _need(q_perm, "q_perm", torch.int32, (H, Nq))
    _need(out, "out", qp.dtype, qp.shape, qp.device)
    _check("svgear_attend_unpermute_noalloc", lib().svgear_attend_unpermute_noalloc(
        _dt(qp), H, Nq, Nk, d, Cq, Ck, float(scale), _ptr(qp), _ptr(kp), _ptr(vp),
        _ptr(q_offsets), _ptr(k_offsets), _ptr(k_centroids), _ptr(v_centroids), _ptr(sel_mask),
        _ptr(q_perm), _ptr(out), _stream()))
    return out


def svgear_unpermute(xp, perm, out=None):
    """X[perm[p]] = Xp[p] per head."""
    _need(xp, "xp")
    H, N, d = xp.shape
    _need(perm, "perm", torch.int32, (H, N))
    x = torch.empty_like(xp) if out is None else out
    _need(x, "out", xp.dtype, xp.shape, xp.device)
    _check("svgear_unpermute", lib().svgear_unpermute(_dt(xp), H, N, d, _ptr(perm), _ptr(xp),
                                                      _ptr(x), _stream()))
    return x


# ----------------------------------------------------------------------------
class RoutedAttention:
    """The whole path with every buffer allocated once, for repeated calls.

    Construct for fixed sizes; each call enqueues cluster + permute of Q,
    cluster + permute of K (with V), probe, route, attend and unpermute on the
    current stream and returns the output tensor (owned by this object).
    ``routing``, ``budget`` and ``probe`` are as in ``routed_attention``:
    exact keys per query cluster ("cluster") or exact entries per head
    ("global"); weight-gap ("weight") or value-aware ("value") block errors.
    With ``stage_events`` the call also records a HIP event pair around each
    stage (``last_stage_ms()`` reads them after a synchronisation).
    """

    # "attend" writes every output row at its query's original position (the
    # unpermutation runs in the attention kernel's epilogue)
    STAGES = ("cluster_permute_q", "cluster_permute_kv", "probe", "route", "attend")

    def __init__(self, H, N, d, cq, ck, budget, iters, dtype=torch.bfloat16, device="cuda",
                 nk=None, scale=None, routing="cluster", probe="weight"):
        if routing not in ("cluster", "global"):
            raise ValueError(f"routing must be 'cluster' or 'global', not {routing!r}")
        if probe not in ("weight", "value"):
            raise ValueError(f"probe must be 'weight' or 'value', not {probe!r}")
        self.routing, self.probe = routing, probe
        nq, nk = N, (N if nk is None else nk)
        self.H, self.nq, self.nk, self.d, self.cq, self.ck = H, nq, nk, d, cq, ck
        self.budget, self.iters = int(budget), int(iters)
        self.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        self.dt = BF16 if dtype == torch.bfloat16 else F32
        e = lambda *s, dt=torch.int32: torch.empty(s, dtype=dt, device=device)
        self.cen_q, self.cen_k = e(H, cq, d, dt=torch.float32), e(H, ck, d, dt=torch.float32)
        self.labels_q, self.labels_k = e(H, nq), e(H, nk)
        self.counts_q, self.counts_k = e(H, cq), e(H, ck)
        self.perm_q, self.perm_k = e(H, nq), e(H, nk)
        self.q_off, self.k_off = e(H, cq + 1), e(H, ck + 1)
        self.qp, self.kp, self.vp = e(H, nq, d, dt=dtype), e(H, nk, d, dt=dtype), e(H, nk, d, dt=dtype)
        self.q_bar = e(H, cq, d, dt=torch.float32)
        self.k_bar, self.v_bar = e(H, ck, d, dt=torch.float32), e(H, ck, d, dt=torch.float32)
        self.ratio, self.log_norm = e(H, cq, ck, dt=torch.float32), e(H, cq, dt=torch.float32)
        self.sel_mask = e(H, cq, ck, dt=torch.uint8)
        self.sel_list, self.sel_count, self.sel_keys = e(H, cq, ck), e(H, cq), e(H, cq)
        self.o = e(H, nq, d, dt=dtype)
        self.used_entries = e(H, dt=torch.int64)
        L = lib()
        wsz = max(L.svgear_route_global_workspace(H, cq, ck) if routing == "global" else 0,
                  L.svgear_cluster_permute_workspace(self.dt, H, nq, d, cq),
                  L.svgear_cluster_permute_workspace(self.dt, H, nk, d, ck),
                  L.svgear_probe_workspace(H, nk, cq, ck),
                  L.svgear_probe_values_workspace(H, nk, cq, ck) if probe == "value" else 0,
                  L.svgear_attend_workspace(self.dt, H, ck, d))
        self.ws = _ws(wsz, device)
        self._events = None

    def check_inputs(self, q, k, v, init_q, init_k):
        """Raises unless the inputs match the sizes, dtype and device this
        object was built for (the kernels read exactly those extents)."""
        H, nq, nk, d, cq, ck = self.H, self.nq, self.nk, self.d, self.cq, self.ck
        dev = self.o.device
        _need(q, "q", self.o.dtype, (H, nq, d), dev)
        _need(k, "k", self.o.dtype, (H, nk, d), dev)
        _need(v, "v", self.o.dtype, (H, nk, d), dev)
        _need(init_q, "init_q", torch.float32, (H, cq, d), dev)
        _need(init_k, "init_k", torch.float32, (H, ck, d), dev)

    def __call__(self, q, k, v, init_q, init_k, stage_events: bool = False):
        self.check_inputs(q, k, v, init_q, init_k)
        L, s, dt = lib(), _stream(), self.dt
        H, nq, nk, d, cq, ck = self.H, self.nq, self.nk, self.d, self.cq, self.ck
        ws, wn = _ptr(self.ws), self.ws.numel()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(self.STAGES))] \
            if stage_events else None
        mark = (lambda i: ev[i].record()) if ev else (lambda i: None)
        self.cen_q.copy_(init_q)
        self.cen_k.copy_(init_k)
        vpp = ctypes.c_void_p
        mark(0)
        _check("svgear_cluster_permute", L.svgear_cluster_permute(
            dt, H, nq, d, cq, self.iters, 1, (vpp * 1)(q.data_ptr()),
            (vpp * 1)(self.qp.data_ptr()), (vpp * 1)(self.q_bar.data_ptr()), _ptr(self.cen_q),
            _ptr(self.labels_q), _ptr(self.counts_q), _ptr(self.perm_q), _ptr(self.q_off), ws, wn,
            s))
        mark(1); mark(2)
        _check("svgear_cluster_permute", L.svgear_cluster_permute(
            dt, H, nk, d, ck, self.iters, 2, (vpp * 2)(k.data_ptr(), v.data_ptr()),
            (vpp * 2)(self.kp.data_ptr(), self.vp.data_ptr()),
            (vpp * 2)(self.k_bar.data_ptr(), self.v_bar.data_ptr()), _ptr(self.cen_k),
            _ptr(self.labels_k), _ptr(self.counts_k), _ptr(self.perm_k), _ptr(self.k_off), ws, wn,
            s))
        mark(3); mark(4)
        if self.probe == "weight":
            _check("svgear_probe", L.svgear_probe(
                dt, H, nk, d, cq, ck, self.scale, _ptr(self.q_bar), _ptr(self.kp),
                _ptr(self.k_bar), _ptr(self.k_off), _ptr(self.ratio), _ptr(self.log_norm), ws, wn,
                s))
        else:
            _check("svgear_probe_values", L.svgear_probe_values(
                dt, H, nk, d, cq, ck, self.scale, _ptr(self.q_bar), _ptr(self.kp),
                _ptr(self.k_bar), _ptr(self.vp), _ptr(self.v_bar), _ptr(self.k_off),
                _ptr(self.ratio), _ptr(self.log_norm), ws, wn, s))
        mark(5); mark(6)
        if self.routing == "cluster":
            _check("svgear_route", L.svgear_route(H, cq, ck, _ptr(self.ratio), _ptr(self.q_off),
                                                  _ptr(self.k_off), self.budget,
                                                  _ptr(self.sel_mask), _ptr(self.sel_list),
                                                  _ptr(self.sel_count), _ptr(self.sel_keys), ws,
                                                  wn, s))
        else:
            _check("svgear_route_global", L.svgear_route_global(
                H, cq, ck, _ptr(self.ratio), _ptr(self.q_off), _ptr(self.k_off), self.budget,
                _ptr(self.sel_mask), _ptr(self.sel_list), _ptr(self.sel_count),
                _ptr(self.sel_keys), _ptr(self.used_entries), ws, wn, s))
        mark(7); mark(8)
        _check("svgear_attend_unpermute", L.svgear_attend_unpermute(
            dt, H, nq, nk, d, cq, ck, self.scale, _ptr(self.qp), _ptr(self.kp), _ptr(self.vp),
            _ptr(self.q_off), _ptr(self.k_off), _ptr(self.k_bar), _ptr(self.v_bar),
            _ptr(self.sel_mask), _ptr(self.perm_q), _ptr(self.o), ws, wn, s))
        mark(9)
        self._events = ev
        return self.o

    def last_stage_ms(self):
        """Per-stage milliseconds of the last call made with stage_events=True."""
        ev = self._events
        return {n: ev[2 * i].elapsed_time(ev[2 * i + 1]) for i, n in enumerate(self.STAGES)}


def budget_keys(rho: float, nk: int) -> int:
    """floor(rho * N_k), evaluated in double precision on the host."""
    return int(math.floor(float(rho) * nk))


def svgear_block_scores(q_centroids, k_centroids, k_offsets, scale: float):
    """Centroid-estimated attention mass of every block [H, Cq, Ck] (-1: empty)."""
    _need(q_centroids, "q_centroids", torch.float32)
    H, Cq, d = q_centroids.shape
    Ck = k_centroids.shape[1]
    _need(k_centroids, "k_centroids", torch.float32, (H, Ck, d))
    _need(k_offsets, "k_offsets", torch.int32, (H, Ck + 1))
    scores = torch.empty((H, Cq, Ck), dtype=torch.float32, device=q_centroids.device)
    _check("svgear_block_scores", lib().svgear_block_scores(
        H, d, Cq, Ck, float(scale), _ptr(q_centroids), _ptr(k_centroids), _ptr(k_offsets),
        _ptr(scores), _stream()))
    return scores


def svgear_map_error(qp, kp, q_offsets, k_offsets, k_centroids, sel_mask, scale: float,
                     compensate: bool = True):
    """Per-query squared map error and both normalisers, each [H, Nq] f32."""
    _need(qp, "qp")
    H, Nq, d = qp.shape
    Nk = kp.shape[1]
    Cq, Ck = q_offsets.shape[1] - 1, k_offsets.shape[1] - 1
    _need(kp, "kp", qp.dtype, (H, Nk, d))
    _need(q_offsets, "q_offsets", torch.int32, (H, Cq + 1))
    _need(k_offsets, "k_offsets", torch.int32, (H, Ck + 1))
    _need(k_centroids, "k_centroids", torch.float32, (H, Ck, d))
    _need(sel_mask, "sel_mask", torch.uint8, (H, Cq, Ck))
    dev = qp.device
    err, zf, zs = (torch.empty((H, Nq), dtype=torch.float32, device=dev) for _ in range(3))
    L = lib()
    ws = _ws(L.svgear_map_error_workspace(H, Nq, Ck), dev)
    _check("svgear_map_error", L.svgear_map_error(
        _dt(qp), H, Nq, Nk, d, Cq, Ck, float(scale), _ptr(qp), _ptr(kp), _ptr(q_offsets),
        _ptr(k_offsets), _ptr(k_centroids), _ptr(sel_mask), int(bool(compensate)), _ptr(err),
        _ptr(zf), _ptr(zs), _ptr(ws), ws.numel(), _stream()))
    return err, zf, zs


def svgear_row_spread(xp, means, offsets):
    """||xp[h, p] - means[h, cluster(p)]||^2 for every permuted row, [H, N] f32."""
    _need(xp, "xp")
    H, N, d = xp.shape
    C = means.shape[1]
    _need(means, "means", torch.float32, (H, C, d))
    _need(offsets, "offsets", torch.int32, (H, C + 1))
    out = torch.empty((H, N), dtype=torch.float32, device=xp.device)
    _check("svgear_row_spread", lib().svgear_row_spread(_dt(xp), H, N, d, C, _ptr(xp),
                                                        _ptr(means), _ptr(offsets), _ptr(out),
                                                        _stream()))
    return out


def svgear_clock_probe(blocks: int, iters: int, device="cuda"):
    """Enqueue the clock probe; returns its [4 + blocks] int64 output buffer
    (shader clock at start and end, real-time counter at start and end, then
    one checksum per block), valid once the stream has reached it."""
    out = torch.zeros(4 + int(blocks), dtype=torch.int64, device=device)
    _check("svgear_clock_probe", lib().svgear_clock_probe(int(blocks), int(iters), _ptr(out),
                                                          _stream()))
    return out


def svgear_realtime_khz() -> int:
    """Rate of the real-time counter that svgear_clock_probe reads (kHz)."""
    khz = ctypes.c_int(0)
    _check("svgear_realtime_khz", lib().svgear_realtime_khz(ctypes.byref(khz)))
    return khz.value


def routed_attention(q, k, v, cq: int, ck: int, budget: int, iters: int, init_q, init_k,
                     scale: float | None = None, labels_q=None, labels_k=None,
                     routing: str = "cluster", probe: str = "weight"):
    """The whole path: cluster -> permute -> probe -> route -> attend -> unpermute.

    ``init_q``/``init_k`` ([H, C, d] f32) are consumed (updated to the final
    centroids); clustering and permutation run as one call per tensor.
    ``labels_q``/``labels_k`` skip the clustering when given.
    ``routing="cluster"`` gives every query cluster ``budget`` exact keys;
    ``routing="global"`` lets all blocks of a head share ``budget`` exact
    (query, key) entries. ``probe="value"`` ranks blocks by the value-aware
    error instead of the weight gap. Returns a dict with every intermediate.
    """
    if routing not in ("cluster", "global"):
        raise ValueError(f"routing must be 'cluster' or 'global', not {routing!r}")
    if probe not in ("weight", "value"):
        raise ValueError(f"probe must be 'weight' or 'value', not {probe!r}")
    d = q.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    res = {}
    if labels_q is None:
        labels_q, res["counts_q"], perm_q, q_off, (qp,), (q_bar,) = \
            svgear_cluster_permute([q], init_q, iters)
    else:
        perm_q, q_off, (qp,), (q_bar,) = svgear_permute(labels_q, cq, [q])
    if labels_k is None:
        labels_k, res["counts_k"], perm_k, k_off, (kp, vp), (k_bar, v_bar) = \
            svgear_cluster_permute([k, v], init_k, iters)
    else:
        perm_k, k_off, (kp, vp), (k_bar, v_bar) = svgear_permute(labels_k, ck, [k, v])
    if probe == "weight":
        ratio, log_norm = svgear_probe(q_bar, kp, k_bar, k_off, scale)
    else:
        ratio, log_norm = svgear_probe_values(q_bar, kp, k_bar, vp, v_bar, k_off, scale)
    if routing == "cluster":
        mask, lst, cnt, keys = svgear_route(ratio, k_off, budget, q_off)
    else:
        mask, lst, cnt, keys, res["used_entries"] = svgear_route_global(ratio, q_off, k_off,
                                                                        budget)
    op = svgear_attend(qp, kp, vp, q_off, k_off, k_bar, v_bar, mask, scale)
    o = svgear_unpermute(op, perm_q)
    res.update(labels_q=labels_q, labels_k=labels_k, perm_q=perm_q, perm_k=perm_k, q_off=q_off,
               k_off=k_off, qp=qp, kp=kp, vp=vp, q_bar=q_bar, k_bar=k_bar, v_bar=v_bar,
               ratio=ratio, log_norm=log_norm, sel_mask=mask, sel_list=lst, sel_count=cnt,
               sel_keys=keys, op=op, o=o)
    return res
