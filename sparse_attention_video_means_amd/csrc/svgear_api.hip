// C ABI of libsvgear: argument validation, workspace carving and launches.
// Every entry point checks all of its arguments before it enqueues anything,
// never allocates or synchronises, and returns the first launch error.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/svgear.h"
#include "svgear_internal.hpp"

using namespace svg;

namespace {

// The kernels are built for gfx950 only. The architecture of the calling
// thread's current device is looked up once per device and cached; a call on
// any other device (or with no device at all) is refused before anything is
// enqueued.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

svgear_status device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();  // leave no sticky error behind for the caller
    return SVGEAR_ERR_UNSUPPORTED;
  }
  int state = dev < kMaxDevices ? g_arch_state[dev].load(std::memory_order_relaxed) : 0;
  if (state == 0) {
    hipDeviceProp_t prop;
    bool ok = hipGetDeviceProperties(&prop, dev) == hipSuccess;
    if (!ok) (void)hipGetLastError();
    // gcnArchName is "gfx950" optionally followed by ":feature+..." flags
    ok = ok && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
         (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
    state = ok ? 1 : 2;
    if (dev < kMaxDevices) g_arch_state[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? SVGEAR_OK : SVGEAR_ERR_UNSUPPORTED;
}

// A C caller may pass any int where the ABI names an enum, and C++ may not
// read an enum object holding a value outside its enumerators. Entry points
// therefore take the bytes of such a parameter as a plain int, without ever
// reading it as the enum type.
template <typename E>
int enum_code(const E* e) {
  static_assert(sizeof(E) == sizeof(int), "ABI enums are int-sized");
  int v;
  std::memcpy(&v, e, sizeof v);
  return v;
}

// Scratch memory of svgear_attend_unpermute_noalloc, for callers that cannot
// allocate: one array per GPU, alive until the process ends. Host code never
// uses the array's name as an address (on the host it only names the symbol);
// the device address is looked up once per device with that device current
// and kept in g_scratch.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of the current device's scratch array.
svgear_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return SVGEAR_ERR_UNSUPPORTED;
  }
  void* p = dev < kMaxDevices ? g_scratch[dev].load(std::memory_order_acquire) : nullptr;
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return SVGEAR_ERR_HIP;
    }
    if (dev < kMaxDevices) g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SVGEAR_OK;
}

int elem_bytes(int dt) {
  return dt == SVGEAR_BF16 ? 2 : (dt == SVGEAR_F32 ? 4 : 0);
}

bool dim_ok(int d) { return d == 64 || d == 128; }

// Common shape check for a tensor family clustered into C clusters.
svgear_status check_shape(int dt, int H, int N, int d, int C) {
  if (H < 1 || N < 1 || C < 1 || C > N || C > kMaxClusters) return SVGEAR_ERR_INVALID_ARG;
  if (elem_bytes(dt) == 0 || !dim_ok(d)) return SVGEAR_ERR_UNSUPPORTED;
  if (size_t(H) * N * d > (size_t(1) << 40)) return SVGEAR_ERR_INVALID_ARG;
  if (size_t(N) * d >= (size_t(1) << 31)) return SVGEAR_ERR_INVALID_ARG;  // 32-bit row offsets
  return SVGEAR_OK;
}

hipStream_t as_stream(svgear_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

struct ClusterWs {
  SortWs sort;
  int32_t* perm;
  int32_t* offsets;
  void* table;
  float* norms;
};

// nt: tensors whose segment sums the workspace holds (1 for the k-means
// iterations; 2 when the last iteration also permutes K and V).
size_t cluster_ws_bytes(int eb, int H, int N, int d, int C, int nt = 1) {
  return sort_ws_bytes(H, N, d, C, nt) + align256(sizeof(int32_t) * size_t(H) * N) +
         align256(sizeof(int32_t) * size_t(H) * (C + 1)) + align256(size_t(eb) * H * C * d) +
         align256(sizeof(float) * size_t(H) * C);
}

ClusterWs cluster_ws_carve(void* ws, int eb, int H, int N, int d, int C, int nt = 1) {
  ClusterWs w;
  w.sort = sort_ws_carve(ws, H, N, d, C, nt);
  char* p = static_cast<char*>(ws) + sort_ws_bytes(H, N, d, C, nt);
  w.perm = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(H) * N);
  w.offsets = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(H) * (C + 1));
  w.table = p;
  p += align256(size_t(eb) * H * C * d);
  w.norms = reinterpret_cast<float*>(p);
  return w;
}


#define SVG_TRY(expr)                                      \
  do {                                                     \
    if ((expr) != hipSuccess) return SVGEAR_ERR_HIP;       \
  } while (0)

// After the arguments are validated: refuse devices the kernels were not built for.
#define SVG_NEED_DEVICE()                                  \
  do {                                                     \
    const svgear_status dev_st_ = device_ok();             \
    if (dev_st_ != SVGEAR_OK) return dev_st_;              \
  } while (0)

svgear_status attend_common(int dt, int H, int Nq, int Nk, int d, int Cq, int Ck,
                            float scale, const void* Qp, const void* Kp, const void* Vp,
                            const int32_t* q_offsets, const int32_t* k_offsets,
                            const float* k_centroids, const float* v_centroids,
                            const uint8_t* sel_mask, const int32_t* q_perm, void* Op, void* ws,
                            size_t ws_bytes, svgear_stream_t s) {
  svgear_status st = check_shape(dt, H, Nq, d, Cq);
  if (st != SVGEAR_OK) return st;
  st = check_shape(dt, H, Nk, d, Ck);
  if (st != SVGEAR_OK) return st;
  if (!(scale > 0.f) || !Qp || !Kp || !Vp || !q_offsets || !k_offsets || !k_centroids ||
      !v_centroids || !sel_mask || !Op)
    return SVGEAR_ERR_INVALID_ARG;
  // the tile copies address one head's K or V with 32-bit byte offsets
  if (size_t(Nk) * d * elem_bytes(dt) >= (size_t(1) << 32)) return SVGEAR_ERR_INVALID_ARG;
  const size_t need = attend_ws_bytes(elem_bytes(dt), H, Ck, d);
  if (need > 0 && (!ws || ws_bytes < need)) return SVGEAR_ERR_WORKSPACE;
  SVG_NEED_DEVICE();
  SVG_TRY(launch_attend(elem_bytes(dt), H, Nq, Nk, d, Cq, Ck, scale, Qp, Kp, Vp, q_offsets,
                        k_offsets, k_centroids, v_centroids, sel_mask, q_perm, Op, ws,
                        as_stream(s)));
  return SVGEAR_OK;
}

}  // namespace

extern "C" {

const char* svgear_status_string(svgear_status st_in) {
  switch (enum_code(&st_in)) {
    case SVGEAR_OK: return "ok";
    case SVGEAR_ERR_INVALID_ARG: return "invalid argument";
    case SVGEAR_ERR_UNSUPPORTED: return "unsupported dtype, head dimension or device";
    case SVGEAR_ERR_WORKSPACE: return "workspace too small";
    case SVGEAR_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

size_t svgear_cluster_workspace(svgear_dtype dt_in, int H, int N, int d, int C) {
  const int dt = enum_code(&dt_in);
  if (check_shape(dt, H, N, d, C) != SVGEAR_OK) return 0;
  return cluster_ws_bytes(elem_bytes(dt), H, N, d, C);
}

svgear_status svgear_cluster(svgear_dtype dt_in, int H, int N, int d, int C, int iters,
                             const void* X, float* centroids, int32_t* labels, int32_t* counts,
                             void* ws, size_t ws_bytes, svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  const svgear_status st = check_shape(dt, H, N, d, C);
  if (st != SVGEAR_OK) return st;
  if (iters < 1 || !X || !centroids || !labels || !counts) return SVGEAR_ERR_INVALID_ARG;
  const int eb = elem_bytes(dt);
  if (!ws || ws_bytes < cluster_ws_bytes(eb, H, N, d, C)) return SVGEAR_ERR_WORKSPACE;
  SVG_NEED_DEVICE();
  const hipStream_t hs = as_stream(s);
  ClusterWs w = cluster_ws_carve(ws, eb, H, N, d, C);
  SVG_TRY(launch_table(eb, H, d, C, centroids, w.table, w.norms, hs));
  for (int it = 0; it < iters; ++it) {
    SVG_TRY(launch_assign(eb, H, N, d, C, X, w.table, w.norms, labels, w.sort.rank, w.sort.hist, hs));
    SVG_TRY(launch_sort_scan(H, N, C, w.sort.hist, w.sort.sizes, w.offsets, counts,
                             w.sort.chunk_prefix, hs));
    SVG_TRY(launch_scatter(labels, w.sort.rank, w.sort.hist, w.offsets, H, N, C, w.perm, hs));
    const void* src[1] = {X};
    SVG_TRY(launch_segsum(eb, H, N, d, C, w.perm, w.offsets, w.sort.chunk_prefix, 1, src, nullptr,
                          w.sort.partial, hs));
    float* means[1] = {centroids};
    const bool last = it + 1 == iters;
    SVG_TRY(launch_combine(eb, H, d, C, 1, w.offsets, w.sort.chunk_prefix, w.sort.partial, N, means,
                           /*mode=*/1, last ? nullptr : w.table, w.norms, hs));
  }
  return SVGEAR_OK;
}

size_t svgear_cluster_permute_workspace(svgear_dtype dt_in, int H, int N, int d, int C) {
  const int dt = enum_code(&dt_in);
  if (check_shape(dt, H, N, d, C) != SVGEAR_OK) return 0;
  return cluster_ws_bytes(elem_bytes(dt), H, N, d, C, 2);
}

svgear_status svgear_cluster_permute(svgear_dtype dt_in, int H, int N, int d, int C, int iters,
                                     int ntensors, const void* const* src, void* const* dst,
                                     float* const* means, float* centroids, int32_t* labels,
                                     int32_t* counts, int32_t* perm, int32_t* offsets, void* ws,
                                     size_t ws_bytes, svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  const svgear_status st = check_shape(dt, H, N, d, C);
  if (st != SVGEAR_OK) return st;
  if (iters < 1 || ntensors < 1 || ntensors > 2 || !src || !dst || !centroids || !labels ||
      !counts || !perm || !offsets)
    return SVGEAR_ERR_INVALID_ARG;
  for (int k = 0; k < ntensors; ++k)
    if (!src[k] || !dst[k] || src[k] == dst[k]) return SVGEAR_ERR_INVALID_ARG;
  const int eb = elem_bytes(dt);
  if (!ws || ws_bytes < cluster_ws_bytes(eb, H, N, d, C, 2)) return SVGEAR_ERR_WORKSPACE;
  SVG_NEED_DEVICE();
  const hipStream_t hs = as_stream(s);
  ClusterWs w = cluster_ws_carve(ws, eb, H, N, d, C, 2);
  const void* X = src[0];
  SVG_TRY(launch_table(eb, H, d, C, centroids, w.table, w.norms, hs));
  for (int it = 0; it < iters; ++it) {
    const bool last = it + 1 == iters;
    int32_t* off = last ? offsets : w.offsets;
    int32_t* pm = last ? perm : w.perm;
    SVG_TRY(launch_assign(eb, H, N, d, C, X, w.table, w.norms, labels, w.sort.rank, w.sort.hist, hs));
    SVG_TRY(launch_sort_scan(H, N, C, w.sort.hist, w.sort.sizes, off, counts, w.sort.chunk_prefix,
                             hs));
    SVG_TRY(launch_scatter(labels, w.sort.rank, w.sort.hist, off, H, N, C, pm, hs));
    if (!last) {
      const void* one[1] = {X};
      SVG_TRY(launch_segsum(eb, H, N, d, C, pm, off, w.sort.chunk_prefix, 1, one, nullptr,
                            w.sort.partial, hs));
      float* cm[1] = {centroids};
      SVG_TRY(launch_combine(eb, H, d, C, 1, off, w.sort.chunk_prefix, w.sort.partial, N, cm,
                             /*mode=*/1, w.table, w.norms, hs));
    } else {
      // the final labels' permutation: one pass writes the permuted copies and
      // the segment sums of every tensor
      SVG_TRY(launch_segsum(eb, H, N, d, C, pm, off, w.sort.chunk_prefix, ntensors, src, dst,
                            w.sort.partial, hs));
      float* cm[2] = {centroids, nullptr};
      SVG_TRY(launch_combine(eb, H, d, C, ntensors, off, w.sort.chunk_prefix, w.sort.partial, N,
                             cm, /*mode=*/1, nullptr, nullptr, hs));
      bool any = false;
      if (means)
        for (int k = 0; k < ntensors; ++k) any = any || means[k];
      if (any)
        SVG_TRY(launch_combine(eb, H, d, C, ntensors, off, w.sort.chunk_prefix, w.sort.partial, N,
                               means, /*mode=*/0, nullptr, nullptr, hs));
    }
  }
  return SVGEAR_OK;
}

size_t svgear_permute_workspace(svgear_dtype dt_in, int H, int N, int d, int C) {
  const int dt = enum_code(&dt_in);
  if (check_shape(dt, H, N, d, C) != SVGEAR_OK) return 0;
  return sort_ws_bytes(H, N, d, C, 2);
}

svgear_status svgear_permute(svgear_dtype dt_in, int H, int N, int d, int C, const int32_t* labels,
                             int32_t* perm, int32_t* offsets, int ntensors,
                             const void* const* src, void* const* dst, float* const* means,
                             void* ws, size_t ws_bytes, svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  const svgear_status st = check_shape(dt, H, N, d, C);
  if (st != SVGEAR_OK) return st;
  if (!labels || !perm || !offsets || ntensors < 1 || ntensors > 2 || !src || !dst)
    return SVGEAR_ERR_INVALID_ARG;
  for (int k = 0; k < ntensors; ++k)
    if (!src[k] || !dst[k] || src[k] == dst[k]) return SVGEAR_ERR_INVALID_ARG;
  if (!ws || ws_bytes < sort_ws_bytes(H, N, d, C, 2)) return SVGEAR_ERR_WORKSPACE;
  const int eb = elem_bytes(dt);
  SVG_NEED_DEVICE();
  const hipStream_t hs = as_stream(s);
  SortWs w = sort_ws_carve(ws, H, N, d, C, 2);
  SVG_TRY(launch_label_rank(labels, H, N, C, w.rank, w.hist, hs));
  SVG_TRY(launch_sort_scan(H, N, C, w.hist, w.sizes, offsets, nullptr, w.chunk_prefix, hs));
  SVG_TRY(launch_scatter(labels, w.rank, w.hist, offsets, H, N, C, perm, hs));
  SVG_TRY(launch_segsum(eb, H, N, d, C, perm, offsets, w.chunk_prefix, ntensors, src, dst,
                        w.partial, hs));
  bool any = false;
  if (means)
    for (int k = 0; k < ntensors; ++k) any = any || means[k];
  if (any)
    SVG_TRY(launch_combine(eb, H, d, C, ntensors, offsets, w.chunk_prefix, w.partial, N, means,
                           /*mode=*/0, nullptr, nullptr, hs));
  return SVGEAR_OK;
}

size_t svgear_probe_workspace(int H, int Nk, int Cq, int Ck) {
  if (H < 1 || Nk < 1 || Cq < 1 || Ck < 1 || Ck > Nk || Ck > kMaxClusters || Cq > kMaxClusters)
    return 0;
  return probe_ws_bytes(H, Nk, Cq, Ck, false);
}

size_t svgear_probe_values_workspace(int H, int Nk, int Cq, int Ck) {
  if (H < 1 || Nk < 1 || Cq < 1 || Ck < 1 || Ck > Nk || Ck > kMaxClusters || Cq > kMaxClusters)
    return 0;
  return probe_ws_bytes(H, Nk, Cq, Ck, true);
}

svgear_status svgear_probe_values(svgear_dtype dt_in, int H, int Nk, int d, int Cq, int Ck,
                                  float scale, const float* q_centroids, const void* Kp,
                                  const float* k_centroids, const void* Vp,
                                  const float* v_centroids, const int32_t* k_offsets,
                                  float* ratio, float* log_norm, void* ws, size_t ws_bytes,
                                  svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  const svgear_status st = check_shape(dt, H, Nk, d, Ck);
  if (st != SVGEAR_OK) return st;
  if (Cq < 1 || Cq > kMaxClusters || !(scale > 0.f) || !q_centroids || !Kp || !k_centroids ||
      !Vp || !v_centroids || !k_offsets || !ratio)
    return SVGEAR_ERR_INVALID_ARG;
  if (!ws || ws_bytes < probe_ws_bytes(H, Nk, Cq, Ck, true)) return SVGEAR_ERR_WORKSPACE;
  SVG_NEED_DEVICE();
  SVG_TRY(launch_probe(elem_bytes(dt), H, Nk, d, Cq, Ck, scale, q_centroids, Kp, k_centroids, Vp,
                       v_centroids, k_offsets, ws, ratio, log_norm, as_stream(s)));
  return SVGEAR_OK;
}

svgear_status svgear_probe(svgear_dtype dt_in, int H, int Nk, int d, int Cq, int Ck, float scale,
                           const float* q_centroids, const void* Kp, const float* k_centroids,
                           const int32_t* k_offsets, float* ratio, float* log_norm, void* ws,
                           size_t ws_bytes, svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  const svgear_status st = check_shape(dt, H, Nk, d, Ck);
  if (st != SVGEAR_OK) return st;
  if (Cq < 1 || Cq > kMaxClusters || !(scale > 0.f) || !q_centroids || !Kp || !k_centroids ||
      !k_offsets || !ratio)
    return SVGEAR_ERR_INVALID_ARG;
  if (!ws || ws_bytes < probe_ws_bytes(H, Nk, Cq, Ck, false)) return SVGEAR_ERR_WORKSPACE;
  SVG_NEED_DEVICE();
  SVG_TRY(launch_probe(elem_bytes(dt), H, Nk, d, Cq, Ck, scale, q_centroids, Kp, k_centroids,
                       nullptr, nullptr, k_offsets, ws, ratio, log_norm, as_stream(s)));
  return SVGEAR_OK;
}

size_t svgear_route_workspace(int H, int Cq, int Ck) {
  (void)H; (void)Cq; (void)Ck;
  return 0;  // the per-query-cluster router keeps its sort in LDS
}

svgear_status svgear_route(int H, int Cq, int Ck, const float* ratio, const int32_t* q_offsets,
                           const int32_t* k_offsets, int32_t budget_keys, uint8_t* sel_mask,
                           int32_t* sel_list, int32_t* sel_count, int32_t* sel_keys, void* ws,
                           size_t ws_bytes, svgear_stream_t s) {
  if (H < 1 || Cq < 1 || Ck < 1 || Cq > kMaxClusters || Ck > kMaxClusters || budget_keys < 0 ||
      !ratio || !k_offsets || !sel_mask)
    return SVGEAR_ERR_INVALID_ARG;
  (void)ws; (void)ws_bytes;  // svgear_route_workspace() is 0: nothing to check
  SVG_NEED_DEVICE();
  SVG_TRY(launch_route(H, Cq, Ck, ratio, q_offsets, k_offsets, budget_keys, sel_mask, sel_list,
                       sel_count, sel_keys, as_stream(s)));
  return SVGEAR_OK;
}

size_t svgear_route_global_workspace(int H, int Cq, int Ck) {
  if (H < 1 || Cq < 1 || Ck < 1 || Cq > kMaxClusters || Ck > kMaxClusters) return 0;
  return route_global_ws_bytes(H, Cq, Ck);
}

svgear_status svgear_route_global(int H, int Cq, int Ck, const float* ratio,
                                  const int32_t* q_offsets, const int32_t* k_offsets,
                                  int64_t budget_entries, uint8_t* sel_mask, int32_t* sel_list,
                                  int32_t* sel_count, int32_t* sel_keys, int64_t* used_entries,
                                  void* ws, size_t ws_bytes, svgear_stream_t s) {
  if (H < 1 || Cq < 1 || Ck < 1 || Cq > kMaxClusters || Ck > kMaxClusters ||
      budget_entries < 0 || !ratio || !q_offsets || !k_offsets || !sel_mask)
    return SVGEAR_ERR_INVALID_ARG;
  if (!ws || ws_bytes < route_global_ws_bytes(H, Cq, Ck)) return SVGEAR_ERR_WORKSPACE;
  SVG_NEED_DEVICE();
  SVG_TRY(launch_route_global(H, Cq, Ck, ratio, q_offsets, k_offsets, budget_entries, sel_mask,
                              sel_list, sel_count, sel_keys, used_entries, ws, as_stream(s)));
  return SVGEAR_OK;
}

size_t svgear_attend_workspace(svgear_dtype dt_in, int H, int Ck, int d) {
  const int dt = enum_code(&dt_in);
  if (H < 1 || Ck < 1 || Ck > kMaxClusters || elem_bytes(dt) == 0 || !dim_ok(d)) return 0;
  return attend_ws_bytes(elem_bytes(dt), H, Ck, d);
}

svgear_status svgear_attend(svgear_dtype dt_in, int H, int Nq, int Nk, int d, int Cq, int Ck,
                            float scale, const void* Qp, const void* Kp, const void* Vp,
                            const int32_t* q_offsets, const int32_t* k_offsets,
                            const float* k_centroids, const float* v_centroids,
                            const uint8_t* sel_mask, void* Op, void* ws, size_t ws_bytes,
                            svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  return attend_common(dt, H, Nq, Nk, d, Cq, Ck, scale, Qp, Kp, Vp, q_offsets, k_offsets,
                       k_centroids, v_centroids, sel_mask, nullptr, Op, ws, ws_bytes, s);
}

svgear_status svgear_attend_unpermute(svgear_dtype dt_in, int H, int Nq, int Nk, int d, int Cq,
                                      int Ck, float scale, const void* Qp, const void* Kp,
                                      const void* Vp, const int32_t* q_offsets,
                                      const int32_t* k_offsets, const float* k_centroids,
                                      const float* v_centroids, const uint8_t* sel_mask,
                                      const int32_t* q_perm, void* O, void* ws, size_t ws_bytes,
                                      svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  if (!q_perm || O == Qp) return SVGEAR_ERR_INVALID_ARG;
  return attend_common(dt, H, Nq, Nk, d, Cq, Ck, scale, Qp, Kp, Vp, q_offsets, k_offsets,
                       k_centroids, v_centroids, sel_mask, q_perm, O, ws, ws_bytes, s);
}

svgear_status svgear_attend_unpermute_noalloc(svgear_dtype dt_in, int H, int Nq, int Nk, int d,
                                              int Cq, int Ck, float scale, const void* Qp,
                                              const void* Kp, const void* Vp,
                                              const int32_t* q_offsets, const int32_t* k_offsets,
                                              const float* k_centroids, const float* v_centroids,
                                              const uint8_t* sel_mask, const int32_t* q_perm,
                                              void* O, svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  if (!q_perm || O == Qp) return SVGEAR_ERR_INVALID_ARG;
  svgear_status st = check_shape(dt, H, Nq, d, Cq);
  if (st != SVGEAR_OK) return st;
  st = check_shape(dt, H, Nk, d, Ck);
  if (st != SVGEAR_OK) return st;
  if (!(scale > 0.f) || !Qp || !Kp || !Vp || !q_offsets || !k_offsets || !k_centroids ||
      !v_centroids || !sel_mask || !O)
    return SVGEAR_ERR_INVALID_ARG;
  // the centroid rows rounded to dt must fit the scratch array
  if (attend_ws_bytes(elem_bytes(dt), H, Ck, d) > kNoallocScratchBytes)
    return SVGEAR_ERR_WORKSPACE;
  // attend_common repeats the full argument check before its launch
  SVG_NEED_DEVICE();
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != SVGEAR_OK) return st;
  return attend_common(dt, H, Nq, Nk, d, Cq, Ck, scale, Qp, Kp, Vp, q_offsets, k_offsets,
                       k_centroids, v_centroids, sel_mask, q_perm, O, ws, kNoallocScratchBytes,
                       s);
}

svgear_status svgear_unpermute(svgear_dtype dt_in, int H, int N, int d, const int32_t* perm,
                               const void* Xp, void* X, svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  const svgear_status st = check_shape(dt, H, N, d, 1);
  if (st != SVGEAR_OK) return st;
  if (!perm || !Xp || !X || Xp == X) return SVGEAR_ERR_INVALID_ARG;
  SVG_NEED_DEVICE();
  SVG_TRY(launch_unpermute(elem_bytes(dt), H, N, d, perm, Xp, X, as_stream(s)));
  return SVGEAR_OK;
}

svgear_status svgear_block_scores(int H, int d, int Cq, int Ck, float scale,
                                  const float* q_centroids, const float* k_centroids,
                                  const int32_t* k_offsets, float* scores, svgear_stream_t s) {
  if (H < 1 || Cq < 1 || Ck < 1 || Cq > kMaxClusters || Ck > kMaxClusters || !dim_ok(d) ||
      !(scale > 0.f) || !q_centroids || !k_centroids || !k_offsets || !scores)
    return SVGEAR_ERR_INVALID_ARG;
  SVG_NEED_DEVICE();
  SVG_TRY(launch_block_scores(H, d, Cq, Ck, scale, q_centroids, k_centroids, k_offsets, scores,
                              as_stream(s)));
  return SVGEAR_OK;
}

size_t svgear_map_error_workspace(int H, int Nq, int Ck) {
  if (H < 1 || Nq < 1 || Ck < 1 || Ck > kMaxClusters) return 0;
  return map_error_ws_bytes(H, Nq, Ck);
}

svgear_status svgear_map_error(svgear_dtype dt_in, int H, int Nq, int Nk, int d, int Cq, int Ck,
                               float scale, const void* Qp, const void* Kp,
                               const int32_t* q_offsets, const int32_t* k_offsets,
                               const float* k_centroids, const uint8_t* sel_mask, int compensate,
                               float* err, float* z_full, float* z_sparse, void* ws,
                               size_t ws_bytes, svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  svgear_status st = check_shape(dt, H, Nq, d, Cq);
  if (st != SVGEAR_OK) return st;
  st = check_shape(dt, H, Nk, d, Ck);
  if (st != SVGEAR_OK) return st;
  if (!(scale > 0.f) || !Qp || !Kp || !q_offsets || !k_offsets || !k_centroids || !sel_mask ||
      !err || !z_full || !z_sparse)
    return SVGEAR_ERR_INVALID_ARG;
  if (!ws || ws_bytes < map_error_ws_bytes(H, Nq, Ck)) return SVGEAR_ERR_WORKSPACE;
  SVG_NEED_DEVICE();
  SVG_TRY(launch_map_error(elem_bytes(dt), H, Nq, Nk, d, Cq, Ck, scale, Qp, Kp, q_offsets,
                           k_offsets, k_centroids, sel_mask, compensate ? 1 : 0, err, z_full,
                           z_sparse, ws, as_stream(s)));
  return SVGEAR_OK;
}

svgear_status svgear_row_spread(svgear_dtype dt_in, int H, int N, int d, int C, const void* Xp,
                                const float* means, const int32_t* offsets, float* spread,
                                svgear_stream_t s) {
  const int dt = enum_code(&dt_in);
  const svgear_status st = check_shape(dt, H, N, d, C);
  if (st != SVGEAR_OK) return st;
  if (!Xp || !means || !offsets || !spread) return SVGEAR_ERR_INVALID_ARG;
  SVG_NEED_DEVICE();
  SVG_TRY(launch_row_spread(elem_bytes(dt), H, N, d, C, Xp, means, offsets, spread,
                            as_stream(s)));
  return SVGEAR_OK;
}

svgear_status svgear_clock_probe(int blocks, int iters, uint64_t* out, svgear_stream_t s) {
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20) || !out)
    return SVGEAR_ERR_INVALID_ARG;
  SVG_NEED_DEVICE();
  SVG_TRY(launch_clock_probe(blocks, iters, out, as_stream(s)));
  return SVGEAR_OK;
}

svgear_status svgear_realtime_khz(int* khz) {
  if (!khz) return SVGEAR_ERR_INVALID_ARG;
  SVG_NEED_DEVICE();
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || *khz <= 0) {
    (void)hipGetLastError();
    return SVGEAR_ERR_HIP;
  }
  return SVGEAR_OK;
}

}  // extern "C"
