// Host-side launchers shared between the svgear translation units. Not part
// of the public ABI (include/svgear.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace svg {

constexpr int kTile = 256;        // rows per counting-sort tile (one block)
constexpr int kChunk = 1024;      // rows per segment-sum chunk
constexpr int kProbeUnit = 256;   // keys per probe work unit
constexpr int kProbeGroup = 128;  // query centroids per probe block
constexpr int kMaxClusters = 1024;
constexpr int kXcds = 8;          // accelerator complex dies of an MI355X

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int sort_tiles(int N) { return ceil_div(N, kTile); }
inline int max_chunks(int N, int C) { return ceil_div(N, kChunk) + C; }
inline int max_units(int Nk, int Ck) { return ceil_div(Nk, kProbeUnit) + Ck; }

// Workspace carve-up for a counting sort + segment means over H heads.
struct SortWs {
  int32_t* rank;          // [H][N]
  int32_t* hist;          // [H][tiles][C] -> exclusive bases after the scan
  int32_t* chunk_prefix;  // [H][C+1]
  int32_t* sizes;         // [H][C]
  float* partial;         // [H][ntensors][max_chunks][d]
};
size_t sort_ws_bytes(int H, int N, int d, int C, int ntensors);
SortWs sort_ws_carve(void* ws, int H, int N, int d, int C, int ntensors);

// sort.hip
hipError_t launch_label_rank(const int32_t* labels, int H, int N, int C, int32_t* rank,
                             int32_t* hist, hipStream_t s);
// hist [H][tiles][C] becomes every tile's exclusive prefix within its cluster.
hipError_t launch_sort_scan(int H, int N, int C, int32_t* hist, int32_t* sizes, int32_t* offsets,
                            int32_t* counts, int32_t* chunk_prefix, hipStream_t s);
hipError_t launch_scatter(const int32_t* labels, const int32_t* rank, const int32_t* hist,
                          const int32_t* offsets, int H, int N, int C, int32_t* perm,
                          hipStream_t s);
// Gathers rows of up to three tensors in permuted order (dst entries may be
// null) and writes per-chunk f32 column sums to `partial`.
hipError_t launch_segsum(int elem_bytes, int H, int N, int d, int C, const int32_t* perm,
                         const int32_t* offsets, const int32_t* chunk_prefix, int ntensors,
                         const void* const* src, void* const* dst, float* partial,
                         hipStream_t s);
// mode 0: empty cluster -> zero row; mode 1: empty cluster keeps `means`.
// When `table` is non-null also writes table = -2 * round_T(mean) and
// norms = ||round_T(mean)||^2 (k-means distance operands).
hipError_t launch_combine(int elem_bytes, int H, int d, int C, int ntensors,
                          const int32_t* offsets, const int32_t* chunk_prefix,
                          const float* partial, int N, float* const* means, int mode,
                          void* table, float* norms, hipStream_t s);
hipError_t launch_unpermute(int elem_bytes, int H, int N, int d, const int32_t* perm,
                            const void* Xp, void* X, hipStream_t s);

// kmeans.hip
hipError_t launch_table(int elem_bytes, int H, int d, int C, const float* mu, void* table,
                        float* norms, hipStream_t s);
hipError_t launch_assign(int elem_bytes, int H, int N, int d, int C, const void* X,
                         const void* table, const float* norms, int32_t* labels, int32_t* rank,
                         int32_t* hist, hipStream_t s);

// probe.hip
size_t probe_ws_bytes(int H, int Nk, int Cq, int Ck, bool values);
// Vp == nullptr: the weight-gap probe; otherwise the value-aware one (vc = vbar).
hipError_t launch_probe(int elem_bytes, int H, int Nk, int d, int Cq, int Ck, float scale,
                        const float* qc, const void* Kp, const float* kc, const void* Vp,
                        const float* vc, const int32_t* koff, void* ws, float* ratio,
                        float* log_norm, hipStream_t s);

// route.hip
// qoff may be null (every query cluster routed); an empty query cluster selects nothing.
hipError_t launch_route(int H, int Cq, int Ck, const float* ratio, const int32_t* qoff,
                        const int32_t* koff, int32_t budget, uint8_t* mask, int32_t* list,
                        int32_t* count, int32_t* keys, hipStream_t s);
size_t route_global_ws_bytes(int H, int Cq, int Ck);
hipError_t launch_route_global(int H, int Cq, int Ck, const float* ratio, const int32_t* qoff,
                               const int32_t* koff, int64_t budget, uint8_t* mask,
                               int32_t* list, int32_t* count, int32_t* keys, int64_t* used,
                               void* ws, hipStream_t s);

// attend.hip
hipError_t launch_attend(int elem_bytes, int H, int Nq, int Nk, int d, int Cq, int Ck,
                         float scale, const void* Qp, const void* Kp, const void* Vp,
                         const int32_t* qoff, const int32_t* koff, const float* kc,
                         const float* vc, const uint8_t* mask, const int32_t* qperm, void* Op,
                         void* ws, hipStream_t s);
size_t attend_ws_bytes(int elem_bytes, int H, int Ck, int d);

// analysis.hip
size_t map_error_ws_bytes(int H, int Nq, int Ck);
hipError_t launch_map_error(int elem_bytes, int H, int Nq, int Nk, int d, int Cq, int Ck,
                            float scale, const void* Qp, const void* Kp, const int32_t* qoff,
                            const int32_t* koff, const float* kc, const uint8_t* mask,
                            int compensate, float* err, float* zfull, float* zsparse, void* ws,
                            hipStream_t s);
hipError_t launch_block_scores(int H, int d, int Cq, int Ck, float scale, const float* qc,
                               const float* kc, const int32_t* koff, float* scores,
                               hipStream_t s);
hipError_t launch_row_spread(int elem_bytes, int H, int N, int d, int C, const void* Xp,
                             const float* mu, const int32_t* off, float* d2, hipStream_t s);

// clock.hip
hipError_t launch_clock_probe(int blocks, int iters, uint64_t* out, hipStream_t s);

}  // namespace svg
