// Deterministic counting sort of cluster labels, gathered copies and segment
// means (the permutation and centroid stages of SVG-EAR, paper §3.1 / §4.1:
// tokens of a cluster are laid out contiguously and summarised by their mean).
//
// Pipeline for one tensor family, all heads at once:
//   label_rank  : per 256-row tile, stable rank of each row among equal labels
//                 of the tile (wave ballots, no atomics) + tile histogram.
//   sort_scan   : per head, exclusive scan over tiles of the [tile][cluster]
//                 histogram (each tile writes one contiguous row) -> every
//                 tile's base slot per cluster, cluster offsets and the
//                 per-cluster chunk list.
//   scatter     : perm[base + rank] = row (stable by construction).
//   segsum      : per chunk of <= 1024 slots of one cluster, gather the rows
//                 (optionally storing the permuted copy) and sum them in f32 in a
//                 fixed order.
//   combine     : per cluster, add its chunk sums in chunk order and divide.
// Every step has a fixed reduction order, so results are bitwise repeatable.
#include "svgear_common.hpp"
#include "svgear_internal.hpp"

namespace svg {

size_t sort_ws_bytes(int H, int N, int d, int C, int ntensors) {
  size_t b = 0;
  b += align256(sizeof(int32_t) * size_t(H) * N);
  b += align256(sizeof(int32_t) * size_t(H) * C * sort_tiles(N));
  b += align256(sizeof(int32_t) * size_t(H) * (C + 1));
  b += align256(sizeof(int32_t) * size_t(H) * C);
  b += align256(sizeof(float) * size_t(H) * ntensors * max_chunks(N, C) * d);
  return b;
}

SortWs sort_ws_carve(void* ws, int H, int N, int d, int C, int ntensors) {
  char* p = static_cast<char*>(ws);
  SortWs w;
  w.rank = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(H) * N);
  w.hist = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(H) * C * sort_tiles(N));
  w.chunk_prefix = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(H) * (C + 1));
  w.sizes = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(H) * C);
  w.partial = reinterpret_cast<float*>(p);
  return w;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void label_rank_kernel(const int32_t* __restrict__ labels,
                                                         int N, int C, int tiles,
                                                         int32_t* __restrict__ rank,
                                                         int32_t* __restrict__ hist) {
  extern __shared__ int wave_hist[];
  const int h = blockIdx.y, t = blockIdx.x, tid = threadIdx.x;
  const int n = t * kTile + tid;
  const bool valid = n < N;
  // labels outside [0, C) are clamped so that no access leaves its buffer
  const int label = valid ? min(max(labels[size_t(h) * N + n], 0), C - 1) : 0;
  const int r = tile_rank(label, valid, C, wave_hist);
  if (valid) rank[size_t(h) * N + n] = r;
  for (int c = tid; c < C; c += 256)
    hist[(size_t(h) * tiles + t) * C + c] =
        wave_hist[c] + wave_hist[C + c] + wave_hist[2 * C + c] + wave_hist[3 * C + c];
}

// Per (head, 64 clusters): exclusive prefix over tiles of the cluster counts,
// in place, and the cluster sizes. Each of the block's wavefronts sums a
// contiguous run of tiles (lane = cluster, so every read covers 64 adjacent
// counts of one tile), the runs' totals are combined in run order through LDS,
// and a second pass over the run writes the prefixes.
constexpr int kPrefixWaves = 16;
__global__ __launch_bounds__(64 * kPrefixWaves) void tile_prefix_kernel(int C, int tiles,
                                                                       int32_t* __restrict__ hist,
                                                                       int32_t* __restrict__ sizes) {
  __shared__ int run_sum[kPrefixWaves][64];
  const int h = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 64 + lane;
  const bool ok = c < C;
  const int per = (tiles + kPrefixWaves - 1) / kPrefixWaves;
  const int t0 = min(tiles, w * per), t1 = min(tiles, t0 + per);
  int32_t* col = hist + size_t(h) * tiles * C + (ok ? c : 0);
  // reads go out kBatch at a time, so a run costs a few memory round trips
  constexpr int kBatch = 24;
  int sum = 0;
  if (ok)
    for (int tb = t0; tb < t1; tb += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = (tb + i < t1) ? col[size_t(tb + i) * C] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) sum += v[i];
    }
  run_sum[w][lane] = sum;
  __syncthreads();
  int carry = 0;
  for (int i = 0; i < w; ++i) carry += run_sum[i][lane];
  if (ok) {
    for (int tb = t0; tb < t1; tb += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = (tb + i < t1) ? col[size_t(tb + i) * C] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (tb + i < t1) {
          col[size_t(tb + i) * C] = carry;
          carry += v[i];
        }
    }
    if (w == kPrefixWaves - 1) sizes[size_t(h) * C + c] = carry;
  }
}

// Per head: cluster offsets and the chunk list of the segment sums.
__global__ __launch_bounds__(1024) void cluster_offsets_kernel(int C,
                                                               const int32_t* __restrict__ sizes,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ chunk_prefix) {
  __shared__ int scratch[16];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int cnt = tid < C ? sizes[size_t(h) * C + tid] : 0;
  int total;
  const int ex = block_exclusive_scan(cnt, scratch, &total);
  const int chunks = (cnt + kChunk - 1) / kChunk;
  int ctotal;
  const int cex = block_exclusive_scan(chunks, scratch, &ctotal);
  if (tid < C) {
    offsets[size_t(h) * (C + 1) + tid] = ex;
    if (counts) counts[size_t(h) * C + tid] = cnt;
    chunk_prefix[size_t(h) * (C + 1) + tid] = cex;
  }
  if (tid == 0) {
    offsets[size_t(h) * (C + 1) + C] = total;
    chunk_prefix[size_t(h) * (C + 1) + C] = ctotal;
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ labels,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ tpre,
                                                      const int32_t* __restrict__ offsets, int N,
                                                      int C, int tiles,
                                                      int32_t* __restrict__ perm) {
  const int h = blockIdx.y, t = blockIdx.x;
  const int n = t * kTile + threadIdx.x;
  if (n >= N) return;
  const int lab = min(max(labels[size_t(h) * N + n], 0), C - 1);
  const int p = offsets[size_t(h) * (C + 1) + lab] + tpre[(size_t(h) * tiles + t) * C + lab] +
                rank[size_t(h) * N + n];
  perm[size_t(h) * N + p] = n;
}

// Cluster c owning chunk q: the largest c with chunk_prefix[c] <= q.
__device__ __forceinline__ int find_segment(const int32_t* prefix, int C, int q) {
  int lo = 0, hi = C;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= q) lo = mid; else hi = mid;
  }
  return lo;
}

struct Ptr3 {
  const void* p[3];
};
struct MutPtr3 {
  void* p[3];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void segsum_kernel(int N, int C, int nt, int maxch,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ chunk_prefix,
                                                     Ptr3 src, MutPtr3 dst,
                                                     float* __restrict__ partial) {
  constexpr int EPT = 16 / sizeof(T);       // elements per 16-byte access
  constexpr int TPR = D / EPT;              // threads per row
  constexpr int RPI = 256 / TPR;            // rows per iteration
  __shared__ float red[RPI][D];
  // heads in reverse launch order: the assignment pass before this one walked
  // them forwards, so the rows it read last are the ones still in the
  // last-level cache when this pass starts (and the next assignment, walking
  // forwards again, starts on what this pass read last)
  const int h = int(gridDim.y) - 1 - int(blockIdx.y), q = blockIdx.x, tid = threadIdx.x;
  const int32_t* cp = chunk_prefix + size_t(h) * (C + 1);
  if (q >= cp[C]) return;
  const int c = find_segment(cp, C, q);
  const int32_t* off = offsets + size_t(h) * (C + 1);
  const int p0 = off[c] + (q - cp[c]) * kChunk;
  const int p1 = min(off[c + 1], p0 + kChunk);
  const int rg = tid / TPR, col = tid % TPR;
  // the chunk's source rows, read once (coalesced) for every tensor
  __shared__ int prow[kChunk];
  const int len = p1 - p0;
  for (int i = tid; i < len; i += 256) prow[i] = perm[size_t(h) * N + p0 + i];
  __syncthreads();
  for (int k = 0; k < nt; ++k) {
    const T* s = static_cast<const T*>(src.p[k]) + size_t(h) * N * D;
    T* dd = dst.p[k] ? static_cast<T*>(dst.p[k]) + size_t(h) * N * D : nullptr;
    float acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
    // sixteen rows in flight per thread; rows are still added in slot order
    constexpr int U = 16;
    for (int j = rg; j < len; j += U * RPI) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int jj = j + u * RPI;
        v[u] = jj < len ? *reinterpret_cast<const uint4*>(s + size_t(prow[jj]) * D + col * EPT)
                        : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int jj = j + u * RPI;
        if (jj >= len) break;
        if (dd) *reinterpret_cast<uint4*>(dd + size_t(p0 + jj) * D + col * EPT) = v[u];
        const T* el = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] += to_f32(el[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) red[rg][col * EPT + e] = acc[e];
    __syncthreads();
    if (tid < D) {
      float sum = 0.f;
      for (int r = 0; r < RPI; ++r) sum += red[r][tid];
      partial[((size_t(h) * nt + k) * maxch + q) * D + tid] = sum;
    }
    __syncthreads();
  }
}

struct FPtr3 {
  float* p[3];
};

// One wavefront per cluster (four per block), each lane holding dims lane and
// lane + 64: the chunk sums of a dim are added in chunk order as before, and
// ||round(mean)||^2 is the same two 64-lane shuffle trees added in the same
// order, so the results are bitwise those of one thread per dim.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(int C, int nt, int maxch,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ chunk_prefix,
                                                     const float* __restrict__ partial, FPtr3 means,
                                                     int mode, T* __restrict__ table,
                                                     float* __restrict__ norms) {
  constexpr int EPL = D / 64;  // dims per lane
  const int h = blockIdx.y, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= C) return;  // a whole wavefront; nothing below synchronises the block
  const int32_t* off = offsets + size_t(h) * (C + 1);
  const int32_t* cp = chunk_prefix + size_t(h) * (C + 1);
  const int n = off[c + 1] - off[c];
  const int q0 = cp[c], q1 = cp[c + 1];
  for (int k = 0; k < nt; ++k) {
    float* mk = means.p[k];
    float m[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int j = lane + 64 * e;
      if (n > 0) {
        float s = 0.f;
        for (int q = q0; q < q1; ++q) s += partial[((size_t(h) * nt + k) * maxch + q) * D + j];
        m[e] = s / float(n);
      } else {
        m[e] = (mode == 0 || !mk) ? 0.f : mk[(size_t(h) * C + c) * D + j];
      }
      if (mk) mk[(size_t(h) * C + c) * D + j] = m[e];
    }
    if (k == 0 && table) {
      float sq[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int j = lane + 64 * e;
        const T r = from_f32<T>(m[e]);
        const float rf = to_f32(r);
        table[(size_t(h) * C + c) * D + j] = from_f32<T>(-2.f * rf);
        sq[e] = rf * rf;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sq[e] += __shfl_xor(sq[e], o, 64);
      }
      if (lane == 0) norms[size_t(h) * C + c] = (D > 64) ? sq[0] + sq[EPL - 1] : sq[0];
    }
  }
}

__global__ void unpermute_kernel(int N, int cpr, const int32_t* __restrict__ perm,
                                 const uint4* __restrict__ Xp, uint4* __restrict__ X) {
  const int h = blockIdx.y;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= size_t(N) * cpr) return;
  const int p = int(idx / cpr), k = int(idx % cpr);
  const int row = perm[size_t(h) * N + p];
  X[(size_t(h) * N + row) * cpr + k] = Xp[(size_t(h) * N + p) * cpr + k];
}

// ---------------------------------------------------------------------------
hipError_t launch_label_rank(const int32_t* labels, int H, int N, int C, int32_t* rank,
                             int32_t* hist, hipStream_t s) {
  const int tiles = sort_tiles(N);
  hipLaunchKernelGGL(label_rank_kernel, dim3(tiles, H), dim3(256), 4 * C * sizeof(int), s, labels,
                     N, C, tiles, rank, hist);
  return hipGetLastError();
}

hipError_t launch_sort_scan(int H, int N, int C, int32_t* hist, int32_t* sizes, int32_t* offsets,
                            int32_t* counts, int32_t* chunk_prefix, hipStream_t s) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(ceil_div(C, 64), H), dim3(64 * kPrefixWaves), 0, s,
                     C,
                     sort_tiles(N), hist, sizes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cluster_offsets_kernel, dim3(H), dim3(1024), 0, s, C, sizes, offsets, counts,
                     chunk_prefix);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* labels, const int32_t* rank, const int32_t* hist,
                          const int32_t* offsets, int H, int N, int C, int32_t* perm,
                          hipStream_t s) {
  const int tiles = sort_tiles(N);
  hipLaunchKernelGGL(scatter_kernel, dim3(tiles, H), dim3(256), 0, s, labels, rank, hist, offsets,
                     N, C, tiles, perm);
  return hipGetLastError();
}

template <typename T, int D>
static void segsum_t(int H, int N, int C, const int32_t* perm, const int32_t* offsets,
                     const int32_t* cp, int nt, const void* const* src, void* const* dst,
                     float* partial, hipStream_t s) {
  Ptr3 sp{};
  MutPtr3 dp{};
  for (int k = 0; k < nt; ++k) {
    sp.p[k] = src[k];
    dp.p[k] = dst ? dst[k] : nullptr;
  }
  const int maxch = max_chunks(N, C);
  hipLaunchKernelGGL((segsum_kernel<T, D>), dim3(maxch, H), dim3(256), 0, s, N, C, nt, maxch,
                     perm, offsets, cp, sp, dp, partial);
}

hipError_t launch_segsum(int elem_bytes, int H, int N, int d, int C, const int32_t* perm,
                         const int32_t* offsets, const int32_t* chunk_prefix, int ntensors,
                         const void* const* src, void* const* dst, float* partial,
                         hipStream_t s) {
  if (elem_bytes == 2) {
    if (d == 128) segsum_t<__bf16, 128>(H, N, C, perm, offsets, chunk_prefix, ntensors, src, dst, partial, s);
    else segsum_t<__bf16, 64>(H, N, C, perm, offsets, chunk_prefix, ntensors, src, dst, partial, s);
  } else {
    if (d == 128) segsum_t<float, 128>(H, N, C, perm, offsets, chunk_prefix, ntensors, src, dst, partial, s);
    else segsum_t<float, 64>(H, N, C, perm, offsets, chunk_prefix, ntensors, src, dst, partial, s);
  }
  return hipGetLastError();
}

template <typename T, int D>
static void combine_t(int H, int C, int nt, const int32_t* offsets, const int32_t* cp,
                      const float* partial, int N, float* const* means, int mode, void* table,
                      float* norms, hipStream_t s) {
  FPtr3 mp{};
  for (int k = 0; k < nt; ++k) mp.p[k] = means ? means[k] : nullptr;
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(ceil_div(C, 4), H), dim3(256), 0, s, C, nt,
                     max_chunks(N, C),
                     offsets, cp, partial, mp, mode, static_cast<T*>(table), norms);
}

hipError_t launch_combine(int elem_bytes, int H, int d, int C, int ntensors,
                          const int32_t* offsets, const int32_t* chunk_prefix,
                          const float* partial, int N, float* const* means, int mode,
                          void* table, float* norms, hipStream_t s) {
  if (elem_bytes == 2) {
    if (d == 128) combine_t<__bf16, 128>(H, C, ntensors, offsets, chunk_prefix, partial, N, means, mode, table, norms, s);
    else combine_t<__bf16, 64>(H, C, ntensors, offsets, chunk_prefix, partial, N, means, mode, table, norms, s);
  } else {
    if (d == 128) combine_t<float, 128>(H, C, ntensors, offsets, chunk_prefix, partial, N, means, mode, table, norms, s);
    else combine_t<float, 64>(H, C, ntensors, offsets, chunk_prefix, partial, N, means, mode, table, norms, s);
  }
  return hipGetLastError();
}

hipError_t launch_unpermute(int elem_bytes, int H, int N, int d, const int32_t* perm,
                            const void* Xp, void* X, hipStream_t s) {
  const int cpr = d * elem_bytes / 16;
  const size_t total = size_t(N) * cpr;
  const int blocks = int((total + 255) / 256);
  hipLaunchKernelGGL(unpermute_kernel, dim3(blocks, H), dim3(256), 0, s, N, cpr, perm,
                     static_cast<const uint4*>(Xp), static_cast<uint4*>(X));
  return hipGetLastError();
}

}  // namespace svg
