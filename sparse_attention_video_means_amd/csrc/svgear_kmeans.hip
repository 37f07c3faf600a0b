// k-means assignment on matrix cores (paper §4.1: Q and K are clustered with
// k-means before permutation).
//
// Each block takes 256 rows of one head. Its four wavefronts keep their 64
// rows as MFMA B operands in registers and stream the centroid table through
// LDS in chunks of 128 centroids (64 for f32), fetching the next chunk into
// registers while the current one is multiplied. The table already holds
// -2 * round(mu) in the input element type and ||round(mu)||^2 in f32, so one
// chain of MFMAs seeded with the norms yields ||mu||^2 - 2 x.mu directly. Each
// lane keeps a running (distance, index) minimum over the centroids it sees in
// increasing index order, two candidates at a time; four lanes share a row and
// are merged with the lower index winning ties. The block then ranks its rows
// among equal labels (for the counting sort that follows) without atomics.
#include "svgear_common.hpp"
#include "svgear_internal.hpp"

namespace svg {


template <typename T, int D>
__global__ __launch_bounds__(256) void assign_kernel(const T* __restrict__ X,
                                                     const T* __restrict__ table,
                                                     const float* __restrict__ norms, int N, int C,
                                                     int tiles, int32_t* __restrict__ labels,
                                                     int32_t* __restrict__ rank,
                                                     int32_t* __restrict__ hist) {
  constexpr int KC = D / 32;                       // 32-wide k chunks
  // centroids staged per LDS pass (f32 rows are twice as wide: half as many)
  constexpr int kAssignChunk = sizeof(T) == 2 ? 128 : 64;
  constexpr int LDR = D + 16 / sizeof(T);          // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) T tab[kAssignChunk * LDR];
  __shared__ float nrm[kAssignChunk];
  __shared__ int wave_hist[4 * kMaxClusters];

  const int h = blockIdx.y, t = blockIdx.x, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int row0 = t * kTile + w * 64;
  const T* Xh = X + size_t(h) * N * D;

  Frag<T> xb[4][KC];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int n = row0 + tb * 16 + r;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      xb[tb][kc] = (n < N) ? load8(Xh + size_t(n) * D + kc * 32 + g * 8) : zero_frag<T>();
  }

  float best[4];
  int bidx[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) { best[tb] = __builtin_inff(); bidx[tb] = 0; }

  const T* tabh = table + size_t(h) * C * D;
  const float* nrmh = norms + size_t(h) * C;
  constexpr int EPT = 16 / sizeof(T);
  constexpr int CPR = D / EPT;                      // 16-byte pieces per row
  constexpr int PPT = kAssignChunk * CPR / 256;     // pieces per thread per chunk
  // The next chunk of the table is fetched into registers while the current
  // one is multiplied, so the table's load latency is paid once per block.
  uint4 pre[PPT];
  float pre_nrm = 0.f;
  auto fetch = [&](int cbase) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int i = tid + p * 256, row = i / CPR, piece = i % CPR;
      pre[p] = (cbase + row < C)
                   ? *reinterpret_cast<const uint4*>(tabh + size_t(cbase + row) * D + piece * EPT)
                   : make_uint4(0, 0, 0, 0);
    }
    if (tid < kAssignChunk) pre_nrm = (cbase + tid < C) ? nrmh[cbase + tid] : __builtin_inff();
  };
  fetch(0);
  for (int cbase = 0; cbase < C; cbase += kAssignChunk) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int i = tid + p * 256, row = i / CPR, piece = i % CPR;
      *reinterpret_cast<uint4*>(&tab[row * LDR + piece * EPT]) = pre[p];
    }
    if (tid < kAssignChunk) nrm[tid] = pre_nrm;
    __syncthreads();
    if (cbase + kAssignChunk < C) fetch(cbase + kAssignChunk);
    const int nblk = min(kAssignChunk, C - cbase + 15) / 16;
    for (int cb = 0; cb < nblk; ++cb) {
      Frag<T> a[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) a[kc] = load8(&tab[(cb * 16 + r) * LDR + kc * 32 + g * 8]);
      f32x4 init;
#pragma unroll
      for (int i = 0; i < 4; ++i) init[i] = nrm[cb * 16 + g * 4 + i];
      const int c0 = cbase + cb * 16 + g * 4;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 acc = init;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) mma(acc, a[kc], xb[tb][kc]);
        // two candidates per step: the new minimum of (best, a, b) in one
        // instruction, then its index; ties keep the lower index (the running
        // best, then a before b)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float nb = __builtin_fminf(best[tb], __builtin_fminf(acc[i], acc[i + 1]));
          const bool keep = nb == best[tb];
          const int cand = (nb == acc[i]) ? c0 + i : c0 + i + 1;
          bidx[tb] = keep ? bidx[tb] : cand;
          best[tb] = nb;
        }
      }
    }
  }

  // merge the four lanes that hold the same row (lanes r, r+16, r+32, r+48)
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float ob = __shfl_xor(best[tb], o, 64);
      const int oi = __shfl_xor(bidx[tb], o, 64);
      if (ob < best[tb] || (ob == best[tb] && oi < bidx[tb])) { best[tb] = ob; bidx[tb] = oi; }
    }
  }
  // lane (g, r) now owns row row0 + 16 g + r = row0 + lane. (Padding
  // centroids past C carry an infinite norm and never win; the clamp keeps
  // the rank, the histogram and the scatter that reads them in range anyway.)
  int my = bidx[0];
#pragma unroll
  for (int tb = 1; tb < 4; ++tb) my = (g == tb) ? bidx[tb] : my;
  my = min(my, C - 1);
  const int n = row0 + lane;
  const bool valid = n < N;
  if (valid) labels[size_t(h) * N + n] = my;
  const int rk = tile_rank(my, valid, C, wave_hist);
  if (valid) rank[size_t(h) * N + n] = rk;
  for (int c = tid; c < C; c += 256)
    hist[(size_t(h) * tiles + t) * C + c] =
        wave_hist[c] + wave_hist[C + c] + wave_hist[2 * C + c] + wave_hist[3 * C + c];
}

// table = -2 * round_T(mu), norms = ||round_T(mu)||^2 for the first assignment.
template <typename T, int D>
__global__ __launch_bounds__(D) void table_kernel(int C, const float* __restrict__ mu,
                                                  T* __restrict__ table, float* __restrict__ norms) {
  __shared__ float wsum[2];
  const int h = blockIdx.y, c = blockIdx.x, j = threadIdx.x;
  const size_t i = (size_t(h) * C + c) * D + j;
  const float rf = to_f32(from_f32<T>(mu[i]));
  table[i] = from_f32<T>(-2.f * rf);
  float sq = rf * rf;
  for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
  if ((j & 63) == 0) wsum[j >> 6] = sq;
  __syncthreads();
  if (j == 0) norms[size_t(h) * C + c] = (D > 64) ? wsum[0] + wsum[1] : wsum[0];
}

hipError_t launch_table(int elem_bytes, int H, int d, int C, const float* mu, void* table,
                        float* norms, hipStream_t s) {
  const dim3 grid(C, H);
  if (elem_bytes == 2) {
    if (d == 128) hipLaunchKernelGGL((table_kernel<__bf16, 128>), grid, dim3(128), 0, s, C, mu, (__bf16*)table, norms);
    else hipLaunchKernelGGL((table_kernel<__bf16, 64>), grid, dim3(64), 0, s, C, mu, (__bf16*)table, norms);
  } else {
    if (d == 128) hipLaunchKernelGGL((table_kernel<float, 128>), grid, dim3(128), 0, s, C, mu, (float*)table, norms);
    else hipLaunchKernelGGL((table_kernel<float, 64>), grid, dim3(64), 0, s, C, mu, (float*)table, norms);
  }
  return hipGetLastError();
}

hipError_t launch_assign(int elem_bytes, int H, int N, int d, int C, const void* X,
                         const void* table, const float* norms, int32_t* labels, int32_t* rank,
                         int32_t* hist, hipStream_t s) {
  const int tiles = sort_tiles(N);
  const dim3 grid(tiles, H), block(256);
  if (elem_bytes == 2) {
    if (d == 128)
      hipLaunchKernelGGL((assign_kernel<__bf16, 128>), grid, block, 0, s, (const __bf16*)X,
                         (const __bf16*)table, norms, N, C, tiles, labels, rank, hist);
    else
      hipLaunchKernelGGL((assign_kernel<__bf16, 64>), grid, block, 0, s, (const __bf16*)X,
                         (const __bf16*)table, norms, N, C, tiles, labels, rank, hist);
  } else {
    if (d == 128)
      hipLaunchKernelGGL((assign_kernel<float, 128>), grid, block, 0, s, (const float*)X,
                         (const float*)table, norms, N, C, tiles, labels, rank, hist);
    else
      hipLaunchKernelGGL((assign_kernel<float, 64>), grid, block, 0, s, (const float*)X,
                         (const float*)table, norms, N, C, tiles, labels, rank, hist);
  }
  return hipGetLastError();
}

}  // namespace svg
