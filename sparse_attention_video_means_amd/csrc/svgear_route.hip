// Greedy error-to-cost routers (paper §4.2 "Error estimation": highest
// error-to-size ratio first until the budget is exhausted).
//
// route_kernel: one block per (head, query cluster), a budget of exact keys
// per query cluster (§5 "Implementation": routing per query cluster).
//
// The block sorts the key clusters by the 64-bit key (~bits(ratio) << 32 | id)
// with a bitonic network in LDS: for non-negative f32 the bit pattern orders
// like the value, so ascending keys are "ratio descending, index ascending".
// Empty key clusters get the all-ones key and sort last. One thread then
// walks the order and keeps every cluster that still fits the budget, and the
// block writes the mask, the ascending list, the count and the keys used.
#include "svgear_common.hpp"
#include "svgear_internal.hpp"

namespace svg {

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ ratio,
                                                    const int32_t* __restrict__ qoff,
                                                    const int32_t* __restrict__ koff, int Cq,
                                                    int Ck, int P, int budget_keys,
                                                    uint8_t* __restrict__ mask,
                                                    int32_t* __restrict__ list,
                                                    int32_t* __restrict__ count,
                                                    int32_t* __restrict__ keys) {
  __shared__ uint64_t key[kMaxClusters];
  __shared__ int cnt[kMaxClusters];
  __shared__ int sel[kMaxClusters];
  __shared__ int scratch[16];
  __shared__ int used_s;
  const int h = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  const float* rr = ratio + (size_t(h) * Cq + c) * Ck;
  // a query cluster without queries has no row to route: it selects nothing
  const int32_t* qo = qoff ? qoff + size_t(h) * (Cq + 1) : nullptr;
  const int budget = (qo && qo[c + 1] - qo[c] <= 0) ? 0 : budget_keys;
  for (int i = tid; i < P; i += 256) {
    uint64_t k = ~0ull;
    if (i < Ck) {
      const int n = ko[i + 1] - ko[i];
      cnt[i] = n;
      sel[i] = 0;
      if (n > 0) {
        const float v = rr[i];
        const uint32_t b = (v > 0.f) ? __float_as_uint(v) : 0u;  // NaN and negatives count as 0
        k = (uint64_t(~b) << 32) | uint32_t(i);
      }
    }
    key[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= (budget > 0 ? P : 1); k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += 256) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = key[i], b = key[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) { key[i] = b; key[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
  // Greedy fill by wavefront 0, 64 candidates at a time: within a window the
  // first candidate (in order) that fits is taken, the budget shrinks, and the
  // search resumes after it. Candidates passed over did not fit when their turn
  // came and the remaining budget only shrinks, so this is the same walk as a
  // one-at-a-time loop.
  if (tid < 64) {
    const int lane = tid;
    int rem = budget;
    for (int base = 0; base < Ck && rem > 0; base += 64) {
      const int i = base + lane;
      const uint64_t k = (i < Ck) ? key[i] : ~0ull;
      const bool valid = k != ~0ull;
      const int id = valid ? int(uint32_t(k)) : 0;
      const int n = valid ? cnt[id] : 0;
      uint64_t pending = __ballot(valid);
      while (pending) {
        const uint64_t fits = __ballot(valid && n <= rem) & pending;
        if (!fits) break;
        const int f = __ffsll((unsigned long long)fits) - 1;
        const int nf = __shfl(n, f, 64);
        if (lane == f) sel[id] = 1;
        rem -= nf;
        pending &= (f == 63) ? 0ull : (~0ull << (f + 1));
      }
      if (__ballot(!valid)) break;  // the sorted keys of empty clusters start here
    }
    if (lane == 0) used_s = budget - rem;
  }
  __syncthreads();
  uint8_t* mk = mask + (size_t(h) * Cq + c) * Ck;
  for (int i = tid; i < Ck; i += 256) mk[i] = uint8_t(sel[i]);
  int carry = 0;
  int32_t* ls = list ? list + (size_t(h) * Cq + c) * Ck : nullptr;
  for (int b = 0; b < Ck; b += 256) {
    const int i = b + tid;
    const int f = (i < Ck) ? sel[i] : 0;
    int tot;
    const int ex = block_exclusive_scan(f, scratch, &tot);
    if (ls && f) ls[carry + ex] = i;
    carry += tot;
  }
  if (ls)
    for (int i = carry + tid; i < Ck; i += 256) ls[i] = -1;
  if (tid == 0) {
    if (count) count[size_t(h) * Cq + c] = carry;
    if (keys) keys[size_t(h) * Cq + c] = used_s;
  }
}

// ---- one budget for the whole head ------------------------------------------
//
// route_global_kernel (paper §4.1: at most rho * Nq * Nk exact entries in the
// block mask of the map; §4.2: greedy by ratio): one 1024-thread block per
// head. Every block (c, c') of the map gets a 32-bit key that orders ratio
// descending (non-negative f32 bit patterns order like their values; NaN and
// negatives count as 0) and puts blocks of empty clusters last. A stable LSD
// radix sort on 8-bit digits, carrying the flat index c * Ck + c', leaves equal
// ratios in index order, i.e. lower query cluster first, then lower key
// cluster. Digits that every key shares are skipped. The block then walks
// the order with the entry budget: whole 1024-block chunks are taken by
// prefix sum while they fit; from the first chunk that overflows on, blocks
// are taken one at a time in order while they still fit.
// route_lists_kernel turns each mask row into the ascending list, the count
// and the exact keys of the query cluster.

constexpr int kGrThreads = 1024;
constexpr int kGrWaves = kGrThreads / 64;
constexpr uint32_t kGrDead = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t global_key(float v, bool live) {
  if (!live) return kGrDead;
  const uint32_t b = (v > 0.f) ? min(__float_as_uint(v), 0x7F800000u) : 0u;
  return 0x7F800000u - b;
}

__device__ __forceinline__ int64_t shfl64(int64_t v, int src) {
  const int lo = __shfl(int(uint32_t(v)), src, 64), hi = __shfl(int(v >> 32), src, 64);
  return (int64_t(hi) << 32) | uint32_t(lo);
}

__device__ __forceinline__ int64_t wave_inclusive_scan64(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int lo = __shfl_up(int(uint32_t(v)), o, 64), hi = __shfl_up(int(v >> 32), o, 64);
    if (lane >= o) v += (int64_t(hi) << 32) | uint32_t(lo);
  }
  return v;
}

__global__ __launch_bounds__(kGrThreads) void route_global_kernel(
    const float* __restrict__ ratio, const int32_t* __restrict__ qoff,
    const int32_t* __restrict__ koff, int Cq, int Ck, int64_t budget,
    uint8_t* __restrict__ mask, int64_t* __restrict__ used_out, uint32_t* __restrict__ wkeys,
    int32_t* __restrict__ widx) {
  __shared__ int hist_s[4][256];
  __shared__ int base_s[256];
  __shared__ int wc_s[2][kGrWaves][256];  // per-wave digit counts, two tiles in flight
  __shared__ int nq_s[kMaxClusters], nk_s[kMaxClusters];
  __shared__ int scan_s[kGrWaves];
  __shared__ int64_t tot_s[kGrWaves];
  __shared__ int64_t cand_cost_s[kGrThreads];
  __shared__ int cand_idx_s[kGrThreads];
  __shared__ int64_t used_s;
  const int h = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n = Cq * Ck;
  uint32_t* ka = wkeys + size_t(h) * 2 * n;
  uint32_t* kb = ka + n;
  int32_t* ia = widx + size_t(h) * 2 * n;
  int32_t* ib = ia + n;
  uint8_t* mh = mask + size_t(h) * n;
  const float* rh = ratio + size_t(h) * n;

  for (int c = tid; c < Cq; c += kGrThreads)
    nq_s[c] = qoff[size_t(h) * (Cq + 1) + c + 1] - qoff[size_t(h) * (Cq + 1) + c];
  for (int c = tid; c < Ck; c += kGrThreads)
    nk_s[c] = koff[size_t(h) * (Ck + 1) + c + 1] - koff[size_t(h) * (Ck + 1) + c];
  for (int i = tid; i < 4 * 256; i += kGrThreads) (&hist_s[0][0])[i] = 0;
  for (int i = tid; i < 2 * kGrWaves * 256; i += kGrThreads) (&wc_s[0][0][0])[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kGrThreads) {
    const int c = i / Ck, j = i - c * Ck;
    const uint32_t key = global_key(rh[i], nq_s[c] > 0 && nk_s[j] > 0);
    ka[i] = key;
    ia[i] = i;
    mh[i] = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) atomicAdd(&hist_s[p][(key >> (8 * p)) & 255], 1);
  }
  __syncthreads();

  uint32_t *ks = ka, *kd = kb;
  int32_t *is = ia, *id = ib;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int p = 0; p < 4; ++p) {
    if (__syncthreads_or(tid < 256 && hist_s[p][tid] == n)) continue;  // one digit value
    int tot;
    const int ex = block_exclusive_scan(tid < 256 ? hist_s[p][tid] : 0, scan_s, &tot);
    if (tid < 256) base_s[tid] = ex;
    __syncthreads();
    // Tile k (1024 keys) counts into wc_s[k & 1]; the table is cleared while
    // tile k + 1 counts into the other one, so two barriers per tile suffice.
    // The next tile's keys are loaded while this one is ranked.
    uint32_t key_n = (tid < n) ? ks[tid] : 0u;
    int32_t idx_n = (tid < n) ? is[tid] : 0;
    for (int t = 0, k = 0; t < n; t += kGrThreads, ++k) {
      const int i = t + tid;
      const bool valid = i < n;
      const uint32_t key = key_n;
      const int32_t idx = idx_n;
      if (i + kGrThreads < n) {
        key_n = ks[i + kGrThreads];
        idx_n = is[i + kGrThreads];
      }
      int(*wc)[256] = wc_s[k & 1];
      const int dg = (key >> (8 * p)) & 255;
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bool bit = (dg >> b) & 1;
        const uint64_t bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      const int rank_w = __popcll(peers & below);
      if (valid && rank_w == 0) wc[w][dg] = __popcll(peers);
      __syncthreads();
      if (valid) {
        int off = base_s[dg] + rank_w;
        for (int v = 0; v < w; ++v) off += wc[v][dg];
        kd[off] = key;
        id[off] = idx;
      }
      __syncthreads();
      if (tid < 256) {
        int add = 0;
        for (int v = 0; v < kGrWaves; ++v) {
          add += wc[v][tid];
          wc[v][tid] = 0;
        }
        base_s[tid] += add;
      }
    }
    __syncthreads();
    uint32_t* tk = ks; ks = kd; kd = tk;
    int32_t* ti = is; is = id; id = ti;
  }

  // Fill, 1024 sorted blocks at a time. Until the first chunk that does not
  // fit whole, chunks are taken by a block-wide prefix sum of their costs.
  // From that chunk on, the blocks that could still fit (cost <= the budget
  // left at the start of the chunk; the budget only shrinks) are compacted in
  // order into LDS and wavefront 0 walks them one at a time.
  bool over = false;
  int64_t used = 0;  // the same in every thread
  for (int t = 0; t < n; t += kGrThreads) {
    const int i = t + tid;
    const uint32_t key = (i < n) ? ks[i] : kGrDead;
    const bool live = key != kGrDead;
    if (!__syncthreads_or(live)) break;  // the blocks of empty clusters sort last
    const int idx = live ? is[i] : 0;
    const int c = idx / Ck, j = idx - c * Ck;
    const int64_t cost = live ? int64_t(nq_s[c]) * nk_s[j] : 0;
    if (!over) {
      const int64_t incl = wave_inclusive_scan64(cost);
      if (lane == 63) tot_s[w] = incl;
      __syncthreads();
      int64_t total = 0;
      for (int v = 0; v < kGrWaves; ++v) total += tot_s[v];
      __syncthreads();
      if (used + total <= budget) {
        if (live) mh[idx] = 1;
        used += total;
        continue;
      }
      over = true;
    }
    const bool cand = live && cost <= budget - used;
    int ncand;
    const int pos = block_exclusive_scan(cand ? 1 : 0, scan_s, &ncand);
    if (cand) {
      cand_cost_s[pos] = cost;
      cand_idx_s[pos] = idx;
    }
    __syncthreads();
    if (w == 0) {
      for (int b = 0; b < ncand; b += 64) {
        const int q = b + lane;
        const bool in = q < ncand;
        const int64_t cq = in ? cand_cost_s[q] : 0;
        uint64_t pending = __ballot(in);
        while (pending) {
          const uint64_t fits = __ballot(in && used + cq <= budget) & pending;
          if (!fits) break;
          const int f = __ffsll((unsigned long long)fits) - 1;
          if (lane == f) mh[cand_idx_s[q]] = 1;
          used += shfl64(cq, f);
          pending &= (f == 63) ? 0ull : (~0ull << (f + 1));
        }
      }
      if (lane == 0) used_s = used;
    }
    __syncthreads();
    used = used_s;
  }
  if (tid == 0 && used_out) used_out[h] = used;
}

__global__ __launch_bounds__(64) void route_lists_kernel(const uint8_t* __restrict__ mask,
                                                         const int32_t* __restrict__ koff,
                                                         int Cq, int Ck,
                                                         int32_t* __restrict__ list,
                                                         int32_t* __restrict__ count,
                                                         int32_t* __restrict__ keys) {
  const int h = blockIdx.y, c = blockIdx.x, lane = threadIdx.x;
  const uint8_t* mr = mask + (size_t(h) * Cq + c) * Ck;
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  int32_t* ls = list ? list + (size_t(h) * Cq + c) * Ck : nullptr;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int carry = 0, ksum = 0;
  for (int b = 0; b < Ck; b += 64) {
    const int j = b + lane;
    const bool m = j < Ck && mr[j] != 0;
    const uint64_t bal = __ballot(m);
    if (m) {
      if (ls) ls[carry + __popcll(bal & below)] = j;
      ksum += ko[j + 1] - ko[j];
    }
    carry += __popcll(bal);
  }
  if (ls)
    for (int j = carry + lane; j < Ck; j += 64) ls[j] = -1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ksum += __shfl_xor(ksum, o, 64);
  if (lane == 0) {
    if (count) count[size_t(h) * Cq + c] = carry;
    if (keys) keys[size_t(h) * Cq + c] = ksum;
  }
}

size_t route_global_ws_bytes(int H, int Cq, int Ck) {
  return size_t(H) * Cq * Ck * 2 * (sizeof(uint32_t) + sizeof(int32_t));
}

hipError_t launch_route_global(int H, int Cq, int Ck, const float* ratio, const int32_t* qoff,
                               const int32_t* koff, int64_t budget, uint8_t* mask,
                               int32_t* list, int32_t* count, int32_t* keys, int64_t* used,
                               void* ws, hipStream_t s) {
  uint32_t* wkeys = static_cast<uint32_t*>(ws);
  int32_t* widx = reinterpret_cast<int32_t*>(wkeys + size_t(H) * Cq * Ck * 2);
  hipLaunchKernelGGL(route_global_kernel, dim3(H), dim3(kGrThreads), 0, s, ratio, qoff, koff, Cq,
                     Ck, budget, mask, used, wkeys, widx);
  hipLaunchKernelGGL(route_lists_kernel, dim3(Cq, H), dim3(64), 0, s, mask, koff, Cq, Ck, list,
                     count, keys);
  return hipGetLastError();
}

hipError_t launch_route(int H, int Cq, int Ck, const float* ratio, const int32_t* qoff,
                        const int32_t* koff, int32_t budget, uint8_t* mask, int32_t* list,
                        int32_t* count, int32_t* keys, hipStream_t s) {
  int P = 1;
  while (P < Ck) P <<= 1;
  hipLaunchKernelGGL(route_kernel, dim3(Cq, H), dim3(256), 0, s, ratio, qoff, koff, Cq, Ck, P,
                     budget, mask, list, count, keys);
  return hipGetLastError();
}

}  // namespace svg
