// Greedy error-to-cost routers (paper §4.2, error estimation: blocks are
// taken in decreasing order of estimated error per entry while the budget
// lasts).
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
// Global routing (paper §4.1: at most rho * Nq * Nk exact entries in the block
// mask of the map; §4.2: greedy by ratio). Every block (c, c') of the map gets
// a 32-bit key that orders ratio descending (non-negative f32 bit patterns
// order like their values; NaN and negatives count as 0) and puts blocks of
// empty clusters last. A stable LSD radix sort in four passes of 8-bit digits,
// carrying the flat index c * Ck + c', leaves equal ratios in index order,
// i.e. lower query cluster first, then lower key cluster. Each pass is spread
// over tiles of 2048 entries of every head: a digit histogram per tile, then
// a scatter in which each tile finds its digits' first output positions from
// the histograms, ranks its entries stably per digit, sorts them by digit in
// LDS and writes each digit's run contiguously. The fill then takes the sorted
// blocks in order while their costs n_q n_k fit the budget: per-tile cost sums
// locate the first block that does not fit (every block before it is taken);
// from there on one wavefront walks the tiles whose cheapest block still fits
// the budget left and takes, in order, every block that fits, until no
// remaining block is cheap enough (per-tile minimum costs).
// route_lists_kernel completes each mask row (the blocks sorted before the
// first misfit, plus those the walk took) and turns it into the ascending
// list, the count and the exact keys of the query cluster.

constexpr int kGtThreads = 256;   // threads per tile block
constexpr int kGtPer = 8;         // entries per thread
constexpr int kGtTile = kGtThreads * kGtPer;
constexpr int kGtBins = 256;      // 8-bit digits
constexpr int kGtPasses = 4;
constexpr int kGtMaxTiles = (kMaxClusters * kMaxClusters + kGtTile - 1) / kGtTile;
constexpr uint32_t kGrDead = 0xFFFFFFFFu;
constexpr int64_t kGtNoCost = 0x7FFFFFFFFFFFFFFFll;

__device__ __forceinline__ uint32_t global_key(float v, bool live) {
  if (!live) return kGrDead;
  const uint32_t b = (v > 0.f) ? min(__float_as_uint(v), 0x7F800000u) : 0u;
  return 0x7F800000u - b;
}

__device__ __forceinline__ int gt_digit(uint32_t key, int pass) {
  return int(key >> (8 * pass)) & (kGtBins - 1);
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

// exclusive prefix over the block (int64); scratch holds one value per wavefront
__device__ __forceinline__ int64_t block_exclusive_scan64(int64_t v, int64_t* scratch,
                                                          int64_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int64_t inc = wave_inclusive_scan64(v);
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int i = 0; i < nw; ++i) {
    const int64_t x = scratch[i];
    before += (i < w) ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Pass 0's tile: the keys from the ratios, the identity index, a cleared mask
// and the tile's histogram of the first digit (hist[h][tile][digit]).
__global__ __launch_bounds__(kGtThreads) void gt_keys_kernel(
    const float* __restrict__ ratio, const int32_t* __restrict__ qoff,
    const int32_t* __restrict__ koff, int Cq, int Ck, int T, uint32_t* __restrict__ ka,
    int32_t* __restrict__ ia, uint8_t* __restrict__ mask, int32_t* __restrict__ hist) {
  __shared__ int cnt[kGtBins];
  __shared__ uint8_t nq_live[kMaxClusters], nk_live[kMaxClusters];
  const int h = blockIdx.y, t = blockIdx.x, tid = threadIdx.x;
  const int n = Cq * Ck;
  const int32_t* qo = qoff + size_t(h) * (Cq + 1);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  cnt[tid] = 0;
  for (int c = tid; c < Cq; c += kGtThreads) nq_live[c] = qo[c + 1] > qo[c];
  for (int c = tid; c < Ck; c += kGtThreads) nk_live[c] = ko[c + 1] > ko[c];
  __syncthreads();
  const size_t hb = size_t(h) * n;
  // every load first, unconditional from clamped positions (no branch per
  // element), then the work
  float rv[kGtPer];
#pragma unroll
  for (int e = 0; e < kGtPer; ++e) rv[e] = ratio[hb + min(t * kGtTile + e * kGtThreads + tid, n - 1)];
#pragma unroll
  for (int e = 0; e < kGtPer; ++e) {
    const int i = t * kGtTile + e * kGtThreads + tid;
    if (i < n) {
      const int c = i / Ck, j = i - c * Ck;
      const uint32_t key = global_key(rv[e], nq_live[c] && nk_live[j]);
      ka[hb + i] = key;
      ia[hb + i] = i;
      mask[hb + i] = 0;
      atomicAdd(&cnt[gt_digit(key, 0)], 1);
    }
  }
  __syncthreads();
  hist[(size_t(h) * T + t) * kGtBins + tid] = cnt[tid];
}

// a later pass's tile histogram
__global__ __launch_bounds__(kGtThreads) void gt_hist_kernel(const uint32_t* __restrict__ ks,
                                                             int n, int T, int pass,
                                                             int32_t* __restrict__ hist) {
  __shared__ int cnt[kGtBins];
  const int h = blockIdx.y, t = blockIdx.x, tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const uint32_t* kh = ks + size_t(h) * n;
  uint32_t kv[kGtPer];
#pragma unroll
  for (int e = 0; e < kGtPer; ++e) kv[e] = kh[min(t * kGtTile + e * kGtThreads + tid, n - 1)];
#pragma unroll
  for (int e = 0; e < kGtPer; ++e)
    if (t * kGtTile + e * kGtThreads + tid < n) atomicAdd(&cnt[gt_digit(kv[e], pass)], 1);
  __syncthreads();
  hist[(size_t(h) * T + t) * kGtBins + tid] = cnt[tid];
}

// One pass's scatter, one tile per block.
// - Thread d finds digit d's first output position for this tile: the counts
//   of all smaller digits in the head plus the counts of digit d in earlier
//   tiles.
// - Wavefront w ranks the tile's entries w*512 .. w*512+511 in order, 64
//   at a time, in a count table of its own (equal digits found by ballots
//   over the digit's bits).
// - The entries are sorted by digit into LDS (stable: earlier quarters first)
//   and written out so that consecutive threads write consecutive positions
//   of a digit's run.
__global__ __launch_bounds__(kGtThreads) void gt_scatter_kernel(
    const uint32_t* __restrict__ ks, const int32_t* __restrict__ is, uint32_t* __restrict__ kd,
    int32_t* __restrict__ id, int H, int n, int T, int pass, const int32_t* __restrict__ hist,
    int32_t* __restrict__ pos_of) {
  __shared__ int wt[4][kGtBins];
  __shared__ int base_s[kGtBins];   // first output position of each digit
  __shared__ int local_s[kGtBins];  // first position of each digit in the tile's order
  __shared__ int scratch[4];
  __shared__ uint32_t skey[kGtTile];
  __shared__ int32_t sidx[kGtTile];
  // Blocks are dealt to the 8 accelerator dies in turn; the (head, tile) of a
  // block is chosen so that each die takes a contiguous run of tiles, and the
  // neighbouring runs of one digit are written through one L2.
  const int nb = T * H, per = (nb + kXcds - 1) / kXcds;
  const int hw = int(blockIdx.x), logical = (hw % kXcds) * per + hw / kXcds;
  if (logical >= nb) return;
  const int h = logical / T, t = logical % T, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const size_t hb = size_t(h) * n;
  uint32_t key[kGtPer];
  int32_t idx[kGtPer];
  int rk[kGtPer];
#pragma unroll
  for (int s = 0; s < kGtPer; ++s) {
    const int i = t * kGtTile + w * (kGtTile / 4) + s * 64 + lane;
    const int ic = min(i, n - 1);  // (past the end: loaded from the last entry, never stored)
    key[s] = ks[hb + ic];
    idx[s] = is[hb + ic];
    if (i >= n) {
      key[s] = kGrDead;
      idx[s] = -1;
    }
  }
  {
    const int32_t* hh = hist + size_t(h) * T * kGtBins + tid;
    int before = 0, total = 0;
    for (int u0 = 0; u0 < T; u0 += 32) {
      int c[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) c[e] = hh[size_t(min(u0 + e, T - 1)) * kGtBins];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        before += (u0 + e < t) ? c[e] : 0;
        total += (u0 + e < T) ? c[e] : 0;
      }
    }
    int all;
    base_s[tid] = block_exclusive_scan(total, scratch, &all) + before;
  }
  for (int i = tid; i < 4 * kGtBins; i += kGtThreads) (&wt[0][0])[i] = 0;
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int s = 0; s < kGtPer; ++s) {
    const bool ok = idx[s] >= 0;
    const int dg = gt_digit(key[s], pass);
    uint64_t peers = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (dg >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int r = __popcll(peers & below);
    rk[s] = (ok ? wt[w][dg] : 0) + r;
    // every lane has read the count before the first lane of its digit adds
    // the wavefront's share (one instruction stream: the read comes first)
    if (ok && r == 0) wt[w][dg] += __popcll(peers);
  }
  __syncthreads();
  {
    const int cnt = wt[0][tid] + wt[1][tid] + wt[2][tid] + wt[3][tid];
    int all;
    local_s[tid] = block_exclusive_scan(cnt, scratch, &all);
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kGtPer; ++s) {
    if (idx[s] < 0) continue;
    const int dg = gt_digit(key[s], pass);
    int pos = local_s[dg] + rk[s];
    for (int v = 0; v < w; ++v) pos += wt[v][dg];
    skey[pos] = key[s];
    sidx[pos] = idx[s];
  }
  __syncthreads();
  const int valid = min(kGtTile, n - t * kGtTile);
#pragma unroll
  for (int s = 0; s < kGtPer; ++s) {
    const int q = s * kGtThreads + tid;
    if (q < valid) {
      const uint32_t k = skey[q];
      const int dg = gt_digit(k, pass);
      const int off = base_s[dg] + (q - local_s[dg]);
      kd[hb + off] = k;
      id[hb + off] = sidx[q];
      if (pos_of) pos_of[hb + sidx[q]] = off;
    }
  }
}

// The sorted entries' costs (0 for a block of an empty cluster), and per tile
// their sum and the smallest cost of a live block.
__global__ __launch_bounds__(kGtThreads) void gt_cost_kernel(
    const uint32_t* __restrict__ ks, const int32_t* __restrict__ is,
    const int32_t* __restrict__ qoff, const int32_t* __restrict__ koff, int Cq, int Ck, int T,
    int64_t* __restrict__ cost, int64_t* __restrict__ tcost, int64_t* __restrict__ tmin) {
  __shared__ int nq_s[kMaxClusters], nk_s[kMaxClusters];
  __shared__ int64_t sum_s[kGtThreads / 64], min_s[kGtThreads / 64];
  const int h = blockIdx.y, t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = Cq * Ck;
  const int32_t* qo = qoff + size_t(h) * (Cq + 1);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  for (int c = tid; c < Cq; c += kGtThreads) nq_s[c] = qo[c + 1] - qo[c];
  for (int c = tid; c < Ck; c += kGtThreads) nk_s[c] = ko[c + 1] - ko[c];
  __syncthreads();
  const size_t hb = size_t(h) * n;
  int64_t sum = 0, mn = kGtNoCost;
  uint32_t kv[kGtPer];
  int32_t iv[kGtPer];
#pragma unroll
  for (int e = 0; e < kGtPer; ++e) {
    const int ic = min(t * kGtTile + e * kGtThreads + tid, n - 1);
    kv[e] = ks[hb + ic];
    iv[e] = is[hb + ic];
  }
#pragma unroll
  for (int e = 0; e < kGtPer; ++e) {
    const int i = t * kGtTile + e * kGtThreads + tid;
    if (i < n) {
      int64_t c = 0;
      if (kv[e] != kGrDead) {
        const int a = iv[e] / Ck;
        c = int64_t(nq_s[a]) * nk_s[iv[e] - a * Ck];
        mn = min(mn, c);
      }
      cost[hb + i] = (kv[e] == kGrDead) ? kGtNoCost : c;
      sum += c;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sum += shfl64(sum, lane ^ o);
    mn = min(mn, shfl64(mn, lane ^ o));
  }
  if (lane == 0) {
    sum_s[w] = sum;
    min_s[w] = mn;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t a = 0, m = kGtNoCost;
    for (int v = 0; v < kGtThreads / 64; ++v) {
      a += sum_s[v];
      m = min(m, min_s[v]);
    }
    tcost[size_t(h) * T + t] = a;
    tmin[size_t(h) * T + t] = m;
  }
}

// The greedy fill of one head over its sorted blocks (one block per head,
// one thread per tile). cost[] holds kGtNoCost for blocks of empty clusters
// (never taken).
constexpr int kGfThreads = 512;
static_assert(kGtMaxTiles <= kGfThreads, "one fill thread per tile");

__global__ __launch_bounds__(kGfThreads) void gt_fill_kernel(
    const int32_t* __restrict__ is, const int64_t* __restrict__ cost, int n, int T,
    int64_t budget, const int64_t* __restrict__ tcost, const int64_t* __restrict__ tmin,
    uint8_t* __restrict__ mask, int32_t* __restrict__ cross_out, int64_t* __restrict__ used_out) {
  constexpr int NW = kGfThreads / 64;
  __shared__ int64_t scratch64[NW];
  __shared__ int64_t suf_s[kGtMaxTiles];  // smallest live cost from tile t on
  __shared__ int64_t tmin_s[kGtMaxTiles]; // smallest live cost of tile t
  __shared__ int first_s;
  __shared__ int64_t before_s, used_s;
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const size_t hb = size_t(h) * n;
  const int32_t* ih = is + hb;
  const int64_t* ch = cost + hb;
  uint8_t* mh = mask + hb;

  // 1. the first tile whose blocks do not all fit, and the suffix minima
  const int64_t my_c = (tid < T) ? tcost[size_t(h) * T + tid] : 0;
  int64_t my_m = (tid < T) ? tmin[size_t(h) * T + tid] : kGtNoCost;
  if (tid < kGtMaxTiles) tmin_s[tid] = my_m;
  if (tid == 0) first_s = T;
  int64_t total;
  const int64_t run = block_exclusive_scan64(my_c, scratch64, &total);  // (barriers)
  if (tid < T && run <= budget && run + my_c > budget) atomicMin(&first_s, tid);
  {
    // suffix minimum: within the wavefront, then over the later wavefronts
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t x = shfl64(my_m, min(lane + o, 63));
      if (lane + o < 64) my_m = min(my_m, x);
    }
    if (lane == 0) scratch64[w] = my_m;
    __syncthreads();
    for (int v = w + 1; v < NW; ++v) my_m = min(my_m, scratch64[v]);
    if (tid < kGtMaxTiles) suf_s[tid] = my_m;
  }
  __syncthreads();
  const int tfirst = first_s;
  if (tid == tfirst) before_s = run;
  __syncthreads();
  if (tfirst == T) {
    // every block fits: every live block is taken
    if (tid == 0) {
      cross_out[h] = n;
      if (used_out) used_out[h] = total;
    }
    return;
  }
  // 2. the first block that does not fit, inside that tile (threads 0..255:
  // entries 8 tid .. 8 tid + 7; the others add nothing)
  if (tid == 0) first_s = kGtTile;
  int64_t cs[kGtPer];
  int64_t mine = 0;
#pragma unroll
  for (int e = 0; e < kGtPer; ++e) {
    const int q = tid * kGtPer + e, i = tfirst * kGtTile + q;
    const int64_t c = ch[min(i, n - 1)];
    cs[e] = (q >= kGtTile || i >= n || c == kGtNoCost) ? 0 : c;
    mine += cs[e];
  }
  int64_t tot2;
  int64_t pre = before_s + block_exclusive_scan64(mine, scratch64, &tot2);
  int mine_q = kGtTile;
  int64_t mine_pre = 0;
#pragma unroll
  for (int e = 0; e < kGtPer; ++e) {
    if (mine_q == kGtTile && pre + cs[e] > budget) {
      mine_q = tid * kGtPer + e;
      mine_pre = pre;
    }
    pre += cs[e];
  }
  if (mine_q < kGtTile) atomicMin(&first_s, mine_q);
  __syncthreads();
  if (mine_q == first_s) used_s = mine_pre;
  __syncthreads();
  // the sorted position of the first misfit: every block before it is taken
  // (route_lists_kernel marks them)
  const int cross = tfirst * kGtTile + first_s;
  if (tid == 0) cross_out[h] = cross;
  int64_t used = used_s;
  // 3. from the misfit on, in order, every block that still fits (wavefront 0
  // alone). Lane l holds entries 64 e + l (e = 0..31) of a tile. Only tiles
  // whose cheapest block fits the budget left (which only shrinks) are read,
  // the next such tile while this one is walked.
  if (w != 0) return;
  constexpr int PF = kGtTile / 64;
  int64_t nc[PF];
  int32_t ni[PF];
  auto load = [&](int t) {
#pragma unroll
    for (int e = 0; e < PF; ++e) {
      const int i = t * kGtTile + e * 64 + lane;
      const bool in = i < n && i > cross;
      const int ic = min(i, n - 1);
      nc[e] = ch[ic];
      ni[e] = ih[ic];
      if (!in) nc[e] = kGtNoCost;
    }
  };
  // the first tile from t on that holds a block no dearer than the budget left
  auto next_tile = [&](int t) {
    if (t < T && budget - used < suf_s[t]) return T;
    while (t < T && tmin_s[t] > budget - used) ++t;
    return t;
  };
  int t = next_tile(tfirst), loaded = -1;
  while (t < T) {
    if (loaded != t) load(t);
    int64_t c[PF];
    int32_t ix[PF];
#pragma unroll
    for (int e = 0; e < PF; ++e) {
      c[e] = nc[e];
      ix[e] = ni[e];
    }
    const int tn = next_tile(t + 1);
    loaded = -1;
    if (tn < T) {
      load(tn);
      loaded = tn;
    }
    // per chunk of 64: among the blocks that could still fit, the longest run
    // (in order) whose running cost fits is taken at once; the block after it
    // does not fit and is dropped; the rest are filtered again
#pragma unroll
    for (int e = 0; e < PF; ++e) {
      uint64_t open = __ballot(c[e] <= budget - used);
      while (open) {
        const bool mine = (open >> lane) & 1;
        const int64_t run = wave_inclusive_scan64(mine ? c[e] : 0);
        const uint64_t take = __ballot(mine && run <= budget - used);
        if ((take >> lane) & 1) mh[ix[e]] = 1;
        if (take) used += shfl64(run, 63 - __clzll((long long)take));
        open &= ~take;
        if (open) open &= open - 1;  // the next open block exceeded the budget left
        open &= __ballot(c[e] <= budget - used);
      }
    }
    t = next_tile(tn);
  }
  if (lane == 0 && used_out) used_out[h] = used;
}

__global__ __launch_bounds__(64) void route_lists_kernel(uint8_t* __restrict__ mask,
                                                         const int32_t* __restrict__ pos_of,
                                                         const int32_t* __restrict__ cross,
                                                         const int32_t* __restrict__ qoff,
                                                         const int32_t* __restrict__ koff,
                                                         int Cq, int Ck,
                                                         int32_t* __restrict__ list,
                                                         int32_t* __restrict__ count,
                                                         int32_t* __restrict__ keys) {
  const int h = blockIdx.y, c = blockIdx.x, lane = threadIdx.x;
  uint8_t* mr = mask + (size_t(h) * Cq + c) * Ck;
  const int32_t* po = pos_of + (size_t(h) * Cq + c) * Ck;
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  const int32_t* qo = qoff + size_t(h) * (Cq + 1);
  const bool qlive = qo[c + 1] > qo[c];
  const int cr = cross[h];
  int32_t* ls = list ? list + (size_t(h) * Cq + c) * Ck : nullptr;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int carry = 0, ksum = 0;
  for (int b = 0; b < Ck; b += 64) {
    const int j = b + lane;
    bool m = false;
    if (j < Ck) {
      const int nk = ko[j + 1] - ko[j];
      m = (qlive && nk > 0 && po[j] < cr) || mr[j] != 0;
      mr[j] = m;
      if (m) ksum += nk;
    }
    const uint64_t bal = __ballot(m);
    if (m && ls) ls[carry + __popcll(bal & below)] = j;
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

static int gt_tiles(int n) { return ceil_div(n, kGtTile); }

size_t route_global_ws_bytes(int H, int Cq, int Ck) {
  const size_t n = size_t(Cq) * Ck;
  const int T = gt_tiles(int(n));
  return align256(size_t(H) * n * 4) * 5 + align256(size_t(H) * n * 8) +
         align256(size_t(H) * T * kGtBins * 4) + align256(size_t(H) * T * 8) * 2 +
         align256(size_t(H) * 4);
}

hipError_t launch_route_global(int H, int Cq, int Ck, const float* ratio, const int32_t* qoff,
                               const int32_t* koff, int64_t budget, uint8_t* mask,
                               int32_t* list, int32_t* count, int32_t* keys, int64_t* used,
                               void* ws, hipStream_t s) {
  const int n = Cq * Ck, T = gt_tiles(n);
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* q = p;
    p += align256(bytes);
    return q;
  };
  uint32_t* ka = reinterpret_cast<uint32_t*>(take(size_t(H) * n * 4));
  uint32_t* kb = reinterpret_cast<uint32_t*>(take(size_t(H) * n * 4));
  int32_t* ia = reinterpret_cast<int32_t*>(take(size_t(H) * n * 4));
  int32_t* ib = reinterpret_cast<int32_t*>(take(size_t(H) * n * 4));
  int64_t* cost = reinterpret_cast<int64_t*>(take(size_t(H) * n * 8));
  int32_t* hist = reinterpret_cast<int32_t*>(take(size_t(H) * T * kGtBins * 4));
  int64_t* tcost = reinterpret_cast<int64_t*>(take(size_t(H) * T * 8));
  int64_t* tmin = reinterpret_cast<int64_t*>(take(size_t(H) * T * 8));
  int32_t* pos_of = reinterpret_cast<int32_t*>(take(size_t(H) * n * 4));
  int32_t* cross = reinterpret_cast<int32_t*>(take(size_t(H) * 4));
  const dim3 tiles(T, H);
  hipLaunchKernelGGL(gt_keys_kernel, tiles, dim3(kGtThreads), 0, s, ratio, qoff, koff, Cq, Ck, T,
                     ka, ia, mask, hist);
  uint32_t *ks = ka, *kd = kb;
  int32_t *is = ia, *id = ib;
  for (int pass = 0; pass < kGtPasses; ++pass) {
    if (pass > 0)
      hipLaunchKernelGGL(gt_hist_kernel, tiles, dim3(kGtThreads), 0, s, ks, n, T, pass, hist);
    hipLaunchKernelGGL(gt_scatter_kernel, dim3(ceil_div(T * H, kXcds) * kXcds),
                       dim3(kGtThreads), 0, s, ks, is, kd, id, H, n, T, pass, hist,
                       pass + 1 == kGtPasses ? pos_of : nullptr);
    uint32_t* tk = ks; ks = kd; kd = tk;
    int32_t* ti = is; is = id; id = ti;
  }
  hipLaunchKernelGGL(gt_cost_kernel, tiles, dim3(kGtThreads), 0, s, ks, is, qoff, koff, Cq, Ck,
                     T, cost, tcost, tmin);
  hipLaunchKernelGGL(gt_fill_kernel, dim3(H), dim3(kGfThreads), 0, s, is, cost, n, T, budget,
                     tcost, tmin, mask, cross, used);
  hipLaunchKernelGGL(route_lists_kernel, dim3(Cq, H), dim3(64), 0, s, mask, pos_of, cross, qoff,
                     koff, Cq, Ck, list, count, keys);
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
