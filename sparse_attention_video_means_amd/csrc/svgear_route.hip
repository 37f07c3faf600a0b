// Greedy error-to-cost router, one block per (head, query cluster)
// (paper §4.2 "Error estimation": highest error-to-size ratio first until the
// budget is exhausted; §5 "Implementation": routing per query cluster).
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
                                                    const int32_t* __restrict__ koff, int Cq,
                                                    int Ck, int P, int budget,
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
  for (int k = 2; k <= P; k <<= 1) {
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

hipError_t launch_route(int H, int Cq, int Ck, const float* ratio, const int32_t* koff,
                        int32_t budget, uint8_t* mask, int32_t* list, int32_t* count,
                        int32_t* keys, hipStream_t s) {
  int P = 1;
  while (P < Ck) P <<= 1;
  hipLaunchKernelGGL(route_kernel, dim3(Cq, H), dim3(256), 0, s, ratio, koff, Cq, Ck, P, budget,
                     mask, list, count, keys);
  return hipGetLastError();
}

}  // namespace svg
