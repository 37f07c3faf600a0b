// Query-centroid error probe (paper §4.2, Eq. 5; streaming kernel of §4.4).
//
// Work is split into units of at most 256 consecutive permuted keys that all
// belong to ONE key cluster c'. A block takes one unit and up to 128 query
// centroids (32 per wavefront). Keys are staged through LDS in 64-row tiles
// and multiplied against the centroids on matrix cores (S^T = K qbar^T); the
// f32 centroids enter as a bf16 high part plus a bf16 remainder, so the logits
// carry about 16 significant bits. Because the unit lies inside one cluster,
// the centroid logit s~ is the same for every key of the unit, and each lane
// keeps a streaming triple relative to a running maximum m (initialised to s~):
//     Z = sum exp(s - m),   E = sum (exp(s - m) - exp(s~ - m))^2.
// The squared gap is accumulated directly rather than expanded, so tight
// blocks (s ~ s~) do not lose their small error to cancellation. A finalize
// pass rescales the unit triples of each query centroid to the global maximum
// and forms ratio = E / (Z^2 |k_c'|). All exponentials are base 2 with log2(e)
// folded into the scale. No atomics: results are bitwise repeatable.
#include "svgear_common.hpp"
#include "svgear_internal.hpp"

namespace svg {

__global__ __launch_bounds__(1024) void probe_units_kernel(int Ck, const int32_t* __restrict__ koff,
                                                           int32_t* __restrict__ unit_prefix) {
  __shared__ int scratch[16];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  int units = 0;
  if (tid < Ck) units = (ko[tid + 1] - ko[tid] + kProbeUnit - 1) / kProbeUnit;
  int total;
  const int ex = block_exclusive_scan(units, scratch, &total);
  if (tid < Ck) unit_prefix[size_t(h) * (Ck + 1) + tid] = ex;
  if (tid == 0) unit_prefix[size_t(h) * (Ck + 1) + Ck] = total;
}

__device__ __forceinline__ int find_unit_cluster(const int32_t* prefix, int C, int q) {
  int lo = 0, hi = C;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= q) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename T>
__device__ __forceinline__ void split_centroid(const float (&x)[8], Frag<T>& hi, Frag<T>& lo,
                                               float (&val)[8]);

template <>
__device__ __forceinline__ void split_centroid<__bf16>(const float (&x)[8], Frag<__bf16>& hi,
                                                       Frag<__bf16>& lo, float (&val)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 a = __bf16(x[e]);
    const __bf16 b = __bf16(x[e] - float(a));
    hi.v[e] = a;
    lo.v[e] = b;
    val[e] = float(a) + float(b);
  }
}

template <>
__device__ __forceinline__ void split_centroid<float>(const float (&x)[8], Frag<float>& hi,
                                                      Frag<float>& lo, float (&val)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi.v[e] = x[e];
    lo.v[e] = 0.f;
    val[e] = x[e];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void probe_kernel(const float* __restrict__ qc,
                                                    const T* __restrict__ Kp,
                                                    const float* __restrict__ kc,
                                                    const int32_t* __restrict__ koff,
                                                    const int32_t* __restrict__ unit_prefix,
                                                    int Nk, int Cq, int Ck, int maxu, float sl2,
                                                    float* __restrict__ rec) {
  constexpr int KC = D / 32;
  constexpr int LDR = D + 16 / sizeof(T);
  constexpr bool kSplit = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) T ks[64 * LDR];

  const int h = blockIdx.y, u = blockIdx.x, grp = blockIdx.z, tid = threadIdx.x;
  const int32_t* up = unit_prefix + size_t(h) * (Ck + 1);
  if (u >= up[Ck]) return;
  const int cc = find_unit_cluster(up, Ck, u);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  const int j0 = ko[cc] + (u - up[cc]) * kProbeUnit;
  const int j1 = min(ko[cc + 1], j0 + kProbeUnit);
  const int w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;

  Frag<T> bhi[2][KC], blo[2][KC];
  float st[2];
  const float* kbar = kc + (size_t(h) * Ck + cc) * D;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = grp * kProbeGroup + w * 32 + cb * 16 + r;
    const bool ok = c < Cq;
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float x[8], val[8];
      const float* qrow = qc + (size_t(h) * Cq + (ok ? c : 0)) * D + k * 32 + g * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ok ? qrow[e] : 0.f;
      split_centroid<T>(x, bhi[cb][k], blo[cb][k], val);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(val[e], kbar[k * 32 + g * 8 + e], dot);
    }
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    st[cb] = dot * sl2;
  }

  float m[2], Z[2], E[2], e2[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) { m[cb] = st[cb]; Z[cb] = 0.f; E[cb] = 0.f; e2[cb] = 1.f; }

  const T* Kh = Kp + size_t(h) * Nk * D;
  constexpr int EPT = 16 / sizeof(T);
  constexpr int CPR = D / EPT;
  for (int tj = j0; tj < j1; tj += 64) {
    __syncthreads();
    for (int i = tid; i < 64 * CPR; i += 256) {
      const int row = i / CPR, piece = i % CPR;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tj + row < j1) v = *reinterpret_cast<const uint4*>(Kh + size_t(tj + row) * D + piece * EPT);
      *reinterpret_cast<uint4*>(&ks[row * LDR + piece * EPT]) = v;
    }
    __syncthreads();
    const int nvalid = min(64, j1 - tj);
    for (int kb = 0; kb * 16 < nvalid; ++kb) {
      Frag<T> a[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) a[k] = load8(&ks[(kb * 16 + r) * LDR + k * 32 + g * 8]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          mma(acc, a[k], bhi[cb][k]);
          if (kSplit) mma(acc, a[k], blo[cb][k]);
        }
        float s2[4];
        float tmax = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = kb * 16 + g * 4 + i < nvalid;
          s2[i] = ok ? acc[i] * sl2 : -__builtin_inff();
          tmax = fmaxf(tmax, s2[i]);
        }
        if (tmax > m[cb]) {
          const float al = fast_exp2(m[cb] - tmax);
          Z[cb] *= al;
          E[cb] *= al * al;
          m[cb] = tmax;
          e2[cb] = fast_exp2(st[cb] - tmax);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kb * 16 + g * 4 + i < nvalid) {
            const float e = fast_exp2(s2[i] - m[cb]);
            Z[cb] += e;
            const float dd = e - e2[cb];
            E[cb] = fmaf(dd, dd, E[cb]);
          }
        }
      }
    }
  }

#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float om = __shfl_xor(m[cb], o, 64);
      const float oZ = __shfl_xor(Z[cb], o, 64);
      const float oE = __shfl_xor(E[cb], o, 64);
      const float M = fmaxf(m[cb], om);
      const float a1 = fast_exp2(m[cb] - M), a2 = fast_exp2(om - M);
      Z[cb] = Z[cb] * a1 + oZ * a2;
      E[cb] = E[cb] * (a1 * a1) + oE * (a2 * a2);
      m[cb] = M;
    }
    const int c = grp * kProbeGroup + w * 32 + cb * 16 + r;
    if (g == 0 && c < Cq) {
      float* o = rec + ((size_t(h) * maxu + u) * Cq + c) * 3;
      o[0] = m[cb];
      o[1] = Z[cb];
      o[2] = E[cb];
    }
  }
}

__global__ __launch_bounds__(256) void probe_finalize_kernel(int Cq, int Ck, int maxu,
                                                             const int32_t* __restrict__ koff,
                                                             const int32_t* __restrict__ unit_prefix,
                                                             const float* __restrict__ rec,
                                                             float* __restrict__ ratio,
                                                             float* __restrict__ log_norm) {
  __shared__ float red[256];
  const int h = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int32_t* up = unit_prefix + size_t(h) * (Ck + 1);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  const int nu = up[Ck];
  auto R = [&](int u, int k) { return rec[((size_t(h) * maxu + u) * Cq + c) * 3 + k]; };

  float mx = -__builtin_inff();
  for (int u = tid; u < nu; u += 256) mx = fmaxf(mx, R(u, 0));
  red[tid] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  const float m = red[0];
  __syncthreads();
  float z = 0.f;
  for (int u = tid; u < nu; u += 256) z += R(u, 1) * fast_exp2(R(u, 0) - m);
  red[tid] = z;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float Z = red[0];
  const float inv = 1.f / (Z * Z);
  for (int k = tid; k < Ck; k += 256) {
    const int n = ko[k + 1] - ko[k];
    // a one-key cluster is its own centroid: its error is exactly zero
    float out = (n == 1) ? 0.f : -1.f;
    if (n > 1) {
      float e = 0.f;
      for (int u = up[k]; u < up[k + 1]; ++u) {
        const float a = fast_exp2(R(u, 0) - m);
        e += R(u, 2) * (a * a);
      }
      out = e * inv / float(n);
    }
    ratio[(size_t(h) * Cq + c) * Ck + k] = out;
  }
  if (tid == 0 && log_norm) log_norm[size_t(h) * Cq + c] = (m + __log2f(Z)) * 0.69314718055994530942f;
}

template <typename T, int D>
static void probe_t(int H, int Nk, int Cq, int Ck, float sl2, const float* qc, const void* Kp,
                    const float* kc, const int32_t* koff, const int32_t* up, float* rec,
                    hipStream_t s) {
  const int maxu = max_units(Nk, Ck);
  hipLaunchKernelGGL((probe_kernel<T, D>), dim3(maxu, H, ceil_div(Cq, kProbeGroup)), dim3(256), 0,
                     s, qc, static_cast<const T*>(Kp), kc, koff, up, Nk, Cq, Ck, maxu, sl2, rec);
}

hipError_t launch_probe(int elem_bytes, int H, int Nk, int d, int Cq, int Ck, float scale,
                        const float* qc, const void* Kp, const float* kc, const int32_t* koff,
                        int32_t* unit_prefix, float* rec, float* ratio, float* log_norm,
                        hipStream_t s) {
  hipLaunchKernelGGL(probe_units_kernel, dim3(H), dim3(1024), 0, s, Ck, koff, unit_prefix);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = scale * 1.44269504088896340736f;
  if (elem_bytes == 2) {
    if (d == 128) probe_t<__bf16, 128>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, unit_prefix, rec, s);
    else probe_t<__bf16, 64>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, unit_prefix, rec, s);
  } else {
    if (d == 128) probe_t<float, 128>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, unit_prefix, rec, s);
    else probe_t<float, 64>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, unit_prefix, rec, s);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(probe_finalize_kernel, dim3(Cq, H), dim3(256), 0, s, Cq, Ck,
                     max_units(Nk, Ck), koff, unit_prefix, rec, ratio, log_norm);
  return hipGetLastError();
}

}  // namespace svg
