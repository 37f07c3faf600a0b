// Error analysis of block selections (paper §5.3 "Strategy of block
// selection", Fig. 6a): how far a block-sparse attention map lies from the
// full one, and the score-based block ranking of the top-p baseline.
//
// map_error_kernel: one wavefront per 16 permuted queries. S^T = K Q^T comes
// from the matrix cores 16 keys at a time, walking the key clusters in order so
// that the selection flag of a lane's query cluster and its centroid logit are
// per-cluster registers. Pass 1 streams the row maximum m, the full normaliser
// Z = sum exp(s - m) and the kept part of the sparse one; the centroid part
// sum over skipped non-empty clusters of |k_c'| exp(s~ - m) (§4.3) is added from
// the centroid logits s~, which the wavefront first computes in f32 and keeps
// in the workspace. Pass 2 recomputes S and sums (a_sparse - a_full)^2 over all
// keys. Exponentials are base 2 with log2(e) folded into the scale; both
// normalisers are relative to the row maximum.
//
// block_scores_kernel: score[c][c'] = |k_c'| exp(scale qbar_c.kbar_c') / sum,
// the centroid estimate of the block's attention mass (top-p ranking); -1 for
// empty key clusters.
//
// row_spread_kernel: ||x_p - xbar_c||^2 for every permuted row (the clustering
// error whose mean is delta_q^2 for the queries, §5.3 Fig. 6b), 16 lanes per
// row, f32.
#include "svgear_common.hpp"
#include "svgear_internal.hpp"

namespace svg {

template <typename T, int D>
__global__ __launch_bounds__(256) void map_error_kernel(
    const T* __restrict__ Qp, const T* __restrict__ Kp, const float* __restrict__ kc,
    const int32_t* __restrict__ qoff, const int32_t* __restrict__ koff,
    const uint8_t* __restrict__ mask, int Nq, int Nk, int Cq, int Ck, float sl2, int compensate,
    float* __restrict__ stl, float* __restrict__ err, float* __restrict__ zfull,
    float* __restrict__ zsparse) {
  constexpr int KC = D / 32;
  const int h = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int q0 = blockIdx.x * 64 + w * 16;
  if (q0 >= Nq) return;  // whole wavefront; the kernel has no block barriers
  const int qi = q0 + r;
  const bool qok = qi < Nq;
  const int qc = qok ? qi : Nq - 1;
  const int32_t* qo = qoff + size_t(h) * (Cq + 1);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  int lo = 0, hi = Cq;  // query cluster of this lane's query
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qo[mid] <= qc) lo = mid; else hi = mid;
  }
  const uint8_t* mrow = mask + (size_t(h) * Cq + lo) * Ck;
  const T* Qh = Qp + size_t(h) * Nq * D;
  const T* Kh = Kp + size_t(h) * Nk * D;

  // Q^T as the B operand: lane (r, g) holds q[qi][32 kc + 8 g + e]
  Frag<T> qf[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) qf[k] = qok ? load8(Qh + size_t(qi) * D + k * 32 + g * 8)
                                           : zero_frag<T>();

  // centroid logits (base-2 units) in f32; the four lanes of a query each keep
  // the entries c' = g (mod 4), so every later read is of the lane's own write
  float* st_row = stl + (size_t(h) * Nq + qc) * Ck;
  for (int c2 = 0; c2 < Ck; ++c2) {
    const float* kb = kc + (size_t(h) * Ck + c2) * D + g * 8;
    float p = 0.f;
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) p = fmaf(to_f32(qf[k].v[e]), kb[k * 32 + e], p);
    p += __shfl_xor(p, 16, 64);
    p += __shfl_xor(p, 32, 64);
    if (qok && (c2 & 3) == g) st_row[c2] = p * sl2;
  }
  __threadfence_block();  // the lanes read these entries back below

  auto logits = [&](int jb, int j1, f32x4& acc) {
    Frag<T> kf[KC];
    const int kj = jb + r;
    const bool kok = kj < j1;
#pragma unroll
    for (int k = 0; k < KC; ++k)
      kf[k] = kok ? load8(Kh + size_t(kj) * D + k * 32 + g * 8) : zero_frag<T>();
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KC; ++k) mma(acc, kf[k], qf[k]);
  };

  // pass 1: m, Z and the kept part of the sparse normaliser
  float m = -__builtin_inff(), Z = 0.f, Zk = 0.f;
  for (int c2 = 0; c2 < Ck; ++c2) {
    const int j0 = ko[c2], j1 = ko[c2 + 1];
    if (j1 == j0) continue;
    const bool sel = mrow[c2] != 0;
    for (int jb = j0; jb < j1; jb += 16) {
      f32x4 acc;
      logits(jb, j1, acc);
      float s[4], tm = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = (jb + g * 4 + i < j1) ? acc[i] * sl2 : -__builtin_inff();
        tm = fmaxf(tm, s[i]);
      }
      if (tm > m) {
        const float a = fast_exp2(m - tm);
        Z *= a;
        Zk *= a;
        m = tm;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = (s[i] > -__builtin_inff()) ? fast_exp2(s[i] - m) : 0.f;
        Z += e;
        Zk += sel ? e : 0.f;
      }
    }
  }
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float om = __shfl_xor(m, o, 64), oZ = __shfl_xor(Z, o, 64), oK = __shfl_xor(Zk, o, 64);
    const float M = fmaxf(m, om);
    const float a1 = (m == -__builtin_inff()) ? 0.f : fast_exp2(m - M);
    const float a2 = (om == -__builtin_inff()) ? 0.f : fast_exp2(om - M);
    Z = Z * a1 + oZ * a2;
    Zk = Zk * a1 + oK * a2;
    m = M;
  }
  float Zc = 0.f;  // skipped non-empty clusters, each |k_c'| copies of the centroid weight
  if (compensate) {
    for (int c2 = g; c2 < Ck; c2 += 4) {
      const int n = ko[c2 + 1] - ko[c2];
      if (qok && n > 0 && mrow[c2] == 0) Zc += float(n) * fast_exp2(st_row[c2] - m);
    }
    Zc += __shfl_xor(Zc, 16, 64);
    Zc += __shfl_xor(Zc, 32, 64);
  }
  const float Zs = Zk + Zc;
  const float inv_f = 1.f / Z, inv_s = Zs > 0.f ? 1.f / Zs : 0.f;

  // pass 2: sum of (a_sparse - a_full)^2 over every key
  float E = 0.f;
  for (int c2 = 0; c2 < Ck; ++c2) {
    const int j0 = ko[c2], j1 = ko[c2 + 1];
    if (j1 == j0) continue;
    const bool sel = mrow[c2] != 0;
    const float own = ((c2 & 3) == g && qok) ? st_row[c2] : 0.f;
    const float stc = __shfl(own, r + 16 * (c2 & 3), 64);
    const float wu = (!sel && compensate) ? fast_exp2(stc - m) * inv_s : 0.f;
    for (int jb = j0; jb < j1; jb += 16) {
      f32x4 acc;
      logits(jb, j1, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (jb + g * 4 + i < j1) {
          const float e = fast_exp2(acc[i] * sl2 - m);
          const float df = (sel ? e * inv_s : wu) - e * inv_f;
          E = fmaf(df, df, E);
        }
      }
    }
  }
  E += __shfl_xor(E, 16, 64);
  E += __shfl_xor(E, 32, 64);
  if (qok && g == 0) {
    err[size_t(h) * Nq + qi] = E;
    zfull[size_t(h) * Nq + qi] = Z;
    zsparse[size_t(h) * Nq + qi] = Zs;
  }
}

__global__ __launch_bounds__(256) void block_scores_kernel(int Ck, int D, float sl2,
                                                           const float* __restrict__ qc,
                                                           const float* __restrict__ kc,
                                                           const int32_t* __restrict__ koff,
                                                           int Cq, float* __restrict__ scores) {
  __shared__ float lg[kMaxClusters];
  __shared__ float red[256];
  const int h = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const float* q = qc + (size_t(h) * Cq + c) * D;
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  float mx = -__builtin_inff();
  for (int c2 = tid; c2 < Ck; c2 += 256) {
    const int n = ko[c2 + 1] - ko[c2];
    const float* k = kc + (size_t(h) * Ck + c2) * D;
    float dot = 0.f;
    for (int e = 0; e < D; ++e) dot = fmaf(q[e], k[e], dot);
    const float l = n > 0 ? dot * sl2 + __log2f(float(n)) : -__builtin_inff();
    lg[c2] = l;
    mx = fmaxf(mx, l);
  }
  red[tid] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  const float m = red[0];
  __syncthreads();
  float z = 0.f;
  for (int c2 = tid; c2 < Ck; c2 += 256) z += (lg[c2] == -__builtin_inff()) ? 0.f : fast_exp2(lg[c2] - m);
  red[tid] = z;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float inv = 1.f / red[0];
  for (int c2 = tid; c2 < Ck; c2 += 256)
    scores[(size_t(h) * Cq + c) * Ck + c2] =
        (lg[c2] == -__builtin_inff()) ? -1.f : fast_exp2(lg[c2] - m) * inv;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void row_spread_kernel(const T* __restrict__ Xp,
                                                         const float* __restrict__ mu,
                                                         const int32_t* __restrict__ off, int N,
                                                         int C, float* __restrict__ d2) {
  constexpr int EL = D / 16;
  const int h = blockIdx.y, tid = threadIdx.x, sub = tid & 15;
  const int j = blockIdx.x * 16 + (tid >> 4);
  const bool ok = j < N;
  const int jj = ok ? j : N - 1;
  const int32_t* o = off + size_t(h) * (C + 1);
  int lo = 0, hi = C;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (o[mid] <= jj) lo = mid; else hi = mid;
  }
  const T* x = Xp + (size_t(h) * N + jj) * D + sub * EL;
  const float* m = mu + (size_t(h) * C + lo) * D + sub * EL;
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    const float df = to_f32(x[e]) - m[e];
    a = fmaf(df, df, a);
  }
#pragma unroll
  for (int s2 = 8; s2 > 0; s2 >>= 1) a += __shfl_xor(a, s2, 64);
  if (ok && sub == 0) d2[size_t(h) * N + j] = a;
}

hipError_t launch_row_spread(int elem_bytes, int H, int N, int d, int C, const void* Xp,
                             const float* mu, const int32_t* off, float* d2, hipStream_t s) {
  const dim3 grid(ceil_div(N, 16), H), block(256);
  if (elem_bytes == 2) {
    if (d == 128)
      hipLaunchKernelGGL((row_spread_kernel<__bf16, 128>), grid, block, 0, s, (const __bf16*)Xp, mu, off, N, C, d2);
    else
      hipLaunchKernelGGL((row_spread_kernel<__bf16, 64>), grid, block, 0, s, (const __bf16*)Xp, mu, off, N, C, d2);
  } else {
    if (d == 128)
      hipLaunchKernelGGL((row_spread_kernel<float, 128>), grid, block, 0, s, (const float*)Xp, mu, off, N, C, d2);
    else
      hipLaunchKernelGGL((row_spread_kernel<float, 64>), grid, block, 0, s, (const float*)Xp, mu, off, N, C, d2);
  }
  return hipGetLastError();
}

size_t map_error_ws_bytes(int H, int Nq, int Ck) { return sizeof(float) * size_t(H) * Nq * Ck; }

hipError_t launch_map_error(int elem_bytes, int H, int Nq, int Nk, int d, int Cq, int Ck,
                            float scale, const void* Qp, const void* Kp, const int32_t* qoff,
                            const int32_t* koff, const float* kc, const uint8_t* mask,
                            int compensate, float* err, float* zfull, float* zsparse, void* ws,
                            hipStream_t s) {
  const float sl2 = scale * 1.44269504088896340736f;
  const dim3 grid(ceil_div(Nq, 64), H), block(256);
  float* stl = static_cast<float*>(ws);
  if (elem_bytes == 2) {
    if (d == 128)
      hipLaunchKernelGGL((map_error_kernel<__bf16, 128>), grid, block, 0, s, (const __bf16*)Qp,
                         (const __bf16*)Kp, kc, qoff, koff, mask, Nq, Nk, Cq, Ck, sl2, compensate,
                         stl, err, zfull, zsparse);
    else
      hipLaunchKernelGGL((map_error_kernel<__bf16, 64>), grid, block, 0, s, (const __bf16*)Qp,
                         (const __bf16*)Kp, kc, qoff, koff, mask, Nq, Nk, Cq, Ck, sl2, compensate,
                         stl, err, zfull, zsparse);
  } else {
    if (d == 128)
      hipLaunchKernelGGL((map_error_kernel<float, 128>), grid, block, 0, s, (const float*)Qp,
                         (const float*)Kp, kc, qoff, koff, mask, Nq, Nk, Cq, Ck, sl2, compensate,
                         stl, err, zfull, zsparse);
    else
      hipLaunchKernelGGL((map_error_kernel<float, 64>), grid, block, 0, s, (const float*)Qp,
                         (const float*)Kp, kc, qoff, koff, mask, Nq, Nk, Cq, Ck, sl2, compensate,
                         stl, err, zfull, zsparse);
  }
  return hipGetLastError();
}

hipError_t launch_block_scores(int H, int d, int Cq, int Ck, float scale, const float* qc,
                               const float* kc, const int32_t* koff, float* scores,
                               hipStream_t s) {
  hipLaunchKernelGGL(block_scores_kernel, dim3(Cq, H), dim3(256), 0, s, Ck, d,
                     scale * 1.44269504088896340736f, qc, kc, koff, Cq, scores);
  return hipGetLastError();
}

}  // namespace svg
