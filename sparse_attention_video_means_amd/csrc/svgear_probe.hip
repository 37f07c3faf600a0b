// Query-centroid error probe (paper §4.2, Eq. 5; streaming kernel of §4.4).
//
// For query centroid c and key j of key cluster c' the raw logit is
// s = s~ + delta with s~ = scale*qbar_c.kbar_c' (the centroid logit, the same for
// the whole block) and delta = scale*qbar_c.(k_j - kbar_c'). The kernels use
// exactly this split:
//   * centroid_logits: s~ for every (c, c') in f32 (a small Cq x Ck x d product);
//   * probe: keys are staged through LDS as (k_j - kbar_c') rounded to the element
//     type, and delta comes from the matrix cores against qbar_c. Because the
//     differences are small, their rounding error is small in absolute terms,
//     so tight blocks (delta ~ 0) keep an accurate error; the centroid side is
//     split into a bf16 high part and a bf16 remainder (two products).
// Work is split into units of at most 256 consecutive permuted keys of ONE key
// cluster; persistent blocks walk the units of a head, keeping their 128 query
// centroids as MFMA B operands in registers. Each lane keeps a streaming triple
// relative to a running reference m >= s~ (base-2 logits):
//     Z = sum exp2(s - m),   E = sum (exp2(s - m) - exp2(s~ - m))^2,
// accumulated directly (the squared gap is never expanded). A finalize pass
// rescales the unit triples of each query centroid to the global maximum and
// forms ratio = E / (Z^2 |k_c'|). No atomics: results are bitwise repeatable.
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

// st2[h][c][c'] = sl2 * qbar_c . kbar_c'  (16 x 16 pairs per block, rows from LDS)
template <int D>
__global__ __launch_bounds__(256) void centroid_logits_kernel(int Cq, int Ck, float sl2,
                                                              const float* __restrict__ qc,
                                                              const float* __restrict__ kc,
                                                              float* __restrict__ st2) {
  __shared__ float qs[16][D + 1];
  __shared__ float kcs[16][D + 1];
  const int h = blockIdx.z, c0 = blockIdx.y * 16, k0 = blockIdx.x * 16, tid = threadIdx.x;
  for (int i = tid; i < 16 * D; i += 256) {
    const int r = i / D, j = i % D;
    qs[r][j] = (c0 + r < Cq) ? qc[(size_t(h) * Cq + c0 + r) * D + j] : 0.f;
    kcs[r][j] = (k0 + r < Ck) ? kc[(size_t(h) * Ck + k0 + r) * D + j] : 0.f;
  }
  __syncthreads();
  const int a = tid / 16, b = tid % 16;
  float dot = 0.f;
#pragma unroll 8
  for (int j = 0; j < D; ++j) dot = fmaf(qs[a][j], kcs[b][j], dot);
  if (c0 + a < Cq && k0 + b < Ck) st2[(size_t(h) * Cq + c0 + a) * Ck + k0 + b] = dot * sl2;
}

__device__ __forceinline__ int find_unit_cluster(const int32_t* prefix, int C, int q) {
  int lo = 0, hi = C;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= q) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void probe_kernel(const float* __restrict__ qc,
                                                    const T* __restrict__ Kp,
                                                    const float* __restrict__ kc,
                                                    const int32_t* __restrict__ koff,
                                                    const int32_t* __restrict__ unit_prefix,
                                                    const float* __restrict__ st2g,
                                                    int Nk, int Cq, int Ck, int maxu, float sl2,
                                                    float* __restrict__ rec) {
  constexpr int KC = D / 32;
  constexpr int LDR = D + 16 / sizeof(T);
  constexpr int QD = D / 4;  // dims staged per thread (4 threads per key row)
  __shared__ __attribute__((aligned(16))) T ks[64 * LDR];
  __shared__ __attribute__((aligned(16))) T kl[sizeof(T) == 2 ? 64 * LDR : 8];

  const int h = blockIdx.y, grp = blockIdx.z, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int32_t* up = unit_prefix + size_t(h) * (Ck + 1);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  const int nunits = up[Ck];

  // centroid blocks of this wave: block w and w + 4 of the group's 8. For bf16
  // the f32 centroid enters as a bf16 high part plus a bf16 remainder (about 16
  // significant bits), two products accumulated in f32.
  constexpr bool kSplit = sizeof(T) == 2;
  Frag<T> bq[2][KC], bl[2][KC];
  int cidx[2];
  bool cok[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = grp * kProbeGroup + (w + 4 * cb) * 16 + r;
    cidx[cb] = c;
    cok[cb] = c < Cq;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const float* qrow = qc + (size_t(h) * Cq + (cok[cb] ? c : 0)) * D + k * 32 + g * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = cok[cb] ? qrow[e] : 0.f;
        bq[cb][k].v[e] = from_f32<T>(x);
        bl[cb][k].v[e] = from_f32<T>(x - to_f32(bq[cb][k].v[e]));
      }
    }
  }
  // blocks that hold no centroid skip their matrix work (wave-uniform)
  const bool blk_live[2] = {grp * kProbeGroup + w * 16 < Cq, grp * kProbeGroup + (w + 4) * 16 < Cq};

  const T* Kh = Kp + size_t(h) * Nk * D;
  const int srow = tid >> 2, sq = tid & 3;
  constexpr int RAW = QD * int(sizeof(T)) / 16;  // 16-byte loads per thread and tile

  // The block walks its units u = blockIdx.x, +gridDim.x, ... and each unit
  // in 64-key tiles. The raw key rows (and, at a unit's first tile, the key
  // centroid) of the next tile are loaded into registers while the current
  // tile is multiplied, so their latency is off the critical path.
  struct Tile {
    int u, cc, j0, j1, tj;
  };
  auto unit_tile = [&](int u) {
    Tile t;
    t.u = u;
    t.cc = find_unit_cluster(up, Ck, u);
    t.j0 = ko[t.cc] + (u - up[t.cc]) * kProbeUnit;
    t.j1 = min(ko[t.cc + 1], t.j0 + kProbeUnit);
    t.tj = t.j0;
    return t;
  };
  auto load_raw = [&](const Tile& t, uint4 (&raw)[RAW]) {
    const bool ok = t.tj + srow < t.j1;
    const T* src = Kh + size_t(ok ? t.tj + srow : 0) * D + sq * QD;
#pragma unroll
    for (int i = 0; i < RAW; ++i) raw[i] = reinterpret_cast<const uint4*>(src)[i];
  };
  auto load_kbar = [&](int cc, float (&kb)[QD]) {
    const float* kr = kc + (size_t(h) * Ck + cc) * D + sq * QD;
#pragma unroll
    for (int i = 0; i < QD; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(kr + i);
      kb[i] = v.x; kb[i + 1] = v.y; kb[i + 2] = v.z; kb[i + 3] = v.w;
    }
  };

  if (int(blockIdx.x) >= nunits) return;
  Tile cur = unit_tile(blockIdx.x);
  uint4 raw[RAW];
  float kb[QD], kbn[QD];
  load_raw(cur, raw);
  load_kbar(cur.cc, kb);
  float st[2], mp[2], Z[2], E[2], e2[2];
  auto unit_start = [&](int cc) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      st[cb] = cok[cb] ? st2g[(size_t(h) * Cq + cidx[cb]) * Ck + cc] : 0.f;
      mp[cb] = 0.f;  // reference relative to s~: m = s~ + mp, mp >= 0
      Z[cb] = 0.f;
      E[cb] = 0.f;
      e2[cb] = 1.f;
    }
  };
  unit_start(cur.cc);

  while (true) {
    __syncthreads();
    {  // stage (k - kbar) as T high part + T remainder; rows past the unit are zero
      const bool ok = cur.tj + srow < cur.j1;
      T* dst = ks + srow * LDR + sq * QD;
      T* dlo = kl + srow * LDR + sq * QD;
#pragma unroll
      for (int i = 0; i < RAW; ++i) {
        const T* el = reinterpret_cast<const T*>(&raw[i]);
        constexpr int E8 = 16 / sizeof(T);
        T out[E8], rem[E8];
#pragma unroll
        for (int e = 0; e < E8; ++e) {
          const float dlt = ok ? to_f32(el[e]) - kb[i * E8 + e] : 0.f;
          out[e] = from_f32<T>(dlt);
          rem[e] = from_f32<T>(dlt - to_f32(out[e]));
        }
        *reinterpret_cast<uint4*>(dst + i * E8) = *reinterpret_cast<const uint4*>(out);
        if (kSplit) *reinterpret_cast<uint4*>(dlo + i * E8) = *reinterpret_cast<const uint4*>(rem);
      }
    }
    __syncthreads();
    // the next tile: the rest of this unit, else the first tile of the next
    Tile nxt = cur;
    nxt.tj += 64;
    const bool new_unit = nxt.tj >= cur.j1;
    if (new_unit) {
      const int un = cur.u + int(gridDim.x);
      if (un < nunits) nxt = unit_tile(un);
      else nxt.u = nunits;  // no next tile
    }
    const bool more = nxt.u < nunits;
    if (more) {
      load_raw(nxt, raw);
      if (new_unit) load_kbar(nxt.cc, kbn);
    }
    const int nvalid = min(64, cur.j1 - cur.tj);
    for (int kb16 = 0; kb16 * 16 < nvalid; ++kb16) {
      Frag<T> a[KC], al[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        a[k] = load8(&ks[(kb16 * 16 + r) * LDR + k * 32 + g * 8]);
        if (kSplit) al[k] = load8(&kl[(kb16 * 16 + r) * LDR + k * 32 + g * 8]);
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        if (!blk_live[cb]) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        // (qhi + qlo).(dhi + dlo) without the qlo.dlo term (below 2^-16 relative)
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          mma(acc, a[k], bq[cb][k]);
          if (kSplit) {
            mma(acc, a[k], bl[cb][k]);
            mma(acc, al[k], bq[cb][k]);
          }
        }
        // lane holds delta for keys kb16*16 + 4g + i of centroid cidx[cb]
        float d2[4];
        float tmax = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = kb16 * 16 + g * 4 + i < nvalid;
          d2[i] = ok ? acc[i] * sl2 : -__builtin_inff();
          tmax = fmaxf(tmax, d2[i]);
        }
        if (tmax > mp[cb]) {
          const float al = fast_exp2(mp[cb] - tmax);
          Z[cb] *= al;
          E[cb] *= al * al;
          mp[cb] = tmax;
          e2[cb] = fast_exp2(-tmax);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kb16 * 16 + g * 4 + i < nvalid) {
            const float e = fast_exp2(d2[i] - mp[cb]);
            Z[cb] += e;
            const float dd = e - e2[cb];
            E[cb] = fmaf(dd, dd, E[cb]);
          }
        }
      }
    }
    if (new_unit) {
      // the unit is done: merge the four lanes of each centroid and record
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
          const float om = __shfl_xor(mp[cb], o, 64);
          const float oZ = __shfl_xor(Z[cb], o, 64);
          const float oE = __shfl_xor(E[cb], o, 64);
          const float M = fmaxf(mp[cb], om);
          const float a1 = fast_exp2(mp[cb] - M), a2 = fast_exp2(om - M);
          Z[cb] = Z[cb] * a1 + oZ * a2;
          E[cb] = E[cb] * (a1 * a1) + oE * (a2 * a2);
          mp[cb] = M;
        }
        if (g == 0 && cok[cb]) {
          float* o = rec + ((size_t(h) * maxu + cur.u) * Cq + cidx[cb]) * 3;
          o[0] = st[cb] + mp[cb];  // absolute base-2 reference of this unit
          o[1] = Z[cb];
          o[2] = E[cb];
        }
      }
      if (!more) break;
#pragma unroll
      for (int i = 0; i < QD; ++i) kb[i] = kbn[i];
      unit_start(nxt.cc);
    }
    cur = nxt;
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

size_t probe_ws_bytes(int H, int Nk, int Cq, int Ck) {
  return align256(sizeof(int32_t) * size_t(H) * (Ck + 1)) +
         align256(sizeof(float) * size_t(H) * Cq * Ck) +
         align256(sizeof(float) * 3 * size_t(H) * max_units(Nk, Ck) * Cq);
}

template <typename T, int D>
static hipError_t probe_t(int H, int Nk, int Cq, int Ck, float sl2, const float* qc,
                          const void* Kp, const float* kc, const int32_t* koff, const int32_t* up,
                          float* st2, float* rec, hipStream_t s) {
  hipLaunchKernelGGL((centroid_logits_kernel<D>), dim3(ceil_div(Ck, 16), ceil_div(Cq, 16), H),
                     dim3(256), 0, s, Cq, Ck, sl2, qc, kc, st2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int maxu = max_units(Nk, Ck);
  const int groups = ceil_div(Cq, kProbeGroup);
  int per_head = ceil_div(2048, H * groups);
  per_head = per_head < 1 ? 1 : (per_head > maxu ? maxu : per_head);
  hipLaunchKernelGGL((probe_kernel<T, D>), dim3(per_head, H, groups), dim3(256), 0, s, qc,
                     static_cast<const T*>(Kp), kc, koff, up, st2, Nk, Cq, Ck, maxu, sl2, rec);
  return hipGetLastError();
}

hipError_t launch_probe(int elem_bytes, int H, int Nk, int d, int Cq, int Ck, float scale,
                        const float* qc, const void* Kp, const float* kc, const int32_t* koff,
                        void* ws, float* ratio, float* log_norm, hipStream_t s) {
  char* p = static_cast<char*>(ws);
  int32_t* up = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(H) * (Ck + 1));
  float* st2 = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * size_t(H) * Cq * Ck);
  float* rec = reinterpret_cast<float*>(p);
  hipLaunchKernelGGL(probe_units_kernel, dim3(H), dim3(1024), 0, s, Ck, koff, up);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = scale * 1.44269504088896340736f;
  if (elem_bytes == 2) {
    e = (d == 128) ? probe_t<__bf16, 128>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, rec, s)
                   : probe_t<__bf16, 64>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, rec, s);
  } else {
    e = (d == 128) ? probe_t<float, 128>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, rec, s)
                   : probe_t<float, 64>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, rec, s);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(probe_finalize_kernel, dim3(Cq, H), dim3(256), 0, s, Cq, Ck,
                     max_units(Nk, Ck), koff, up, rec, ratio, log_norm);
  return hipGetLastError();
}

}  // namespace svg
