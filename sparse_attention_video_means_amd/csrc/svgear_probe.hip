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
//
// Value-aware variant (§4.2's value-aware estimate; its display was lost, the
// reading taken is eps = ||p v_j - p~ vbar||^2 with the two weights above). With
// delta_p = p - p~ it splits as
//     ||p (v_j - vbar) + delta_p vbar||^2
//       = p^2 a_j + p delta_p b_j + delta_p^2 w,
// a_j = ||v_j - vbar||^2, b_j = 2 (v_j - vbar).vbar, w = ||vbar||^2, so that no
// term is a difference of nearly equal large numbers. value_stats writes
// (a_j, b_j) per permuted key and w per key cluster; the probe then also
// streams Ev = sum e (e a_j + dd b_j) (e = exp2(s - m), dd = e - exp2(s~ - m))
// and the finalize pass forms (Ev + w E) / (Z^2 |k_c'|).
#include <type_traits>

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

// st2[h][c'][c] = sl2 * qbar_c . kbar_c'  (16 x 16 pairs per block, rows from LDS;
// query centroid fastest, so that one key cluster's logits are contiguous)
template <int D>
__global__ __launch_bounds__(256) void centroid_logits_kernel(int Cq, int Ck, float sl2,
                                                              const float* __restrict__ qc,
                                                              const float* __restrict__ kc,
                                                              float* __restrict__ st2) {
  __shared__ __attribute__((aligned(16))) float qs[16][D + 4];
  __shared__ __attribute__((aligned(16))) float kcs[16][D + 4];
  const int h = blockIdx.z, c0 = blockIdx.y * 16, k0 = blockIdx.x * 16, tid = threadIdx.x;
  constexpr int V = D / 4;  // float4 pieces per row
  for (int i = tid; i < 16 * V; i += 256) {
    const int r = i / V, j = (i % V) * 4;
    // clamped rows, loaded unconditionally; rows past the end become zero
    float4 x = *reinterpret_cast<const float4*>(qc + (size_t(h) * Cq + min(c0 + r, Cq - 1)) * D + j);
    float4 y = *reinterpret_cast<const float4*>(kc + (size_t(h) * Ck + min(k0 + r, Ck - 1)) * D + j);
    if (c0 + r >= Cq) x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k0 + r >= Ck) y = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(&qs[r][j]) = x;
    *reinterpret_cast<float4*>(&kcs[r][j]) = y;
  }
  __syncthreads();
  const int a = tid / 16, b = tid % 16;
  // in double: the probe subtracts this logit from each raw key's, so its
  // rounding is the only error the pair shares (one f32 rounding at the end);
  // four interleaved partial sums shorten the dependent chain
  double dot[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
  for (int j = 0; j < D; j += 4) {
    const float4 x = *reinterpret_cast<const float4*>(&qs[a][j]);
    const float4 y = *reinterpret_cast<const float4*>(&kcs[b][j]);
    dot[0] = fma(double(x.x), double(y.x), dot[0]);
    dot[1] = fma(double(x.y), double(y.y), dot[1]);
    dot[2] = fma(double(x.z), double(y.z), dot[2]);
    dot[3] = fma(double(x.w), double(y.w), dot[3]);
  }
  if (c0 + a < Cq && k0 + b < Ck)
    st2[(size_t(h) * Ck + k0 + b) * Cq + c0 + a] =
        float(((dot[0] + dot[1]) + (dot[2] + dot[3])) * double(sl2));
}

__device__ __forceinline__ int find_unit_cluster(const int32_t* prefix, int C, int q) {
  int lo = 0, hi = C;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= q) lo = mid; else hi = mid;
  }
  return lo;
}

// (a_j, b_j) = (||v_j - vbar||^2, 2 (v_j - vbar).vbar) for every permuted key j.
// One block per key cluster, whose keys are the consecutive rows
// [koff[c], koff[c+1]) of the permuted tensor: its mean row stays in
// registers, 16 lanes per key row, 16 rows per pass.
template <typename T, int D>
__global__ __launch_bounds__(256) void value_stats_kernel(const T* __restrict__ Vp,
                                                          const float* __restrict__ vc,
                                                          const int32_t* __restrict__ koff,
                                                          int Nk, int Ck,
                                                          float2* __restrict__ stats) {
  constexpr int EL = D / 16;  // elements per lane
  const int h = blockIdx.y, c = blockIdx.x, tid = threadIdx.x, sub = tid & 15;
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  const int j0 = max(ko[c], 0), j1 = min(ko[c + 1], Nk);
  const float* vb = vc + (size_t(h) * Ck + c) * D + sub * EL;
  float m[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) m[e] = vb[e];
  // (every lane of a 16-lane row group takes the same trip count, so the
  // group's lane swaps below only read lanes of that group)
  for (int j = j0 + (tid >> 4); j < j1; j += 16) {
    const T* v = Vp + (size_t(h) * Nk + j) * D + sub * EL;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const float df = to_f32(v[e]) - m[e];
      a = fmaf(df, df, a);
      b = fmaf(df, m[e], b);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      a += __shfl_xor(a, o, 64);
      b += __shfl_xor(b, o, 64);
    }
    if (sub == 0) stats[size_t(h) * Nk + j] = make_float2(a, 2.f * b);
  }
}

// w[h][k] = ||vbar_k||^2, one wavefront per key cluster.
template <int D>
__global__ __launch_bounds__(256) void vbar_norm_kernel(int Ck, const float* __restrict__ vc,
                                                        float* __restrict__ w) {
  const int h = blockIdx.y, k = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (k >= Ck) return;  // whole wavefronts
  const float* vb = vc + (size_t(h) * Ck + k) * D;
  float x = 0.f;
  for (int e = lane; e < D; e += 64) x = fmaf(vb[e], vb[e], x);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  if (lane == 0) w[size_t(h) * Ck + k] = x;
}

template <typename T, int D, bool VALUE>
__global__ __launch_bounds__(256) void probe_kernel(const float* __restrict__ qc,
                                                    const T* __restrict__ Kp,
                                                    const float* __restrict__ kc,
                                                    const int32_t* __restrict__ koff,
                                                    const int32_t* __restrict__ unit_prefix,
                                                    const float* __restrict__ st2g,
                                                    const float2* __restrict__ vstat,
                                                    int Nk, int Cq, int Ck, int maxu, float sl2,
                                                    float* __restrict__ rec) {
  constexpr int RS = VALUE ? 4 : 3;  // floats per unit record
  constexpr int KC = D / 32;
  constexpr int LDR = D + 16 / sizeof(T);
  constexpr int QD = D / 4;  // dims staged per thread (4 threads per key row)
  __shared__ __attribute__((aligned(16))) T ks[64 * LDR];
  __shared__ __attribute__((aligned(16))) T kl[sizeof(T) == 2 ? 64 * LDR : 8];
  __shared__ __attribute__((aligned(16))) float2 vs[VALUE ? 64 : 2];  // (a_j, b_j) of the tile

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
  auto load_raw = [&](const Tile& t, uint4 (&raw)[RAW], float2& vraw) {
    const bool ok = t.tj + srow < t.j1;
    const T* src = Kh + size_t(ok ? t.tj + srow : 0) * D + sq * QD;
#pragma unroll
    for (int i = 0; i < RAW; ++i) raw[i] = reinterpret_cast<const uint4*>(src)[i];
    if (VALUE && sq == 0)
      vraw = ok ? vstat[size_t(h) * Nk + t.tj + srow] : make_float2(0.f, 0.f);
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
  float2 vraw = make_float2(0.f, 0.f);
  float kb[QD], kbn[QD];
  load_raw(cur, raw, vraw);
  load_kbar(cur.cc, kb);
  float st[2], mp[2], Z[2], E[2], Ev[2], e2[2];
  auto unit_start = [&](int cc) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      st[cb] = cok[cb] ? st2g[(size_t(h) * Ck + cc) * Cq + cidx[cb]] : 0.f;
      mp[cb] = 0.f;  // reference relative to s~: m = s~ + mp, mp >= 0
      Z[cb] = 0.f;
      E[cb] = 0.f;
      Ev[cb] = 0.f;
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
        constexpr int E8 = 16 / sizeof(T);
        if constexpr (kSplit) {
          // bf16 pairs: unpack, subtract kbar, round to the high part and the
          // remainder two at a time (the same round-to-nearest-even values as
          // element by element)
          typedef float f2 __attribute__((ext_vector_type(2)));
          typedef __bf16 b2 __attribute__((ext_vector_type(2)));
          uint32_t hi4[4], lo4[4];
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            const uint32_t wd = (&raw[i].x)[w2];
            const f2 x = {__uint_as_float(wd << 16), __uint_as_float(wd & 0xffff0000u)};
            const f2 dl = x - f2{kb[i * E8 + 2 * w2], kb[i * E8 + 2 * w2 + 1]};
            const b2 hb = __builtin_convertvector(dl, b2);
            const uint32_t hw = __builtin_bit_cast(uint32_t, hb);
            const f2 hf = {__uint_as_float(hw << 16), __uint_as_float(hw & 0xffff0000u)};
            hi4[w2] = hw;
            lo4[w2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(dl - hf, b2));
          }
          const uint4 hv = ok ? make_uint4(hi4[0], hi4[1], hi4[2], hi4[3]) : make_uint4(0, 0, 0, 0);
          const uint4 lv = ok ? make_uint4(lo4[0], lo4[1], lo4[2], lo4[3]) : make_uint4(0, 0, 0, 0);
          *reinterpret_cast<uint4*>(dst + i * E8) = hv;
          *reinterpret_cast<uint4*>(dlo + i * E8) = lv;
        } else {
          const T* el = reinterpret_cast<const T*>(&raw[i]);
          T out[E8];
#pragma unroll
          for (int e = 0; e < E8; ++e) out[e] = ok ? el[e] - kb[i * E8 + e] : 0.f;
          *reinterpret_cast<uint4*>(dst + i * E8) = *reinterpret_cast<const uint4*>(out);
        }
      }
      if (VALUE && sq == 0) vs[srow] = vraw;
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
      load_raw(nxt, raw, vraw);
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
          if (VALUE) Ev[cb] *= al * al;
          mp[cb] = tmax;
          e2[cb] = fast_exp2(-tmax);
        }
        float2 vk[4];
        if (VALUE) {
          const float4* vp4 = reinterpret_cast<const float4*>(&vs[kb16 * 16 + g * 4]);
          const float4 x0 = vp4[0], x1 = vp4[1];
          vk[0] = make_float2(x0.x, x0.y); vk[1] = make_float2(x0.z, x0.w);
          vk[2] = make_float2(x1.x, x1.y); vk[3] = make_float2(x1.z, x1.w);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kb16 * 16 + g * 4 + i < nvalid) {
            const float e = fast_exp2(d2[i] - mp[cb]);
            Z[cb] += e;
            const float dd = e - e2[cb];
            E[cb] = fmaf(dd, dd, E[cb]);
            if (VALUE) Ev[cb] = fmaf(e, fmaf(dd, vk[i].y, e * vk[i].x), Ev[cb]);
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
          const float oV = VALUE ? __shfl_xor(Ev[cb], o, 64) : 0.f;
          const float M = fmaxf(mp[cb], om);
          const float a1 = fast_exp2(mp[cb] - M), a2 = fast_exp2(om - M);
          Z[cb] = Z[cb] * a1 + oZ * a2;
          E[cb] = E[cb] * (a1 * a1) + oE * (a2 * a2);
          if (VALUE) Ev[cb] = Ev[cb] * (a1 * a1) + oV * (a2 * a2);
          mp[cb] = M;
        }
        if (g == 0 && cok[cb]) {
          // records are centroid-major ([h][c][unit]), so that the finalize
          // pass reads each centroid's units contiguously
          float* o = rec + ((size_t(h) * Cq + cidx[cb]) * maxu + cur.u) * RS;
          o[0] = st[cb] + mp[cb];  // absolute base-2 reference of this unit
          o[1] = Z[cb];
          o[2] = E[cb];
          if (VALUE) o[3] = Ev[cb];
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

// ---- bf16 keys: raw key tiles copied straight into LDS ---------------------
//
// For bf16 keys the kernel below replaces the staging of (k - kbar): the
// matrix cores take the raw keys (exact bf16) against q' = sl2 qbar carried
// as two bf16 parts (q' = p0 + p1 to about 2^-17 relative), and every
// accumulator starts at -sl2 qbar.kbar (the centroid logit, formed in double
// and rounded once), so that the result is the base-2 delta logit D_j =
// sl2 qbar.(k_j - kbar) with no vector work per key before the
// exponentials. Tiles of 64 keys are copied from HBM into LDS by the buffer
// unit, already in MFMA fragment order (fragment (rb, kc) = keys 16 rb .. +15,
// dims 32 kc .. +31: lane (r, g) holds key 16 rb + r, dims 32 kc + 8 g .. +7),
// through three buffers, so that the next two tiles are in flight while the
// current one is multiplied.
typedef __attribute__((address_space(3))) void probe_lds_void;

// 16 (or 4) bytes at byte offset voff of [base, base + bytes) into LDS at
// dst + size * lane (kept out of the kernel template's body, like the
// attention kernel's copy helper).
__device__ __forceinline__ void probe_copy_lds(const void* base, uint32_t bytes, uint32_t voff,
                                               probe_lds_void* dst, int size) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
  if (size == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, 0, 0, 0);
}

template <int D, bool VALUE>
__global__ __launch_bounds__(256) void probe_bf16_kernel(
    const float* __restrict__ qc, const __bf16* __restrict__ Kp, const int32_t* __restrict__ koff,
    const int32_t* __restrict__ unit_prefix, const float* __restrict__ st2g,
    const float2* __restrict__ vstat, int Nk, int Cq, int Ck, int maxu, float sl2,
    float* __restrict__ rec) {
  constexpr int RS = VALUE ? 4 : 3;
  constexpr int KC = D / 32;
  constexpr int FR = 4 * KC;   // 1 KB fragments per 64-key tile
  constexpr int NI = FR / 4;   // copy instructions per wave and tile
  constexpr int TILE = 64 * D;
  // three tile buffers (copies run two tiles ahead), each a distinct LDS
  // object so that the compiler tells the asynchronous fill of one from the
  // reads of another
  __shared__ __attribute__((aligned(16))) __bf16 kt0[TILE];
  __shared__ __attribute__((aligned(16))) __bf16 kt1[TILE];
  __shared__ __attribute__((aligned(16))) __bf16 kt2[TILE];
  // (a_j, b_j) of the tile's keys, as two arrays of 64 floats
  __shared__ __attribute__((aligned(16))) float va0[VALUE ? 64 : 4];
  __shared__ __attribute__((aligned(16))) float vb0[VALUE ? 64 : 4];
  __shared__ __attribute__((aligned(16))) float va1[VALUE ? 64 : 4];
  __shared__ __attribute__((aligned(16))) float vb1[VALUE ? 64 : 4];
  __shared__ __attribute__((aligned(16))) float va2[VALUE ? 64 : 4];
  __shared__ __attribute__((aligned(16))) float vb2[VALUE ? 64 : 4];
  // the centroid logits of the tile's key cluster: wave w's 64 floats hold its
  // two centroid blocks at [64 w + 16 cb + r]
  __shared__ __attribute__((aligned(16))) float sb0[256];
  __shared__ __attribute__((aligned(16))) float sb1[256];
  __shared__ __attribute__((aligned(16))) float sb2[256];
  // copy instructions per wave and tile (the vmcnt of one tile's copies)
  constexpr int CPT = NI + 1 + (VALUE ? 2 : 0);
  static_assert(CPT < 16, "vmcnt field");

  const int h = blockIdx.y, grp = blockIdx.z, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int32_t* up = unit_prefix + size_t(h) * (Ck + 1);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  if (up[Ck] == 0) return;  // no keys in this head (uniform over the block)

  // B operands: centroid blocks w and w + 4 of the group's 8, q' in two parts
  Frag<__bf16> bq[2][KC][2];
  int cidx[2];
  bool cok[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = grp * kProbeGroup + (w + 4 * cb) * 16 + r;
    cidx[cb] = c;
    cok[cb] = c < Cq;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      // (a clamped row, loaded unconditionally: no branch per element)
      const float4* qrow = reinterpret_cast<const float4*>(
          qc + (size_t(h) * Cq + (cok[cb] ? c : 0)) * D + k * 32 + g * 8);
      const float4 q0 = qrow[0], q1 = qrow[1];
      const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = cok[cb] ? qv[e] * sl2 : 0.f;
        const __bf16 p0 = __bf16(x);
        bq[cb][k][0].v[e] = p0;
        bq[cb][k][1].v[e] = __bf16(x - float(p0));  // the difference is exact
      }
    }
  }
  const uint32_t kbytes = uint32_t(size_t(Nk) * D * 2);
  const __bf16* Kh = Kp + size_t(h) * Nk * D;
  const float2* Vs = VALUE ? vstat + size_t(h) * Nk : nullptr;
  const uint32_t vbytes = uint32_t(size_t(Nk) * 8);
  const int wu = __builtin_amdgcn_readfirstlane(w);

  // A tile: unit u (keys [j0, j1) of cluster cc, whose keys end at kend),
  // keys tj .. tj + 63 of it. u == kNone: no tile.
  struct Tile {
    int u, cc, j0, j1, tj, kend;
  };
  constexpr int kNone = 0x7fffffff;
  // The block's share of the head: the units whose first key lies in
  // [J0, J1), where the head's blocks split its keys evenly. That is a run of
  // consecutive units, which the block walks in order, so that finding the
  // next unit takes at most a read of the next cluster's end (no search).
  const int J0 = int(int64_t(Nk) * blockIdx.x / gridDim.x);
  const int J1 = int(int64_t(Nk) * (blockIdx.x + 1) / gridDim.x);
  // the unit after t (skipping empty clusters), or none
  auto next_unit = [&](const Tile& t) {
    Tile n = t;
    n.u = t.u + 1;
    if (t.j1 < t.kend) {
      n.j0 = t.j1;
    } else {
      int c = t.cc + 1;
      while (c < Ck && ko[c + 1] == t.kend) ++c;
      if (c >= Ck) {
        n.u = kNone;
        return n;
      }
      n.cc = c;
      n.j0 = t.kend;
      n.kend = ko[c + 1];
    }
    if (n.j0 >= J1) n.u = kNone;
    n.j1 = min(n.j0 + kProbeUnit, n.kend);
    n.tj = n.j0;
    return n;
  };
  // copies of one tile into (kt, va, vb); rows past the unit read its first
  // row (finite data, masked out below)
  const uint32_t sbytes = uint32_t(size_t(Ck) * Cq * 4);
  const float* sth = st2g + size_t(h) * Ck * Cq;
  // the centroid this lane copies the logit of (lanes 32..63 repeat 0..31)
  const int scid = min(grp * kProbeGroup + (wu + 4 * ((lane >> 4) & 1)) * 16 + r, Cq - 1);
  auto issue = [&](const Tile& t, __bf16* kt, float* va, float* vb, float* sb) {
    probe_copy_lds(sth, sbytes, uint32_t(t.cc * Cq + scid) * 4, (probe_lds_void*)(sb + wu * 64), 4);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int f = wu * NI + i, rb = f / KC, kc = f % KC;
      int row = t.tj + rb * 16 + r;
      row = row < t.j1 ? row : t.j0;
      probe_copy_lds(Kh, kbytes, uint32_t(row) * (D * 2) + (kc * 32 + g * 8) * 2,
                     (probe_lds_void*)(kt + f * 512), 16);
    }
    if (VALUE && lane < 16) {  // wave w: keys 16 w .. 16 w + 15
      const int k = t.tj + wu * 16 + lane;
      const int key = k < t.j1 ? k : t.j0;
      probe_copy_lds(Vs, vbytes, uint32_t(key) * 8, (probe_lds_void*)(va + wu * 16), 4);
      probe_copy_lds(Vs, vbytes, uint32_t(key) * 8 + 4, (probe_lds_void*)(vb + wu * 16), 4);
    }
  };

  float st[2], mp[2], Z[2], E[2], Ev[2], e2[2];
  auto reset = [&]() {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      mp[cb] = 0.f;  // reference relative to s~: m = s~ + mp, mp >= 0
      Z[cb] = 0.f;
      E[cb] = 0.f;
      Ev[cb] = 0.f;
      e2[cb] = 1.f;
    }
  };
  // the next tile: the rest of this unit, else the first tile of the next
  auto next_of = [&](const Tile& cur) {
    if (cur.tj + 64 < cur.j1) {
      Tile nxt = cur;
      nxt.tj += 64;
      return nxt;
    }
    return next_unit(cur);
  };
  // products and streaming sums of one tile held in (kt, va, vb, sb), in two
  // halves of 32 keys: both halves are multiplied first (the two centroid
  // blocks' chains interleaved), then each half takes its own rescale of
  // the running reference (branch-free) and its exponentials. A full tile
  // (64 keys of the unit) takes a branch-free path; the unit's last, partial
  // tile masks the keys past its end. Both centroid blocks are always multiplied: a block without live
  // centroids has zero operands and is never recorded.
  auto compute_impl = [&](auto full_tag, const Tile& cur, const __bf16* kt, const float* va,
                          const float* vb, const float* sb) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int nvalid = FULL ? 64 : min(64, cur.j1 - cur.tj);
    const int ngrp = FULL ? 4 : (nvalid + 15) >> 4;  // groups holding a key (uniform)
    st[0] = sb[wu * 64 + r];
    st[1] = sb[wu * 64 + 16 + r];
    const f32x4 seed[2] = {f32x4{-st[0], -st[0], -st[0], -st[0]},
                           f32x4{-st[1], -st[1], -st[1], -st[1]}};
    f32x4 acc[2][4];
    // products of groups kb0, kb0 + 1
    auto products = [&](int kb0) {
#pragma unroll
      for (int kb = kb0; kb < kb0 + 2; ++kb) {
        if (FULL || kb < ngrp) {
          Frag<__bf16> a[KC];
#pragma unroll
          for (int k = 0; k < KC; ++k) a[k] = load8(kt + (kb * KC + k) * 512 + lane * 8);
          acc[0][kb] = seed[0];
          acc[1][kb] = seed[1];
#pragma unroll
          for (int k = 0; k < KC; ++k)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              mma(acc[0][kb], a[k], bq[0][k][p]);
              mma(acc[1][kb], a[k], bq[1][k][p]);
            }
        }
      }
    };
    // rescale test and streamed sums of groups kb0, kb0 + 1
    auto sums = [&](int kb0) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float tmax = mp[cb];
#pragma unroll
        for (int kb = kb0; kb < kb0 + 2; ++kb) {
          if (FULL || kb < ngrp) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (!FULL && kb * 16 + g * 4 + i >= nvalid) acc[cb][kb][i] = -__builtin_inff();
              tmax = fmaxf(tmax, acc[cb][kb][i]);
            }
          }
        }
        // the reference follows the maximum without a branch (al = 1 when it
        // stays), so that a full tile is one straight block of code
        {
          const float mn = fmaxf(mp[cb], tmax);
          const float al = fast_exp2(mp[cb] - mn);
          Z[cb] *= al;
          E[cb] *= al * al;
          if (VALUE) Ev[cb] *= al * al;
          mp[cb] = mn;
          e2[cb] = fast_exp2(-mn);
        }
        const float m = mp[cb], ee = e2[cb];
        float zs[2] = {0.f, 0.f}, es[2] = {0.f, 0.f}, vs2[2] = {0.f, 0.f};
#pragma unroll
        for (int kb = kb0; kb < kb0 + 2; ++kb) {
          if (FULL || kb < ngrp) {
            float ax[4], bx[4];
            if (VALUE) {
              const float4 xa = *reinterpret_cast<const float4*>(va + kb * 16 + g * 4);
              const float4 xb = *reinterpret_cast<const float4*>(vb + kb * 16 + g * 4);
              ax[0] = xa.x; ax[1] = xa.y; ax[2] = xa.z; ax[3] = xa.w;
              bx[0] = xb.x; bx[1] = xb.y; bx[2] = xb.z; bx[3] = xb.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // a masked key gives e = 0 and dd = -ee: its square is dropped
              const int pp = i & 1;
              const float e = fast_exp2(acc[cb][kb][i] - m);
              zs[pp] += e;
              const float dd = (FULL || kb * 16 + g * 4 + i < nvalid) ? e - ee : 0.f;
              es[pp] = fmaf(dd, dd, es[pp]);
              if (VALUE) vs2[pp] = fmaf(e, fmaf(dd, bx[i], e * ax[i]), vs2[pp]);
            }
          }
        }
        Z[cb] += zs[0] + zs[1];
        E[cb] += es[0] + es[1];
        if (VALUE) Ev[cb] += vs2[0] + vs2[1];
      }
    };
    // the second half's products overlap the first half's sums: in a full
    // tile (one block of straight code) the scheduler is asked to alternate
    // one matrix instruction with a few vector ones
    products(0);
    products(2);
    sums(0);
    sums(2);
  };
  auto compute = [&](const Tile& cur, const __bf16* kt, const float* va, const float* vb,
                     const float* sb) {
    if (cur.j1 - cur.tj >= 64) compute_impl(std::true_type{}, cur, kt, va, vb, sb);
    else compute_impl(std::false_type{}, cur, kt, va, vb, sb);
  };
  // a unit is done: merge the four lanes of each centroid and record it
  auto record = [&](const Tile& cur) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float om = __shfl_xor(mp[cb], o, 64);
        const float oZ = __shfl_xor(Z[cb], o, 64);
        const float oE = __shfl_xor(E[cb], o, 64);
        const float oV = VALUE ? __shfl_xor(Ev[cb], o, 64) : 0.f;
        const float M = fmaxf(mp[cb], om);
        const float a1 = fast_exp2(mp[cb] - M), a2 = fast_exp2(om - M);
        Z[cb] = Z[cb] * a1 + oZ * a2;
        E[cb] = E[cb] * (a1 * a1) + oE * (a2 * a2);
        if (VALUE) Ev[cb] = Ev[cb] * (a1 * a1) + oV * (a2 * a2);
        mp[cb] = M;
      }
      if (g == 0 && cok[cb]) {
        float* o = rec + ((size_t(h) * Cq + cidx[cb]) * maxu + cur.u) * RS;
        o[0] = st[cb] + mp[cb];  // absolute base-2 reference of this unit
        o[1] = Z[cb];
        o[2] = E[cb];
        if (VALUE) o[3] = Ev[cb];
      }
    }
  };
  // one step: wait for the current tile's copies (leaving the next tile's in
  // flight), start the copies two tiles ahead, multiply the current tile.
  // cur, n1, n2 are the current tile and the next two (u == kNone: none);
  // past the last tile the copies repeat the current one, so that every step
  // issues and waits for the same number of copies.
  // Returns false after the last tile.
  auto step = [&](Tile& cur, Tile& n1, Tile& n2, const __bf16* kt, const float* va,
                  const float* vb, const float* sb, __bf16* ktn, float* van, float* vbn,
                  float* sbn) -> bool {
    // vmcnt(CPT), lgkmcnt(0): every copy but n1's has landed
    __builtin_amdgcn_s_waitcnt((CPT & 15) | (7 << 4) | ((CPT >> 4) << 14));
    // every wave's copies of this tile have landed, and every wave is done
    // with the buffer the new copies fill (the barrier adds no wait of its own)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(n2.u != kNone ? n2 : cur, ktn, van, vbn, sbn);
    compute(cur, kt, va, vb, sb);
    if (n1.u != cur.u) {
      record(cur);
      reset();
    }
    cur = n1;
    n1 = n2;
    if (n2.u != kNone) n2 = next_of(n2);
    return cur.u != kNone;
  };

  // the first unit: the one after the (possibly empty) stretch of the cluster
  // holding key J0 that starts before J0
  Tile cur;
  {
    int lo = 0, hi = Ck;  // the last cluster c with ko[c] <= J0 (a non-empty one)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ko[mid] <= J0) lo = mid; else hi = mid;
    }
    const int k = (J0 - ko[lo] + kProbeUnit - 1) / kProbeUnit;  // units starting before J0
    Tile before;
    before.cc = lo;
    before.kend = ko[lo + 1];
    before.u = up[lo] + k - 1;
    before.j0 = before.j1 = min(ko[lo] + k * kProbeUnit, before.kend);
    cur = next_unit(before);
  }
  if (cur.u == kNone) return;  // uniform: no unit starts in this block's keys
  reset();
  Tile n1 = next_of(cur);
  Tile n2 = n1.u != kNone ? next_of(n1) : n1;
  issue(cur, kt0, va0, vb0, sb0);
  issue(n1.u != kNone ? n1 : cur, kt1, va1, vb1, sb1);
  while (step(cur, n1, n2, kt0, va0, vb0, sb0, kt2, va2, vb2, sb2) &&
         step(cur, n1, n2, kt1, va1, vb1, sb1, kt0, va0, vb0, sb0) &&
         step(cur, n1, n2, kt2, va2, vb2, sb2, kt1, va1, vb1, sb1)) {
  }
  __builtin_amdgcn_s_waitcnt(0);
}

template <bool VALUE>
__global__ __launch_bounds__(256) void probe_finalize_kernel(int Cq, int Ck, int maxu,
                                                             const int32_t* __restrict__ koff,
                                                             const int32_t* __restrict__ unit_prefix,
                                                             const float* __restrict__ rec,
                                                             const float* __restrict__ wv,
                                                             float* __restrict__ ratio,
                                                             float* __restrict__ log_norm) {
  constexpr int RS = VALUE ? 4 : 3;
  __shared__ float red[256];
  const int h = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int32_t* up = unit_prefix + size_t(h) * (Ck + 1);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);
  const int nu = up[Ck];
  auto R = [&](int u, int k) { return rec[((size_t(h) * Cq + c) * maxu + u) * RS + k]; };

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
      const float wk = VALUE ? wv[size_t(h) * Ck + k] : 0.f;
      for (int u = up[k]; u < up[k + 1]; ++u) {
        const float a = fast_exp2(R(u, 0) - m);
        e += (VALUE ? fmaf(R(u, 2), wk, R(u, 3)) : R(u, 2)) * (a * a);
      }
      out = e * inv / float(n);
    }
    ratio[(size_t(h) * Cq + c) * Ck + k] = out;
  }
  if (tid == 0 && log_norm) log_norm[size_t(h) * Cq + c] = (m + __log2f(Z)) * 0.69314718055994530942f;
}

size_t probe_ws_bytes(int H, int Nk, int Cq, int Ck, bool values) {
  return align256(sizeof(int32_t) * size_t(H) * (Ck + 1)) +
         align256(sizeof(float) * size_t(H) * Cq * Ck) +
         align256(sizeof(float) * (values ? 4 : 3) * size_t(H) * max_units(Nk, Ck) * Cq) +
         (values ? align256(sizeof(float2) * size_t(H) * Nk) + align256(sizeof(float) * size_t(H) * Ck)
                 : 0);
}

// Blocks of 256 threads of `kernel` that the current device holds at once
// (compute units times blocks per unit), or 0 on failure.
static int resident_blocks(const void* kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess)
    return 0;
  return cus * per_cu;
}

template <typename T, int D, bool VALUE>
static hipError_t probe_t(int H, int Nk, int Cq, int Ck, float sl2, const float* qc,
                          const void* Kp, const float* kc, const int32_t* koff, const int32_t* up,
                          float* st2, const float2* vstat, float* rec, hipStream_t s) {
  hipLaunchKernelGGL((centroid_logits_kernel<D>), dim3(ceil_div(Ck, 16), ceil_div(Cq, 16), H),
                     dim3(256), 0, s, Cq, Ck, sl2, qc, kc, st2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int maxu = max_units(Nk, Ck);
  const int groups = ceil_div(Cq, kProbeGroup);
  if constexpr (sizeof(T) == 2) {
    // one wave of resident blocks: the head's keys split evenly over its blocks
    const int cap = resident_blocks(reinterpret_cast<const void*>(&probe_bf16_kernel<D, VALUE>));
    if (cap <= 0) return hipErrorInvalidDeviceFunction;
    int per_head = cap / (H * groups);
    per_head = per_head < 1 ? 1 : (per_head > maxu ? maxu : per_head);
    hipLaunchKernelGGL((probe_bf16_kernel<D, VALUE>), dim3(per_head, H, groups), dim3(256), 0, s,
                       qc, static_cast<const __bf16*>(Kp), koff, up, st2, vstat, Nk, Cq, Ck, maxu,
                       sl2, rec);
  } else {
    int per_head = ceil_div(2048, H * groups);
    per_head = per_head < 1 ? 1 : (per_head > maxu ? maxu : per_head);
    hipLaunchKernelGGL((probe_kernel<T, D, VALUE>), dim3(per_head, H, groups), dim3(256), 0, s,
                       qc, static_cast<const T*>(Kp), kc, koff, up, st2, vstat, Nk, Cq, Ck, maxu,
                       sl2, rec);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t value_stats_t(int H, int Nk, int Ck, const void* Vp, const float* vc,
                                const int32_t* koff, float2* stats, float* wv, hipStream_t s) {
  hipLaunchKernelGGL((value_stats_kernel<T, D>), dim3(Ck, H), dim3(256), 0, s,
                     static_cast<const T*>(Vp), vc, koff, Nk, Ck, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((vbar_norm_kernel<D>), dim3(ceil_div(Ck, 4), H), dim3(256), 0, s, Ck, vc, wv);
  return hipGetLastError();
}

hipError_t launch_probe(int elem_bytes, int H, int Nk, int d, int Cq, int Ck, float scale,
                        const float* qc, const void* Kp, const float* kc, const void* Vp,
                        const float* vc, const int32_t* koff, void* ws, float* ratio,
                        float* log_norm, hipStream_t s) {
  const bool values = Vp != nullptr;
  char* p = static_cast<char*>(ws);
  int32_t* up = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(H) * (Ck + 1));
  float* st2 = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * size_t(H) * Cq * Ck);
  float* rec = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * (values ? 4 : 3) * size_t(H) * max_units(Nk, Ck) * Cq);
  float2* vstat = values ? reinterpret_cast<float2*>(p) : nullptr;
  if (values) p += align256(sizeof(float2) * size_t(H) * Nk);
  float* wv = values ? reinterpret_cast<float*>(p) : nullptr;
  hipLaunchKernelGGL(probe_units_kernel, dim3(H), dim3(1024), 0, s, Ck, koff, up);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = scale * 1.44269504088896340736f;
  const bool bf = elem_bytes == 2, wide = d == 128;
  if (values) {
    e = bf ? (wide ? value_stats_t<__bf16, 128>(H, Nk, Ck, Vp, vc, koff, vstat, wv, s)
                   : value_stats_t<__bf16, 64>(H, Nk, Ck, Vp, vc, koff, vstat, wv, s))
           : (wide ? value_stats_t<float, 128>(H, Nk, Ck, Vp, vc, koff, vstat, wv, s)
                   : value_stats_t<float, 64>(H, Nk, Ck, Vp, vc, koff, vstat, wv, s));
    if (e != hipSuccess) return e;
    e = bf ? (wide ? probe_t<__bf16, 128, true>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, vstat, rec, s)
                   : probe_t<__bf16, 64, true>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, vstat, rec, s))
           : (wide ? probe_t<float, 128, true>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, vstat, rec, s)
                   : probe_t<float, 64, true>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, vstat, rec, s));
  } else {
    e = bf ? (wide ? probe_t<__bf16, 128, false>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, nullptr, rec, s)
                   : probe_t<__bf16, 64, false>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, nullptr, rec, s))
           : (wide ? probe_t<float, 128, false>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, nullptr, rec, s)
                   : probe_t<float, 64, false>(H, Nk, Cq, Ck, sl2, qc, Kp, kc, koff, up, st2, nullptr, rec, s));
  }
  if (e != hipSuccess) return e;
  if (values)
    hipLaunchKernelGGL(probe_finalize_kernel<true>, dim3(Cq, H), dim3(256), 0, s, Cq, Ck,
                       max_units(Nk, Ck), koff, up, rec, wv, ratio, log_norm);
  else
    hipLaunchKernelGGL(probe_finalize_kernel<false>, dim3(Cq, H), dim3(256), 0, s, Cq, Ck,
                       max_units(Nk, Ck), koff, up, rec, nullptr, ratio, log_norm);
  return hipGetLastError();
}

}  // namespace svg
