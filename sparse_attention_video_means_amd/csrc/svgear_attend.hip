// Compensated block-sparse attention (paper §4.1 block mask, §4.3 linear
// compensation): every query of query cluster c sees one softmax over the
// exact keys of its selected key clusters and one centroid logit (+ ln|k_c'|)
// per skipped non-empty key cluster, with mean values for the latter.
//
// Block = 4 wavefronts x 32 queries of one query cluster. The selected key
// clusters are packed back to back into 64-key tiles (a tile may span several
// clusters, so ragged cluster ends waste no matrix work); the skipped clusters'
// centroid rows follow as further 64-row tiles carrying the ln|k_c'| bias.
// Both kinds of tile run through the same online softmax:
//   S^T = K Q^T   (A = K rows from LDS, B = Q^T held in registers)
//   O^T += V^T P^T (A = V^T read from row-major LDS with ds_read_b64_tr_b16,
//                   B = P^T taken straight from the S^T accumulators)
// so P never leaves registers. Exponentials are base 2 with log2(e) folded
// into the scale; the running maximum is only raised (and O, l rescaled) when
// a tile's maximum exceeds it by more than 8, which keeps every p <= 2^8.
#include "svgear_common.hpp"
#include "svgear_internal.hpp"

namespace svg {

constexpr int kAttBM = 128;  // queries per block
constexpr int kAttBK = 64;   // keys per tile
constexpr float kRescaleSlack = 8.0f;

// A operand V^T (16 dims x 32 keys) for key chunk kc2 and dim block db; key
// slot e of lane (r, g) is tile row 32*kc2 + 4g + (e < 4 ? e : 12 + e).
template <int LDR>
__device__ __forceinline__ Frag<__bf16> load_vt(const __bf16* vs, int kc2, int db, int r, int g) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int row = kc2 * 32 + g * 4 + (r >> 2);
  const int col = db * 16 + (r & 3) * 4;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)(vs + row * LDR + col));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)(vs + (row + 16) * LDR + col));
  Frag<__bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

template <int LDR>
__device__ __forceinline__ Frag<float> load_vt(const float* vs, int kc2, int db, int r, int g) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = kc2 * 32 + g * 4 + (e < 4 ? e : 12 + e);
    f.v[e] = vs[key * LDR + db * 16 + r];
  }
  return f;
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4]);

template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, const float (&v)[4]) {
  bf16x4 x;
  x[0] = __bf16(v[0]); x[1] = __bf16(v[1]); x[2] = __bf16(v[2]); x[3] = __bf16(v[3]);
  *reinterpret_cast<bf16x4*>(p) = x;
}

template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&v)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attend_kernel(
    const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
    const int32_t* __restrict__ qoff, const int32_t* __restrict__ koff,
    const float* __restrict__ kcen, const float* __restrict__ vcen,
    const uint8_t* __restrict__ mask, int Nq, int Nk, int Cq, int Ck, float sl2,
    T* __restrict__ Op) {
  constexpr int KC = D / 32;
  constexpr int DB = D / 16;
  constexpr int LDR = D + 16 / sizeof(T);
  constexpr int EPT = 16 / sizeof(T);
  constexpr int PIECES = D / EPT / 4;  // 16-byte pieces each of 4 threads copies per row
  __shared__ __attribute__((aligned(16))) T ks[kAttBK * LDR];
  __shared__ __attribute__((aligned(16))) T vs[kAttBK * LDR];
  __shared__ int sel_s[kMaxClusters];
  __shared__ int comp_s[kMaxClusters];
  __shared__ int pref_s[kMaxClusters + 1];
  __shared__ float bias_s[kAttBK];
  __shared__ int scratch[16];
  __shared__ int info[2];

  const int h = blockIdx.y, t = blockIdx.x, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int32_t* qo = qoff + size_t(h) * (Cq + 1);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);

  // ---- which query cluster / tile this block owns
  int carry = 0;
  for (int b = 0; b < Cq; b += 256) {
    const int i = b + tid;
    const int nt = (i < Cq) ? (qo[i + 1] - qo[i] + kAttBM - 1) / kAttBM : 0;
    int tot;
    const int ex = block_exclusive_scan(nt, scratch, &tot);
    if (nt > 0 && t >= carry + ex && t < carry + ex + nt) {
      info[0] = i;
      info[1] = t - carry - ex;
    }
    carry += tot;
  }
  if (t >= carry) return;  // uniform: every thread computed the same total
  __syncthreads();
  const int c = info[0];
  const int q0 = qo[c] + info[1] * kAttBM;
  const int q1 = min(qo[c + 1], q0 + kAttBM);

  // ---- selected (packed) and compensated key-cluster lists
  const uint8_t* mk = mask + (size_t(h) * Cq + c) * Ck;
  int nsel = 0, nkeys = 0, ncomp = 0;
  for (int b = 0; b < Ck; b += 256) {
    const int i = b + tid;
    int n = 0, is_sel = 0, is_comp = 0;
    if (i < Ck) {
      n = ko[i + 1] - ko[i];
      is_sel = (mk[i] != 0) && n > 0;
      is_comp = (mk[i] == 0) && n > 0;
    }
    int t1, t2, t3;
    const int e1 = block_exclusive_scan(is_sel, scratch, &t1);
    const int e2 = block_exclusive_scan(is_sel ? n : 0, scratch, &t2);
    const int e3 = block_exclusive_scan(is_comp, scratch, &t3);
    if (is_sel) { sel_s[nsel + e1] = i; pref_s[nsel + e1] = nkeys + e2; }
    if (is_comp) comp_s[ncomp + e3] = i;
    nsel += t1; nkeys += t2; ncomp += t3;
  }
  if (tid == 0) pref_s[nsel] = nkeys;
  __syncthreads();

  // ---- Q^T fragments
  const T* Qh = Qp + size_t(h) * Nq * D;
  const int qw = q0 + w * 32;
  const bool active = qw < q1;
  Frag<T> qf[2][KC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + qb * 16 + r;
#pragma unroll
    for (int k = 0; k < KC; ++k)
      qf[qb][k] = (qi < q1) ? load8(Qh + size_t(qi) * D + k * 32 + g * 8) : zero_frag<T>();
  }

  f32x4 o[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-__builtin_inff(), -__builtin_inff()};
  float lsum[2] = {0.f, 0.f};

  const T* Kh = Kp + size_t(h) * Nk * D;
  const T* Vh = Vp + size_t(h) * Nk * D;
  const float* KCh = kcen + size_t(h) * Ck * D;
  const float* VCh = vcen + size_t(h) * Ck * D;
  const int nt_exact = (nkeys + kAttBK - 1) / kAttBK;
  const int nt_all = nt_exact + (ncomp + kAttBK - 1) / kAttBK;
  const int srow = tid >> 2, sq = tid & 3;

  for (int tile = 0; tile < nt_all; ++tile) {
    __syncthreads();
    // ---- stage 64 key rows and value rows (4 threads per row)
    {
      T* kd = ks + srow * LDR + sq * (D / 4);
      T* vd = vs + srow * LDR + sq * (D / 4);
      float bias = -__builtin_inff();
      if (tile < nt_exact) {
        const int p = tile * kAttBK + srow;
        if (p < nkeys) {
          int lo = 0, hi = nsel;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pref_s[mid] <= p) lo = mid; else hi = mid;
          }
          const int krow = ko[sel_s[lo]] + (p - pref_s[lo]);
          const T* kg = Kh + size_t(krow) * D + sq * (D / 4);
          const T* vg = Vh + size_t(krow) * D + sq * (D / 4);
#pragma unroll
          for (int i = 0; i < PIECES; ++i) {
            copy16(kd + i * EPT, kg + i * EPT);
            copy16(vd + i * EPT, vg + i * EPT);
          }
          bias = 0.f;
        } else {
#pragma unroll
          for (int i = 0; i < PIECES; ++i) {
            *reinterpret_cast<uint4*>(kd + i * EPT) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(vd + i * EPT) = make_uint4(0, 0, 0, 0);
          }
        }
      } else {
        const int p = (tile - nt_exact) * kAttBK + srow;
        if (p < ncomp) {
          const int cc = comp_s[p];
          const float* kg = KCh + size_t(cc) * D + sq * (D / 4);
          const float* vg = VCh + size_t(cc) * D + sq * (D / 4);
#pragma unroll
          for (int i = 0; i < D / 4; i += 4) {
            const float4 a = *reinterpret_cast<const float4*>(kg + i);
            const float4 b = *reinterpret_cast<const float4*>(vg + i);
            kd[i] = from_f32<T>(a.x); kd[i + 1] = from_f32<T>(a.y);
            kd[i + 2] = from_f32<T>(a.z); kd[i + 3] = from_f32<T>(a.w);
            vd[i] = from_f32<T>(b.x); vd[i + 1] = from_f32<T>(b.y);
            vd[i + 2] = from_f32<T>(b.z); vd[i + 3] = from_f32<T>(b.w);
          }
          bias = __log2f(float(ko[cc + 1] - ko[cc]));
        } else {
#pragma unroll
          for (int i = 0; i < PIECES; ++i) {
            *reinterpret_cast<uint4*>(kd + i * EPT) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(vd + i * EPT) = make_uint4(0, 0, 0, 0);
          }
        }
      }
      if (sq == 0) bias_s[srow] = bias;
    }
    __syncthreads();
    if (!active) continue;

    // ---- S^T = K Q^T
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag<T> a[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) a[k] = load8(&ks[(kb * 16 + r) * LDR + k * 32 + g * 8]);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KC; ++k) mma(s[kb][qb], a[k], qf[qb][k]);
      }
    }
    // ---- logits (base 2), tile maxima per query
    float bias4[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) bias4[kb][i] = bias_s[kb * 16 + g * 4 + i];
    float tmax[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = fmaf(s[kb][qb][i], sl2, bias4[kb][i]);
          s[kb][qb][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      tmax[qb] = mx;
    }
    const bool need0 = tmax[0] > mrow[0] + kRescaleSlack;
    const bool need1 = tmax[1] > mrow[1] + kRescaleSlack;
    if (__ballot(need0 || need1) != 0ull) {
      const float mn0 = need0 ? tmax[0] : mrow[0];
      const float mn1 = need1 ? tmax[1] : mrow[1];
      const float a0 = fast_exp2(mrow[0] - mn0), a1 = fast_exp2(mrow[1] - mn1);
      mrow[0] = mn0; mrow[1] = mn1;
      lsum[0] *= a0; lsum[1] *= a1;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        o[db][0] *= a0;
        o[db][1] *= a1;
      }
    }
    // ---- P^T fragments straight from the accumulators
    Frag<T> pb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float ls = 0.f;
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(s[kc2 * 2 + (e >> 2)][qb][e & 3] - mrow[qb]);
          ls += p;
          pb[qb][kc2].v[e] = from_f32<T>(p);
        }
      lsum[qb] += ls;
    }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        const Frag<T> va = load_vt<LDR>(vs, kc2, db, r, g);
        mma(o[db][0], va, pb[0][kc2]);
        mma(o[db][1], va, pb[1][kc2]);
      }
  }

  if (!active) return;
  T* Oh = Op + size_t(h) * Nq * D;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = lsum[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.f / l;
    const int qi = qw + qb * 16 + r;
    if (qi < q1) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = o[db][qb][i] * inv;
        store4<T>(Oh + size_t(qi) * D + db * 16 + g * 4, v);
      }
    }
  }
}

template <typename T, int D>
static void attend_t(int H, int Nq, int Nk, int Cq, int Ck, float sl2, const void* Qp,
                     const void* Kp, const void* Vp, const int32_t* qoff, const int32_t* koff,
                     const float* kc, const float* vc, const uint8_t* mask, void* Op,
                     hipStream_t s) {
  const int grid_x = ceil_div(Nq, kAttBM) + Cq;
  hipLaunchKernelGGL((attend_kernel<T, D>), dim3(grid_x, H), dim3(256), 0, s,
                     static_cast<const T*>(Qp), static_cast<const T*>(Kp),
                     static_cast<const T*>(Vp), qoff, koff, kc, vc, mask, Nq, Nk, Cq, Ck, sl2,
                     static_cast<T*>(Op));
}

hipError_t launch_attend(int elem_bytes, int H, int Nq, int Nk, int d, int Cq, int Ck,
                         float scale, const void* Qp, const void* Kp, const void* Vp,
                         const int32_t* qoff, const int32_t* koff, const float* kc,
                         const float* vc, const uint8_t* mask, void* Op, hipStream_t s) {
  const float sl2 = scale * 1.44269504088896340736f;
  if (elem_bytes == 2) {
    if (d == 128) attend_t<__bf16, 128>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, kc, vc, mask, Op, s);
    else attend_t<__bf16, 64>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, kc, vc, mask, Op, s);
  } else {
    if (d == 128) attend_t<float, 128>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, kc, vc, mask, Op, s);
    else attend_t<float, 64>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, kc, vc, mask, Op, s);
  }
  return hipGetLastError();
}

}  // namespace svg
