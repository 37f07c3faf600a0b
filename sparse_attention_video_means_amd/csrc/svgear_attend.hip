// Compensated block-sparse attention (paper §4.1 block mask, §4.3 linear
// compensation): every query of query cluster c sees one softmax over the
// exact keys of its selected key clusters and one centroid logit (+ ln|k_c'|)
// per skipped non-empty key cluster, with mean values for the latter.
//
// Block = 4 wavefronts x (16*QB) queries of one query cluster. The selected key
// clusters are packed back to back into 64-key tiles (a tile may span several
// clusters, so ragged cluster ends waste no matrix work); the skipped clusters'
// centroid rows (pre-rounded to the element type) follow as further 64-row
// tiles carrying the log2|k_c'| bias. Both kinds of tile run through the same
// online softmax:
//   S^T = K Q^T     (A = K rows from LDS, B = Q^T held in registers)
//   O^T += V^T P^T  (A = V^T read from row-major LDS with ds_read_b64_tr_b16,
//                    B = P^T taken straight from the S^T accumulators)
// so P never leaves registers.
//
// Tiles are double-buffered in LDS and filled by global_load_lds_dwordx4: each
// lane's 16-byte piece lands at (LDS pointer + 16 * lane), so no registers are
// spent on staging. Rows are stored unpadded with their 16-byte pieces XOR-
// swizzled by a function of the row, chosen so that both the K reads (16 rows,
// same piece) and the transposed V reads (8 rows, two adjacent pieces) hit
// distinct LDS banks. The loads of tile t+1 are issued before tile t is
// computed; one wait and one barrier per tile.
//
// Exponentials are base 2 with log2(e) folded into the scale; the running
// maximum is only raised (and O, l rescaled) when a tile's maximum exceeds it
// by more than 8, which keeps every p <= 2^8.
#include "svgear_common.hpp"
#include "svgear_internal.hpp"

namespace svg {

constexpr int kAttBK = 64;  // keys per tile
constexpr float kRescaleSlack = 8.0f;

template <typename T>
struct AttCfg;
#ifndef SVGEAR_ATT_QB_BF16
#define SVGEAR_ATT_QB_BF16 2
#endif
template <>
struct AttCfg<__bf16> {
  static constexpr int QB = SVGEAR_ATT_QB_BF16;  // 16-query blocks per wavefront
};
template <>
struct AttCfg<float> {
  static constexpr int QB = 2;
};

typedef __attribute__((address_space(3))) void lds_void;

// Swizzle of the 16-byte pieces of one LDS row; CPR = pieces per row.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPR == 16) {
    return ((row & 7) << 1) | ((row >> 3) & 1);
  } else if constexpr (CPR == 8) {
    const int a = row >> 1;
    return ((a & 3) << 1) | ((a >> 2) & 1);
  } else {
    return row & (CPR - 1);
  }
}

// Element (row, col) of a swizzled tile.
template <typename T, int D>
__device__ __forceinline__ int lds_index(int row, int col) {
  constexpr int EPT = 16 / sizeof(T);
  constexpr int CPR = D / EPT;
  return row * D + (((col / EPT) ^ swz<CPR>(row)) * EPT) + (col % EPT);
}

// A operand K (16 keys x 32 dims): lane (r, g) holds K[row0 + r][k*32 + g*8 .. +7].
template <int D>
__device__ __forceinline__ Frag<__bf16> load_k(const __bf16* ks, int row, int k, int g) {
  return load8(ks + lds_index<__bf16, D>(row, k * 32 + g * 8));
}

template <int D>
__device__ __forceinline__ Frag<float> load_k(const float* ks, int row, int k, int g) {
  Frag<float> f;
  const float4 a = *reinterpret_cast<const float4*>(ks + lds_index<float, D>(row, k * 32 + g * 8));
  const float4 b = *reinterpret_cast<const float4*>(ks + lds_index<float, D>(row, k * 32 + g * 8 + 4));
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}

// A operand V^T (16 dims x 32 keys) for key chunk kc2 and dim block db; key
// slot e of lane (r, g) is tile row 32*kc2 + 4g + (e < 4 ? e : 12 + e).
template <int D>
__device__ __forceinline__ Frag<__bf16> load_vt(const __bf16* vs, int kc2, int db, int r, int g) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int row = kc2 * 32 + g * 4 + (r >> 2);
  const int col = db * 16 + (r & 3) * 4;
  const bf16x4 lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vs + lds_index<__bf16, D>(row, col)));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)(vs + lds_index<__bf16, D>(row + 16, col)));
  Frag<__bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

template <int D>
__device__ __forceinline__ Frag<float> load_vt(const float* vs, int kc2, int db, int r, int g) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = kc2 * 32 + g * 4 + (e < 4 ? e : 12 + e);
    f.v[e] = vs[lds_index<float, D>(key, db * 16 + r)];
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

// max / sum of x over lanes l, l^16, l^32, l^48 (VALU lane swaps, no LDS).
__device__ __forceinline__ float quad_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}

__device__ __forceinline__ float quad_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(a[0]) + __int_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void attend_kernel(
    const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
    const int32_t* __restrict__ qoff, const int32_t* __restrict__ koff,
    const T* __restrict__ kcen, const T* __restrict__ vcen, const uint8_t* __restrict__ mask,
    int Nq, int Nk, int Cq, int Ck, float sl2, T* __restrict__ Op) {
  constexpr int QB = AttCfg<T>::QB;
  constexpr int BM = 64 * QB;
  constexpr int KC = D / 32;
  constexpr int DB = D / 16;
  constexpr int EPT = 16 / sizeof(T);
  constexpr int CPR = D / EPT;       // 16-byte pieces per row
  constexpr int NI = CPR / 4;        // load instructions per wave per tensor per tile
  constexpr int TILE = kAttBK * D;   // elements per tile
  // two buffers per tensor as distinct objects: the compiler can then tell
  // the asynchronous fill of one from the reads of the other and inserts no
  // wait between them
  __shared__ __attribute__((aligned(16))) T ks0[TILE];
  __shared__ __attribute__((aligned(16))) T ks1[TILE];
  __shared__ __attribute__((aligned(16))) T vs0[TILE];
  __shared__ __attribute__((aligned(16))) T vs1[TILE];
  __shared__ float bias0[kAttBK];
  __shared__ float bias1[kAttBK];
  // per-block lists, sized by Ck at launch (5 * Ck + 1 words):
  extern __shared__ int lists[];
  int* sel_s = lists;                  // selected key cluster ids, ascending
  int* start_s = lists + Ck;           // first key row of a selection minus its packed offset
  int* comp_s = lists + 2 * Ck;        // compensated (skipped, non-empty) key clusters
  float* cbias_s = reinterpret_cast<float*>(lists + 3 * Ck);  // log2 |k_c'| of those
  int* pref_s = lists + 4 * Ck;        // packed offset of every selected cluster (+ total)
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
    const int nt = (i < Cq) ? (qo[i + 1] - qo[i] + BM - 1) / BM : 0;
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
  const int q0 = qo[c] + info[1] * BM;
  const int q1 = min(qo[c + 1], q0 + BM);

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
    if (is_sel) {
      sel_s[nsel + e1] = i;
      pref_s[nsel + e1] = nkeys + e2;
      start_s[nsel + e1] = ko[i] - (nkeys + e2);
    }
    if (is_comp) {
      comp_s[ncomp + e3] = i;
      cbias_s[ncomp + e3] = __log2f(float(n));
    }
    nsel += t1; nkeys += t2; ncomp += t3;
  }
  if (tid == 0) pref_s[nsel] = nkeys;
  __syncthreads();

  const T* Kh = Kp + size_t(h) * Nk * D;
  const T* Vh = Vp + size_t(h) * Nk * D;
  const T* KCh = kcen + size_t(h) * Ck * D;
  const T* VCh = vcen + size_t(h) * Ck * D;
  const int nt_exact = (nkeys + kAttBK - 1) / kAttBK;
  const int nt_all = nt_exact + (ncomp + kAttBK - 1) / kAttBK;

  // ---- asynchronous tile loads: lane `lane` of instruction i fills LDS slot
  // (w*NI + i)*64 + lane, i.e. row slot/CPR, swizzled piece slot%CPR.
  int cur[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) cur[i] = 0;
  auto issue = [&](int tile, T* kd0, T* vd0, float* bd) {
    const bool exact = tile < nt_exact;  // uniform over the block
    const T* kbase = exact ? Kh : KCh;
    const T* vbase = exact ? Vh : VCh;
    int offs[NI];  // element offset of this lane's piece in every load
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = (w * NI + i) * 64 + lane;
      const int row = slot / CPR, pos = slot % CPR;
      const int piece = pos ^ swz<CPR>(row);
      int src = 0;  // filler row 0: finite data whose weight is exactly 0
      float bias = -__builtin_inff();
      if (exact) {
        const int p = tile * kAttBK + row;
        if (p < nkeys) {
          int cu = cur[i];
          while (cu + 1 < nsel && pref_s[cu + 1] <= p) ++cu;
          cur[i] = cu;
          src = start_s[cu] + p;
          bias = 0.f;
        }
      } else {
        const int p = (tile - nt_exact) * kAttBK + row;
        if (p < ncomp) {
          src = comp_s[p];
          bias = cbias_s[p];
        }
      }
      offs[i] = src * D + piece * EPT;
      if (pos == 0) bd[row] = bias;
    }
    // all LDS traffic of this step is above: nothing below touches LDS
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kbase + offs[i]),
                                       (lds_void*)(kd0 + (w * NI + i) * 64 * EPT), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(vbase + offs[i]),
                                       (lds_void*)(vd0 + (w * NI + i) * 64 * EPT), 16, 0, 0);
    }
  };

  // ---- Q^T fragments
  const T* Qh = Qp + size_t(h) * Nq * D;
  const int qw = q0 + w * 16 * QB;
  const bool active = qw < q1;
  Frag<T> qf[QB][KC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw + qb * 16 + r;
#pragma unroll
    for (int k = 0; k < KC; ++k)
      qf[qb][k] = (qi < q1) ? load8(Qh + size_t(qi) * D + k * 32 + g * 8) : zero_frag<T>();
  }

  f32x4 o[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { mrow[qb] = -__builtin_inff(); lsum[qb] = 0.f; }

  // one tile: start filling the other buffer with tile+1, compute this one
  auto step = [&](int tile, const T* kb_s, const T* vb_s, const float* bb_s, T* kn_s, T* vn_s,
                  float* bn_s) {
    if (tile + 1 < nt_all) issue(tile + 1, kn_s, vn_s, bn_s);
    if (active) {
      // the 64-key tile is processed as two 32-key halves to bound registers
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        // ---- S^T = K Q^T for keys 32*kh .. 32*kh+31
        f32x4 s[2][QB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < KC; ++k) {
            const Frag<T> a = load_k<D>(kb_s, kh * 32 + kb * 16 + r, k, g);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) mma(s[kb][qb], a, qf[qb][k]);
          }
        }
        // ---- logits (base 2) and maxima per query
        float bias4[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) bias4[kb][i] = bb_s[kh * 32 + kb * 16 + g * 4 + i];
        bool need = false;
        float tmax[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float mx = -__builtin_inff();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float v = fmaf(s[kb][qb][i], sl2, bias4[kb][i]);
              s[kb][qb][i] = v;
              mx = fmaxf(mx, v);
            }
          mx = quad_max(mx);
          tmax[qb] = mx;
          need = need || (mx > mrow[qb] + kRescaleSlack);
        }
        if (__ballot(need) != 0ull) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float mn = (tmax[qb] > mrow[qb] + kRescaleSlack) ? tmax[qb] : mrow[qb];
            const float al = fast_exp2(mrow[qb] - mn);
            mrow[qb] = mn;
            lsum[qb] *= al;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db][qb] *= al;
          }
        }
        // ---- P^T fragments straight from the accumulators
        Frag<T> pb[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float ls = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = fast_exp2(s[e >> 2][qb][e & 3] - mrow[qb]);
            ls += p;
            pb[qb].v[e] = from_f32<T>(p);
          }
          lsum[qb] += ls;
        }
        // ---- O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const Frag<T> va = load_vt<D>(vb_s, kh, db, r, g);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) mma(o[db][qb], va, pb[qb]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue(0, ks0, vs0, bias0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int tile = 0; tile < nt_all; tile += 2) {
    step(tile, ks0, vs0, bias0, ks1, vs1, bias1);
    if (tile + 1 < nt_all) step(tile + 1, ks1, vs1, bias1, ks0, vs0, bias0);
  }

  if (!active) return;
  T* Oh = Op + size_t(h) * Nq * D;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.f / quad_sum(lsum[qb]);
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

// Centroid rows rounded to the element type once per call.
template <typename T>
__global__ void round_rows_kernel(size_t n, const float* __restrict__ a, const float* __restrict__ b,
                                  T* __restrict__ ra, T* __restrict__ rb) {
  const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) {
    ra[i] = from_f32<T>(a[i]);
    rb[i] = from_f32<T>(b[i]);
  }
}

size_t attend_ws_bytes(int elem_bytes, int H, int Ck, int d) {
  return elem_bytes == 4 ? 0 : 2 * align256(size_t(elem_bytes) * H * Ck * d);
}

template <typename T, int D>
static void attend_t(int H, int Nq, int Nk, int Cq, int Ck, float sl2, const void* Qp,
                     const void* Kp, const void* Vp, const int32_t* qoff, const int32_t* koff,
                     const void* kc, const void* vc, const uint8_t* mask, void* Op,
                     hipStream_t s) {
  constexpr int BM = 64 * AttCfg<T>::QB;
  const int grid_x = ceil_div(Nq, BM) + Cq;
  const size_t lds_lists = sizeof(int) * (5 * size_t(Ck) + 1);
  hipLaunchKernelGGL((attend_kernel<T, D>), dim3(grid_x, H), dim3(256), lds_lists, s,
                     static_cast<const T*>(Qp), static_cast<const T*>(Kp),
                     static_cast<const T*>(Vp), qoff, koff, static_cast<const T*>(kc),
                     static_cast<const T*>(vc), mask, Nq, Nk, Cq, Ck, sl2, static_cast<T*>(Op));
}

hipError_t launch_attend(int elem_bytes, int H, int Nq, int Nk, int d, int Cq, int Ck,
                         float scale, const void* Qp, const void* Kp, const void* Vp,
                         const int32_t* qoff, const int32_t* koff, const float* kc,
                         const float* vc, const uint8_t* mask, void* Op, void* ws,
                         hipStream_t s) {
  const float sl2 = scale * 1.44269504088896340736f;
  if (elem_bytes == 2) {
    const size_t n = size_t(H) * Ck * d;
    __bf16* rk = static_cast<__bf16*>(ws);
    __bf16* rv = reinterpret_cast<__bf16*>(static_cast<char*>(ws) + align256(2 * n));
    hipLaunchKernelGGL(round_rows_kernel<__bf16>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s,
                       n, kc, vc, rk, rv);
    if (d == 128) attend_t<__bf16, 128>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, rk, rv, mask, Op, s);
    else attend_t<__bf16, 64>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, rk, rv, mask, Op, s);
  } else {
    if (d == 128) attend_t<float, 128>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, kc, vc, mask, Op, s);
    else attend_t<float, 64>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, kc, vc, mask, Op, s);
  }
  return hipGetLastError();
}

}  // namespace svg
