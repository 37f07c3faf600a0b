// Compensated block-sparse attention (paper §4.1 block mask, §4.3 linear
// compensation): every query of query cluster c sees one softmax over the
// exact keys of its selected key clusters and one centroid logit (+ ln|k_c'|)
// per skipped non-empty key cluster, with mean values for the latter.
//
// Block = NW wavefronts x (16*QB) queries of one query cluster; wavefront w
// takes the 16-query groups w, w + NW, ..., so that a partial block's groups
// spread evenly over the SIMDs. The selected
// key clusters are packed back to back into 64-key tiles (a tile may span
// several clusters, so ragged cluster ends waste no matrix work); the skipped
// clusters' centroid rows (pre-rounded to the element type) follow as further
// 64-row tiles carrying the log|k_c'| bias. Both kinds of tile run through the
// same online softmax:
//   S^T = K Q^T     (A = K fragments from LDS, B = Q^T held in registers)
//   O^T += V^T P^T  (A = V^T fragments from LDS, B = P^T taken straight from
//                    the S^T accumulators)
// so P never leaves registers.
//
// LDS layout. Tiles are filled by buffer_load_dwordx4 ... lds, which puts
// lane l's 16-byte piece at (LDS pointer + 16 l) while its source is free.
// The copy therefore writes every piece where the matrix operands will read
// it: for bf16, K in MFMA fragment order (one 1 KB fragment per 16 keys x 32
// dims, lane order) and V in the order of the transposing read
// ds_read_b64_tr_b16 (512 contiguous bytes per read), so every LDS read of the
// inner loop is one contiguous, conflict-free block. (f32 tiles, the
// reference-precision path, use plain row-major rows with XOR-swizzled
// 16-byte pieces.) The source rows of the packed keys are tabulated in LDS
// once per block (a window of positions at a time), so a copy lane finds its
// row's source with one LDS read.
//
// Softmax. Exponentials are base 2 with log2(e) folded into the scale. The
// row biases (0 for exact keys, ln|k_c'| for centroid rows, -inf for filler)
// seed the S accumulators, so every logit leaves the matrix core complete.
// The running maximum m of a query is only raised when a logit exceeds it by
// more than kRescaleSlack, so every weight stays below 2^kRescaleSlack; the
// test uses each lane's own maximum (a row exceeds the bound exactly when one
// of its lanes does), and the cross-lane row maximum and the O, l rescale are
// only computed on the rare tiles that raise m.
//
// Per tile the two 32-key halves are skewed so that matrix and vector work
// of different halves sit next to each other:
//   S0 | S1 + exp(S0) | PV0 + exp(S1) | PV1
//
// Pipeline. bf16 tiles cycle through three LDS buffers: while tile t is
// computed, tile t+1 is in flight, and the copies of tile t+2 are issued at
// the end of the step. Each step ends with one wait (this wave's copies of
// tile t+1) and one barrier. f32 tiles are twice as large and use two
// buffers, one tile ahead.
#include <type_traits>

#include "svgear_common.hpp"
#include "svgear_internal.hpp"

namespace svg {

constexpr int kAttBK = 64;              // keys per tile
constexpr float kRescaleSlack = 16.0f;  // weights stay below 2^16 between rescales

template <typename T>
struct AttCfg;
#ifndef SVGEAR_ATT_NW
#define SVGEAR_ATT_NW 8
#endif
template <>
struct AttCfg<__bf16> {
  static constexpr int QB = 2;              // 16-query blocks per wavefront
  static constexpr int NW = SVGEAR_ATT_NW;  // wavefronts per block
  static constexpr int ROWS = 8192;         // packed key positions per source-row window
  static constexpr int STAGES = 3;          // tile buffers (copies run STAGES - 1 tiles ahead)
};
template <>
struct AttCfg<float> {
  static constexpr int QB = 1;
  static constexpr int NW = 4;
  static constexpr int ROWS = 1024;
  static constexpr int STAGES = 2;
};
// The short last blocks of the query clusters (at most 128 queries): four
// wavefronts, two tile buffers and a small source-row window, so that two
// such blocks share a compute unit (a full-size block with few active
// wavefronts holds a whole unit).
struct AttTailCfg {
  static constexpr int QB = 2;
  static constexpr int NW = 4;
  static constexpr int ROWS = 1024;
  static constexpr int STAGES = 2;
};
// Which query tiles a launch covers: every tile of BM queries (kAllTiles);
// the tiles of 256 queries except a last one of at most 128 (kFullTiles);
// only those last ones (kShortTails).
constexpr int kAllTiles = 0, kFullTiles = 1, kShortTails = 2;
constexpr int kTailMax = 128;

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier that leaves the caller's own s_waitcnt in charge: unlike
// __syncthreads it adds no wait for outstanding loads (tile copies still in
// flight). The caller has waited for its LDS accesses (lgkmcnt 0) and for the
// copies the other waves will read; the empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Raw buffer resource over [p, p + bytes), bytes < 2^32 (the host checks a
// head's K or V fits): 32-bit data format, no swizzle.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           int(uint32_t(bytes)), 0x00020000);
}

// 16 bytes at byte offset voff of [base, base + bytes) into LDS at dst (lane l
// at dst + 16 l). (Kept out of the kernel: with the buffer builtin written
// inside the kernel template's body the host pass drops the kernel's stub.)
__device__ __forceinline__ void copy16_lds(const void* base, size_t bytes, uint32_t voff,
                                           lds_void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base, bytes), dst, 16, voff, 0, 0, 0);
}

// Where the 16-byte piece slot j of a K or V tile comes from (key row of the
// tile and 16-byte piece of that row), and how the matrix operands are read.
template <typename T, int D>
struct TileLayout;

// bf16: fragment-ordered K, transposed-read-ordered V.
template <int D>
struct TileLayout<__bf16, D> {
  static constexpr int KC = D / 32;  // 32-dim chunks (K fragments per 16 keys)
  static constexpr int DB = D / 16;  // 16-dim blocks (V^T fragments per 32 keys)
  // fragment f = (16-key block rb, chunk k) occupies slots 64f .. 64f+63 in
  // lane order: lane (r, g) holds K[16 rb + r][32 k + 8 g .. +7]
  __device__ static void k_slot(int j, int& row, int& piece) {
    const int f = j >> 6, l = j & 63;
    row = (f / KC) * 16 + (l & 15);
    piece = (f % KC) * 4 + (l >> 4);
  }
  // transposed read (32-key half h, upper 16 keys u, dim block db) occupies
  // slots 32 i .. 32 i + 31, i = (2 h + u) DB + db; lane group g of the read
  // takes keys 32 h + 16 u + 4 g + e (e = 0..3), 16 dims each, as two pieces.
  // (db varies fastest, so one 64-slot copy instruction reads 16 keys x 64
  // contiguous bytes, as for K, rather than 32 keys x 32 bytes.)
  static_assert(DB % 2 == 0, "a copy instruction covers two dim blocks");
  __device__ static void v_slot(int j, int& row, int& piece) {
    const int i = j >> 5, q = j & 31;
    const int db = i % DB, u = (i / DB) & 1, h = i / (2 * DB);
    row = h * 32 + u * 16 + 4 * (q >> 3) + ((q & 7) >> 1);
    piece = 2 * db + (q & 1);
  }
  // A operand K (16 keys x 32 dims) of block rb, chunk k
  __device__ static Frag<__bf16> k_frag(const __bf16* ks, int rb, int k, int lane) {
    return load8(ks + (rb * KC + k) * 512 + lane * 8);
  }
  // A operand V^T (16 dims x 32 keys) of half h, dim block db; key slot e of
  // lane (r, g) is tile key 32 h + 4 g + (e < 4 ? e : 12 + e)
  __device__ static Frag<__bf16> vt_frag(const __bf16* vs, int h, int db, int lane) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const __bf16* p = vs + (2 * h * DB + db) * 256 + lane * 4;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + DB * 256));
    Frag<__bf16> f;
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
  }
};

// f32: row-major rows whose 16-byte pieces are XOR-swizzled by the row.
template <int D>
struct TileLayout<float, D> {
  static constexpr int CPR = D / 4;  // pieces per row
  __device__ static int swz(int row) { return row & (CPR - 1); }
  __device__ static int index(int row, int col) {
    return row * D + (((col >> 2) ^ swz(row)) << 2) + (col & 3);
  }
  __device__ static void k_slot(int j, int& row, int& piece) {
    row = j / CPR;
    piece = (j % CPR) ^ swz(row);
  }
  __device__ static void v_slot(int j, int& row, int& piece) { k_slot(j, row, piece); }
  __device__ static Frag<float> k_frag(const float* ks, int rb, int k, int lane) {
    const int row = rb * 16 + (lane & 15), col = k * 32 + (lane >> 4) * 8;
    Frag<float> f;
    const float4 a = *reinterpret_cast<const float4*>(ks + index(row, col));
    const float4 b = *reinterpret_cast<const float4*>(ks + index(row, col + 4));
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
  __device__ static Frag<float> vt_frag(const float* vs, int h, int db, int lane) {
    const int r = lane & 15, g = lane >> 4;
    Frag<float> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = vs[index(h * 32 + g * 4 + (e < 4 ? e : 12 + e), db * 16 + r)];
    return f;
  }
};

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

// acc + sum of the eight elements of a fragment (bf16: four v_dot2 with ones).
__device__ __forceinline__ float frag_sum(const Frag<__bf16>& f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {__bf16(1.0f), __bf16(1.0f)};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f.v, f.v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f.v, f.v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f.v, f.v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f.v, f.v, 6, 7), one, acc, false);
  return acc;
}

__device__ __forceinline__ float frag_sum(const Frag<float>& f, float acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc += f.v[e];
  return acc;
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

template <typename T, int D, typename Cfg>
__global__ __launch_bounds__(64 * Cfg::NW, 8 / Cfg::NW) void attend_kernel(
    const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
    const int32_t* __restrict__ qoff, const int32_t* __restrict__ koff,
    const T* __restrict__ kcen, const T* __restrict__ vcen, const uint8_t* __restrict__ mask,
    int H, int Nq, int Nk, int Cq, int Ck, float sl2, int per_head, int span, int mode,
    const int32_t* __restrict__ qperm, T* __restrict__ Op) {
  using L = TileLayout<T, D>;
  constexpr int QB = Cfg::QB;
  constexpr int NW = Cfg::NW;
  constexpr int BM = 16 * NW * QB;
  constexpr int KC = D / 32;
  constexpr int DB = D / 16;
  constexpr int EPT = 16 / sizeof(T);
  constexpr int PIECES = kAttBK * D / EPT;  // 16-byte pieces per tile and tensor
  constexpr int NI = PIECES / (64 * NW);    // copy instructions per wave, tensor and tile
  static_assert(NI * 64 * NW == PIECES, "tile pieces must split evenly over the waves");
  constexpr int TILE = kAttBK * D;          // elements per tile
  // bf16 tiles are triple-buffered (copies run two tiles ahead); f32 tiles
  // are twice as large and double-buffered
  constexpr int kStages = Cfg::STAGES;
  static_assert(kStages == 2 || kStages == 3, "two or three tile buffers");
  constexpr int kAhead = kStages - 1;
  // two buffers per tensor as distinct objects: the compiler can then tell
  // the asynchronous fill of one from the reads of the other and inserts no
  // wait between them
  __shared__ __attribute__((aligned(16))) T ks0[TILE];
  __shared__ __attribute__((aligned(16))) T ks1[TILE];
  __shared__ __attribute__((aligned(16))) T ks2[kStages > 2 ? TILE : 8];
  __shared__ __attribute__((aligned(16))) T vs0[TILE];
  __shared__ __attribute__((aligned(16))) T vs1[TILE];
  __shared__ __attribute__((aligned(16))) T vs2[kStages > 2 ? TILE : 8];
  __shared__ __attribute__((aligned(16))) float bias0[kAttBK];
  __shared__ __attribute__((aligned(16))) float bias1[kAttBK];
  __shared__ __attribute__((aligned(16))) float bias2[kAttBK];
  // per-block lists, sized by Ck at launch (5 * Ck + 1 words):
  extern __shared__ int lists[];
  int* sel_s = lists;                  // selected key cluster ids, ascending
  int* start_s = lists + Ck;           // first key row of a selection minus its packed offset
  int* comp_s = lists + 2 * Ck;        // compensated (skipped, non-empty) key clusters
  float* cbias_s = reinterpret_cast<float*>(lists + 3 * Ck);  // ln |k_c'| / scale of those
  int* pref_s = lists + 4 * Ck;        // packed offset of every selected cluster (+ total)
  // source row of every packed exact key position in [rbase, rbase + ROWS)
  __shared__ int rows_s[Cfg::ROWS];
  __shared__ int scratch[16];
  __shared__ int info[2];

  // Blocks are dealt to the XCDs round-robin (block b runs on XCD b % 8).
  // Renumber so that every XCD walks one contiguous range of (head, tile):
  // the tiles of one query cluster then run side by side on one XCD and read
  // the same key/value rows through its L2.
  const int logical = int(blockIdx.x % kXcds) * span + int(blockIdx.x / kXcds);
  const int h = logical / per_head, t = logical % per_head, tid = threadIdx.x;
  if (h >= H) return;  // padding of the grid to a multiple of the XCD count
  const int w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int32_t* qo = qoff + size_t(h) * (Cq + 1);
  const int32_t* ko = koff + size_t(h) * (Ck + 1);

  // ---- which query cluster / tile this block owns
  // (a cluster of n queries: n / 256 tiles of 256 and a last one of n % 256,
  // split between the kFullTiles and kShortTails launches by its size)
  auto tiles_of = [&](int n) __attribute__((always_inline)) {
    if (mode == kAllTiles) return (n + BM - 1) / BM;
    const int rem = n % 256;
    const bool short_tail = rem > 0 && rem <= kTailMax;
    if (mode == kFullTiles) return n / 256 + ((rem > 0 && !short_tail) ? 1 : 0);
    return short_tail ? 1 : 0;
  };
  int carry = 0;
  for (int b = 0; b < Cq; b += 64 * NW) {
    const int i = b + tid;
    const int nt = (i < Cq) ? tiles_of(qo[i + 1] - qo[i]) : 0;
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
  const int q0 = qo[c] + (mode == kShortTails ? (qo[c + 1] - qo[c]) / 256 * 256 : info[1] * BM);
  const int q1 = min(qo[c + 1], q0 + BM);

  // ---- selected (packed) and compensated key-cluster lists
  const uint8_t* mk = mask + (size_t(h) * Cq + c) * Ck;
  int nsel = 0, nkeys = 0, ncomp = 0;
  for (int b = 0; b < Ck; b += 64 * NW) {
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
      cbias_s[ncomp + e3] = __log2f(float(n)) / sl2;  // raw logit units
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

  // ---- source rows of the packed exact keys, one window of ROWS positions at
  // a time: wave w walks selected clusters w, w + NW, ... and its lanes write
  // consecutive positions (the keys of a selected cluster are consecutive rows
  // of the permuted tensors)
  constexpr int ROWS = Cfg::ROWS;
  static_assert(ROWS % kAttBK == 0, "windows hold whole tiles");
  int rbase = 0;
  auto fill_rows = [&](int base) __attribute__((always_inline)) {
    for (int j = w; j < nsel; j += NW) {
      const int a = max(pref_s[j], base), b = min(pref_s[j + 1], base + ROWS);
      const int st = start_s[j];
      for (int p = a + lane; p < b; p += 64) rows_s[p - base] = st + p;
    }
  };
  fill_rows(0);
  __syncthreads();

  // ---- asynchronous tile loads. The tile row and 16-byte piece behind every
  // copy lane's slot are fixed for the whole loop; per tile a lane only looks
  // up its rows' sources (filler rows read row 0: finite data whose weight is
  // exactly 0). The row biases are kept in raw logit units (divided by the
  // log2 scale) so that they can seed the S accumulators.
  int krow[NI], kpc[NI], vrow[NI], vpc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = (w * NI + i) * 64 + lane;
    L::k_slot(j, krow[i], kpc[i]);
    L::v_slot(j, vrow[i], vpc[i]);
    kpc[i] *= 16;  // byte offset of the piece within its row
    vpc[i] *= 16;
  }
  // The copies address rows through buffer resources of this head's tensors:
  // a 32-bit byte offset per lane (row * row bytes + piece) instead of a
  // 64-bit pointer, and a wave-uniform LDS destination.
  constexpr int RB = D * int(sizeof(T));
  const size_t kv_bytes = size_t(Nk) * RB, cen_bytes = size_t(Ck) * RB;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // sources of this lane's K and V rows of `tile`, its row bias, and the copies
  auto issue = [&](int tile, T* kd, T* vd, float* bd) __attribute__((always_inline)) {
    const bool exact = tile < nt_exact;  // uniform over the block
    int ksrc[NI], vsrc[NI];
    float bias;
    if (exact) {
      const int p0 = tile * kAttBK;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        ksrc[i] = (p0 + krow[i] < nkeys) ? rows_s[p0 - rbase + krow[i]] : 0;
        vsrc[i] = (p0 + vrow[i] < nkeys) ? rows_s[p0 - rbase + vrow[i]] : 0;
      }
      bias = (p0 + lane < nkeys) ? 0.f : -__builtin_inff();
    } else {
      const int p0 = (tile - nt_exact) * kAttBK;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        ksrc[i] = (p0 + krow[i] < ncomp) ? comp_s[p0 + krow[i]] : 0;
        vsrc[i] = (p0 + vrow[i] < ncomp) ? comp_s[p0 + vrow[i]] : 0;
      }
      bias = (p0 + lane < ncomp) ? cbias_s[p0 + lane] : -__builtin_inff();
    }
    if (w == 0) bd[lane] = bias;
    const T* kb = exact ? Kh : KCh;
    const T* vb = exact ? Vh : VCh;
    const size_t nb = exact ? kv_bytes : cen_bytes;
    // all LDS traffic of this call is above: nothing below touches LDS
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      copy16_lds(kb, nb, uint32_t(ksrc[i]) * RB + kpc[i], (lds_void*)(kd + (wu * NI + i) * 64 * EPT));
      copy16_lds(vb, nb, uint32_t(vsrc[i]) * RB + vpc[i], (lds_void*)(vd + (wu * NI + i) * 64 * EPT));
    }
  };

  // s_waitcnt leaving this wave's copies of the newest kAhead - 1 tiles in
  // flight (2 NI each): vmcnt = that count, expcnt untouched (7), lgkmcnt 0
  // (gfx9 field layout: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4]
  // at [15:14])
  constexpr int kInFlight = (kAhead - 1) * 2 * NI;
  static_assert(kInFlight < 64, "vmcnt field");
  auto wait_copies_but_newest = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt((kInFlight & 15) | (7 << 4) | ((kInFlight >> 4) << 14));
  };

  // ---- Q^T fragments
  const T* Qh = Qp + size_t(h) * Nq * D;
  // query group qb of this wave: 16 rows from q0 + 16 (w + NW qb). The
  // wavefronts of a block are dealt to the SIMDs in turn (w and w + NW/2 share
  // one), so spread this way a partial tile's groups load the SIMDs evenly; a
  // wave whose last group lies past the tile runs a loop without it (nq).
  auto qbase = [&](int qb) __attribute__((always_inline)) { return q0 + 16 * (w + NW * qb); };
  const bool active = qbase(0) < q1;
  int nq = 0;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) nq += (qbase(qb) < q1) ? 1 : 0;
  nq = __builtin_amdgcn_readfirstlane(nq);
  Frag<T> qf[QB][KC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qbase(qb) + r;
#pragma unroll
    for (int k = 0; k < KC; ++k)
      qf[qb][k] = (qi < q1) ? load8(Qh + size_t(qi) * D + k * 32 + g * 8) : zero_frag<T>();
  }

  f32x4 o[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float inv_sl2 = 1.f / sl2;
  // running maximum (log2 units), its rescale threshold in raw logit units,
  // and the running denominator of every query of this lane
  // The row sums of the rounded weights: for bf16 one more MFMA per query
  // block with an all-ones A operand puts query r's sum in every entry of
  // column r (no vector adds, no final lane reduction); f32 sums per lane.
  constexpr bool kOnesSum = sizeof(T) == 2;
  Frag<T> ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones.v[e] = T(1.0f);
  f32x4 lacc[QB];
  float mrow[QB], thr[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrow[qb] = -__builtin_inff();
    thr[qb] = -__builtin_inff();
    lsum[qb] = 0.f;
    lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- the pieces of one 32-key half kh (keys 32 kh .. 32 kh + 31 of a tile)
  auto kfrags = [&](Frag<T> (&ka)[2][KC], const T* kb_s, int kh) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int k = 0; k < KC; ++k) ka[kb][k] = L::k_frag(kb_s, kh * 2 + kb, k, lane);
  };
  auto vfrags = [&](Frag<T> (&va)[DB], const T* vb_s, int kh) {
#pragma unroll
    for (int db = 0; db < DB; ++db) va[db] = L::vt_frag(vb_s, kh, db, lane);
  };
  // S^T in raw logit units, accumulators seeded with the rows' biases
  // (NQ: the number of this wave's query blocks, a compile-time constant)
  auto qk = [&](auto NQ, f32x4 (&sh)[2][QB], const Frag<T> (&ka)[2][KC], const float* bb_s,
                int kh) {
    constexpr int nqc = decltype(NQ)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(bb_s + kh * 32 + kb * 16 + g * 4);
#pragma unroll
      for (int qb = 0; qb < nqc; ++qb) sh[kb][qb] = b4;
    }
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < nqc; ++qb) mma(sh[kb][qb], ka[kb][k], qf[qb][k]);
  };
  // raise the running maxima if a logit of the half exceeds its threshold;
  // l is scaled down to the new maximum at once and the factors are returned
  // for O (true if any is not 1), which the caller scales once every weight
  // computed under the old maxima has been added to it
  auto check = [&](auto NQ, const f32x4 (&sh)[2][QB], float (&al)[QB]) -> bool {
    constexpr int nqc = decltype(NQ)::value;
    float mx[QB];
    bool up = false;
#pragma unroll
    for (int qb = 0; qb < nqc; ++qb) {
      float m = sh[0][qb][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) m = fmaxf(m, sh[e >> 2][qb][e & 3]);
      mx[qb] = m;
      up = up || (m > thr[qb]);
    }
    if (__ballot(up) == 0ull) return false;
#pragma unroll
    for (int qb = 0; qb < nqc; ++qb) {
      const float mn = fmaxf(mrow[qb], quad_max(mx[qb]) * sl2);  // the scale is positive
      al[qb] = (mn > mrow[qb]) ? fast_exp2(mrow[qb] - mn) : 1.f;
      mrow[qb] = mn;
      thr[qb] = (mn + kRescaleSlack) * inv_sl2;
      if (kOnesSum) lacc[qb] *= al[qb];
      else lsum[qb] *= al[qb];
    }
    return true;
  };
  auto scale_o = [&](auto NQ, const float (&al)[QB]) {
    constexpr int nqc = decltype(NQ)::value;
#pragma unroll
    for (int qb = 0; qb < nqc; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db][qb] *= al[qb];
  };
  // P^T fragments and their sums (the denominator adds the same rounded
  // weights the numerator uses)
  auto weights = [&](auto NQ, const f32x4 (&sh)[2][QB], Frag<T> (&pb)[QB]) {
    constexpr int nqc = decltype(NQ)::value;
#pragma unroll
    for (int qb = 0; qb < nqc; ++qb) {
      const float nm = -mrow[qb];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[qb].v[e] = from_f32<T>(fast_exp2(fmaf(sh[e >> 2][qb][e & 3], sl2, nm)));
      if (kOnesSum) mma(lacc[qb], ones, pb[qb]);
      else lsum[qb] = frag_sum(pb[qb], lsum[qb]);
    }
  };
  auto pv = [&](auto NQ, const Frag<T> (&va)[DB], const Frag<T> (&pb)[QB]) {
    constexpr int nqc = decltype(NQ)::value;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qb = 0; qb < nqc; ++qb) mma(o[db][qb], va[db], pb[qb]);
  };

  // copies of tile+kAhead into the buffer that tile-1 used. Past the last
  // tile the copies still run (filler rows), so that every step ends with
  // the same wait: all but this wave's newest copies.
  auto copy_ahead = [&](int tile, T* kn_s, T* vn_s, float* bn_s) __attribute__((always_inline)) {
    const int nxt = tile + kAhead;
    if (nxt < nt_exact && nxt * kAttBK == rbase + ROWS) {
      // the tile copied next starts a new window of source rows (every wave
      // is past its reads of the current window: the last barrier)
      rbase += ROWS;
      fill_rows(rbase);
      __syncthreads();
    }
    issue(nxt, kn_s, vn_s, bn_s);
  };
  // one tile. Two tiles ahead (bf16), the copies are issued after this
  // tile's matrix work, so that its first LDS reads start the step; one tile
  // ahead (f32), before it, so that they overlap it.
  auto step = [&](auto NQ, int tile, const T* kb_s, const T* vb_s, const float* bb_s, T* kn_s,
                  T* vn_s, float* bn_s) __attribute__((always_inline)) {
    if (kAhead == 1) copy_ahead(tile, kn_s, vn_s, bn_s);
    if (active && tile >= 0) {
      Frag<T> ka0[2][KC], ka1[2][KC], va0[DB], va1[DB], pb0[QB], pb1[QB];
      f32x4 s0[2][QB], s1[2][QB];
      kfrags(ka0, kb_s, 0);
      kfrags(ka1, kb_s, 1);
      float al0[QB], al1[QB];
      qk(NQ, s0, ka0, bb_s, 0);
      if (check(NQ, s0, al0)) scale_o(NQ, al0);
      vfrags(va0, vb_s, 0);
      qk(NQ, s1, ka1, bb_s, 1);
      weights(NQ, s0, pb0);
      const bool up1 = check(NQ, s1, al1);
      vfrags(va1, vb_s, 1);
      pv(NQ, va0, pb0);             // weights of the old maxima first,
      weights(NQ, s1, pb1);
      if (up1) scale_o(NQ, al1);    // then O follows l to the new maxima
      pv(NQ, va1, pb1);
    }
    if (kAhead > 1) copy_ahead(tile, kn_s, vn_s, bn_s);
    wait_copies_but_newest();
    lds_barrier();
  };

  // The loop starts kAhead tiles early: those steps only issue copies, so
  // every copy comes from the issue sites inside the loop, whose LDS
  // destinations the compiler tells apart (it then inserts no wait between
  // the copies into one buffer and the reads of another). The guards are
  // nested so that no path reaches a step without the one before it.
  // one copy of the loop per query-block count, so that a wave without its
  // last block runs no matrix or vector work for it
  auto run = [&](auto NQ) __attribute__((always_inline)) {
    if constexpr (kStages == 3) {
      for (int tile = -2; tile < nt_all; tile += 3) {
        step(NQ, tile, ks1, vs1, bias1, ks0, vs0, bias0);
        if (tile + 1 < nt_all) {
          step(NQ, tile + 1, ks2, vs2, bias2, ks1, vs1, bias1);
          if (tile + 2 < nt_all) step(NQ, tile + 2, ks0, vs0, bias0, ks2, vs2, bias2);
        }
      }
    } else {
      for (int tile = -1; tile < nt_all; tile += 2) {
        step(NQ, tile, ks1, vs1, bias1, ks0, vs0, bias0);
        if (tile + 1 < nt_all) step(NQ, tile + 1, ks0, vs0, bias0, ks1, vs1, bias1);
      }
    }
  };
  if constexpr (QB > 1) {
    if (nq < QB) run(std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, QB>{});
  } else {
    run(std::integral_constant<int, 1>{});
  }
  // the filler copies of the last steps land before the block's LDS is freed
  __builtin_amdgcn_s_waitcnt(0);

  if (!active) return;
  T* Oh = Op + size_t(h) * Nq * D;
  // with a query permutation, row qi of the permuted order is written to the
  // query's original row (rows outside [0, Nq) are dropped)
  const int32_t* ph = qperm ? qperm + size_t(h) * Nq : nullptr;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (qb >= nq) break;
    const float inv = 1.f / (kOnesSum ? lacc[qb][0] : quad_sum(lsum[qb]));
    const int qp = qbase(qb) + r;
    const int qi = (ph && qp < q1) ? ph[qp] : qp;
    if (qp < q1 && unsigned(qi) < unsigned(Nq)) {
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

template <typename T, int D, typename Cfg>
static void attend_launch(int mode, int per_head, int H, int Nq, int Nk, int Cq, int Ck, float sl2,
                          const void* Qp, const void* Kp, const void* Vp, const int32_t* qoff,
                          const int32_t* koff, const void* kc, const void* vc,
                          const uint8_t* mask, const int32_t* qperm, void* Op, hipStream_t s) {
  const int span = ceil_div(H * per_head, kXcds);
  const size_t lds_lists = sizeof(int) * (5 * size_t(Ck) + 1);
  hipLaunchKernelGGL((attend_kernel<T, D, Cfg>), dim3(span * kXcds), dim3(64 * Cfg::NW), lds_lists,
                     s, static_cast<const T*>(Qp), static_cast<const T*>(Kp),
                     static_cast<const T*>(Vp), qoff, koff, static_cast<const T*>(kc),
                     static_cast<const T*>(vc), mask, H, Nq, Nk, Cq, Ck, sl2, per_head, span,
                     mode, qperm, static_cast<T*>(Op));
}

template <typename T, int D>
static void attend_t(int H, int Nq, int Nk, int Cq, int Ck, float sl2, const void* Qp,
                     const void* Kp, const void* Vp, const int32_t* qoff, const int32_t* koff,
                     const void* kc, const void* vc, const uint8_t* mask,
                     const int32_t* qperm, void* Op, hipStream_t s) {
  using C = AttCfg<T>;
  constexpr int BM = 16 * C::NW * C::QB;
  if constexpr (sizeof(T) == 2 && BM == 256) {
    // blocks of 256 queries, then the short last blocks two to a compute unit
    attend_launch<T, D, C>(kFullTiles, ceil_div(Nq, BM) + Cq, H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp,
                           qoff, koff, kc, vc, mask, qperm, Op, s);
    attend_launch<T, D, AttTailCfg>(kShortTails, Cq, H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff,
                                    koff, kc, vc, mask, qperm, Op, s);
  } else {
    attend_launch<T, D, C>(kAllTiles, ceil_div(Nq, BM) + Cq, H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp,
                           qoff, koff, kc, vc, mask, qperm, Op, s);
  }
}

hipError_t launch_attend(int elem_bytes, int H, int Nq, int Nk, int d, int Cq, int Ck,
                         float scale, const void* Qp, const void* Kp, const void* Vp,
                         const int32_t* qoff, const int32_t* koff, const float* kc,
                         const float* vc, const uint8_t* mask, const int32_t* qperm, void* Op,
                         void* ws, hipStream_t s) {
  const float sl2 = scale * 1.44269504088896340736f;
  if (elem_bytes == 2) {
    const size_t n = size_t(H) * Ck * d;
    __bf16* rk = static_cast<__bf16*>(ws);
    __bf16* rv = reinterpret_cast<__bf16*>(static_cast<char*>(ws) + align256(2 * n));
    hipLaunchKernelGGL(round_rows_kernel<__bf16>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s,
                       n, kc, vc, rk, rv);
    if (d == 128) attend_t<__bf16, 128>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, rk, rv, mask, qperm, Op, s);
    else attend_t<__bf16, 64>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, rk, rv, mask, qperm, Op, s);
  } else {
    if (d == 128) attend_t<float, 128>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, kc, vc, mask, qperm, Op, s);
    else attend_t<float, 64>(H, Nq, Nk, Cq, Ck, sl2, Qp, Kp, Vp, qoff, koff, kc, vc, mask, qperm, Op, s);
  }
  return hipGetLastError();
}

}  // namespace svg
