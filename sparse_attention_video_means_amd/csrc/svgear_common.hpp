// Device-side building blocks shared by the svgear kernels (gfx950 / CDNA4).
//
// Matrix-core convention used throughout: one 64-lane wavefront computes a
// 16x16 f32 tile D += A(16 x 32) * B(32 x 16). Lane l (r = l % 16, g = l / 16)
// supplies A[r][8g .. 8g+7] and B[8g .. 8g+7][r] and receives D[4g .. 4g+3][r].
// For bf16 operands that is one v_mfma_f32_16x16x32_bf16; for f32 operands the
// same per-lane data feeds eight v_mfma_f32_16x16x4_f32 steps, step e
// contracting k = {e, 8+e, 16+e, 24+e}, so every kernel is written once for
// both element types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

template <typename T>
struct Frag;

template <>
struct Frag<__bf16> {
  bf16x8 v;
};

template <>
struct Frag<float> {
  float v[8];
};

__device__ __forceinline__ void mma(f32x4& acc, const Frag<__bf16>& a, const Frag<__bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Eight consecutive elements starting at p (16-byte aligned for bf16, 32 for f32).
__device__ __forceinline__ Frag<__bf16> load8(const __bf16* p) {
  Frag<__bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}

__device__ __forceinline__ Frag<float> load8(const float* p) {
  Frag<float> f;
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}

template <typename T>
__device__ __forceinline__ Frag<T> zero_frag() {
  Frag<T> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = T(0.0f);
  return f;
}

// Element conversions (round to nearest even for bf16).
template <typename T>
__device__ __forceinline__ T from_f32(float x) { return T(x); }

__device__ __forceinline__ float to_f32(__bf16 x) { return float(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Copy of 16 bytes.
__device__ __forceinline__ void copy16(void* dst, const void* src) {
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-wide inclusive scan of an int (lane order).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Block-wide exclusive scan of one int per thread; `scratch` holds >= blockDim/64 ints.
// Returns the exclusive prefix; *total receives the block sum. Contains barriers.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < nw; ++i) {
    const int s = scratch[i];
    before += (i < w) ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Number of bits needed to tell C labels apart.
__device__ __forceinline__ int label_bits(int C) { return C <= 1 ? 0 : 32 - __clz(C - 1); }

// Stable rank of every thread's label among the equal labels of lower thread
// index in the block, and the block's label histogram. Thread order is the
// row order of the tile. `wave_hist` holds 4*C ints of LDS (blockDim = 256).
// Invalid threads (valid = false) take no part. Contains barriers.
__device__ __forceinline__ int tile_rank(int label, bool valid, int C, int* wave_hist) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 4 * C; i += 256) wave_hist[i] = 0;
  __syncthreads();
  uint64_t peers = __ballot(valid);
  const int nb = label_bits(C);
  for (int b = 0; b < nb; ++b) {
    const bool bit = (label >> b) & 1;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank_w = __popcll(peers & below);
  if (valid && rank_w == 0) wave_hist[w * C + label] = __popcll(peers);
  __syncthreads();
  int r = rank_w;
  if (valid)
    for (int i = 0; i < w; ++i) r += wave_hist[i * C + label];
  return r;
}

}  // namespace svg
