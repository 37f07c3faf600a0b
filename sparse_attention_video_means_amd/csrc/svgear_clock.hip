// Shader clock under matrix-core load, for a fraction of peak that follows
// the clock the chip actually holds (it runs below the nominal 2.4 GHz while
// the matrix cores are busy).
//
// Every wavefront runs eight independent chains of bf16 16x16x32 MFMAs on
// register operands. The first wavefront of block 0 reads the shader clock
// counter and the constant-rate real-time counter before and after its
// chains; with enough resident blocks the whole chip is busy meanwhile, so
// the ratio of the two deltas is the clock under that load.
#include "svgear_common.hpp"
#include "svgear_internal.hpp"

namespace svg {

__global__ __launch_bounds__(256) void clock_probe_kernel(int iters, uint64_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  Frag<__bf16> a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a.v[e] = __bf16(float((lane + e) & 7) * 0.125f);
    b.v[e] = __bf16(float((3 * lane + e) & 7) * 0.125f);
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool lead = blockIdx.x == 0 && threadIdx.x == 0;
  uint64_t c0 = 0, r0 = 0;
  if (lead) {
    c0 = uint64_t(clock64());
    r0 = uint64_t(wall_clock64());
  }
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) mma(acc[j], a, b);
  if (lead) {
    const uint64_t c1 = uint64_t(clock64()), r1 = uint64_t(wall_clock64());
    out[0] = c0;
    out[1] = c1;
    out[2] = r0;
    out[3] = r1;
  }
  // one checksum per block keeps the products from being dropped
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  if (threadIdx.x == 0) out[4 + blockIdx.x] = uint64_t(__float_as_uint(s));
}

hipError_t launch_clock_probe(int blocks, int iters, uint64_t* out, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace svg
