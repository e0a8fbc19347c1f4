// Measurement helper: the sustained rate of the bf16 matrix pipes on this
// device, and the shader clock observed while they run.
//
// Every wavefront keeps four independent v_mfma_f32_32x32x16_bf16
// accumulator chains busy for `iters` rounds (no memory traffic inside the
// loop), so the matrix pipe of each SIMD never waits on a dependency; the
// grid holds two wavefronts per SIMD on every CU.  Wavefront 0 of each
// workgroup reads the shader-cycle counter (s_memtime) and the constant-rate
// real-time counter (s_memrealtime) around its loop; their ratio gives the
// shader clock the loop ran at.
#include "common.h"
#include "kernels.h"

namespace stb {

namespace {

constexpr int kChains = 4;

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ out,
                                                        long long* __restrict__ clocks) {
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  // small operands (2^-10 and neighbours): the sums stay far from overflow
  const uint32_t v = 0x3a803a80u + (threadIdx.x & 7);
  const uint4 a = make_uint4(v, v, v, v);
  const uint4 b = make_uint4(v ^ 1u, v, v, v ^ 1u);
  const long long c0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = mfma32x32x16(a, b, acc[c], bf16_t{});
  }
  const long long c1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[static_cast<long long>(blockIdx.x) * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

int mfma_probe_grid(int cus) { return 2 * cus; }

long long mfma_probe_flops(int grid, int iters) {
  // 4 wavefronts per workgroup, kChains MFMAs of 32*32*16 multiply-adds
  return static_cast<long long>(grid) * 4 * iters * kChains * 2LL * 32 * 32 * 16;
}

hipError_t mfma_probe(int grid, int iters, float* out, long long* clocks, hipStream_t s) {
  mfma_loop_kernel<<<grid, 256, 0, s>>>(iters, out, clocks);
  return hipGetLastError();
}

}  // namespace stb
