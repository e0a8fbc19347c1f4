// Shared device-side definitions of the Spatial-Transformer block kernels
// (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stb {

typedef uint16_t bf16_t;   // bfloat16 storage (upper half of an fp32)
typedef _Float16 f16_t;    // IEEE half storage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kHeadDim = 64;
constexpr int kCtxLen = 77;
constexpr int kGroups = 32;

__device__ __forceinline__ float bf2f(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f2bf(float v) {
  __bf16 b = static_cast<__bf16>(v);
  return __builtin_bit_cast(bf16_t, b);
}

__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  bf16x2 r;
  r[0] = static_cast<__bf16>(lo);
  r[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
  f16x2 r;
  r[0] = static_cast<_Float16>(lo);
  r[1] = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

// Two 16-bit values of type T packed in one dword, rounded to nearest even.
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) { return pack2bf(lo, hi); }
template <> __device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi) { return pack2h(lo, hi); }

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf2f(v); }
template <> __device__ __forceinline__ float to_f32<f16_t>(f16_t v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float v) { return static_cast<f16_t>(v); }

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Wavefront sum without LDS: DPP within each row of 16 lanes (swap
// neighbours, swap pairs, half-row mirror, row mirror: every lane then holds
// its row's sum), then row_bcast15 / row_bcast31 carry the row sums up to
// lane 63, whose value is broadcast.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_f32<0x140, 0xF>(v);  // row_mirror
  v += dpp_f32<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  v += dpp_f32<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// GELU in its exact form: g * Phi(g) = g/2 * (1 + erf(g / sqrt 2)).
__device__ __forceinline__ float gelu_erf(float g) {
  return 0.5f * g * (1.0f + erff(g * 0.70710678118654752f));
}

// The same GELU with erf from Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: erf(x) = 1 - P(t) exp(-x^2), P(t) = t (a1 + t
// (a2 + t (a3 + t (a4 + t a5)))), t = 1 / (1 + p x), x >= 0, |error| <=
// 1.5e-7; erf is odd.  With x = |g| / sqrt 2, g erf(g / sqrt 2) = |g| (1 - P
// exp(-g^2 / 2)), so GELU(g) = max(g, 0) - |g| / 2 * P * exp(-g^2 / 2).
// Used where the result is rounded to a 16-bit type, whose rounding (>=
// 2^-12 relative) is far larger than that error.
__device__ __forceinline__ float gelu_as(float g) {
  const float a = fabsf(g);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.2316418882663604f, a, 1.0f));  // p / sqrt 2
  float poly = fmaf(t, 1.061405429f, -1.453152027f);
  poly = fmaf(t, poly, 1.421413741f);
  poly = fmaf(t, poly, -0.284496736f);
  poly = fmaf(t, poly, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(g * g * -0.7213475204444817f);  // exp(-g^2 / 2)
  return fmaf(-0.5f * a, poly * t * e, fmaxf(g, 0.0f));
}

// 32x32x16 MFMA with fp32 accumulation, bf16 or fp16 operands (8 per lane).
__device__ __forceinline__ floatx16 mfma32x32x16(const uint4& a, const uint4& b,
                                                 floatx16 c, bf16_t) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma32x32x16(const uint4& a, const uint4& b,
                                                 floatx16 c, f16_t) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// True when one of the fp16 values packed in the dwords is infinite or NaN
// (exponent field all ones).
__device__ __forceinline__ bool f16_pair_nonfinite(uint32_t d) {
  return ((d & 0x7c00u) == 0x7c00u) | ((d & 0x7c000000u) == 0x7c000000u);
}
__device__ __forceinline__ bool f16x8_nonfinite(const uint4& w) {
  // the four tests OR-ed without branches
  const int any = static_cast<int>(f16_pair_nonfinite(w.x)) | static_cast<int>(f16_pair_nonfinite(w.y)) |
                  static_cast<int>(f16_pair_nonfinite(w.z)) | static_cast<int>(f16_pair_nonfinite(w.w));
  return any != 0;
}

// s_waitcnt that waits for vmcnt <= n and for every LDS access of this
// wavefront (lgkmcnt 0), expcnt left at its maximum.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without the release fence of __syncthreads(), which
// would wait for every outstanding global load -- including the LDS DMA of
// later pipeline stages.  Callers wait for exactly what they need first
// (wait_vmcnt_lds).  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace stb
