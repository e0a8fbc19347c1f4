// GroupNorm, LayerNorm and small helper kernels of the Spatial-Transformer
// block (gfx950).  All of these are HBM-bound: each reads and writes every
// element once with coalesced 16-byte accesses where the layout allows.
#include "common.h"
#include "kernels.h"

namespace stb {

// ---------------------------------------------------------------- GroupNorm
// x is NCHW, so one (sample, group) is a contiguous run of (C/32)*N elements.
// Stage 1: `split` workgroups per group each reduce a slice to the sum and
// sum of squares of (x - shift), shift = the group's first element (shifted
// sums keep the variance free of cancellation for data with a large mean).
// Stage 2 (in the apply kernel): the partials are added in fp64 into
// (mean, 1/sqrt(var + 1e-6)), population variance.

constexpr int kGnThreads = 256;
constexpr int kGnSliceMin = 4096;  // elements per workgroup at least

template <typename T>
__device__ __forceinline__ void load8(const T* p, float v[8]);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float v[8]) {
  uint4 r = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float v[8]) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(kGnThreads) void gn_partial_kernel(
    const T* __restrict__ x, long long group_elems, int split,
    float2* __restrict__ partial) {
  const int g = blockIdx.x;  // b*32 + group
  const int s = blockIdx.y;
  // absolute element indices into x (x itself is 16-byte aligned), so the
  // 8-wide vector body stays aligned whatever the group size is
  const long long gbase = static_cast<long long>(g) * group_elems;
  const float shift = to_f32<T>(x[gbase]);
  const long long slice = (group_elems + split - 1) / split;
  const long long lo = gbase + min(group_elems, s * slice);
  const long long hi = gbase + min(group_elems, (s + 1) * slice);
  float s1 = 0.f, s2 = 0.f;
  long long vlo = (lo + 7) & ~7LL;
  long long vhi = hi & ~7LL;
  if (vlo > hi) vlo = hi;
  if (vhi < vlo) vhi = vlo;
  for (long long i = lo + threadIdx.x; i < vlo; i += kGnThreads) {
    float d = to_f32<T>(x[i]) - shift;
    s1 += d; s2 += d * d;
  }
  // two vectors per thread and step, both loads issued before either is
  // summed (the same order of additions as one vector per step)
  constexpr long long kStep = 8LL * kGnThreads;
  for (long long i = vlo + 8LL * threadIdx.x; i < vhi; i += 2 * kStep) {
    float v[8], w[8];
    const bool two = i + kStep < vhi;
    load8<T>(x + i, v);
    if (two) load8<T>(x + i + kStep, w);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float d = v[j] - shift;
      s1 += d; s2 += d * d;
    }
    if (two) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float d = w[j] - shift;
        s1 += d; s2 += d * d;
      }
    }
  }
  for (long long i = vhi + threadIdx.x; i < hi; i += kGnThreads) {
    float d = to_f32<T>(x[i]) - shift;
    s1 += d; s2 += d * d;
  }
  s1 = warp_sum(s1);
  s2 = warp_sum(s2);
  __shared__ float red[2][kGnThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][w] = s1; red[1][w] = s2; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 0.f, b = 0.f;
    for (int i = 0; i < kGnThreads / 64; ++i) { a += red[0][i]; b += red[1][i]; }
    partial[g * split + s] = make_float2(a, b);
  }
}

int gn_split(int C, int N, int max_split) {
  long long elems = static_cast<long long>(C / kGroups) * N;
  long long s = (elems + kGnSliceMin - 1) / kGnSliceMin;
  if (s < 1) s = 1;
  if (s > max_split) s = max_split;
  return static_cast<int>(s);
}

hipError_t gn_stats(const void* x, bool bf16, int B, int C, int N,
                    float2* partial, int max_split, hipStream_t s) {
  const long long group_elems = static_cast<long long>(C / kGroups) * N;
  const int split = gn_split(C, N, max_split);
  dim3 grid(B * kGroups, split);
  if (bf16)
    gn_partial_kernel<bf16_t><<<grid, kGnThreads, 0, s>>>(
        static_cast<const bf16_t*>(x), group_elems, split, partial);
  else
    gn_partial_kernel<float><<<grid, kGnThreads, 0, s>>>(
        static_cast<const float*>(x), group_elems, split, partial);
  return hipGetLastError();
}

// Eight values stored; returns true when a stored value is not finite
// (fp16 only: fp32 keeps the range of its inputs).
template <typename T>
__device__ __forceinline__ bool store8(T* p, const float v[8]);
template <>
__device__ __forceinline__ bool store8<f16_t>(f16_t* p, const float v[8]) {
  const uint4 w = make_uint4(pack2h(v[0], v[1]), pack2h(v[2], v[3]), pack2h(v[4], v[5]),
                             pack2h(v[6], v[7]));
  *reinterpret_cast<uint4*>(p) = w;
  return f16x8_nonfinite(w);
}
template <>
__device__ __forceinline__ bool store8<float>(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  return false;
}

// Apply GroupNorm and transpose NCHW -> tokens [B*N][C] through LDS.  A
// workgroup owns 64 channels x 64 tokens of one sample.  Its 64 threads
// first turn the group partial sums into per-channel (scale, offset) =
// (rstd * gamma, beta - mean * rstd * gamma), combining the slices in fp64
// (mean = shift + E[x - shift], population variance); then every thread
// reads 8 consecutive tokens of one channel (16 bytes of bf16) and writes 8
// consecutive channels of one token.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void gn_apply_tokens_kernel(
    const TI* __restrict__ x, const float2* __restrict__ partial, int split,
    const float* __restrict__ gamma, const float* __restrict__ beta,
    TO* __restrict__ out, int C, int N, int* __restrict__ range_flag) {
  __shared__ float2 coef[64];
  __shared__ float tile[64][64 + 4];  // [channel][token]
  const int n0 = blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int b = blockIdx.z;
  const int cg = C / kGroups;
  const int tid = threadIdx.x;
  // The tile's loads go out first: they do not depend on the coefficients,
  // whose chain of dependent loads and fp64 sums then runs in their shadow.
  const bool vec_n = (N & 7) == 0;
  float v[2][8];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cl = pass * 32 + (tid >> 3);
    const int n = n0 + 8 * (tid & 7);
    const TI* src = x + (static_cast<long long>(b) * C + c0 + cl) * N + n;
    if (vec_n && n + 7 < N) {
      load8<TI>(src, v[pass]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[pass][j] = n + j < N ? to_f32<TI>(src[j]) : 0.f;
    }
  }
  if (tid < 64) {
    const int c = c0 + tid;
    const int g = b * kGroups + c / cg;
    const double shift = to_f32<TI>(x[static_cast<long long>(g) * cg * N]);
    double s1 = 0.0, s2 = 0.0;
#pragma unroll 4
    for (int i = 0; i < split; ++i) {
      const float2 pr = partial[g * split + i];
      s1 += pr.x;
      s2 += pr.y;
    }
    const double n = static_cast<double>(cg) * N;
    const double dm = s1 / n;
    double var = s2 / n - dm * dm;
    if (var < 0.0) var = 0.0;
    const float rstd = static_cast<float>(1.0 / sqrt(var + 1e-6));
    const float scale = rstd * gamma[c];
    coef[tid] = make_float2(scale, beta[c] - static_cast<float>(shift + dm) * scale);
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cl = pass * 32 + (tid >> 3);
    const int nl = 8 * (tid & 7);
    const float2 k = coef[cl];
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[cl][nl + j] = v[pass][j] * k.x + k.y;
  }
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int nl = pass * 32 + (tid >> 3);
    const int cl = 8 * (tid & 7);
    const int n = n0 + nl;
    if (n >= N) continue;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = tile[cl + j][nl];
    bad |= store8<TO>(out + (static_cast<long long>(b) * N + n) * C + c0 + cl, v);
  }
  if (bad && range_flag) *range_flag = 1;
}

hipError_t gn_apply_tokens(const void* x, bool bf16, const float2* partial,
                           int max_split, const float* gamma, const float* beta,
                           void* out, int out_type, int B, int C, int N,
                           int* range_flag, hipStream_t s) {
  const int split = gn_split(C, N, max_split);
  dim3 grid((N + 63) / 64, C / 64, B);
  if (bf16 && out_type == ACT_F16)
    gn_apply_tokens_kernel<bf16_t, f16_t><<<grid, 256, 0, s>>>(
        static_cast<const bf16_t*>(x), partial, split, gamma, beta,
        static_cast<f16_t*>(out), C, N, range_flag);
  else if (!bf16 && out_type == ACT_F32)
    gn_apply_tokens_kernel<float, float><<<grid, 256, 0, s>>>(
        static_cast<const float*>(x), partial, split, gamma, beta,
        static_cast<float*>(out), C, N, nullptr);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// GroupNorm apply on NCHW -> NCHW (the standalone GroupNorm op), optionally
// followed by SiLU.  A workgroup takes 2048 elements of one (sample,
// channel) plane: wavefront 0 first combines the group's partial sums in
// fp64 into the channel's (scale, offset), then every thread moves eight
// consecutive elements (16-byte accesses when the plane allows).
template <typename T>
__global__ __launch_bounds__(256) void gn_apply_nchw_kernel(
    const T* __restrict__ x, const float2* __restrict__ partial, int split,
    const T* __restrict__ gamma, const T* __restrict__ beta, T* __restrict__ y, int C, int N,
    float eps, int silu) {
  __shared__ float2 coef;
  const int c = blockIdx.y, b = blockIdx.z;
  const int cg = C / kGroups;
  const int g = b * kGroups + c / cg;
  if (threadIdx.x < 64) {
    double s1 = 0.0, s2 = 0.0;
    for (int i = threadIdx.x; i < split; i += 64) {
      const float2 pr = partial[g * split + i];
      s1 += pr.x;
      s2 += pr.y;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      s1 += __shfl_xor(s1, o, 64);
      s2 += __shfl_xor(s2, o, 64);
    }
    if (threadIdx.x == 0) {
      const double n = static_cast<double>(cg) * N;
      const double shift = to_f32<T>(x[static_cast<long long>(g) * cg * N]);
      const double dm = s1 / n;
      double var = s2 / n - dm * dm;
      if (var < 0.0) var = 0.0;
      const float rstd = static_cast<float>(1.0 / sqrt(var + static_cast<double>(eps)));
      const float gm = gamma ? to_f32<T>(gamma[c]) : 1.f;
      const float bt = beta ? to_f32<T>(beta[c]) : 0.f;
      const float scale = rstd * gm;
      coef = make_float2(scale, bt - static_cast<float>(shift + dm) * scale);
    }
  }
  __syncthreads();
  const float2 k = coef;
  const long long plane = (static_cast<long long>(b) * C + c) * N;
  const int n = blockIdx.x * 2048 + threadIdx.x * 8;
  if (n >= N) return;
  const T* src = x + plane + n;
  T* dst = y + plane + n;
  float v[8];
  const bool vec = (N & 7) == 0;
  if (vec) {
    load8<T>(src, v);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = n + j < N ? to_f32<T>(src[j]) : 0.f;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float a = fmaf(v[j], k.x, k.y);
    if (silu) a = a / (1.0f + __expf(-a));
    v[j] = a;
  }
  if (vec) {
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]),
                                                  pack2bf(v[4], v[5]), pack2bf(v[6], v[7]));
    } else {
      reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
      reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (n + j < N) dst[j] = from_f32<T>(v[j]);
  }
}

hipError_t gn_apply_nchw(const void* x, bool bf16, const float2* partial, int max_split,
                         const void* gamma, const void* beta, void* y, int B, int C, int N,
                         float eps, bool silu, hipStream_t s) {
  const int split = gn_split(C, N, max_split);
  dim3 grid((N + 2047) / 2048, C, B);
  if (bf16)
    gn_apply_nchw_kernel<bf16_t><<<grid, 256, 0, s>>>(
        static_cast<const bf16_t*>(x), partial, split, static_cast<const bf16_t*>(gamma),
        static_cast<const bf16_t*>(beta), static_cast<bf16_t*>(y), C, N, eps, silu ? 1 : 0);
  else
    gn_apply_nchw_kernel<float><<<grid, 256, 0, s>>>(
        static_cast<const float*>(x), partial, split, static_cast<const float*>(gamma),
        static_cast<const float*>(beta), static_cast<float*>(y), C, N, eps, silu ? 1 : 0);
  return hipGetLastError();
}

// ------------------------------------------- convolution operand (NHWC)
// The halo of a zero-haloed NHWC operand over an Hg x Wg grid: the pixels a
// 3x3 convolution of stride 1 or 2 reads outside the image, i.e. padded
// rows 0 and Hg + 1 (columns 0 .. Wg + 1) and padded columns 0 and Wg + 1
// of rows 1 .. Hg: 2 (Wg + 2) + 2 Hg pixels per sample.  Columns past Wg + 1
// (the rounding of Wp) and the rows after the last sample are read only for
// the padding outputs the GEMM epilogue drops.  Halo pixel k of sample b:
__device__ __forceinline__ long long halo_row(int b, int k, int Hg, int Wg, int Wp) {
  int ip, jp;
  if (k < Wg + 2) {
    ip = 0; jp = k;
  } else if (k < 2 * (Wg + 2)) {
    ip = Hg + 1; jp = k - (Wg + 2);
  } else {
    const int q = k - 2 * (Wg + 2);
    ip = 1 + (q >> 1);
    jp = (q & 1) ? Wg + 1 : 0;
  }
  return (static_cast<long long>(b) * (Hg + 2) + ip) * Wp + jp;
}
__host__ __device__ inline int halo_pixels(int Hg, int Wg) { return 2 * (Wg + 2) + 2 * Hg; }
// Workgroups past the image's pixel tiles write the halo's zeros: 32 halo
// pixels x 64 channels each, 16 bytes per thread.
constexpr int kHaloPerGroup = 32;

// GroupNorm apply + SiLU from NCHW into the zero-haloed NHWC operand of a
// 3x3 convolution: input pixel (i, j) of sample b goes to row (b * (H + 2) +
// i + 1) * Wp + j + 1 of `out` (L fp16 elements per row, channels from 0),
// and the workgroups after the pixel tiles write the halo's zeros for the
// same channels, so that the buffer needs no clearing beforehand.
// Optionally the raw input also goes to `raw` (same rows, row length L_raw,
// channels from raw_cbase): the operand of a fused 1x1 shortcut.  A
// workgroup owns 64 channels x 64 pixels of one sample, transposed through
// LDS: 16-byte loads along pixels, 16-byte stores along channels.
template <typename TI>
__global__ __launch_bounds__(256) void gn_apply_pad_kernel(
    const TI* __restrict__ x, const float2* __restrict__ partial, int split,
    const float* __restrict__ gamma, const float* __restrict__ beta, f16_t* __restrict__ out,
    int C, int H, int W, int Wp, int L, float eps, f16_t* __restrict__ raw, int L_raw,
    int raw_cbase, int* __restrict__ range_flag) {
  __shared__ float2 coef[64];
  __shared__ float tile[64][64 + 4];  // [channel][pixel], normalised
  __shared__ float rtile[64][64 + 4];  // raw values (only with `raw`)
  const int N = H * W;
  const int n0 = blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int b = blockIdx.z;
  const int cg = C / kGroups;
  const int tid = threadIdx.x;
  const int ntiles = (N + 63) / 64;
  if (static_cast<int>(blockIdx.x) >= ntiles) {  // halo zeros (no barrier below)
    const int k = (blockIdx.x - ntiles) * kHaloPerGroup + (tid >> 3);
    if (k >= halo_pixels(H, W)) return;
    const long long row = halo_row(b, k, H, W, Wp);
    const int cl = 8 * (tid & 7);
    *reinterpret_cast<uint4*>(out + row * L + c0 + cl) = make_uint4(0u, 0u, 0u, 0u);
    if (raw) *reinterpret_cast<uint4*>(raw + row * L_raw + raw_cbase + c0 + cl) = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  if (tid < 64) {
    const int c = c0 + tid;
    const int g = b * kGroups + c / cg;
    double s1 = 0.0, s2 = 0.0;
    for (int i = 0; i < split; ++i) {
      const float2 pr = partial[g * split + i];
      s1 += pr.x;
      s2 += pr.y;
    }
    const double n = static_cast<double>(cg) * N;
    const double shift = to_f32<TI>(x[static_cast<long long>(g) * cg * N]);
    const double dm = s1 / n;
    double var = s2 / n - dm * dm;
    if (var < 0.0) var = 0.0;
    const float rstd = static_cast<float>(1.0 / sqrt(var + static_cast<double>(eps)));
    const float scale = rstd * gamma[c];
    coef[tid] = make_float2(scale, beta[c] - static_cast<float>(shift + dm) * scale);
  }
  __syncthreads();
  const bool vec_n = (N & 7) == 0;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cl = pass * 32 + (tid >> 3);
    const int nl = 8 * (tid & 7);
    const int n = n0 + nl;
    const float2 k = coef[cl];
    const TI* src = x + (static_cast<long long>(b) * C + c0 + cl) * N + n;
    float v[8];
    if (vec_n && n + 7 < N) {
      load8<TI>(src, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = n + j < N ? to_f32<TI>(src[j]) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = fmaf(v[j], k.x, k.y);
      tile[cl][nl + j] = a / (1.0f + __expf(-a));
      if (raw) rtile[cl][nl + j] = v[j];
    }
  }
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int nl = pass * 32 + (tid >> 3);
    const int cl = 8 * (tid & 7);
    const int n = n0 + nl;
    if (n >= N) continue;
    const int i = n / W, j = n - (n / W) * W;
    const long long row = (static_cast<long long>(b) * (H + 2) + i + 1) * Wp + j + 1;
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = tile[cl + q][nl];
    bad |= store8<f16_t>(out + row * L + c0 + cl, v);
    if (raw) {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = rtile[cl + q][nl];
      bad |= store8<f16_t>(raw + row * L_raw + raw_cbase + c0 + cl, v);
    }
  }
  if (bad && range_flag) *range_flag = 1;
}

hipError_t gn_apply_pad(const void* x, const float2* partial, int max_split, const float* gamma,
                        const float* beta, void* out, int B, int C, int H, int W, int Wp, int L,
                        float eps, void* raw, int L_raw, int raw_cbase, int* range_flag,
                        hipStream_t s) {
  if (C % 64 || L % 8 || L_raw % 8 || raw_cbase % 8) return hipErrorInvalidValue;
  const int N = H * W;
  const int split = gn_split(C, N, max_split);
  dim3 grid((N + 63) / 64 + (halo_pixels(H, W) + kHaloPerGroup - 1) / kHaloPerGroup, C / 64, B);
  gn_apply_pad_kernel<bf16_t><<<grid, 256, 0, s>>>(
      static_cast<const bf16_t*>(x), partial, split, gamma, beta, static_cast<f16_t*>(out), C, H,
      W, Wp, L, eps, static_cast<f16_t*>(raw), L_raw, raw_cbase, range_flag);
  return hipGetLastError();
}

// Time-embedding projection of the ResnetBlock2D, plus the constant terms
// the first convolution adds: cadd[b][co] = sum_d w[co][d] SiLU(temb[b][d])
// + temb_b[co] + conv_b[co].  SiLU(temb) of every sample is computed once
// per workgroup into LDS; then one wavefront per output channel, each lane
// taking eight consecutive d of the weight row (one 16-byte load), fp32
// sums reduced across the wavefront.
constexpr int kTembMaxB = 16;
constexpr int kTembMaxFloats = 16384;  // B * Dt floats of SiLU(temb) held in LDS (64 KB)
__global__ __launch_bounds__(256) void temb_proj_kernel(
    const bf16_t* __restrict__ temb, const bf16_t* __restrict__ w,
    const float* __restrict__ temb_b, const float* __restrict__ conv_b, float* __restrict__ cadd,
    int B, int Dt, int Cout) {
  extern __shared__ float st[];  // [B][Dt]
  for (int i = threadIdx.x; i < B * Dt; i += 256) {
    const float t = bf2f(temb[i]);
    st[i] = t / (1.0f + __expf(-t));
  }
  __syncthreads();
  const int co = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (co >= Cout) return;
  float acc[kTembMaxB];
#pragma unroll
  for (int b = 0; b < kTembMaxB; ++b) acc[b] = 0.f;
  const bf16_t* wr = w + static_cast<long long>(co) * Dt;
  for (int d0 = lane * 8; d0 < Dt; d0 += 512) {
    float wv[8];
    load8<bf16_t>(wr + d0, wv);
#pragma unroll
    for (int b = 0; b < kTembMaxB; ++b) {
      if (b < B) {
        const float* sb = st + b * Dt + d0;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[b] = fmaf(wv[q], sb[q], acc[b]);
      }
    }
  }
  const float add = (temb_b ? temb_b[co] : 0.f) + (conv_b ? conv_b[co] : 0.f);
#pragma unroll
  for (int b = 0; b < kTembMaxB; ++b) {
    if (b < B) {
      const float v = warp_sum(acc[b]);
      if (lane == 0) cadd[static_cast<long long>(b) * Cout + co] = v + add;
    }
  }
}

hipError_t temb_proj(const void* temb, const void* w, const float* temb_b, const float* conv_b,
                     float* cadd, int B, int Dt, int Cout, hipStream_t s) {
  // rows of 8-element (16-byte) loads; SiLU(temb) of all samples in LDS
  if (!temb_proj_supported(B, Dt)) return hipErrorInvalidValue;
  temb_proj_kernel<<<(Cout + 3) / 4, 256, sizeof(float) * B * Dt, s>>>(
      static_cast<const bf16_t*>(temb), static_cast<const bf16_t*>(w), temb_b, conv_b, cadd, B, Dt,
      Cout);
  return hipGetLastError();
}
bool temb_proj_supported(int B, int Dt) {
  return B >= 1 && B <= kTembMaxB && Dt >= 8 && Dt % 8 == 0 && B * Dt <= kTembMaxFloats;
}

// Convolution weights to the GEMM operand: w [Cout][Cin][3][3] (bf16) ->
// dst [Cout][ldk] fp16 with dst[co][t * Cp + ci] = w[co][ci][t] (tap t = 3
// di + dj; channels Cin <= ci < Cp are zero: the padding of a narrow input
// to a whole number of 64-deep K stages), and, with a 1x1 shortcut,
// dst[co][9 Cp + ci] = sc[co][ci] (bf16 [Cout][Csc]).  Magnitudes above
// 65504 set *overflow.
__global__ void conv_weight_pack_kernel(const bf16_t* __restrict__ w, const bf16_t* __restrict__ sc,
                                        f16_t* __restrict__ dst, int Cout, int Cin, int Cp, int Csc,
                                        int* __restrict__ overflow) {
  const int ldk = 9 * Cp + Csc;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long long>(Cout) * ldk) return;
  const int co = static_cast<int>(idx / ldk);
  const int k = static_cast<int>(idx - static_cast<long long>(co) * ldk);
  float v = 0.f;
  if (k < 9 * Cp) {
    const int t = k / Cp, ci = k - (k / Cp) * Cp;
    if (ci < Cin) v = bf2f(w[(static_cast<long long>(co) * Cin + ci) * 9 + t]);
  } else {
    v = bf2f(sc[static_cast<long long>(co) * Csc + (k - 9 * Cp)]);
  }
  if (fabsf(v) > 65504.0f) *overflow = 1;
  dst[idx] = static_cast<f16_t>(v);
}

hipError_t conv_weight_pack(const void* w, const void* sc, void* dst, int Cout, int Cin, int Csc,
                            int* overflow, hipStream_t s) {
  return conv_weight_pack_padded(w, sc, dst, Cout, Cin, Cin, Csc, overflow, s);
}

hipError_t conv_weight_pack_padded(const void* w, const void* sc, void* dst, int Cout, int Cin,
                                   int Cp, int Csc, int* overflow, hipStream_t s) {
  if (Cp < Cin) return hipErrorInvalidValue;
  const long long n = static_cast<long long>(Cout) * (9 * Cp + Csc);
  conv_weight_pack_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      static_cast<const bf16_t*>(w), static_cast<const bf16_t*>(sc), static_cast<f16_t*>(dst), Cout,
      Cin, Cp, Csc, overflow);
  return hipGetLastError();
}

// NCHW bf16 -> the zero-haloed NHWC fp16 operand of a 3x3 convolution, no
// normalisation: input pixel (i, j) goes to grid position (i + 1, j + 1)
// (row (b * (Hg + 2) + i + 1) * Wp + j + 1, L elements per row), or, with
// `up`, to the four positions (2i + a + 1, 2j + c + 1) of the 2x grid
// (nearest-neighbour upsampling).  Channels C <= c < L get zeros, and the
// workgroups after the pixel tiles write the halo's zeros (all L channels),
// so that the buffer needs no clearing beforehand.  64 channels x 64
// pixels per workgroup through LDS, as the GroupNorm variant.
__global__ __launch_bounds__(256) void nchw_to_pad_kernel(
    const bf16_t* __restrict__ x, f16_t* __restrict__ out, int C, int H, int W, int Wp, int L,
    int up, int* __restrict__ range_flag) {
  __shared__ float tile[64][64 + 4];
  const int N = H * W;
  const int n0 = blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int Hg = up ? 2 * H : H, Wg = up ? 2 * W : W;
  const int ntiles = (N + 63) / 64;
  if (static_cast<int>(blockIdx.x) >= ntiles) {  // halo zeros (no barrier below)
    const int k = (blockIdx.x - ntiles) * kHaloPerGroup + (tid >> 3);
    const int cl = 8 * (tid & 7);
    if (k >= halo_pixels(Hg, Wg) || c0 + cl >= L) return;
    *reinterpret_cast<uint4*>(out + halo_row(b, k, Hg, Wg, Wp) * L + c0 + cl) = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cl = pass * 32 + (tid >> 3);
    const int nl = 8 * (tid & 7);
    const int c = c0 + cl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + nl + j;
      tile[cl][nl + j] = (c < C && n < N) ? bf2f(x[(static_cast<long long>(b) * C + c) * N + n]) : 0.f;
    }
  }
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int nl = pass * 32 + (tid >> 3);
    const int cl = 8 * (tid & 7);
    const int n = n0 + nl;
    // channels past C hold zeros in the tile
    if (n >= N || c0 + cl >= L) continue;
    const int i = n / W, j = n - (n / W) * W;
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = tile[cl + q][nl];
    const int reps = up ? 4 : 1;
    for (int r = 0; r < reps; ++r) {
      const int oi = up ? 2 * i + (r >> 1) : i, oj = up ? 2 * j + (r & 1) : j;
      const long long row = (static_cast<long long>(b) * (Hg + 2) + oi + 1) * Wp + oj + 1;
      bad |= store8<f16_t>(out + row * L + c0 + cl, v);
    }
  }
  if (bad && range_flag) *range_flag = 1;
}

hipError_t nchw_to_pad(const void* x, void* out, int B, int C, int H, int W, int Wp, int L, bool up,
                       int* range_flag, hipStream_t s) {
  // the channel tiles cover [0, L): L is C rounded up to at most 64
  if (L % 8 || L < C || L > (C + 63) / 64 * 64) return hipErrorInvalidValue;
  const int Hg = up ? 2 * H : H, Wg = up ? 2 * W : W;
  dim3 grid((H * W + 63) / 64 + (halo_pixels(Hg, Wg) + kHaloPerGroup - 1) / kHaloPerGroup, (C + 63) / 64, B);
  nchw_to_pad_kernel<<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(x), static_cast<f16_t*>(out), C,
                                          H, W, Wp, L, up ? 1 : 0, range_flag);
  return hipGetLastError();
}

// Sinusoidal timestep embedding: out[b][i] = cos(t_b f_i), out[b][half + i]
// = sin(t_b f_i), f_i = 10000^(-i / half), fp32.
__global__ void timestep_embed_kernel(const float* __restrict__ t, float* __restrict__ out, int dim) {
  const int b = blockIdx.x;
  const int half = dim / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const float f = expf(-9.210340371976184f * static_cast<float>(i) / static_cast<float>(half));
    float sv, cv;
    sincosf(t[b] * f, &sv, &cv);
    out[static_cast<long long>(b) * dim + i] = cv;
    out[static_cast<long long>(b) * dim + half + i] = sv;
  }
}

hipError_t timestep_embed(const float* t, float* out, int B, int dim, hipStream_t s) {
  if (dim % 2) return hipErrorInvalidValue;
  timestep_embed_kernel<<<B, 128, 0, s>>>(t, out, dim);
  return hipGetLastError();
}

// One Linear of the embedding MLPs, tiny batch: y[b][o] = sum_d w[o][d]
// act(x[b][d]) + bias[o] (+ y[b][o] when accumulating), act = SiLU or the
// identity, x fp32 or bf16, w bf16 [Dout][Din]; with y16 the result is also
// stored in bf16.  act(x) of every sample is staged in LDS once per
// workgroup; one wavefront per output feature, 16-byte weight loads.
template <typename TX>
__global__ __launch_bounds__(256) void mlp_linear_kernel(
    const TX* __restrict__ x, int silu, const bf16_t* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ y, bf16_t* __restrict__ y16, int accumulate, int B, int Din, int Dout) {
  extern __shared__ float sx[];  // [B][Din]
  for (int i = threadIdx.x; i < B * Din; i += 256) {
    const float v = to_f32<TX>(x[i]);
    sx[i] = silu ? v / (1.0f + __expf(-v)) : v;
  }
  __syncthreads();
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (o >= Dout) return;
  float acc[kTembMaxB];
#pragma unroll
  for (int b = 0; b < kTembMaxB; ++b) acc[b] = 0.f;
  const bf16_t* wr = w + static_cast<long long>(o) * Din;
  for (int d0 = lane * 8; d0 < Din; d0 += 512) {
    float wv[8];
    load8<bf16_t>(wr + d0, wv);
#pragma unroll
    for (int b = 0; b < kTembMaxB; ++b) {
      if (b < B) {
        const float* sb = sx + b * Din + d0;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[b] = fmaf(wv[q], sb[q], acc[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < kTembMaxB; ++b) {
    if (b < B) {
      float v = warp_sum(acc[b]) + (bias ? bias[o] : 0.f);
      if (lane == 0) {
        const long long at = static_cast<long long>(b) * Dout + o;
        if (accumulate) v += y[at];
        y[at] = v;
        if (y16) y16[at] = f2bf(v);
      }
    }
  }
}

hipError_t mlp_linear(const void* x, bool x_bf16, bool silu, const void* w, const float* bias,
                      float* y, void* y16, bool accumulate, int B, int Din, int Dout, hipStream_t s) {
  if (!temb_proj_supported(B, Din)) return hipErrorInvalidValue;
  const size_t lds = sizeof(float) * B * Din;
  if (x_bf16)
    mlp_linear_kernel<bf16_t><<<(Dout + 3) / 4, 256, lds, s>>>(
        static_cast<const bf16_t*>(x), silu ? 1 : 0, static_cast<const bf16_t*>(w), bias, y,
        static_cast<bf16_t*>(y16), accumulate ? 1 : 0, B, Din, Dout);
  else
    mlp_linear_kernel<float><<<(Dout + 3) / 4, 256, lds, s>>>(
        static_cast<const float*>(x), silu ? 1 : 0, static_cast<const bf16_t*>(w), bias, y,
        static_cast<bf16_t*>(y16), accumulate ? 1 : 0, B, Din, Dout);
  return hipGetLastError();
}

// ------------------------------------------------------- key padding mask
__global__ __launch_bounds__(64) void mask_to_bits_kernel(const uint8_t* __restrict__ mask,
                                                          uint32_t* __restrict__ bits, int nk) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  // lane k < 32 covers keys k, 32 + k, 64 + k
  uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int key = 32 * i + lane;
    const bool on = lane < 32 && key < nk && mask[static_cast<long long>(b) * nk + key] != 0;
    w[i] = static_cast<uint32_t>(__ballot(on));  // lanes 0..31 of the ballot
  }
  if (lane == 0)
    *reinterpret_cast<uint4*>(bits + 4LL * b) = make_uint4(w[0], w[1], w[2], 0u);
}

hipError_t mask_to_bits(const uint8_t* mask, uint32_t* bits, int B, int nk, hipStream_t s) {
  if (nk > 96) return hipErrorInvalidValue;
  mask_to_bits_kernel<<<B, 64, 0, s>>>(mask, bits, nk);
  return hipGetLastError();
}

// ------------------------------------------------------- guided DDPM step
// x_prev = c1 * (x_t - c2 * eps) + sigma * z with eps = eps_u + scale *
// (eps_c - eps_u), elementwise in fp32; eps_pair holds the unconditional
// prediction in [0, n) and the conditional one in [n, 2n).
template <typename TE>
__global__ __launch_bounds__(256) void guided_ddpm_kernel(
    const TE* __restrict__ eps_pair, const float* __restrict__ x_t,
    const float* __restrict__ noise, float* __restrict__ x_prev, long long n, float scale,
    float c1, float c2, float sigma) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float eu = to_f32<TE>(eps_pair[i]);
    const float ec = to_f32<TE>(eps_pair[n + i]);
    const float e = fmaf(scale, ec - eu, eu);
    float v = c1 * fmaf(-c2, e, x_t[i]);
    if (noise) v = fmaf(sigma, noise[i], v);
    x_prev[i] = v;
  }
}

hipError_t guided_ddpm(const void* eps_pair, bool eps_bf16, const float* x_t, const float* noise,
                       float* x_prev, long long n, float scale, float c1, float c2, float sigma,
                       hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (eps_bf16)
    guided_ddpm_kernel<bf16_t><<<static_cast<unsigned>(blocks), 256, 0, s>>>(
        static_cast<const bf16_t*>(eps_pair), x_t, noise, x_prev, n, scale, c1, c2, sigma);
  else
    guided_ddpm_kernel<float><<<static_cast<unsigned>(blocks), 256, 0, s>>>(
        static_cast<const float*>(eps_pair), x_t, noise, x_prev, n, scale, c1, c2, sigma);
  return hipGetLastError();
}

// ---------------------------------------------------------------- LayerNorm
// One wavefront per token row of the fp32 residual stream; the row, gamma and
// beta are held in registers (VPL float4 each per lane), mean and variance
// are two exact passes over registers with wavefront sums in registers.
template <int VPL, typename TO>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const float* __restrict__ h, const float* __restrict__ gamma,
    const float* __restrict__ beta, TO* __restrict__ u, int T, int C) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= T) return;
  const float4* hr = reinterpret_cast<const float4*>(h + static_cast<long long>(row) * C);
  const int nv = C / 4;
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  const float4* b4 = reinterpret_cast<const float4*>(beta);
  // the row, gamma and beta all in flight at once
  float4 v[VPL], g[VPL], bb[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    const bool in = j < nv;
    v[i] = in ? hr[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    g[i] = in ? g4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    bb[i] = in ? b4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = wave_sum(s) / C;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    if (j < nv) {
      float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      q += (a * a + b * b) + (c * c + d * d);
    }
  }
  const float rstd = rsqrtf(wave_sum(q) / C + 1e-5f);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    if (j < nv) {
      float o0 = (v[i].x - mean) * rstd * g[i].x + bb[i].x;
      float o1 = (v[i].y - mean) * rstd * g[i].y + bb[i].y;
      float o2 = (v[i].z - mean) * rstd * g[i].z + bb[i].z;
      float o3 = (v[i].w - mean) * rstd * g[i].w + bb[i].w;
      TO* dst = u + static_cast<long long>(row) * C + 4 * j;
      if constexpr (sizeof(TO) == 2) {
        uint2 pk = make_uint2(pack2<TO>(o0, o1), pack2<TO>(o2, o3));
        *reinterpret_cast<uint2*>(dst) = pk;
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(o0, o1, o2, o3);
      }
    }
  }
}

// Rows wider than the register path: three passes over global memory.
template <typename TO>
__global__ __launch_bounds__(256) void layernorm_wide_kernel(
    const float* __restrict__ h, const float* __restrict__ gamma,
    const float* __restrict__ beta, TO* __restrict__ u, int T, int C) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= T) return;
  const float* hr = h + static_cast<long long>(row) * C;
  float s = 0.f;
  for (int j = lane; j < C; j += 64) s += hr[j];
  const float mean = warp_sum(s) / C;
  float q = 0.f;
  for (int j = lane; j < C; j += 64) { float d = hr[j] - mean; q += d * d; }
  const float rstd = rsqrtf(warp_sum(q) / C + 1e-5f);
  for (int j = lane; j < C; j += 64)
    u[static_cast<long long>(row) * C + j] =
        from_f32<TO>((hr[j] - mean) * rstd * gamma[j] + beta[j]);
}

template <typename TO>
static void launch_ln(const float* h, const float* g, const float* b, TO* u,
                      int T, int C, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  const int vpl = (C / 4 + 63) / 64;
  switch (vpl) {
    case 1: layernorm_kernel<1, TO><<<grid, 256, 0, s>>>(h, g, b, u, T, C); break;
    case 2: layernorm_kernel<2, TO><<<grid, 256, 0, s>>>(h, g, b, u, T, C); break;
    case 3: layernorm_kernel<3, TO><<<grid, 256, 0, s>>>(h, g, b, u, T, C); break;
    case 4: layernorm_kernel<4, TO><<<grid, 256, 0, s>>>(h, g, b, u, T, C); break;
    case 5: layernorm_kernel<5, TO><<<grid, 256, 0, s>>>(h, g, b, u, T, C); break;
    case 6: layernorm_kernel<6, TO><<<grid, 256, 0, s>>>(h, g, b, u, T, C); break;
    case 7: layernorm_kernel<7, TO><<<grid, 256, 0, s>>>(h, g, b, u, T, C); break;
    case 8: layernorm_kernel<8, TO><<<grid, 256, 0, s>>>(h, g, b, u, T, C); break;
    default: layernorm_wide_kernel<TO><<<grid, 256, 0, s>>>(h, g, b, u, T, C); break;
  }
}

hipError_t layernorm(const float* h, const float* gamma, const float* beta,
                     void* u, int out_type, int T, int C, hipStream_t s) {
  if (out_type == ACT_BF16)
    launch_ln<bf16_t>(h, gamma, beta, static_cast<bf16_t*>(u), T, C, s);
  else if (out_type == ACT_F16)
    launch_ln<f16_t>(h, gamma, beta, static_cast<f16_t*>(u), T, C, s);
  else
    launch_ln<float>(h, gamma, beta, static_cast<float*>(u), T, C, s);
  return hipGetLastError();
}

// ------------------------------------------------------------------ helpers
__global__ void geglu_f32_kernel(const float* __restrict__ z,
                                 float* __restrict__ f, long long total, int F) {
  long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  long long r = i / F;
  int c = static_cast<int>(i - r * F);
  const float* zr = z + r * 2 * F;
  f[i] = zr[c] * gelu_erf(zr[F + c]);
}

hipError_t geglu_f32(const float* z, float* f, long long T, int F,
                     hipStream_t s) {
  long long total = T * F;
  geglu_f32_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, s>>>(z, f, total, F);
  return hipGetLastError();
}

template <typename T>
__global__ void to_f32_kernel(const T* __restrict__ src, float* __restrict__ dst,
                              long long n, float fill) {
  long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  dst[i] = src ? to_f32<T>(src[i]) : fill;
}

hipError_t to_f32(const void* src, bool bf16, float* dst, long long n,
                  float fill, hipStream_t s) {
  unsigned grid = static_cast<unsigned>((n + 255) / 256);
  if (bf16)
    to_f32_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(src), dst, n, fill);
  else
    to_f32_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(src), dst, n, fill);
  return hipGetLastError();
}

__global__ void f16_to_f32_kernel(const f16_t* __restrict__ src, float* __restrict__ dst,
                                  long long n) {
  long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = static_cast<float>(src[i]);
}

hipError_t f16_to_f32(const void* src, float* dst, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  f16_to_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      static_cast<const f16_t*>(src), dst, n);
  return hipGetLastError();
}

__global__ void bf16_to_f16_kernel(uint16_t* __restrict__ buf, long long n,
                                   int* __restrict__ overflow) {
  long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = bf2f(buf[i]);
  if (fabsf(v) > 65504.0f) *overflow = 1;
  buf[i] = __builtin_bit_cast(uint16_t, static_cast<f16_t>(v));
}

hipError_t bf16_to_f16_inplace(void* buf, long long n, int* overflow,
                               hipStream_t s) {
  bf16_to_f16_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      static_cast<uint16_t*>(buf), n, overflow);
  return hipGetLastError();
}

// One wavefront per weight row: the row's elements strided over the lanes,
// fp64 sums reduced across the wavefront.
__global__ __launch_bounds__(64) void weight_fold_layernorm_kernel(
    uint16_t* __restrict__ w, int C, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* __restrict__ bias,
    const int* __restrict__ map, float* __restrict__ g, int* __restrict__ overflow) {
  const int j = blockIdx.x;
  uint16_t* row = w + static_cast<long long>(j) * C;
  double gs = 0.0, bs = 0.0;
  bool big = false;
  for (int c = threadIdx.x; c < C; c += 64) {
    const float v = bf2f(row[c]);
    const f16_t h = static_cast<f16_t>(v * gamma[c]);
    big |= fabsf(v * gamma[c]) > 65504.0f;
    row[c] = __builtin_bit_cast(uint16_t, h);
    gs += static_cast<double>(static_cast<float>(h));
    bs += static_cast<double>(beta[c]) * static_cast<double>(v);
  }
  if (big) *overflow = 1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    gs += __shfl_xor(gs, o, 64);
    bs += __shfl_xor(bs, o, 64);
  }
  if (threadIdx.x == 0) {
    g[j] = static_cast<float>(gs);
    const int bj = map ? map[j] : j;
    bias[bj] = static_cast<float>(static_cast<double>(bias[bj]) + bs);
  }
}

hipError_t weight_fold_layernorm(void* w, int rows, int C, const float* gamma,
                                 const float* beta, float* bias, const int* map,
                                 float* g, int* overflow, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  weight_fold_layernorm_kernel<<<rows, 64, 0, s>>>(static_cast<uint16_t*>(w), C, gamma, beta,
                                                   bias, map, g, overflow);
  return hipGetLastError();
}

__global__ void gather_rows_kernel(const uint4* __restrict__ src,
                                   uint4* __restrict__ dst,
                                   const int* __restrict__ map,
                                   long long row_vec) {
  const int r = blockIdx.x;
  const uint4* s = src + static_cast<long long>(map[r]) * row_vec;
  uint4* d = dst + static_cast<long long>(r) * row_vec;
  for (long long i = threadIdx.x; i < row_vec; i += blockDim.x) d[i] = s[i];
}

hipError_t gather_rows(const void* src, void* dst, const int* map, int rows,
                       long long row_bytes, hipStream_t s) {
  gather_rows_kernel<<<rows, 256, 0, s>>>(static_cast<const uint4*>(src),
                                          static_cast<uint4*>(dst), map,
                                          row_bytes / 16);
  return hipGetLastError();
}

}  // namespace stb
