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
  for (long long i = vlo + 8LL * threadIdx.x; i < vhi; i += 8LL * kGnThreads) {
    float v[8];
    load8<T>(x + i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float d = v[j] - shift;
      s1 += d; s2 += d * d;
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

template <typename T>
__device__ __forceinline__ void store8(T* p, const float v[8]);
template <>
__device__ __forceinline__ void store8<f16_t>(f16_t* p, const float v[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack2h(v[0], v[1]), pack2h(v[2], v[3]),
                                            pack2h(v[4], v[5]), pack2h(v[6], v[7]));
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
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
    TO* __restrict__ out, int C, int N) {
  __shared__ float2 coef[64];
  __shared__ float tile[64][64 + 4];  // [channel][token]
  const int n0 = blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int b = blockIdx.z;
  const int cg = C / kGroups;
  const int tid = threadIdx.x;
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
    const float rstd = static_cast<float>(1.0 / sqrt(var + 1e-6));
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
    for (int j = 0; j < 8; ++j) tile[cl][nl + j] = v[j] * k.x + k.y;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int nl = pass * 32 + (tid >> 3);
    const int cl = 8 * (tid & 7);
    const int n = n0 + nl;
    if (n >= N) continue;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = tile[cl + j][nl];
    store8<TO>(out + (static_cast<long long>(b) * N + n) * C + c0 + cl, v);
  }
}

hipError_t gn_apply_tokens(const void* x, bool bf16, const float2* partial,
                           int max_split, const float* gamma, const float* beta,
                           void* out, int out_type, int B, int C, int N,
                           hipStream_t s) {
  const int split = gn_split(C, N, max_split);
  dim3 grid((N + 63) / 64, C / 64, B);
  if (bf16 && out_type == ACT_F16)
    gn_apply_tokens_kernel<bf16_t, f16_t><<<grid, 256, 0, s>>>(
        static_cast<const bf16_t*>(x), partial, split, gamma, beta,
        static_cast<f16_t*>(out), C, N);
  else if (!bf16 && out_type == ACT_F32)
    gn_apply_tokens_kernel<float, float><<<grid, 256, 0, s>>>(
        static_cast<const float*>(x), partial, split, gamma, beta,
        static_cast<float*>(out), C, N);
  else
    return hipErrorInvalidValue;
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
