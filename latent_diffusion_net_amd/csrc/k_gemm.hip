// GEMMs of the Spatial-Transformer block: C[M][N] = A[M][K] * B[N][K]^T with
// both operands K-contiguous (activations [tokens][in], weights [out][in]).
//
// 16-bit path: v_mfma_f32_32x32x16_{bf16,f16} on gfx950.  A 256-thread workgroup
// owns a 128x128 output tile; each of its four wavefronts owns a 64x64
// quarter as 2x2 MFMA blocks of 32x32 (64 fp32 accumulators per lane).  K
// advances 64 at a time through two LDS buffers: the next tile's global loads
// are issued before the current tile's MFMAs and written to the other buffer
// after them, so one barrier per K step suffices.  LDS rows are 128 bytes
// (64 bf16); the eight 16-byte chunks of a row are XOR-swizzled by the row
// index so that the 32 rows one MFMA operand read touches spread over all
// banks.  Rows beyond M or N are clamped on load and masked on store.
//
// fp32 path (debug builds of the block): a plain LDS-tiled fp32 FMA GEMM with
// the same epilogues.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace stb {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

// One 8-element chunk of B.  SPLIT: B is fp32 and the chunk holds its bf16
// high part (lo == false) or the bf16 rounding of the remainder (lo == true).
template <bool SPLIT>
__device__ __forceinline__ uint4 load_b_chunk(const void* B, long long ldb,
                                              long long row, int k, bool lo) {
  if constexpr (SPLIT) {
    const float4* p = reinterpret_cast<const float4*>(
        static_cast<const float*>(B) + row * ldb + k);
    const float4 x0 = p[0], x1 = p[1];
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if (lo) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] -= bf2f(f2bf(v[i]));
    }
    return make_uint4(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]),
                      pack2bf(v[4], v[5]), pack2bf(v[6], v[7]));
  } else {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(B) +
                                           row * ldb + k);
  }
}

template <int EPI, typename OpT, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void gemm_mfma_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const uint16_t* A = static_cast<const uint16_t*>(p.A);
  const int M = p.M, N = p.N;
  const int nkh = p.K / BK;                 // K steps over the real K
  const int nk = SPLIT ? 2 * nkh : nkh;     // SPLIT: hi pass then lo pass

  // Each thread stages 4 chunks of 8 elements of A and of B per K step.
  uint4 ra[4], rb[4];
  auto load_tile = [&](int kt) {
    const bool lo = SPLIT && kt >= nkh;
    const int k0 = (lo ? kt - nkh : kt) * BK;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = tid + kThreads * r;
      const int row = q >> 3, c = q & 7;
      const long long gm = min(m0 + row, M - 1);
      const long long gn = min(n0 + row, N - 1);
      ra[r] = *reinterpret_cast<const uint4*>(A + gm * p.lda + k0 + c * 8);
      rb[r] = load_b_chunk<SPLIT>(p.B, p.ldb, gn, k0 + c * 8, lo);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = tid + kThreads * r;
      const int row = q >> 3, c = q & 7;
      *reinterpret_cast<uint4*>(&sA[buf][lds_off(row, c)]) = ra[r];
      *reinterpret_cast<uint4*>(&sB[buf][lds_off(row, c)]) = rb[r];
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  const int l32 = lane & 31, lhi = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int chunk = 2 * s + lhi;
      uint4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const uint4*>(&sA[buf][lds_off(wm * 64 + i * 32 + l32, chunk)]);
        b[i] = *reinterpret_cast<const uint4*>(&sB[buf][lds_off(wn * 64 + i * 32 + l32, chunk)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j], OpT{});
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Accumulator layout of a 32x32 block: lane holds column (lane & 31) and
  // rows 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
  if constexpr (EPI == EPI_GEGLU) {
    // Repacked W1: each group of 64 rows is 32 value rows then the 32
    // matching gate rows, so block j=0 holds values and j=1 their gates.
    const int pc0 = n0 + wn * 64;
    if (pc0 < N) {
      const int fcol = (pc0 >> 6) * 32 + l32;
      const int F = p.epi.F;
      const float bv = p.epi.bias ? p.epi.bias[fcol] : 0.f;
      const float bg = p.epi.bias ? p.epi.bias[F + fcol] : 0.f;
      f16_t* out = static_cast<f16_t*>(p.epi.out_act);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
          if (row < M) {
            const float v = acc[i][0][r] + bv;
            const float g = acc[i][1][r] + bg;
            out[static_cast<long long>(row) * F + fcol] = static_cast<f16_t>(v * gelu_erf(g));
          }
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + j * 32 + l32;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
          if (row < M) epi_store<EPI, bf16_t>(p.epi, row, col, acc[i][j][r]);
        }
      }
  }
}

// ---------------------------------------------------------------- fp32 GEMM
constexpr int FT = 64, FK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  __shared__ float sA[FK][FT + 4];
  __shared__ float sB[FK][FT + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
  const float* A = static_cast<const float*>(p.A);
  const float* B = static_cast<const float*>(p.B);
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += FK) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = tid + 256 * r;
      const int row = q >> 4, kk = q & 15;
      const long long gm = min(m0 + row, p.M - 1);
      const long long gn = min(n0 + row, p.N - 1);
      sA[kk][row] = A[gm * p.lda + k0 + kk];
      sB[kk][row] = B[gn * p.ldb + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sA[kk][ty * 4 + i]; b[i] = sB[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
      if (row < p.M && col < p.N) epi_store<EPI, float>(p.epi, row, col, acc[i][j]);
    }
}

}  // namespace

hipError_t gemm_mfma(const GemmParams& p, int op, bool b_split_f32,
                     hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.K % BK) return hipErrorInvalidValue;
  if (b_split_f32 && op != ACT_BF16) return hipErrorInvalidValue;
  dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM);
  switch (p.epi.kind) {
    case EPI_STORE_F32:
      if (op == ACT_F16) gemm_mfma_kernel<EPI_STORE_F32, f16_t, false><<<grid, kThreads, 0, s>>>(p);
      else gemm_mfma_kernel<EPI_STORE_F32, bf16_t, false><<<grid, kThreads, 0, s>>>(p);
      break;
    case EPI_RESID_F32:
      if (op == ACT_F16) gemm_mfma_kernel<EPI_RESID_F32, f16_t, false><<<grid, kThreads, 0, s>>>(p);
      else gemm_mfma_kernel<EPI_RESID_F32, bf16_t, false><<<grid, kThreads, 0, s>>>(p);
      break;
    case EPI_HEADS:
      if (op == ACT_F16) gemm_mfma_kernel<EPI_HEADS, f16_t, false><<<grid, kThreads, 0, s>>>(p);
      else gemm_mfma_kernel<EPI_HEADS, bf16_t, false><<<grid, kThreads, 0, s>>>(p);
      break;
    case EPI_GEGLU:
      if (op == ACT_F16) gemm_mfma_kernel<EPI_GEGLU, f16_t, false><<<grid, kThreads, 0, s>>>(p);
      else gemm_mfma_kernel<EPI_GEGLU, bf16_t, false><<<grid, kThreads, 0, s>>>(p);
      break;
    case EPI_NCHW:
      if (b_split_f32) gemm_mfma_kernel<EPI_NCHW, bf16_t, true><<<grid, kThreads, 0, s>>>(p);
      else if (op == ACT_F16) gemm_mfma_kernel<EPI_NCHW, f16_t, false><<<grid, kThreads, 0, s>>>(p);
      else gemm_mfma_kernel<EPI_NCHW, bf16_t, false><<<grid, kThreads, 0, s>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t gemm_f32(const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  dim3 grid((p.N + FT - 1) / FT, (p.M + FT - 1) / FT);
  switch (p.epi.kind) {
    case EPI_STORE_F32: gemm_f32_kernel<EPI_STORE_F32><<<grid, 256, 0, s>>>(p); break;
    case EPI_RESID_F32: gemm_f32_kernel<EPI_RESID_F32><<<grid, 256, 0, s>>>(p); break;
    case EPI_HEADS: gemm_f32_kernel<EPI_HEADS><<<grid, 256, 0, s>>>(p); break;
    case EPI_NCHW: gemm_f32_kernel<EPI_NCHW><<<grid, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace stb
