// GEMMs of the Spatial-Transformer block: C[M][N] = A[M][K] * B[N][K]^T with
// both operands K-contiguous (activations [tokens][in], weights [out][in]).
//
// 16-bit operands (bf16 or fp16) on v_mfma_f32_32x32x16 with fp32
// accumulation.  A 256-thread workgroup owns a 128x128 output tile; each of
// its four wavefronts owns a 64x64 quarter as 2x2 MFMA blocks of 32x32 (64
// fp32 accumulators per lane).  K advances 64 at a time through a ring of
// LDS stages filled by global_load_lds_dwordx4 (no staging registers), with
// one barrier per stage.  Each stage buffer is its own LDS object: the
// compiler can then tell a DMA into one stage from reads of another and does
// not wait on it.  LDS rows are 128 bytes (64 elements, eight 16-byte
// chunks); chunk c of row r is stored at c ^ ((r >> 1) & 7), which spreads
// the 16 rows of one 16-lane read phase over all 16 bank groups of gfx950's
// 64-bank LDS.  Rows beyond M or N are clamped on load and masked on store.
//
// The residual epilogue can also leave the new fp32 value as two bf16 terms
// (hi, lo) so that proj_out can take the residual stream at ~16 significant
// bits through the same bf16 kernel with K doubled.
//
// fp32 path (debug builds of the block): a plain LDS-tiled fp32 FMA GEMM with
// the same epilogues.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace stb {

namespace {

constexpr int BM = 128, BN = 128;
constexpr int kThreads = 256;

// Output tile of this workgroup (1-D grid of mt * nt workgroups).
// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2, so
// each XCD is given a contiguous run of logical tiles; logical tiles walk
// groups of up to 4 M-tiles, M fastest, then N.  The A rows of a group and
// the few B tiles its resident workgroups share then stay in one L2 instead
// of every XCD streaming all of B.
__device__ __forceinline__ void tile_coords(int mt, int nt, int bid, int& tm, int& tn) {
  constexpr int G = 4;
  const int total = mt * nt;
  int b = bid;
  if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);
  const int group = b / (G * nt);
  const int first = group * G;
  const int gm = min(G, mt - first);
  const int r = b - group * G * nt;
  tn = r / gm;
  tm = first + (r - tn * gm);
}


// Head-split store of four consecutive rows (tokens) of one column.  For a
// V^T destination the four values are contiguous and go out as one 8-byte
// store when they belong to one sample and stay aligned.
__device__ __forceinline__ void store_heads4(const HeadSplit& hs, int row0,
                                             int col, const float v[4],
                                             float bias, int M) {
  const int which = col / hs.C;
  const int s = which % hs.nsplit;
  const int layer = which / hs.nsplit;
  const int within = col - which * hs.C;
  const int head = within >> 6;
  const int dim = within & 63;
  bf16_t* base = static_cast<bf16_t*>(hs.dst[s]) + layer * hs.layer_stride;
  const bool trans = (hs.transposed_mask >> s) & 1;
  const int b0 = row0 / hs.rows_per_batch;
  const int n0 = row0 - b0 * hs.rows_per_batch;
  if (trans && (hs.rows_per_batch & 3) == 0 && row0 + 3 < M) {
    const long long bh = static_cast<long long>(b0) * hs.heads + head;
    const uint2 pk = make_uint2(pack2bf(v[0] + bias, v[1] + bias),
                                pack2bf(v[2] + bias, v[3] + bias));
    *reinterpret_cast<uint2*>(base + (bh * kHeadDim + dim) * hs.npad + n0) = pk;
    return;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = row0 + k;
    if (row >= M) break;
    const int b = row / hs.rows_per_batch;
    const int n = row - b * hs.rows_per_batch;
    const long long bh = static_cast<long long>(b) * hs.heads + head;
    const long long idx = trans ? (bh * kHeadDim + dim) * hs.npad + n
                                : (bh * hs.npad + n) * kHeadDim + dim;
    base[idx] = f2bf(v[k] + bias);
  }
}

// Epilogue through LDS.  The wavefront's 64x64 fp32 tile is written to a
// 16 KB LDS area in the accumulator layout, then read back along whichever
// axis is contiguous in the destination, so every global access is a 8- or
// 16-byte vector on consecutive addresses (rows of h, rows of a head of Q/K,
// runs of tokens of V^T and of an NCHW plane, rows of the GEGLU output).
// Column col of the tile is stored at col ^ (32 * ((row >> 2) & 1)): the
// two lane halves of an accumulator write (rows 4 apart) then use opposite
// bank halves.  Requires N % 64 == 0 except for the NCHW kind (tokens).
__device__ __forceinline__ int stg(int row, int col) {
  return row * 64 + (col ^ (((row >> 2) & 1) << 5));
}

template <int EPI>
__device__ __forceinline__ void epilogue_lds(const GemmParams& p,
                                             const floatx16 (&acc)[2][2],
                                             int m0, int n0, int wm, int wn,
                                             int lane, float* stage) {
  const int l32 = lane & 31, lhi = lane >> 5;
  const int M = p.M, N = p.N;
  const int R0 = m0 + wm * 64, C0 = n0 + wn * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stage[stg(i * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3), j * 32 + l32)] = acc[i][j][r];
  __builtin_amdgcn_s_waitcnt((7 << 4) | (63 & 15) | ((63 >> 4) << 14));  // lgkmcnt(0)
  if (C0 >= N || R0 >= M) return;

  if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_RESID_F32) {
    // lane -> 4 consecutive columns of one row; 4 rows per pass
    const int lc = (lane & 15) * 4;
    const float4 bias = p.epi.bias ? *reinterpret_cast<const float4*>(p.epi.bias + C0 + lc)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
    // all 16 residual rows are loaded before the first store (the compiler
    // cannot prove a store to h disjoint from the next row's load)
    float4 hin[16];
    if constexpr (EPI == EPI_RESID_F32) {
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int row = R0 + it * 4 + (lane >> 4);
        hin[it] = row < M ? *reinterpret_cast<const float4*>(
                                p.epi.out_f32 + static_cast<long long>(row) * p.epi.ldo + C0 + lc)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int lr = it * 4 + (lane >> 4);
      const int row = R0 + lr;
      if (row >= M) break;
      const float4 c = *reinterpret_cast<const float4*>(&stage[stg(lr, lc)]);
      float4 v = make_float4(c.x + bias.x, c.y + bias.y, c.z + bias.z, c.w + bias.w);
      if constexpr (EPI == EPI_RESID_F32) {
        v.x += hin[it].x; v.y += hin[it].y; v.z += hin[it].z; v.w += hin[it].w;
      }
      *reinterpret_cast<float4*>(p.epi.out_f32 + static_cast<long long>(row) * p.epi.ldo + C0 + lc) = v;
      if constexpr (EPI == EPI_RESID_F32) {
        if (p.epi.out_act) {
          // h = hi + lo in bf16: hi in columns [0, ldo), lo in [ldo, 2 ldo)
          const uint32_t h0 = f2bf(v.x), h1 = f2bf(v.y), h2 = f2bf(v.z), h3 = f2bf(v.w);
          bf16_t* hs = static_cast<bf16_t*>(p.epi.out_act) + static_cast<long long>(row) * 2 * p.epi.ldo + C0 + lc;
          *reinterpret_cast<uint2*>(hs) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
          *reinterpret_cast<uint2*>(hs + p.epi.ldo) =
              make_uint2(pack2bf(v.x - bf2f(h0), v.y - bf2f(h1)), pack2bf(v.z - bf2f(h2), v.w - bf2f(h3)));
        }
      }
    }
  } else if constexpr (EPI == EPI_GEGLU) {
    // columns 0..31 are values, 32..63 the matching gates; output
    // f[row][(C0 / 64) * 32 + 0..31] in fp16; lane -> 4 outputs of one row
    const int F = p.epi.F;
    const int fc0 = (C0 >> 6) * 32;
    const int lc = (lane & 7) * 4;
    float bv[4], bg[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bv[k] = p.epi.bias ? p.epi.bias[fc0 + lc + k] : 0.f;
      bg[k] = p.epi.bias ? p.epi.bias[F + fc0 + lc + k] : 0.f;
    }
    f16_t* out = static_cast<f16_t*>(p.epi.out_act);
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
      const int lr = it * 8 + (lane >> 3);
      const int row = R0 + lr;
      if (row >= M) break;
      const float4 v = *reinterpret_cast<const float4*>(&stage[stg(lr, lc)]);
      const float4 g = *reinterpret_cast<const float4*>(&stage[stg(lr, 32 + lc)]);
      const uint2 pk = make_uint2(
          pack2h((v.x + bv[0]) * gelu_as(g.x + bg[0]), (v.y + bv[1]) * gelu_as(g.y + bg[1])),
          pack2h((v.z + bv[2]) * gelu_as(g.z + bg[2]), (v.w + bv[3]) * gelu_as(g.w + bg[3])));
      *reinterpret_cast<uint2*>(out + static_cast<long long>(row) * F + fc0 + lc) = pk;
    }
  } else if constexpr (EPI == EPI_HEADS) {
    // The 64 columns are one head of one split (C0 and C are multiples of
    // 64).
    const HeadSplit& hs = p.epi.hs;
    const int which = C0 / hs.C;
    const int sp = which % hs.nsplit;
    const int layer = which / hs.nsplit;
    const int head = (C0 - which * hs.C) >> 6;
    bf16_t* base = static_cast<bf16_t*>(hs.dst[sp]) + layer * hs.layer_stride;
    const float* bias = p.epi.bias ? p.epi.bias + C0 : nullptr;
    if (!((hs.transposed_mask >> sp) & 1)) {
      // [bh][n][64]: lane -> 4 consecutive dims of one token
      const int lc = (lane & 15) * 4;
      float bb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) bb[k] = bias ? bias[lc + k] : 0.f;
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int lr = it * 4 + (lane >> 4);
        const int row = R0 + lr;
        if (row >= M) break;
        const int b = row / hs.rows_per_batch;
        const int n = row - b * hs.rows_per_batch;
        const float4 c = *reinterpret_cast<const float4*>(&stage[stg(lr, lc)]);
        const uint2 pk = make_uint2(pack2bf(c.x + bb[0], c.y + bb[1]), pack2bf(c.z + bb[2], c.w + bb[3]));
        const long long bh = static_cast<long long>(b) * hs.heads + head;
        *reinterpret_cast<uint2*>(base + (bh * hs.npad + n) * kHeadDim + lc) = pk;
      }
    } else {
      // V^T [bh][64][npad]: lane -> one dim, 4 consecutive tokens
      const int dim = lane;
      const float bb = bias ? bias[dim] : 0.f;
      const bool vec = (hs.rows_per_batch & 3) == 0;
#pragma unroll 2
      for (int it = 0; it < 16; ++it) {
        const int lr0 = it * 4;
        const int row0 = R0 + lr0;
        if (row0 >= M) break;
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = stage[stg(lr0 + k, dim)] + bb;
        if (vec && row0 + 3 < M) {
          const int b = row0 / hs.rows_per_batch;
          const int n = row0 - b * hs.rows_per_batch;
          const long long bh = static_cast<long long>(b) * hs.heads + head;
          *reinterpret_cast<uint2*>(base + (bh * kHeadDim + dim) * hs.npad + n) =
              make_uint2(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]));
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int row = row0 + k;
            if (row >= M) break;
            const int b = row / hs.rows_per_batch;
            const int n = row - b * hs.rows_per_batch;
            const long long bh = static_cast<long long>(b) * hs.heads + head;
            base[(bh * kHeadDim + dim) * hs.npad + n] = f2bf(v[k]);
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_NCHW) {
    // rows = channels, columns = tokens: y[b][c][n] = acc + bias[c] + x[b][c][n];
    // lane -> 4 consecutive tokens of one channel
    const int ntok = p.epi.ntok;
    const int lc = (lane & 15) * 4;
    const bf16_t* xin = static_cast<const bf16_t*>(p.epi.resid_act);
    bf16_t* yout = static_cast<bf16_t*>(p.epi.out_act);
    const int t0 = C0 + lc;
    const int b0 = t0 / ntok;
    const int nn = t0 - b0 * ntok;
    const bool vec = (ntok & 3) == 0 && t0 + 3 < N;
    const long long base0 = static_cast<long long>(b0) * p.epi.ldo * ntok + nn;
    if (vec) {
      // all 16 input runs are loaded before the first store
      uint2 xv[16];
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int c = R0 + it * 4 + (lane >> 4);
        xv[it] = c < M ? *reinterpret_cast<const uint2*>(xin + base0 + static_cast<long long>(c) * ntok)
                       : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int lr = it * 4 + (lane >> 4);
        const int c = R0 + lr;
        if (c >= M) break;
        const float bias = p.epi.bias ? p.epi.bias[c] : 0.f;
        const float4 a = *reinterpret_cast<const float4*>(&stage[stg(lr, lc)]);
        const float y0 = a.x + bias + __uint_as_float(xv[it].x << 16);
        const float y1 = a.y + bias + __uint_as_float(xv[it].x & 0xffff0000u);
        const float y2 = a.z + bias + __uint_as_float(xv[it].y << 16);
        const float y3 = a.w + bias + __uint_as_float(xv[it].y & 0xffff0000u);
        *reinterpret_cast<uint2*>(yout + base0 + static_cast<long long>(c) * ntok) =
            make_uint2(pack2bf(y0, y1), pack2bf(y2, y3));
      }
    } else {
      for (int it = 0; it < 16; ++it) {
        const int lr = it * 4 + (lane >> 4);
        const int c = R0 + lr;
        if (c >= M) break;
        const float bias = p.epi.bias ? p.epi.bias[c] : 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = t0 + k;
          if (t >= N) break;
          const int b = t / ntok;
          const long long off = (static_cast<long long>(b) * p.epi.ldo + c) * ntok + (t - b * ntok);
          yout[off] = f2bf(stage[stg(lr, lc + k)] + bias + bf2f(xin[off]));
        }
      }
    }
  }
}

// ------------------------------------------------------- DMA-ring GEMM
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// Stage rows of BKT elements: 64 (128 bytes, eight chunks, chunk c of row r
// at c ^ ((r >> 1) & 7)) or 32 (64 bytes, four chunks, at c ^ ((r >> 2) &
// 3)); either way the 16 rows of one 16-lane read phase cover all 16 bank
// groups of the 64-bank LDS.
template <int BKT>
__device__ __forceinline__ int swz_k(int row, int chunk) {
  if constexpr (BKT == 64)
    return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
  else
    return row * 32 + ((chunk ^ ((row >> 2) & 3)) << 3);
}

template <int EPI, typename OpT, int BKT, int NST>
__global__ __launch_bounds__(kThreads, 2) void gemm_dma_kernel(GemmParams p) {
  // NST stage buffers per operand, each its own LDS object (see the file
  // comment); unused ones are never referenced and take no LDS.
  __shared__ __attribute__((aligned(16))) uint16_t sA0[BM * BKT];
  __shared__ __attribute__((aligned(16))) uint16_t sA1[BM * BKT];
  __shared__ __attribute__((aligned(16))) uint16_t sA2[BM * BKT];
  __shared__ __attribute__((aligned(16))) uint16_t sB0[BN * BKT];
  __shared__ __attribute__((aligned(16))) uint16_t sB1[BN * BKT];
  __shared__ __attribute__((aligned(16))) uint16_t sB2[BN * BKT];
  static_assert(NST == 2 || NST == 3, "stages");
  constexpr int RPB = 1024 / (BKT * 2);      // rows per 1 KB DMA block
  constexpr int DPW = BM / RPB / 4;          // DMA blocks per wave per operand per stage
  constexpr int CPR = BKT / 8;               // 16-byte chunks per row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // split-K: workgroup blockIdx.x takes tile blockIdx.x % tiles and K slice
  // blockIdx.x / tiles (always 0 without split)
  const int mt = (p.M + BM - 1) / BM, nt = (p.N + BN - 1) / BN;
  const int kz = blockIdx.x / (mt * nt);
  const int kslice = p.K / (p.ksplit > 1 ? p.ksplit : 1);
  int tm, tn;
  tile_coords(mt, nt, blockIdx.x - kz * mt * nt, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int M = p.M, N = p.N;
  const uint16_t* A = static_cast<const uint16_t*>(p.A);
  const uint16_t* Bm = static_cast<const uint16_t*>(p.B);
  const int l32 = lane & 31, lhi = lane >> 5;

  // Lane i of a DMA block lands in slot i: row i / CPR, physical chunk
  // i % CPR, so it fetches the logical chunk that belongs there.
  long long aoff[DPW], boff[DPW];
#pragma unroll
  for (int j2 = 0; j2 < DPW; ++j2) {
    const int row = RPB * (wave * DPW + j2) + lane / CPR;
    const int pc = lane % CPR;
    const int cl = (BKT == 64) ? (pc ^ ((row >> 1) & 7)) : (pc ^ ((row >> 2) & 3));
    aoff[j2] = static_cast<long long>(min(m0 + row, M - 1)) * p.lda + static_cast<long long>(kz) * kslice + cl * 8;
    boff[j2] = static_cast<long long>(min(n0 + row, N - 1)) * p.ldb + static_cast<long long>(kz) * kslice + cl * 8;
  }
  auto issue = [&](int k, uint16_t* sa, uint16_t* sb) {
#pragma unroll
    for (int j2 = 0; j2 < DPW; ++j2) {
      const int blk = (wave * DPW + j2) * 512;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(A + aoff[j2] + k * BKT),
                                       (lds_ptr_t)(sa + blk), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Bm + boff[j2] + k * BKT),
                                       (lds_ptr_t)(sb + blk), 16, 0, 0);
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](const uint16_t* sa, const uint16_t* sb) {
#pragma unroll
    for (int s = 0; s < BKT / 16; ++s) {
      const int chunk = 2 * s + lhi;
      uint4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const uint4*>(sa + swz_k<BKT>(wm * 64 + i * 32 + l32, chunk));
        b[i] = *reinterpret_cast<const uint4*>(sb + swz_k<BKT>(wn * 64 + i * 32 + l32, chunk));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j], OpT{});
    }
  };

  // Iteration k: stage k must have landed (later stages may still be in
  // flight), every wavefront must be past iteration k-1 (whose buffer is
  // refilled now with stage k + NST - 1), then stage k is consumed.
  const int nk = kslice / BKT;
  constexpr int PER = 2 * DPW;  // DMA instructions per stage per wavefront
  issue(0, sA0, sB0);
  if (nk > 1 && NST > 2) issue(1, sA1, sB1);
  auto step = [&](int k, const uint16_t* ca, const uint16_t* cb, uint16_t* wa,
                  uint16_t* wb) {
    if constexpr (NST == 3) {
      if (k + 1 < nk) wait_vmcnt_lds<PER>();
      else wait_vmcnt_lds<0>();
    } else {
      wait_vmcnt_lds<0>();
    }
    stage_barrier();
    if (k + NST - 1 < nk) issue(k + NST - 1, wa, wb);
    compute(ca, cb);
  };
  if constexpr (NST == 3) {
    for (int k = 0; k < nk; k += 3) {
      step(k, sA0, sB0, sA2, sB2);
      if (k + 1 < nk) step(k + 1, sA1, sB1, sA0, sB0);
      if (k + 2 < nk) step(k + 2, sA2, sB2, sA1, sB1);
    }
  } else {
    for (int k = 0; k < nk; k += 2) {
      step(k, sA0, sB0, sA1, sB1);
      if (k + 1 < nk) step(k + 1, sA1, sB1, sA0, sB0);
    }
  }

  // every wavefront is done reading the stage buffers before they hold
  // the epilogue tiles
  stage_barrier();
  float* stage = reinterpret_cast<float*>(wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sB0 : sB1);
  if (p.ksplit > 1) {
    // this slice's product, plain fp32, into ws[kz]
    GemmParams q = p;
    q.epi.kind = EPI_STORE_F32;
    q.epi.bias = nullptr;
    q.epi.out_f32 = p.ws + static_cast<long long>(kz) * M * N;
    q.epi.ldo = N;
    epilogue_lds<EPI_STORE_F32>(q, acc, m0, n0, wm, wn, lane, stage);
  } else {
    epilogue_lds<EPI>(p, acc, m0, n0, wm, wn, lane, stage);
  }
}

// Second pass of split-K: the slices added in order (deterministic), then
// the epilogue of one element.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p) {
  const long long mn = static_cast<long long>(p.M) * p.N;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= mn) return;
  float acc = 0.f;
  for (int z = 0; z < p.ksplit; ++z) acc += p.ws[z * mn + idx];
  const int row = static_cast<int>(idx / p.N);
  epi_store<EPI, bf16_t>(p.epi, row, static_cast<int>(idx - static_cast<long long>(row) * p.N), acc);
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

#ifndef ST_GEMM_BKT
#define ST_GEMM_BKT 64
#endif
#ifndef ST_GEMM_NST
#define ST_GEMM_NST 2
#endif
constexpr int kBKT = ST_GEMM_BKT, kNST = ST_GEMM_NST;

hipError_t gemm_mfma(const GemmParams& p, int op, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.K % kBKT) return hipErrorInvalidValue;
  const int split = p.ksplit > 1 ? p.ksplit : 1;
  if (split > 1 && (!p.ws || p.K % (split * kBKT) || op != ACT_BF16 ||
                    (p.epi.kind != EPI_HEADS && p.epi.kind != EPI_STORE_F32)))
    return hipErrorInvalidValue;
  const dim3 grid(((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM) * split);
  if (split > 1) {
    // the slices (the kernel switches to the plain fp32 store), then the sum
    gemm_dma_kernel<EPI_STORE_F32, bf16_t, kBKT, kNST><<<grid, kThreads, 0, s>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long mn = static_cast<long long>(p.M) * p.N;
    const unsigned blocks = static_cast<unsigned>((mn + 255) / 256);
    if (p.epi.kind == EPI_HEADS) splitk_reduce_kernel<EPI_HEADS><<<blocks, 256, 0, s>>>(p);
    else splitk_reduce_kernel<EPI_STORE_F32><<<blocks, 256, 0, s>>>(p);
    return hipGetLastError();
  }
#define ST_GEMM_CASE(E)                                                     \
  case E:                                                                   \
    if (op == ACT_F16) gemm_dma_kernel<E, f16_t, kBKT, kNST><<<grid, kThreads, 0, s>>>(p); \
    else gemm_dma_kernel<E, bf16_t, kBKT, kNST><<<grid, kThreads, 0, s>>>(p);           \
    break;
  switch (p.epi.kind) {
    ST_GEMM_CASE(EPI_STORE_F32)
    ST_GEMM_CASE(EPI_RESID_F32)
    ST_GEMM_CASE(EPI_HEADS)
    ST_GEMM_CASE(EPI_GEGLU)
    ST_GEMM_CASE(EPI_NCHW)
    default:
      return hipErrorInvalidValue;
  }
#undef ST_GEMM_CASE
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
