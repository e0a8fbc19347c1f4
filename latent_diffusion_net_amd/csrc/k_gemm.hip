// GEMMs of the Spatial-Transformer block: C[M][N] = A[M][K] * B[N][K]^T with
// both operands K-contiguous (activations [tokens][in], weights [out][in]).
//
// 16-bit operands (bf16 or fp16) on v_mfma_f32_32x32x16 with fp32
// accumulation.  A workgroup of WM x WN wavefronts owns a tile of
// (WM*FM*32) x (WN*FN*32) outputs, each wavefront FM x FN MFMA blocks of
// 32x32: 128x128 tiles of four 64x64 wavefronts (two workgroups per CU), or
// 256x256 tiles of eight 128x64 wavefronts when the product has enough of
// them.  K advances 64 at a time through two LDS stages (three, with one
// 128x128 workgroup per CU, when the product has no more tiles than CUs)
// filled by buffer_load_dwordx4 ... lds (no staging registers), with one
// barrier per stage; the LDS operand reads of each 16-wide K step are issued while the
// MFMAs of the previous step run.  Each stage buffer is its own LDS object,
// so the compiler can tell a DMA into one stage from reads of the other and
// does not wait on it.  LDS rows are 128 bytes (64 elements, eight 16-byte
// chunks); chunk c of row r is stored at c ^ ((r >> 1) & 7), which spreads
// the 16 rows of one 16-lane read phase over all 16 bank groups of gfx950's
// 64-bank LDS.  Rows beyond M or N are clamped on load and masked on store.
//
// The store and residual epilogues keep the residual stream either in fp32
// (optionally with an fp16 copy) or, on the bf16 path, in fp16 only (h16,
// 11 significant bits, the operand of the products behind the LayerNorms
// and of proj_out), each with optional per-row sums for a folded LayerNorm.
//
// fp32 path (debug builds of the block): a plain LDS-tiled fp32 FMA GEMM with
// the same epilogues.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace stb {

namespace {

// Fewest 256x256 tiles for which the large-tile configuration is used.
constexpr int kBigTileMin = 192;
// Fewest 256x256 tiles for a product that they cover without padding.
constexpr int kBigTileExact = 128;
// Shallowest product (K) that takes 256x256 tiles.
constexpr int kBigTileMinK = 640;

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

// Sum over the 8 lanes of half a DPP row; each of them gets the sum.
__device__ __forceinline__ float row8_sum(float v) {
  v += dpp_f32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141, 0xF>(v);  // row_half_mirror
  return v;
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_f32<0x140, 0xF>(v);  // row_mirror
  return v;
}

// rstd * a - mean * rstd * g for four columns of one row (k = (rstd, mean * rstd)).
__device__ __forceinline__ float4 ln_fix(float4 a, float2 k, float4 g) {
  return make_float4(fmaf(a.x, k.x, -k.y * g.x), fmaf(a.y, k.x, -k.y * g.y),
                     fmaf(a.z, k.x, -k.y * g.z), fmaf(a.w, k.x, -k.y * g.w));
}

// Key order of a 32-key block of the fused cross-attention: row r of the K
// operand holds key kperm(r) (bits 2 and 3 of r swapped), so that the eight
// scores the accumulator layout gives one lane for one P.V step are eight
// consecutive keys, the keys of one 16-byte V^T operand.
__device__ __forceinline__ int kperm(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Staging of Q in the cross-attention epilogue: the 16-byte chunk k of row r
// is stored at chunk k ^ g(r), g(r) = r mod 16 with bits 2 and 3 swapped.
// The read-back gives each lane its own row (16 consecutive rows per
// 16-lane read phase, one chunk each: 16 distinct chunks, all 64 banks);
// the accumulator stores write rows r and r + 4 (bit 2 of r differs, so
// bit 3 of g differs) into disjoint halves of the banks.
__device__ __forceinline__ int qstg(int row, int col) {
  const int g = (row & 3) | ((row & 8) >> 1) | ((row & 4) << 1);
  return row * 64 + ((((col >> 2) ^ g) << 2) | (col & 3));
}

// EPI_CROSS_ATTN for one 64x64 block (64 queries of one sample, one head):
// Q = (acc [LayerNorm-corrected] + bias) * scale is staged in LDS and read
// back as bf16 B operands; for each 32-query half, S^T = K Q^T over three
// 32-key blocks (keys >= nk masked), an exact one-pass softmax in base 2,
// O^T = V^T P^T over six 16-key steps, O normalised and stored as bf16.  The
// K and V^T operands come straight from memory (L2: 24 KB per sample and
// head), requested before the staging.
template <bool LN>
__device__ __forceinline__ void cross_attn_block(const GemmParams& p, const floatx16 (&acc)[2][2],
                                                 int R0, int C0, int lane, float* stage,
                                                 const float2* ln_rows, const float* ln_cols) {
  const int l32 = lane & 31, lhi = lane >> 5;
  const CrossAttn& ca = p.epi.ca;
  if (R0 >= p.M || C0 >= p.N) return;
  const int sample = R0 / ca.rows_per_batch;
  const long long bh = static_cast<long long>(sample) * ca.heads + (C0 >> 6);
  // key padding mask of this sample (all keys below nk when there is none)
  uint4 kbits = make_uint4(~0u, ~0u, ~0u, 0u);
  if (ca.key_bits) kbits = *reinterpret_cast<const uint4*>(ca.key_bits + 4LL * sample);
  const uint32_t kbw[3] = {kbits.x, kbits.y, kbits.z};
  const uint16_t* Kh = static_cast<const uint16_t*>(ca.k) + bh * ca.kv_pad * kHeadDim;
  const uint16_t* Vh = static_cast<const uint16_t*>(ca.vt) + bh * kHeadDim * ca.kv_pad;
  uint4 kop[3][4], vop[2][6];
#pragma unroll
  for (int kb = 0; kb < 3; ++kb)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      kop[kb][s4] = *reinterpret_cast<const uint4*>(Kh + (kb * 32 + kperm(l32)) * kHeadDim + 16 * s4 + 8 * lhi);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int st = 0; st < 6; ++st)
      vop[db][st] = *reinterpret_cast<const uint4*>(
          Vh + static_cast<long long>(db * 32 + l32) * ca.kv_pad + 16 * st + 8 * lhi);
  float bj[2], gj[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bj[j] = p.epi.bias ? p.epi.bias[C0 + j * 32 + l32] : 0.f;
    if constexpr (LN) gj[j] = ln_cols[j * 32 + l32];
  }
  // rows come in runs of four (r % 4): their (rstd, mean * rstd) pairs are
  // read as two 16-byte words before the run's stores
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int lr0 = i * 32 + 8 * g4 + 4 * lhi;
      float2 k[4] = {make_float2(1.f, 0.f), make_float2(1.f, 0.f), make_float2(1.f, 0.f),
                     make_float2(1.f, 0.f)};
      if constexpr (LN) {
        const float4 u = *reinterpret_cast<const float4*>(ln_rows + lr0);
        const float4 w = *reinterpret_cast<const float4*>(ln_rows + lr0 + 2);
        k[0] = make_float2(u.x, u.y); k[1] = make_float2(u.z, u.w);
        k[2] = make_float2(w.x, w.y); k[3] = make_float2(w.z, w.w);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 4 * g4 + jj;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float v = acc[i][j][r];
          if constexpr (LN) v = fmaf(v, k[jj].x, -k[jj].y * gj[j]);
          stage[qstg(lr0 + jj, j * 32 + l32)] = (v + bj[j]) * ca.scale;
        }
      }
    }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (63 & 15) | ((63 >> 4) << 14));  // lgkmcnt(0)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int lr = qb * 32 + l32;  // this lane's query within the block
    uint4 qop[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const float4 a = *reinterpret_cast<const float4*>(&stage[qstg(lr, 16 * s4 + 8 * lhi)]);
      const float4 c = *reinterpret_cast<const float4*>(&stage[qstg(lr, 16 * s4 + 8 * lhi + 4)]);
      qop[s4] = make_uint4(pack2bf(a.x, a.y), pack2bf(a.z, a.w), pack2bf(c.x, c.y), pack2bf(c.z, c.w));
    }
    floatx16 sc[3];
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) sc[kb] = mfma32x32x16(kop[kb][s4], qop[s4], sc[kb], bf16_t{});
    }
    // keys >= nk (nk > 64: only the third block has any) and masked keys
    // -> -inf
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 3; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = kperm(8 * (r >> 2) + 4 * lhi + (r & 3));
        if ((kb == 2 && 64 + kr >= ca.nk) || !((kbw[kb] >> kr) & 1u)) sc[kb][r] = -INFINITY;
        mx = fmaxf(mx, sc[kb][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx == -INFINITY) mx = 0.f;  // every key masked: all probabilities 0
    // P^T step st: block st / 2, entries 8 (st % 2) + 0..7 = keys 16 st + 8 lhi + 0..7;
    // steps past the last key are zero and skipped
    const int nsteps = (ca.nk + 15) >> 4;
    // row sum of the fp32 exponentials in four independent chains (as the
    // self-attention kernel does)
    uint4 pb[6];
    float pa[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 6; ++st) {
      if (st >= nsteps) {
        pb[st] = make_uint4(0u, 0u, 0u, 0u);
        continue;
      }
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float e0 = __builtin_amdgcn_exp2f(sc[st >> 1][8 * (st & 1) + 2 * jj] - mx);
        const float e1 = __builtin_amdgcn_exp2f(sc[st >> 1][8 * (st & 1) + 2 * jj + 1] - mx);
        bf16x2 pk;
        pk[0] = static_cast<__bf16>(e0);
        pk[1] = static_cast<__bf16>(e1);
        pa[(2 * jj) & 3] += e0;
        pa[(2 * jj + 1) & 3] += e1;
        w[jj] = __builtin_bit_cast(uint32_t, pk);
      }
      pb[st] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    const float ps = (pa[0] + pa[1]) + (pa[2] + pa[3]);
    const float ptot = ps + __shfl_xor(ps, 32, 64);
    const float inv = ptot > 0.f ? 1.0f / ptot : 0.f;  // no key: O = 0
    floatx16 o[2];
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
#pragma unroll
      for (int st = 0; st < 6; ++st)
        if (st < nsteps) o[db] = mfma32x32x16(vop[db][st], pb[st], o[db], bf16_t{});
    }
    // O^T: this lane holds query lr, dims db*32 + 8g + 4lhi + 0..3
    const int row = R0 + lr;
    if (row < p.M) {
      uint16_t* orow = static_cast<uint16_t*>(p.epi.out_act) + static_cast<long long>(row) * p.epi.ldo + C0;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(orow + db * 32 + 8 * g + 4 * lhi) =
              make_uint2(pack2bf(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                         pack2bf(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
    }
  }
}

// PF (EPI_RESID_H16): the residual values of this lane's 8 rows x 8 columns
// arrive in resv (read from LDS after the main loop) instead of from memory.
// Folded LayerNorm (LN: EPI_HEADS, EPI_GEGLU and EPI_CROSS_ATTN only):
// ln_rows (LDS) holds (rstd, mean * rstd) for the 64 rows of this block and
// ln_cols (LDS) the folded weights' sums for its 64 columns; each value read
// back from the staging tile becomes rstd * acc - mean * rstd * g.
template <int EPI, bool LN, bool PF = false>
__device__ __forceinline__ void epilogue_lds(const GemmParams& p,
                                             const floatx16 (&acc)[2][2],
                                             int m0, int n0, int wm, int wn,
                                             int lane, float* stage,
                                             const float2* ln_rows, const float* ln_cols,
                                             const uint4 (&resv)[8]) {
  static_assert(!LN || EPI == EPI_HEADS || EPI == EPI_GEGLU || EPI == EPI_CROSS_ATTN,
                "folded LayerNorm kinds");
  if constexpr (EPI == EPI_CROSS_ATTN) {
    cross_attn_block<LN>(p, acc, m0 + wm * 64, n0 + wn * 64, lane, stage, ln_rows, ln_cols);
    return;
  }
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

  if constexpr (EPI == EPI_STORE_H16 || EPI == EPI_RESID_H16) {
    // The stream is kept in fp16: lane -> 8 consecutive columns of one row
    // (one 16-byte store), 8 rows per pass; the row sums use the stored
    // (rounded) values.
    constexpr bool kRes = EPI == EPI_RESID_H16;
    const int lc = (lane & 7) * 8;
    float bias[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) bias[k] = 0.f;
    if (p.epi.bias) {
      const float4 b0 = *reinterpret_cast<const float4*>(p.epi.bias + C0 + lc);
      const float4 b1 = *reinterpret_cast<const float4*>(p.epi.bias + C0 + lc + 4);
      bias[0] = b0.x; bias[1] = b0.y; bias[2] = b0.z; bias[3] = b0.w;
      bias[4] = b1.x; bias[5] = b1.y; bias[6] = b1.z; bias[7] = b1.w;
    }
    f16_t* h16 = static_cast<f16_t*>(p.epi.out_act);
    bool bad = false;  // a stored value is not finite
    // all residual rows are loaded before the first store (the compiler
    // cannot prove a store to h disjoint from the next row's load)
    uint4 hin[8];
    if constexpr (kRes) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = R0 + it * 8 + (lane >> 3);
        if constexpr (PF) {
          hin[it] = resv[it];  // prefetched during the last stage
        } else {
          hin[it] = row < M ? *reinterpret_cast<const uint4*>(h16 + static_cast<long long>(row) * p.epi.ldo + C0 + lc)
                            : make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int lr = it * 8 + (lane >> 3);
      const int row = R0 + lr;
      if (row >= M) break;
      const float4 c0 = *reinterpret_cast<const float4*>(&stage[stg(lr, lc)]);
      const float4 c1 = *reinterpret_cast<const float4*>(&stage[stg(lr, lc + 4)]);
      float v[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += bias[k];
      if constexpr (kRes) {
        const uint32_t hw[4] = {hin[it].x, hin[it].y, hin[it].z, hin[it].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f16x2 h2 = __builtin_bit_cast(f16x2, hw[k]);
          v[2 * k] += static_cast<float>(h2[0]);
          v[2 * k + 1] += static_cast<float>(h2[1]);
        }
      }
      const uint4 w = make_uint4(pack2h(v[0], v[1]), pack2h(v[2], v[3]), pack2h(v[4], v[5]),
                                 pack2h(v[6], v[7]));
      *reinterpret_cast<uint4*>(h16 + static_cast<long long>(row) * p.epi.ldo + C0 + lc) = w;
      bad |= f16x8_nonfinite(w);
      if (p.epi.row_stats) {
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f16x2 h2 = __builtin_bit_cast(f16x2, ww[k]);
          v[2 * k] = static_cast<float>(h2[0]);
          v[2 * k + 1] = static_cast<float>(h2[1]);
        }
        // the row's 64 values sit in 8 lanes (half a DPP row)
        const float sum = row8_sum(((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])));
        const float mb = sum * (1.0f / 64.0f);
        float q = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) q = fmaf(v[k] - mb, v[k] - mb, q);
        const float m2 = row8_sum(q);
        if ((lane & 7) == 0)
          p.epi.row_stats[static_cast<long long>(row) * (p.epi.ldo >> 6) + (C0 >> 6)] = make_float2(sum, m2);
      }
    }
    if (bad && p.epi.range_flag) *p.epi.range_flag = 1;
  } else if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_RESID_F32) {
    constexpr bool kRes = EPI == EPI_RESID_F32;
    // lane -> 4 consecutive columns of one row; 4 rows per pass
    const int lc = (lane & 15) * 4;
    const float4 bias = p.epi.bias ? *reinterpret_cast<const float4*>(p.epi.bias + C0 + lc)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
    f16_t* h16 = static_cast<f16_t*>(p.epi.out_act);
    // all 16 residual rows are loaded before the first store (the compiler
    // cannot prove a store to h disjoint from the next row's load)
    float4 hin[16];
    if constexpr (kRes) {
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int row = R0 + it * 4 + (lane >> 4);
        const long long off = static_cast<long long>(row) * p.epi.ldo + C0 + lc;
        hin[it] = row < M ? *reinterpret_cast<const float4*>(p.epi.out_f32 + off)
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
      if constexpr (kRes) {
        v.x += hin[it].x; v.y += hin[it].y; v.z += hin[it].z; v.w += hin[it].w;
      }
      const long long off = static_cast<long long>(row) * p.epi.ldo + C0 + lc;
      *reinterpret_cast<float4*>(p.epi.out_f32 + off) = v;
      if (h16) {
        // the new values also as fp16 [M][ldo] (the operand of the next
        // product)
        *reinterpret_cast<uint2*>(h16 + off) = make_uint2(pack2h(v.x, v.y), pack2h(v.z, v.w));
      }
      if (p.epi.row_stats) {
        // the row's 64 values sit in the 16 lanes of one DPP row
        const float sum = row16_sum((v.x + v.y) + (v.z + v.w));
        const float mb = sum * (1.0f / 64.0f);
        const float dx = v.x - mb, dy = v.y - mb, dz = v.z - mb, dw = v.w - mb;
        const float m2 = row16_sum((dx * dx + dy * dy) + (dz * dz + dw * dw));
        if ((lane & 15) == 0)
          p.epi.row_stats[static_cast<long long>(row) * (p.epi.ldo >> 6) + (C0 >> 6)] = make_float2(sum, m2);
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
    float4 lgv = make_float4(0.f, 0.f, 0.f, 0.f), lgg = lgv;
    if constexpr (LN) {
      lgv = *reinterpret_cast<const float4*>(ln_cols + lc);
      lgg = *reinterpret_cast<const float4*>(ln_cols + 32 + lc);
    }
    bool bad = false;  // a stored value is not finite
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
      const int lr = it * 8 + (lane >> 3);
      const int row = R0 + lr;
      if (row >= M) break;
      float4 v = *reinterpret_cast<const float4*>(&stage[stg(lr, lc)]);
      float4 g = *reinterpret_cast<const float4*>(&stage[stg(lr, 32 + lc)]);
      if constexpr (LN) {
        const float2 k = ln_rows[lr];
        v = ln_fix(v, k, lgv);
        g = ln_fix(g, k, lgg);
      }
      const uint2 pk = make_uint2(
          pack2h((v.x + bv[0]) * gelu_as(g.x + bg[0]), (v.y + bv[1]) * gelu_as(g.y + bg[1])),
          pack2h((v.z + bv[2]) * gelu_as(g.z + bg[2]), (v.w + bv[3]) * gelu_as(g.w + bg[3])));
      *reinterpret_cast<uint2*>(out + static_cast<long long>(row) * F + fc0 + lc) = pk;
      bad |= (static_cast<int>(f16_pair_nonfinite(pk.x)) | static_cast<int>(f16_pair_nonfinite(pk.y))) != 0;
    }
    if (bad && p.epi.range_flag) *p.epi.range_flag = 1;
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
    const float sc = hs.scale[sp];
    if (!((hs.transposed_mask >> sp) & 1)) {
      // [bh][n][64]: lane -> 8 consecutive dims of one token (one 16-byte
      // store), 8 tokens per pass
      const int lc = (lane & 7) * 8;
      float bb[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) bb[k] = bias ? bias[lc + k] : 0.f;
      float4 lg[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
      if constexpr (LN) {
        lg[0] = *reinterpret_cast<const float4*>(ln_cols + lc);
        lg[1] = *reinterpret_cast<const float4*>(ln_cols + lc + 4);
      }
#pragma unroll 2
      for (int it = 0; it < 8; ++it) {
        const int lr = it * 8 + (lane >> 3);
        const int row = R0 + lr;
        if (row >= M) break;
        const int b = row / hs.rows_per_batch;
        const int n = row - b * hs.rows_per_batch;
        float4 c0 = *reinterpret_cast<const float4*>(&stage[stg(lr, lc)]);
        float4 c1 = *reinterpret_cast<const float4*>(&stage[stg(lr, lc + 4)]);
        if constexpr (LN) {
          const float2 k = ln_rows[lr];
          c0 = ln_fix(c0, k, lg[0]);
          c1 = ln_fix(c1, k, lg[1]);
        }
        const uint4 pk = make_uint4(pack2bf((c0.x + bb[0]) * sc, (c0.y + bb[1]) * sc),
                                    pack2bf((c0.z + bb[2]) * sc, (c0.w + bb[3]) * sc),
                                    pack2bf((c1.x + bb[4]) * sc, (c1.y + bb[5]) * sc),
                                    pack2bf((c1.z + bb[6]) * sc, (c1.w + bb[7]) * sc));
        const long long bh = static_cast<long long>(b) * hs.heads + head;
        *reinterpret_cast<uint4*>(base + (bh * hs.npad + n) * kHeadDim + lc) = pk;
      }
    } else {
      // V^T [bh][64][npad]: lane -> one dim, 8 consecutive tokens (one
      // 16-byte store)
      const int dim = lane;
      const float bb = bias ? bias[dim] : 0.f;
      float lg = 0.f;
      if constexpr (LN) lg = ln_cols[dim];
      const bool vec = (hs.rows_per_batch & 7) == 0;
#pragma unroll 1
      for (int it = 0; it < 8; ++it) {
        const int lr0 = it * 8;
        const int row0 = R0 + lr0;
        if (row0 >= M) break;
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float a = stage[stg(lr0 + k, dim)];
          if constexpr (LN) {
            const float2 kk = ln_rows[lr0 + k];
            a = fmaf(a, kk.x, -kk.y * lg);
          }
          v[k] = (a + bb) * sc;
        }
        if (vec && row0 + 7 < M) {
          const int b = row0 / hs.rows_per_batch;
          const int n = row0 - b * hs.rows_per_batch;
          const long long bh = static_cast<long long>(b) * hs.heads + head;
          *reinterpret_cast<uint4*>(base + (bh * kHeadDim + dim) * hs.npad + n) =
              make_uint4(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]), pack2bf(v[4], v[5]),
                         pack2bf(v[6], v[7]));
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
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
  } else if constexpr (EPI == EPI_CONV) {
    // rows = output channels, columns = output pixels m of the padded grid
    // (m = (b * Hq + i) * Wp + j; valid when i < Ho and j < Wo): y[b][c][i][j]
    // = acc + cadd[b][c] (+ resid[b][c][i][j]); lane -> 4 consecutive pixels
    // of one channel, 16 channels per pass.  Wp % 4 == 0 and Wo % 4 == 0
    // keep a group of four in one row, all valid or all padding.
    const ConvGemm& cv = p.conv;
    const int lc = (lane & 15) * 4;
    const int m0 = C0 + lc;
    const int per_b = cv.Hq * cv.Wp;
    const int b = m0 / per_b;
    const int rem = m0 - b * per_b;
    const int i = rem / cv.Wp;
    const int j = rem - i * cv.Wp;
    if (m0 >= N || i >= cv.Ho || j >= cv.Wo) return;
    const long long plane = static_cast<long long>(cv.Ho) * cv.Wo;
    const long long pix = static_cast<long long>(i) * cv.Wo + j;
    const bf16_t* rin = static_cast<const bf16_t*>(cv.resid);
    bf16_t* yout = static_cast<bf16_t*>(cv.out);
    uint2 rv[16];
    if (rin) {
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int c = R0 + it * 4 + (lane >> 4);
        rv[it] = c < M ? *reinterpret_cast<const uint2*>(rin + (static_cast<long long>(b) * M + c) * plane + pix)
                       : make_uint2(0u, 0u);
      }
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int lr = it * 4 + (lane >> 4);
      const int c = R0 + lr;
      if (c >= M) break;
      const float add = cv.cadd[static_cast<long long>(b) * M + c];
      const float4 a = *reinterpret_cast<const float4*>(&stage[stg(lr, lc)]);
      float y0 = a.x + add, y1 = a.y + add, y2 = a.z + add, y3 = a.w + add;
      if (rin) {
        y0 += __uint_as_float(rv[it].x << 16);
        y1 += __uint_as_float(rv[it].x & 0xffff0000u);
        y2 += __uint_as_float(rv[it].y << 16);
        y3 += __uint_as_float(rv[it].y & 0xffff0000u);
      }
      *reinterpret_cast<uint2*>(yout + (static_cast<long long>(b) * M + c) * plane + pix) =
          make_uint2(pack2bf(y0, y1), pack2bf(y2, y3));
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

// Offset (in elements) of 16-byte chunk `chunk` of stage row `row`: rows of
// 64 elements, chunk c of row r at c ^ ((r >> 1) & 7), so that the 16 rows
// of one 16-lane read phase cover all 16 bank groups of the 64-bank LDS.
__device__ __forceinline__ int swz_k(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// buffer_load_dwordx4 ... lds: 64 lanes x 16 bytes from `base` + soff + voff
// into the 1 KB of LDS at `lds`, lane i landing in slot i.  Unlike
// global_load_lds (a FLAT instruction, which the compiler must assume may
// also be an LDS access), a buffer load leaves the LDS wait counter alone,
// so the waits for LDS operand reads can stay partial.
__device__ __forceinline__ void dma16(const void* base, int nbytes, uint16_t* lds,
                                      unsigned voff, int soff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// ------------------------------------------------------ DMA-ring GEMM
// WM x WN wavefronts, each owning (FM*32) x (FN*32) outputs as FM x FN MFMA
// blocks; MINB workgroups per CU.  Stage k: wait for its DMA, barrier (every
// wavefront is done with stage k-1), issue the DMA of stage k+1 into the
// other buffers, then the four 16-wide K steps, the LDS operand reads of
// step s+1 issued before the MFMAs of step s (two register sets; the
// scheduling groups keep the compiler from folding them back into one).
template <int EPI, typename OpT, int WM, int WN, int FM, int FN, int MINB, bool LN, int NST>
__global__ __launch_bounds__(64 * WM * WN, MINB) void gemm_pipe_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int TBM = WM * FM * 32, TBN = WN * FN * 32;
  constexpr int BKT = 64;
  constexpr int RPB = 8;                 // rows per 1 KB DMA block
  constexpr int DPA = TBM / RPB / NW;    // A blocks per wavefront per stage
  constexpr int DPB = TBN / RPB / NW;    // B blocks per wavefront per stage
  static_assert(DPA * RPB * NW == TBM && DPB * RPB * NW == TBN, "DMA split");
  static_assert(FM % 2 == 0 && FN % 2 == 0, "epilogue works on 64x64 blocks");
  static_assert(NST * (TBM + TBN) * BKT * 2 >= NW * 16384, "epilogue staging");
  static_assert(NST == 2 || NST == 3, "two or three stages");
  // NST stage buffers per operand, each its own LDS object
  constexpr int kXA2 = NST == 3 ? TBM * BKT : 8, kXB2 = NST == 3 ? TBN * BKT : 8;
  __shared__ __attribute__((aligned(16))) uint16_t sA0[TBM * BKT];
  __shared__ __attribute__((aligned(16))) uint16_t sA1[TBM * BKT];
  __shared__ __attribute__((aligned(16))) uint16_t sA2[kXA2];
  __shared__ __attribute__((aligned(16))) uint16_t sB0[TBN * BKT];
  __shared__ __attribute__((aligned(16))) uint16_t sB1[TBN * BKT];
  __shared__ __attribute__((aligned(16))) uint16_t sB2[kXB2];
  // folded LayerNorm: (rstd, mean * rstd) per row and g per column
  __shared__ __attribute__((aligned(16))) float2 ln_tab[LN ? TBM : 2];
  __shared__ __attribute__((aligned(16))) float ln_gtab[LN ? TBN : 4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  // split-K: workgroup blockIdx.x takes tile blockIdx.x % tiles and K slice
  // blockIdx.x / tiles (always 0 without split)
  const int mt = (p.M + TBM - 1) / TBM, nt = (p.N - p.n_off + TBN - 1) / TBN;
  const int kz = blockIdx.x / (mt * nt);
  const int kslice = p.K / (p.ksplit > 1 ? p.ksplit : 1);
  int tm, tn;
  tile_coords(mt, nt, blockIdx.x - kz * mt * nt, tm, tn);
  const int m0 = tm * TBM;
  const int n0 = p.n_off + tn * TBN;
  const int M = p.M, N = p.N;
  const uint16_t* A = static_cast<const uint16_t*>(p.A);
  const uint16_t* Bm = static_cast<const uint16_t*>(p.B);
  const int l32 = lane & 31, lhi = lane >> 5;

  // DMA through buffer loads: 32-bit byte offsets per lane, the K step as
  // the scalar offset (callers keep each operand below 4 GB)
  unsigned aoff[DPA], boff[DPB];
#pragma unroll
  for (int j2 = 0; j2 < DPA; ++j2) {
    const int row = RPB * (wave * DPA + j2) + (lane >> 3);
    const int cl = (lane & 7) ^ ((row >> 1) & 7);
    aoff[j2] = static_cast<unsigned>((min(m0 + row, M - 1) * p.lda + kz * kslice + cl * 8) * 2);
  }
#pragma unroll
  for (int j2 = 0; j2 < DPB; ++j2) {
    const int row = RPB * (wave * DPB + j2) + (lane >> 3);
    const int cl = (lane & 7) ^ ((row >> 1) & 7);
    // a convolution's B operand takes its K position from the tap offsets
    const int bk0 = EPI == EPI_CONV ? 0 : kz * kslice;
    boff[j2] = static_cast<unsigned>((min(n0 + row, N - 1) * p.ldb + bk0 + cl * 8) * 2);
  }
  const int abytes = M * static_cast<int>(p.lda) * 2;
  const int bbytes = EPI == EPI_CONV ? static_cast<int>(p.conv.b_bytes) : N * static_cast<int>(p.ldb) * 2;
  // Convolution: the byte offset of K stage k within the activation buffer,
  // tracked incrementally (every caller asks for the stages in order, one
  // at a time): tap ct = 3 di + dj at (crow, ccol), stage cj of the tap;
  // a K slice of a split product starts at stage kz * kslice / 64.
  int ct = 0, cj = 0, crow = 0, ccol = 0;
  if constexpr (EPI == EPI_CONV) {
    const int s0 = kz * kslice / BKT;
    const int taps = 9 * p.conv.spt;
    if (s0 < taps) {
      ct = s0 / p.conv.spt;
      cj = s0 - ct * p.conv.spt;
    } else {
      ct = 9;
      cj = s0 - taps;
    }
    crow = ct / 3;
    ccol = ct - crow * 3;
  }
  auto next_boff = [&](int k) -> int {
    if constexpr (EPI != EPI_CONV) {
      return k * BKT * 2;
    } else {
      const ConvGemm& cv = p.conv;
      int off;
      if (ct < 9) off = ((crow * cv.Wp + ccol) * cv.L + cj * BKT) * 2;
      else off = (cv.sc_roff * cv.L + cv.sc_cbase + cj * BKT) * 2;
      if (++cj == (ct < 9 ? cv.spt : cv.sc_spt)) {
        cj = 0;
        ++ct;
        if (++ccol == 3) { ccol = 0; ++crow; }
      }
      return off;
    }
  };
  auto issue = [&](int k, uint16_t* sa, uint16_t* sb) {
    const int bk = next_boff(k);
#pragma unroll
    for (int j2 = 0; j2 < DPA; ++j2)
      dma16(A, abytes, sa + (wave * DPA + j2) * 512, aoff[j2], k * BKT * 2);
#pragma unroll
    for (int j2 = 0; j2 < DPB; ++j2)
      dma16(Bm, bbytes, sb + (wave * DPB + j2) * 512, boff[j2], bk);
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // operands of K step s (16 wide) of a stage
  auto rd = [&](const uint16_t* sa, const uint16_t* sb, int s, uint4 (&a)[FM], uint4 (&b)[FN]) {
    const int chunk = 2 * s + lhi;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      a[i] = *reinterpret_cast<const uint4*>(sa + swz_k(wm * FM * 32 + i * 32 + l32, chunk));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      b[j] = *reinterpret_cast<const uint4*>(sb + swz_k(wn * FN * 32 + j * 32 + l32, chunk));
  };
  auto mm = [&](const uint4 (&a)[FM], const uint4 (&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j], OpT{});
  };

  const int nk = kslice / BKT;
  uint4 xa[FM], xb[FN], ya[FM], yb[FN];
  auto steps = [&](const uint16_t* ca, const uint16_t* cb) {
    rd(ca, cb, 0, xa, xb);
    rd(ca, cb, 1, ya, yb);
    mm(xa, xb);
    rd(ca, cb, 2, xa, xb);
    mm(ya, yb);
    rd(ca, cb, 3, ya, yb);
    mm(xa, xb);
    mm(ya, yb);
    // keep the order: reads of step s+1 ahead of the MFMAs of step s
    constexpr int R = FM + FN, F = FM * FN;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * R, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, F, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, F, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * F, 0);
  };
  // Folded LayerNorm: the folded weights' column sums of the tile, and per
  // row (rstd, mean * rstd) from the 64-column blocks' sums s_k and squared
  // deviations d_k, in fp64: mean = sum s_k / K, var = sum (d_k + s_k^2 /
  // 64) / K - mean^2.  Two threads per row take alternate blocks.  The loads
  // are issued before the first stage's DMA and used after it, so that no
  // wait for them also waits for the DMA (the counter is in order).
  constexpr int kLnRegs = 10;  // blocks per thread held in registers (K <= 1280)
  float2 lnv[kLnRegs];
  float ln_gv = 0.f;
  double ln_sum = 0.0, ln_sq = 0.0, ln_inv_k = 0.0;
  if constexpr (LN) {
    static_assert(2 * TBM == 64 * NW && TBN <= 64 * NW, "two threads per row, one per column");
    const int t = threadIdx.x, half = t & 1;
    ln_gv = p.epi.ln_g[min(n0 + t % TBN, N - 1)];
    const float2* st = p.epi.ln_stats + static_cast<long long>(min(m0 + (t >> 1), M - 1)) * p.epi.ln_blocks;
#pragma unroll
    for (int i = 0; i < kLnRegs; ++i) lnv[i] = make_float2(0.f, 0.f);
    auto load = [&](auto nb_c) {
      constexpr int NB = decltype(nb_c)::value;
      static_assert((NB + 1) / 2 <= kLnRegs, "registers");
      ln_inv_k = 1.0 / (64.0 * NB);
#pragma unroll
      for (int i = 0; i < (NB + 1) / 2; ++i) {
        const float2 x = st[min(2 * i + half, NB - 1)];
        lnv[i] = (NB % 2 == 0 || 2 * i + half < NB) ? x : make_float2(0.f, 0.f);
      }
    };
    switch (p.epi.ln_blocks) {
      case 5: load(std::integral_constant<int, 5>{}); break;
      case 10: load(std::integral_constant<int, 10>{}); break;
      case 20: load(std::integral_constant<int, 20>{}); break;
      default:
        ln_inv_k = 1.0 / (64.0 * p.epi.ln_blocks);
        for (int kb = half; kb < p.epi.ln_blocks; kb += 2) {
          const float2 v = st[kb];
          ln_sum += v.x;
          ln_sq += static_cast<double>(v.y) + static_cast<double>(v.x) * v.x * (1.0 / 64.0);
        }
    }
  }
  // Three-stage ring (NST == 3): every stage issues one DMA, unconditionally
  // (past the last stage with an empty buffer range, which fetches nothing
  // and zeroes buffers no later stage reads), so that every wait is the same
  // partial count and no branch separates a DMA from the reads after it.
  auto issue_at = [&](int k, bool valid, uint16_t* sa, uint16_t* sb) {
    const int bk = next_boff(k);
    const int ab = valid ? abytes : 0, bb = valid ? bbytes : 0, so = valid ? k * BKT * 2 : 0;
    const int sob = valid ? bk : 0;
#pragma unroll
    for (int j2 = 0; j2 < DPA; ++j2) dma16(A, ab, sa + (wave * DPA + j2) * 512, aoff[j2], so);
#pragma unroll
    for (int j2 = 0; j2 < DPB; ++j2) dma16(Bm, bb, sb + (wave * DPB + j2) * 512, boff[j2], sob);
  };
  issue(0, sA0, sB0);
  if constexpr (NST == 3) issue_at(1, nk > 1, sA1, sB1);
  if constexpr (LN) {
    // the sums stay below the DMA issue (the empty statements take the
    // loaded values after it)
#pragma unroll
    for (int i = 0; i < kLnRegs; ++i) asm volatile("" : "+v"(lnv[i].x), "+v"(lnv[i].y)::"memory");
    asm volatile("" : "+v"(ln_gv)::"memory");
    const int t = threadIdx.x, half = t & 1;
    ln_gtab[t % TBN] = ln_gv;
#pragma unroll
    for (int i = 0; i < kLnRegs; ++i) {
      ln_sum += lnv[i].x;
      ln_sq += static_cast<double>(lnv[i].y) + static_cast<double>(lnv[i].x) * lnv[i].x * (1.0 / 64.0);
    }
    ln_sum += __shfl_xor(ln_sum, 1, 64);
    ln_sq += __shfl_xor(ln_sq, 1, 64);
    const double mean = ln_sum * ln_inv_k;
    const float var = static_cast<float>(fmax(ln_sq * ln_inv_k - mean * mean, 0.0));
    const float rstd = rsqrtf(var + p.epi.ln_eps);
    if (!half) ln_tab[t >> 1] = make_float2(rstd, static_cast<float>(mean) * rstd);
  }
  // Residual prefetch (EPI_RESID_H16, 128x128 tiles): at the top of the
  // last stage, the stage buffers that stage does not read (32 KB: one
  // 128x128 fp16 tile, rows 0-63 in the A buffer and 64-127 in the B
  // buffer) receive the tile's residual values by LDS DMA (rows past M read
  // as zero), which land while the last stage computes; each wavefront then
  // takes its 64x64 part into registers before the buffers hold the
  // epilogue tiles.
  constexpr bool kPF = EPI == EPI_RESID_H16 && WM == 2 && WN == 2 && FM == 2 && FN == 2 && NST == 2;
  auto issue_res = [&](uint16_t* wa, uint16_t* wb) {
    const long long lim = static_cast<long long>(M) * p.epi.ldo * 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = wave * 8 + j;  // rows 4 blk .. 4 blk + 3, 16 lanes per row
      const long long off = (static_cast<long long>(m0 + 4 * blk + (lane >> 4)) * p.epi.ldo + n0 +
                             (lane & 15) * 8) * 2;
      dma16(p.epi.out_act, static_cast<int>(lim), blk < 16 ? wa + blk * 512 : wb + (blk - 16) * 512,
            static_cast<unsigned>(off < lim ? off : lim), 0);
    }
  };
  auto stage = [&](int k, const uint16_t* ca, const uint16_t* cb, uint16_t* wa, uint16_t* wb) {
    wait_vmcnt_lds<0>();
    stage_barrier();
    if (k + 1 < nk) issue(k + 1, wa, wb);
    else if (kPF && p.ksplit <= 1) issue_res(wa, wb);
    steps(ca, cb);
  };
  // Stage k of the three-stage ring waits until its own DMA has landed (the
  // one issued after it may still be in flight), and after the barrier
  // refills the buffers that stage k-1 read with stage k+2.
  constexpr int kPer = DPA + DPB;  // DMA instructions per wavefront per stage
  // The three-stage ring issues its DMA spread over the stage's MFMA
  // groups (a quarter after each) instead of all before them.
  // (bk: the B offset of stage k, from next_boff, called once per stage)
  auto dma_one = [&](int j, int k, int bk, bool valid, uint16_t* sa, uint16_t* sb) {
    if (j < DPA) {
      const int ab = valid ? abytes : 0, so = valid ? k * BKT * 2 : 0;
      dma16(A, ab, sa + (wave * DPA + j) * 512, aoff[j], so);
    } else {
      const int bb = valid ? bbytes : 0, sob = valid ? bk : 0;
      dma16(Bm, bb, sb + (wave * DPB + j - DPA) * 512, boff[j - DPA], sob);
    }
  };
  auto steps_dma = [&](const uint16_t* ca, const uint16_t* cb, int k2, bool valid, uint16_t* wa, uint16_t* wb) {
    constexpr int Q = (DPA + DPB) / 4;
    static_assert(4 * Q == DPA + DPB, "DMA quarters");
    const int bk = next_boff(k2);
    rd(ca, cb, 0, xa, xb);
    rd(ca, cb, 1, ya, yb);
#pragma unroll
    for (int j = 0; j < Q; ++j) dma_one(j, k2, bk, valid, wa, wb);
    mm(xa, xb);
    rd(ca, cb, 2, xa, xb);
#pragma unroll
    for (int j = Q; j < 2 * Q; ++j) dma_one(j, k2, bk, valid, wa, wb);
    mm(ya, yb);
    rd(ca, cb, 3, ya, yb);
#pragma unroll
    for (int j = 2 * Q; j < 3 * Q; ++j) dma_one(j, k2, bk, valid, wa, wb);
    mm(xa, xb);
#pragma unroll
    for (int j = 3 * Q; j < 4 * Q; ++j) dma_one(j, k2, bk, valid, wa, wb);
    mm(ya, yb);
    constexpr int R = FM + FN, F = FM * FN;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * R, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, Q, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, F, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, Q, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, F, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, Q, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, F, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, Q, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, F, 0);
  };
  auto stage3 = [&](int k, const uint16_t* ca, const uint16_t* cb, uint16_t* wa, uint16_t* wb) {
    wait_vmcnt_lds<kPer>();
    stage_barrier();
    steps_dma(ca, cb, k + 2, k + 2 < nk, wa, wb);
  };
  if constexpr (NST == 2 && (WM != 2 || WN != 2)) {
    // 256x256 tiles: the next stage's DMA at the top of each stage (spread
    // over the MFMA groups, the stores-only epilogues of these tiles spill)
    for (int k = 0; k < nk; k += 2) {
      stage(k, sA0, sB0, sA1, sB1);
      if (k + 1 < nk) stage(k + 1, sA1, sB1, sA0, sB0);
    }
  } else if constexpr (NST == 2) {
    // every stage but the last issues the next one's DMA spread over its
    // MFMA groups; the last issues the residual prefetch (or nothing)
    auto stage_mid = [&](int k, const uint16_t* ca, const uint16_t* cb, uint16_t* wa, uint16_t* wb) {
      wait_vmcnt_lds<0>();
      stage_barrier();
      steps_dma(ca, cb, k + 1, true, wa, wb);
    };
    int k = 0;
    for (; k + 2 < nk; k += 2) {
      stage_mid(k, sA0, sB0, sA1, sB1);
      stage_mid(k + 1, sA1, sB1, sA0, sB0);
    }
    if (nk - k == 2) {
      stage_mid(k, sA0, sB0, sA1, sB1);
      stage(k + 1, sA1, sB1, sA0, sB0);
    } else {
      stage(k, sA0, sB0, sA1, sB1);
    }
  } else if constexpr (NST == 3) {
    int k = 0;
    for (; k + 3 <= nk; k += 3) {
      stage3(k, sA0, sB0, sA2, sB2);
      stage3(k + 1, sA1, sB1, sA0, sB0);
      stage3(k + 2, sA2, sB2, sA1, sB1);
    }
    const int rem = nk - k;
    if (rem > 0) stage3(k, sA0, sB0, sA2, sB2);
    if (rem > 1) stage3(k + 1, sA1, sB1, sA0, sB0);
    wait_vmcnt_lds<0>();  // the empty DMAs past the last stage
  }

  uint4 resv[8];
  uint16_t* ra = ((nk - 1) & 1) ? sA0 : sA1;
  uint16_t* rb = ((nk - 1) & 1) ? sB0 : sB1;
  if constexpr (kPF) wait_vmcnt_lds<0>();  // the residual tile has landed

  // every wavefront is done reading the stage buffers before they hold
  // the epilogue tiles
  stage_barrier();
  if constexpr (kPF) {
    const uint16_t* rt = (wm ? rb : ra) + wn * 64 + (lane & 7) * 8;
#pragma unroll
    for (int it = 0; it < 8; ++it)
      resv[it] = *reinterpret_cast<const uint4*>(rt + (it * 8 + (lane >> 3)) * 128);
    stage_barrier();
  }
  // 16 KB per wavefront: the stage buffers taken in order
  float* stg_area;
  {
    // wavefront areas in buffer order: sA0, sA1, (sA2,) sB0, sB1, (sB2)
    constexpr int PA = TBM * BKT * 2 / 16384;  // wavefront areas per A buffer
    constexpr int PB = TBN * BKT * 2 / 16384;
    constexpr int PA2 = NST == 3 ? PA : 0, PB2 = NST == 3 ? PB : 0;
    int w = wave;
    if (w < PA) stg_area = reinterpret_cast<float*>(sA0) + w * 4096;
    else if ((w -= PA) < PA) stg_area = reinterpret_cast<float*>(sA1) + w * 4096;
    else if ((w -= PA) < PA2) stg_area = reinterpret_cast<float*>(sA2) + w * 4096;
    else if ((w -= PA2) < PB) stg_area = reinterpret_cast<float*>(sB0) + w * 4096;
    else if ((w -= PB) < PB) stg_area = reinterpret_cast<float*>(sB1) + w * 4096;
    else stg_area = reinterpret_cast<float*>(sB2) + (w - PB) * 4096;
    static_assert(2 * PA + PA2 + 2 * PB + PB2 >= NW, "epilogue areas");
  }
  GemmParams q = p;
  if (p.ksplit > 1) {
    // this slice's product, plain fp32, into ws[kz]
    q.epi.kind = EPI_STORE_F32;
    q.epi.bias = nullptr;
    // slices of rows ldws = N rounded up to 64 (whole 64-wide column blocks)
    const int ldws = (N + 63) & ~63;
    q.epi.out_f32 = p.ws + static_cast<long long>(kz) * M * ldws;
    q.epi.ldo = ldws;
    q.epi.out_act = nullptr;
    q.epi.row_stats = nullptr;
  }
#pragma unroll
  for (int si = 0; si < FM / 2; ++si)
#pragma unroll
    for (int sj = 0; sj < FN / 2; ++sj) {
      const floatx16 sub[2][2] = {{acc[2 * si][2 * sj], acc[2 * si][2 * sj + 1]},
                                  {acc[2 * si + 1][2 * sj], acc[2 * si + 1][2 * sj + 1]}};
      const int r0 = m0 + wm * FM * 32 + si * 64, c0 = n0 + wn * FN * 32 + sj * 64;
      if (p.ksplit > 1)
        epilogue_lds<EPI_STORE_F32, false>(q, sub, r0, c0, 0, 0, lane, stg_area, nullptr, nullptr, resv);
      else
        epilogue_lds<EPI, LN, kPF>(p, sub, r0, c0, 0, 0, lane, stg_area, ln_tab + (r0 - m0),
                                   ln_gtab + (c0 - n0), resv);
    }
}

// Second pass of split-K: the slices added in order (deterministic), then
// the epilogue of one element.
// The reduce kernels issue every slice's loads before the first sum (they
// are latency-bound launches of a few microseconds): at most kMaxSlices
// slices (gemm_mfma checks).
constexpr int kMaxSlices = 8, kMaxConvSlices = 12;

template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p) {
  const long long mn = static_cast<long long>(p.M) * p.N;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= mn) return;
  float v[kMaxSlices];
#pragma unroll
  for (int z = 0; z < kMaxSlices; ++z)
    if (z < p.ksplit) v[z] = p.ws[z * mn + idx];
  float acc = v[0];
#pragma unroll
  for (int z = 1; z < kMaxSlices; ++z)
    if (z < p.ksplit) acc += v[z];
  const int row = static_cast<int>(idx / p.N);
  epi_store<EPI, bf16_t>(p.epi, row, static_cast<int>(idx - static_cast<long long>(row) * p.N), acc);
}

// Second pass of split-K for a convolution: a thread takes four
// consecutive pixels of one output channel, adds the slices in order
// (rows of N rounded up to 64), then the per-(sample, channel) term and the
// residual, and stores the valid pixels NCHW as the EPI_CONV epilogue does.
__global__ __launch_bounds__(256) void splitk_reduce_conv_kernel(GemmParams p) {
  const ConvGemm& cv = p.conv;
  const int ldws = (p.N + 63) & ~63;
  const int per_row = ldws >> 2;
  const long long g = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int c = static_cast<int>(g / per_row);
  if (c >= p.M) return;
  const int m0 = static_cast<int>(g - static_cast<long long>(c) * per_row) * 4;
  if (m0 >= p.N) return;
  const int per_b = cv.Hq * cv.Wp;
  const int b = m0 / per_b;
  const int rem = m0 - b * per_b;
  const int i = rem / cv.Wp;
  const int j = rem - i * cv.Wp;
  if (i >= cv.Ho || j >= cv.Wo) return;
  const long long mn = static_cast<long long>(p.M) * ldws;
  const float* w = p.ws + static_cast<long long>(c) * ldws + m0;
  float4 sl[kMaxConvSlices];
#pragma unroll
  for (int z = 0; z < kMaxConvSlices; ++z)
    if (z < p.ksplit) sl[z] = *reinterpret_cast<const float4*>(w + z * mn);
  float4 a = sl[0];
#pragma unroll
  for (int z = 1; z < kMaxConvSlices; ++z) {
    if (z < p.ksplit) {
      a.x += sl[z].x; a.y += sl[z].y; a.z += sl[z].z; a.w += sl[z].w;
    }
  }
  const float add = cv.cadd[static_cast<long long>(b) * p.M + c];
  float y0 = a.x + add, y1 = a.y + add, y2 = a.z + add, y3 = a.w + add;
  const long long plane = static_cast<long long>(cv.Ho) * cv.Wo;
  const long long off = (static_cast<long long>(b) * p.M + c) * plane + static_cast<long long>(i) * cv.Wo + j;
  if (cv.resid) {
    const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(cv.resid) + off);
    y0 += __uint_as_float(r.x << 16);
    y1 += __uint_as_float(r.x & 0xffff0000u);
    y2 += __uint_as_float(r.y << 16);
    y3 += __uint_as_float(r.y & 0xffff0000u);
  }
  *reinterpret_cast<uint2*>(static_cast<bf16_t*>(cv.out) + off) = make_uint2(pack2bf(y0, y1), pack2bf(y2, y3));
}

// Second pass of split-K for the fp16 stream (EPI_STORE_H16 / EPI_RESID_H16):
// a thread takes 8 consecutive columns of one row, adds the slices in order,
// then the bias (and the residual) and rounds to fp16 as the GEMM epilogue
// does; the 8 threads of a 64-column block give its row sums.
template <bool RES>
__global__ __launch_bounds__(256) void splitk_reduce_h16_kernel(GemmParams p) {
  const int cpr = p.N >> 3;  // threads per row (N % 64 == 0)
  const long long g = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const long long row = g / cpr;
  if (row >= p.M) return;  // whole 8-thread groups
  const int c = static_cast<int>(g - row * cpr) * 8;
  const long long mn = static_cast<long long>(p.M) * p.N;
  const float* w = p.ws + row * p.N + c;
  f16_t* h16 = static_cast<f16_t*>(p.epi.out_act) + row * p.epi.ldo + c;
  float4 sa[kMaxSlices], sb[kMaxSlices];
#pragma unroll
  for (int z = 0; z < kMaxSlices; ++z) {
    if (z < p.ksplit) {
      sa[z] = *reinterpret_cast<const float4*>(w + z * mn);
      sb[z] = *reinterpret_cast<const float4*>(w + z * mn + 4);
    }
  }
  uint4 hin = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (RES) hin = *reinterpret_cast<const uint4*>(h16);
  float v[8] = {sa[0].x, sa[0].y, sa[0].z, sa[0].w, sb[0].x, sb[0].y, sb[0].z, sb[0].w};
#pragma unroll
  for (int z = 1; z < kMaxSlices; ++z) {
    if (z < p.ksplit) {
      v[0] += sa[z].x; v[1] += sa[z].y; v[2] += sa[z].z; v[3] += sa[z].w;
      v[4] += sb[z].x; v[5] += sb[z].y; v[6] += sb[z].z; v[7] += sb[z].w;
    }
  }
  if (p.epi.bias) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] += p.epi.bias[c + k];
  }
  if constexpr (RES) {
    const uint32_t hw[4] = {hin.x, hin.y, hin.z, hin.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16x2 h2 = __builtin_bit_cast(f16x2, hw[k]);
      v[2 * k] += static_cast<float>(h2[0]);
      v[2 * k + 1] += static_cast<float>(h2[1]);
    }
  }
  const uint4 o = make_uint4(pack2h(v[0], v[1]), pack2h(v[2], v[3]), pack2h(v[4], v[5]),
                             pack2h(v[6], v[7]));
  *reinterpret_cast<uint4*>(h16) = o;
  if (p.epi.range_flag && f16x8_nonfinite(o)) *p.epi.range_flag = 1;
  if (p.epi.row_stats) {
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16x2 h2 = __builtin_bit_cast(f16x2, ow[k]);
      v[2 * k] = static_cast<float>(h2[0]);
      v[2 * k + 1] = static_cast<float>(h2[1]);
    }
    const float sum = row8_sum(((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])));
    const float mb = sum * (1.0f / 64.0f);
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) q = fmaf(v[k] - mb, v[k] - mb, q);
    const float m2 = row8_sum(q);
    if ((threadIdx.x & 7) == 0)
      p.epi.row_stats[row * (p.epi.ldo >> 6) + (c >> 6)] = make_float2(sum, m2);
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

namespace {
template <int WM, int WN, int FM, int FN, int MINB, int NST = 2>
hipError_t launch_pipe(const GemmParams& p, int op, int kind, int split, hipStream_t s) {
  constexpr int TBM = WM * FM * 32, TBN = WN * FN * 32;
  const dim3 grid(((p.M + TBM - 1) / TBM) * ((p.N - p.n_off + TBN - 1) / TBN) * split);
  constexpr int threads = 64 * WM * WN;
#define ST_PIPE_LAUNCH(E, LN)                                                                          \
  if (op == ACT_F16) gemm_pipe_kernel<E, f16_t, WM, WN, FM, FN, MINB, LN, NST><<<grid, threads, 0, s>>>(p); \
  else gemm_pipe_kernel<E, bf16_t, WM, WN, FM, FN, MINB, LN, NST><<<grid, threads, 0, s>>>(p);
  const bool ln = p.epi.ln_stats != nullptr;
  switch (kind) {
    case EPI_STORE_F32: ST_PIPE_LAUNCH(EPI_STORE_F32, false) break;
    case EPI_RESID_F32: ST_PIPE_LAUNCH(EPI_RESID_F32, false) break;
    case EPI_STORE_H16: ST_PIPE_LAUNCH(EPI_STORE_H16, false) break;
    case EPI_RESID_H16: ST_PIPE_LAUNCH(EPI_RESID_H16, false) break;
    case EPI_NCHW: ST_PIPE_LAUNCH(EPI_NCHW, false) break;
    case EPI_CONV:
      if (op != ACT_F16) return hipErrorInvalidValue;
      gemm_pipe_kernel<EPI_CONV, f16_t, WM, WN, FM, FN, MINB, false, NST><<<grid, threads, 0, s>>>(p);
      break;
    case EPI_HEADS:
      if (ln) { ST_PIPE_LAUNCH(EPI_HEADS, true) } else { ST_PIPE_LAUNCH(EPI_HEADS, false) }
      break;
    case EPI_GEGLU:
      if (ln) { ST_PIPE_LAUNCH(EPI_GEGLU, true) } else { ST_PIPE_LAUNCH(EPI_GEGLU, false) }
      break;
    case EPI_CROSS_ATTN:  // 64x64 wavefront tiles only (gemm_mfma picks them)
      if constexpr (FM == 2 && FN == 2) {
        if (ln) { ST_PIPE_LAUNCH(EPI_CROSS_ATTN, true) } else { ST_PIPE_LAUNCH(EPI_CROSS_ATTN, false) }
      } else {
        return hipErrorInvalidValue;
      }
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef ST_PIPE_LAUNCH
  return hipGetLastError();
}
}  // namespace

// Compute units of the current device (cached per device; host threads may
// race to fill an entry, with the same value).
static int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Convolutions: 128x128 tiles, two per CU (three-stage ring when there are no
// more tiles than CUs), or 256x256 tiles when there are many of them.
static hipError_t launch_conv(const GemmParams& p, hipStream_t s) {
  if (p.ksplit > 1) {
    // slices one 128x128 workgroup per CU (three-stage ring), then the sum
    const long long wgs = static_cast<long long>((p.M + 127) / 128) * ((p.N + 127) / 128) * p.ksplit;
    hipError_t e = wgs <= cu_count() ? launch_pipe<2, 2, 2, 2, 1, 3>(p, ACT_F16, EPI_CONV, p.ksplit, s)
                                     : launch_pipe<2, 2, 2, 2, 2>(p, ACT_F16, EPI_CONV, p.ksplit, s);
    if (e != hipSuccess) return e;
    const long long n = static_cast<long long>(p.M) * (((p.N + 63) & ~63) >> 2);
    splitk_reduce_conv_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(p);
    return hipGetLastError();
  }
  const long long tiles = static_cast<long long>((p.M + 127) / 128) * ((p.N + 127) / 128);
  const long long big = static_cast<long long>((p.M + 255) / 256) * ((p.N + 255) / 256);
  if (big >= kBigTileMin) return launch_pipe<2, 4, 4, 2, 1>(p, ACT_F16, EPI_CONV, 1, s);
  if (tiles <= cu_count()) return launch_pipe<2, 2, 2, 2, 1, 3>(p, ACT_F16, EPI_CONV, 1, s);
  return launch_pipe<2, 2, 2, 2, 2>(p, ACT_F16, EPI_CONV, 1, s);
}

int conv_ksplit(int M, int N, int K, int cus) {
  const long long tiles = static_cast<long long>((M + 127) / 128) * ((N + 127) / 128);
  if (2 * tiles > cus) return 1;
  const int stages = K / 64;
  for (int sp = 12; sp > 1; --sp)
    if (stages % sp == 0 && stages / sp >= 16 && tiles * sp <= cus) return sp;
  return 1;
}

hipError_t gemm_mfma(const GemmParams& p, int op, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.n_off != 0) return hipErrorInvalidValue;
  if (p.epi.ln_stats && (!p.epi.ln_g || p.epi.ln_blocks * 64 != p.K ||
                         (p.epi.kind != EPI_HEADS && p.epi.kind != EPI_GEGLU &&
                          p.epi.kind != EPI_CROSS_ATTN)))
    return hipErrorInvalidValue;
  if (p.epi.kind == EPI_CROSS_ATTN &&
      (!p.epi.ca.k || !p.epi.ca.vt || !p.epi.out_act || p.epi.ca.nk <= 64 || p.epi.ca.nk > 96 ||
       p.epi.ca.kv_pad < 96 || p.epi.ca.rows_per_batch <= 0 || p.epi.ca.rows_per_batch % 64 ||
       p.N % 64 || p.epi.ldo % 4 || p.N != p.epi.ca.heads * 64))
    return hipErrorInvalidValue;
  if (p.epi.row_stats && (p.epi.ldo % 64 || p.N % 64 ||
                          (p.epi.kind != EPI_STORE_F32 && p.epi.kind != EPI_RESID_F32 &&
                           p.epi.kind != EPI_STORE_H16 && p.epi.kind != EPI_RESID_H16)))
    return hipErrorInvalidValue;
  // fp16 stream rows move as 16-byte vectors
  if ((p.epi.kind == EPI_STORE_H16 || p.epi.kind == EPI_RESID_H16) &&
      (!p.epi.out_act || p.N % 64 || p.epi.ldo % 8))
    return hipErrorInvalidValue;
  if (p.K % 64) return hipErrorInvalidValue;
  if (p.epi.kind == EPI_CONV) {
    const ConvGemm& cv = p.conv;
    if (op != ACT_F16 || (p.ksplit > 1 && (!p.ws || p.ksplit > kMaxConvSlices || p.K % (p.ksplit * 64))) ||
        p.epi.ln_stats ||
        !cv.cadd || !cv.out || cv.spt < 1 ||
        cv.sc_spt < 0 || p.K != (9 * cv.spt + cv.sc_spt) * 64 || cv.Wp % 4 || cv.Wo % 4 ||
        cv.Wo > cv.Wp || cv.Ho > cv.Hq || p.N % (cv.Hq * cv.Wp) || cv.b_bytes <= 0 ||
        cv.b_bytes > 0x7fffffffLL || static_cast<long long>(p.M) * p.lda * 2 > 0x7fffffffLL)
      return hipErrorInvalidValue;
    return launch_conv(p, s);
  }
  // the DMA addresses each operand with 32-bit byte offsets
  if (static_cast<long long>(p.M) * p.lda * 2 > 0x7fffffffLL ||
      static_cast<long long>(p.N) * p.ldb * 2 > 0x7fffffffLL)
    return hipErrorInvalidValue;
  const int split = p.ksplit > 1 ? p.ksplit : 1;
  if (split > 1) {
    const bool h16 = p.epi.kind == EPI_STORE_H16 || p.epi.kind == EPI_RESID_H16;
    if (!p.ws || split > kMaxSlices || p.K % (split * 64) || p.epi.ln_stats ||
        (!h16 && (op != ACT_BF16 || p.epi.row_stats ||
                  (p.epi.kind != EPI_HEADS && p.epi.kind != EPI_STORE_F32))))
      return hipErrorInvalidValue;
    // the slices (the kernel switches to the plain fp32 store; one 128x128
    // workgroup per CU with three stages when they all fit so), then the sum
    const long long slice_wgs = static_cast<long long>((p.M + 127) / 128) * ((p.N + 127) / 128) * split;
    hipError_t e = slice_wgs <= cu_count() ? launch_pipe<2, 2, 2, 2, 1, 3>(p, op, p.epi.kind, split, s)
                                           : launch_pipe<2, 2, 2, 2, 2>(p, op, p.epi.kind, split, s);
    if (e != hipSuccess) return e;
    const long long mn = static_cast<long long>(p.M) * p.N;
    if (h16) {
      const unsigned blocks = static_cast<unsigned>((mn / 8 + 255) / 256);
      if (p.epi.kind == EPI_RESID_H16) splitk_reduce_h16_kernel<true><<<blocks, 256, 0, s>>>(p);
      else splitk_reduce_h16_kernel<false><<<blocks, 256, 0, s>>>(p);
      return hipGetLastError();
    }
    const unsigned blocks = static_cast<unsigned>((mn + 255) / 256);
    if (p.epi.kind == EPI_HEADS) splitk_reduce_kernel<EPI_HEADS><<<blocks, 256, 0, s>>>(p);
    else splitk_reduce_kernel<EPI_STORE_F32><<<blocks, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  // 256x256 tiles (eight wavefronts of 128x64) when there are enough of
  // them to give most CUs one; otherwise 128x128 tiles, two per CU.
  const int mtb = (p.M + 255) / 256, ntb = (p.N + 255) / 256;
  const long long big_tiles = static_cast<long long>(mtb) * ntb;
  const int cus = cu_count();
  // 128x128 tiles: with no more of them than CUs, one per CU with a
  // three-stage ring (96 KB of LDS), else two per CU with two stages
  auto small_tiles = [&](const GemmParams& q) {
    const long long tiles = static_cast<long long>((q.M + 127) / 128) * ((q.N - q.n_off + 127) / 128);
    if (tiles <= cus) return launch_pipe<2, 2, 2, 2, 1, 3>(q, op, q.epi.kind, 1, s);
    return launch_pipe<2, 2, 2, 2, 2>(q, op, q.epi.kind, 1, s);
  };
  // below kBigTileMin, large tiles only where they cover the product with
  // no padding (FF1 of the U-Net's 1024-token levels at batch 1, 160
  // tiles: SDXL-Inpaint timestep 17.8 -> 17.0 ms, same box; with padding,
  // e.g. N = 320, they measured slower)
  const bool exact = p.M % 256 == 0 && p.N % 256 == 0 && big_tiles >= kBigTileExact;
  // Products shallower than 640 (five 64-deep stages at C = 320) keep
  // 128x128 tiles two per CU: the two workgroups of a CU overlap each
  // other's prologue and epilogue, which such short K loops cannot hide
  // (SD2.1 Down0: Q/K/V 33-36 -> 27-32 us, forward -1%; SD2.1-base
  // timestep -0.5-0.8%, same box).
  if ((big_tiles < kBigTileMin && !exact) || p.epi.kind == EPI_CROSS_ATTN || p.K < kBigTileMinK)
    return small_tiles(p);
  // When the last round of large tiles would leave more than a quarter of
  // the CUs idle, the columns of whole rounds take large tiles and the rest
  // 128x128 tiles (two per CU) in a second launch.
  const long long rounds = big_tiles / cus, tail = big_tiles % cus;
  const int nb = rounds > 0 ? static_cast<int>(rounds * cus / mtb) : 0;
  if (tail > 0 && 4 * tail < 3LL * cus && nb >= 1 && nb < ntb) {
    GemmParams q = p;
    q.N = nb * 256;
    hipError_t e = launch_pipe<2, 4, 4, 2, 1>(q, op, p.epi.kind, 1, s);
    if (e != hipSuccess) return e;
    q.N = p.N;
    q.n_off = nb * 256;
    return small_tiles(q);
  }
  return launch_pipe<2, 4, 4, 2, 1>(p, op, p.epi.kind, 1, s);
}

hipError_t gemm_f32(const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.epi.ln_stats || p.epi.row_stats || p.n_off) return hipErrorInvalidValue;
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
