// Multi-head attention of the Spatial-Transformer block (gfx950), head dim 64:
// per (sample, head) O = softmax(Q K^T / sqrt(64)) V over all keys, no mask
// (SD1.5 anatomy article §3.4; self-attention with Q=K=V=image tokens and
// cross-attention with K=V=context, SDXL-Inpaint architecture page §4).
//
// bf16 path: flash-style.  A 256-thread workgroup owns 128 query rows of one
// (sample, head); each wavefront owns 32 of them.  Keys stream through LDS in
// tiles of 64 (K rows and V^T rows, double-buffered, loads of the next tile
// in flight during the current one), and nothing of size Nq x Nk reaches HBM.
// The kernel computes the transposed scores S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 so that each lane's accumulators belong to ONE
// query (lane & 31): the running max, the exponentials and the rescaling of
// the output stay in the lane, and only the row max needs one exchange with
// the other lane half.  The probabilities then feed O^T += V^T P^T directly
// as the B operand of the second MFMA, in the same K order that the V^T
// operand is read from LDS.  Softmax runs in fp32 with exp2 and the scale
// 1/8 * log2(e) folded into one FMA; keys at or beyond Nk get -inf.
//
// fp32 path (debug builds): one thread per query row, K/V tiles in LDS,
// online softmax in fp32.
#include "common.h"
#include "kernels.h"

namespace stb {

namespace {

constexpr int QT = 128;  // query rows per workgroup
constexpr int KT = 64;   // key rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int kswz(int row, int chunk) {  // bf16 element offset
  return row * 64 + ((chunk ^ (row & 7)) << 3);
}

__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KT * 64];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][64 * KT];  // [d][key]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31, lhi = lane >> 5;

  const int qtiles = (p.Nq + QT - 1) / QT;
  const int bh = blockIdx.x / qtiles;
  const int qt = blockIdx.x - bh * qtiles;
  const int b = bh / p.heads;
  const int head = bh - b * p.heads;
  const int q0 = qt * QT + wave * 32;

  const bf16_t* Q = static_cast<const bf16_t*>(p.q) + static_cast<long long>(bh) * p.q_pad * 64;
  const bf16_t* K = static_cast<const bf16_t*>(p.k) + static_cast<long long>(bh) * p.kv_pad * 64;
  const bf16_t* VT = static_cast<const bf16_t*>(p.vt) + static_cast<long long>(bh) * 64 * p.kv_pad;

  // Q^T as the B operand: lane holds query q0 + l32, dims 16s + 8*lhi + 0..7.
  bf16x8 qf[4];
  {
    const int qrow = min(q0 + l32, p.q_pad - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(Q + static_cast<long long>(qrow) * 64 + 16 * s + 8 * lhi);
  }

  // Tile loads: K tile 64 rows x 8 chunks, V^T tile 64 rows (dims) x 8 chunks.
  uint4 rk[2], rv[2];
  auto load_tile = [&](int t) {
    const int k0 = t * KT;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = tid + 256 * r;
      const int row = q >> 3, c = q & 7;
      rk[r] = *reinterpret_cast<const uint4*>(K + static_cast<long long>(k0 + row) * 64 + c * 8);
      rv[r] = *reinterpret_cast<const uint4*>(VT + static_cast<long long>(row) * p.kv_pad + k0 + c * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = tid + 256 * r;
      const int row = q >> 3, c = q & 7;
      *reinterpret_cast<uint4*>(&sK[buf][kswz(row, c)]) = rk[r];
      *reinterpret_cast<uint4*>(&sV[buf][kswz(row, c)]) = rv[r];
    }
  };

  floatx16 o[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's partial row sum (its 32 of every 64 keys)
  const float c = 0.125f * kLog2e;

  const int ntiles = (p.Nk + KT - 1) / KT;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);

    // S^T block kb: keys kb*32 + 8*(r/4) + 4*lhi + r%4, query l32.
    floatx16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sK[buf][kswz(kb * 32 + l32, 2 * s + lhi)]);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc[kb], 0, 0, 0);
      }
    }
    const int kvalid = p.Nk - t * KT;
    if (kvalid < KT) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
          if (key >= kvalid) sc[kb][r] = -INFINITY;
        }
    }
    float mt = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
    const float mc = m_new * c;
    m_run = m_new;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], c, -mc));
        sc[kb][r] = e;
        ls += e;
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;

    // P^T operand of step st (keys 16st..16st+15 of the tile): this lane's
    // keys 16st + 4*lhi + 0..3 and 16st + 8 + 4*lhi + 0..3, i.e. accumulator
    // entries r = 8*(st%2) + 0..7 of block st/2.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = static_cast<__bf16>(sc[st >> 1][8 * (st & 1) + j]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // V^T operand: dim row i*32 + l32, the same eight keys in the same order.
        const int drow = i * 32 + l32;
        const int key0 = 16 * st + 4 * lhi;        // 4 keys, 8 bytes
        const int key1 = 16 * st + 8 + 4 * lhi;    // 4 keys, 8 bytes
        const bf16_t* vrow = &sV[buf][0];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + kswz(drow, key0 >> 3) + (key0 & 7));
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + kswz(drow, key1 >> 3) + (key1 & 7));
        const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8 va = __builtin_bit_cast(bf16x8, vv);
        o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[i], 0, 0, 0);
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Row sum over both lane halves, normalise, store O[token][head*64 + d].
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  const int qrow = q0 + l32;
  if (qrow < p.Nq) {
    bf16_t* orow = static_cast<bf16_t*>(p.o) +
                   (static_cast<long long>(b) * p.Nq + qrow) * p.C + head * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = i * 32 + 8 * g + 4 * lhi;
        const uint2 pk = make_uint2(pack2bf(o[i][4 * g] * inv, o[i][4 * g + 1] * inv),
                                    pack2bf(o[i][4 * g + 2] * inv, o[i][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(orow + d) = pk;
      }
  }
}

// ---------------------------------------------------------------- fp32 path
constexpr int FQ = 64;   // queries per workgroup (one per thread)
constexpr int FKT = 32;  // keys per LDS tile

__global__ __launch_bounds__(FQ) void attn_f32_kernel(AttnParams p) {
  __shared__ float sK[FKT][64];
  __shared__ float sV[64][FKT + 1];
  const int qtiles = (p.Nq + FQ - 1) / FQ;
  const int bh = blockIdx.x / qtiles;
  const int qt = blockIdx.x - bh * qtiles;
  const int b = bh / p.heads;
  const int head = bh - b * p.heads;
  const int qi = qt * FQ + threadIdx.x;
  const float* Q = static_cast<const float*>(p.q) + static_cast<long long>(bh) * p.q_pad * 64;
  const float* K = static_cast<const float*>(p.k) + static_cast<long long>(bh) * p.kv_pad * 64;
  const float* VT = static_cast<const float*>(p.vt) + static_cast<long long>(bh) * 64 * p.kv_pad;
  float q[64], o[64];
  const int qr = min(qi, p.q_pad - 1);
  for (int d = 0; d < 64; ++d) { q[d] = Q[static_cast<long long>(qr) * 64 + d]; o[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 < p.Nk; k0 += FKT) {
    __syncthreads();
    for (int i = threadIdx.x; i < FKT * 64; i += FQ) {
      const int kr = i >> 6, d = i & 63;
      sK[kr][d] = K[static_cast<long long>(k0 + kr) * 64 + d];
      const int dv = i / FKT, kv = i % FKT;
      sV[dv][kv] = VT[static_cast<long long>(dv) * p.kv_pad + k0 + kv];
    }
    __syncthreads();
    const int kn = min(FKT, p.Nk - k0);
    for (int j = 0; j < kn; ++j) {
      float s = 0.f;
      for (int d = 0; d < 64; ++d) s = fmaf(q[d], sK[j][d], s);
      s *= 0.125f;
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn);
      const float e = expf(s - mn);
      l = l * a + e;
      for (int d = 0; d < 64; ++d) o[d] = o[d] * a + e * sV[d][j];
      m = mn;
    }
  }
  if (qi < p.Nq) {
    float* orow = static_cast<float*>(p.o) + (static_cast<long long>(b) * p.Nq + qi) * p.C + head * 64;
    const float inv = 1.f / l;
    for (int d = 0; d < 64; ++d) orow[d] = o[d] * inv;
  }
}

}  // namespace

int attention_bf16_q_tile() { return QT; }
int attention_bf16_kv_tile() { return KT; }

hipError_t attention_bf16(const AttnParams& p, hipStream_t s) {
  const int qtiles = (p.Nq + QT - 1) / QT;
  attn_bf16_kernel<<<p.B * p.heads * qtiles, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t attention_f32(const AttnParams& p, hipStream_t s) {
  const int qtiles = (p.Nq + FQ - 1) / FQ;
  attn_f32_kernel<<<p.B * p.heads * qtiles, FQ, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace stb
