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
// operand is read from LDS.  Softmax runs in fp32 with exp2: the queries
// arrive multiplied by log2(e)/8 (the projection's epilogue does it), and
// each score block starts with one more MFMA step that adds -m, the row's
// reference max, so that the accumulators already hold the exponents and the
// vector units do no per-score arithmetic before exp2.  m is kept equal to
// the sum of two bf16 values (hi + lo, ~16 significant bits), which this
// step adds exactly.  Keys at or beyond Nk get -inf.
//
// fp32 path (debug builds): one thread per query row, K/V tiles in LDS,
// online softmax in fp32.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace stb {

namespace {

constexpr int KT = 64;  // key rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
// Lazy running max: a tile is exponentiated against the row's reference max
// from earlier tiles; only when some lane's probabilities sum past this bound
// (or overflow) is the exact max taken and the output rescaled.
constexpr float kLazyBound = 256.f;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// Word 3 of a gfx9 buffer resource for raw (untyped) dword access.
constexpr int kBufferWord3 = 0x00020000;

// buffer_load_dwordx4 ... lds: 64 lanes x 16 bytes from `base` + soff + voff
// (reads at or past nbytes return 0) into the 1 KB of LDS at `lds`, lane i
// landing in slot i.
__device__ __forceinline__ void tile_dma(const void* base, int nbytes, uint16_t* lds,
                                         unsigned voff, int soff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// Both tiles live in LDS as 64 rows of 64 bf16 (128 bytes = eight 16-byte
// chunks): K as [key][dim], V^T as [dim][key].  gfx950 serves a 16-byte LDS
// read 16 lanes at a time over 64 banks (256 bytes), so two consecutive rows
// fill the banks once; chunk c of row r is stored at c ^ ((r >> 1) & 7),
// which gives the 16 rows of one read phase 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
}
// Key order inside a K tile: LDS row r holds key perm(r), r with its bits 2
// and 3 swapped.  Then the eight scores that the S^T accumulator layout gives
// one lane for one PV step (rows 16st + 4*lhi + 0..3 and 16st + 8 + 4*lhi +
// 0..3) are the keys 16st + 8*lhi + 0..7: contiguous in the V^T tile, so the
// matching V^T operand is a single 16-byte read.
__device__ __forceinline__ int perm(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// QB: 32-row query blocks per wavefront; NW: wavefronts per workgroup.
// KIND only gives self- and cross-attention their own kernel symbols.
template <int KIND, int QB, int NW>
__global__ __launch_bounds__(64 * NW, QB == 1 && NW >= 4 ? 3 : 2) void attn_bf16_kernel(AttnParams p) {
  constexpr int QW = 32 * QB;   // query rows per wavefront
  constexpr int QT = QW * NW;   // query rows per workgroup
  constexpr int BPW = 8 / NW;   // 1 KB DMA blocks of each 8 KB tile per wavefront
  // Three K and three V^T buffers as distinct LDS objects, so that the
  // compiler can tell the DMA into one buffer from the reads of the others
  // and does not wait for the DMA before reading.
  __shared__ __attribute__((aligned(16))) uint16_t sK0[KT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[KT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sK2[KT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[64 * KT];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[64 * KT];
  __shared__ __attribute__((aligned(16))) uint16_t sV2[64 * KT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lhi = lane >> 5;

  // Workgroups [0, n_full) take whole query tiles, the rest one key range
  // (piece) of a split tile.  Within each group, XCD-aware order:
  // workgroups are dealt round-robin to the 8 XCDs, so consecutive logical
  // tiles (the same sample and head, hence the same K and V) are given to
  // one XCD and share its L2.
  const int ntiles_all = (p.Nk + KT - 1) / KT;
  const int nsplit = p.nsplit > 1 ? p.nsplit : 1;
  auto xcd_order = [](int h, int n) { return (n & 7) ? h : (h & 7) * (n >> 3) + (h >> 3); };
  int tile, piece = -1, kt0 = 0, kt1 = ntiles_all;
  if (nsplit == 1 || static_cast<int>(blockIdx.x) < p.n_full) {
    tile = xcd_order(blockIdx.x, nsplit == 1 ? gridDim.x : p.n_full);
  } else {
    const int r = xcd_order(blockIdx.x - p.n_full, gridDim.x - p.n_full);
    tile = p.n_full + r / nsplit;
    piece = r - (r / nsplit) * nsplit;
    kt0 = piece * ntiles_all / nsplit;
    kt1 = (piece + 1) * ntiles_all / nsplit;
  }
  const int qtiles = (p.Nq + QT - 1) / QT;
  const int bh = tile / qtiles;
  const int qt = tile - bh * qtiles;
  const int b = bh / p.heads;
  const int head = bh - b * p.heads;
  const int q0 = qt * QT + wave * QW;

  const uint16_t* Q = static_cast<const uint16_t*>(p.q) + static_cast<long long>(bh) * p.q_pad * 64;
  const uint16_t* K = static_cast<const uint16_t*>(p.k) + static_cast<long long>(bh) * p.kv_pad * 64;
  const uint16_t* VT = static_cast<const uint16_t*>(p.vt) + static_cast<long long>(bh) * 64 * p.kv_pad;

  // Q^T as the B operand: block qb, step s -> query q0 + 32qb + l32,
  // dims 16s + 8*lhi + 0..7.
  uint4 qf[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = min(q0 + qb * 32 + l32, p.q_pad - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[qb][s] = *reinterpret_cast<const uint4*>(Q + static_cast<long long>(qrow) * 64 + 16 * s + 8 * lhi);
  }

  // Tiles move to LDS with tile_dma: one instruction moves 8 rows, so each
  // lane fetches the chunk that belongs in its slot.  The buffer covers this
  // (sample, head)'s K or V^T, the tile's offset is a scalar and each lane
  // adds a fixed 32-bit offset, so nothing per tile lives in vector
  // registers.
  const int kv_bytes = p.kv_pad * 128;  // K or V^T of one (sample, head)
  unsigned koff[BPW], voff[BPW];
#pragma unroll
  for (int j2 = 0; j2 < BPW; ++j2) {
    const int r = 8 * (wave * BPW + j2) + (lane >> 3);
    const int cl = (lane & 7) ^ ((r >> 1) & 7);
    koff[j2] = static_cast<unsigned>(perm(r) * 64 + cl * 8) * 2u;
    voff[j2] = static_cast<unsigned>(r * p.kv_pad + cl * 8) * 2u;
  }
  auto issue_k = [&](int t, uint16_t* dst) {
#pragma unroll
    for (int j2 = 0; j2 < BPW; ++j2)
      tile_dma(K, kv_bytes, dst + (wave * BPW + j2) * 512, koff[j2], t * KT * 128);
  };
  auto issue_v = [&](int t, uint16_t* dst) {
#pragma unroll
    for (int j2 = 0; j2 < BPW; ++j2)
      tile_dma(VT, kv_bytes, dst + (wave * BPW + j2) * 512, voff[j2], t * KT * 2);
  };

  floatx16 o[QB][2];
#pragma unroll
  for (int i = 0; i < QB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][j][r] = 0.f;
  float mref[QB], lsum[QB];  // lsum: this lane's partial row sums
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { mref[qb] = 0.f; lsum[qb] = 0.f; }
  // The max step of the score MFMAs: A = ones in dimensions 0 and 1 (lane
  // half 0), B = -m_hi, -m_lo of the lane's query in the same dimensions.
  const uint4 ones_col = lhi == 0 ? make_uint4(0x3F803F80u, 0u, 0u, 0u) : make_uint4(0u, 0u, 0u, 0u);
  uint4 negm[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) negm[qb] = make_uint4(0u, 0u, 0u, 0u);
  // m := hi + lo with hi = bf16(x), lo = bf16(x - hi); exact in fp32.
  auto set_m = [&](int qb, float x) {
    const uint32_t hi = f2bf(x);
    const uint32_t lo = f2bf(x - bf2f(hi));
    mref[qb] = bf2f(hi) + bf2f(lo);
    negm[qb].x = lhi == 0 ? ((hi ^ 0x8000u) | ((lo ^ 0x8000u) << 16)) : 0u;
  };
  // Byte offset of this lane's operand chunk for step s within a 32-row half
  // tile; rows 32..63 add 4096 bytes (the swizzle key depends on row bits 1-3
  // only).  The empty asm hides how the offset is formed, so that the buffer
  // base and the half-tile step become the read's immediate offset instead
  // of one address register per buffer.
  unsigned lo[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    lo[s4] = static_cast<unsigned>(swz(l32, 2 * s4 + lhi)) * 2u;
    asm volatile("" : "+v"(lo[s4]));
  }
  auto lds_operand = [&](const uint16_t* buf, int half, int s4) -> uint4 {
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(buf) + half * 4096 + lo[s4]);
  };

  // S^T = K Q^T for one tile; sc[qb][kb] entry r: tile row
  // kb*32 + 8*(r/4) + 4*lhi + r%4 (key perm of it), query q0 + 32qb + l32.
  // qk reads each K operand right before its MFMAs; qk_ops takes operands
  // read earlier (ka[kb][s]: block kb, step s) and alternates the two score
  // blocks, so that consecutive MFMAs do not depend on each other.
  auto qk_ops = [&](const uint4 (&ka)[2][4], floatx16 (&sc)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        floatx16 z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.f;
        sc[qb][kb] = mfma32x32x16(ones_col, negm[qb], z, bf16_t{});
      }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc[qb][kb] = mfma32x32x16(ka[kb][s], qf[qb][s], sc[qb][kb], bf16_t{});
  };
  auto qk = [&](const uint16_t* kbuf, floatx16 (&sc)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        floatx16 z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.f;
        sc[qb][kb] = mfma32x32x16(ones_col, negm[qb], z, bf16_t{});
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 a = lds_operand(kbuf, kb, s);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc[qb][kb] = mfma32x32x16(a, qf[qb][s], sc[qb][kb], bf16_t{});
      }
  };

  // Exact row max of the tile, whose scores are relative to the reference
  // max m: raises m by the excess (rounded to hi + lo), rescales the running
  // sum and output by 2^-excess and shifts the tile's scores to the new m.
  auto exact_max = [&](floatx16 (&sc)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mt = sc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[qb][kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_old = mref[qb];
      set_m(qb, m_old + fmaxf(mt, 0.f));
      const float delta = mref[qb] - m_old;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      lsum[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[qb][kb][r] -= delta;
    }
  };
  // The first tile sets m from its own max (whatever its sign).
  auto first_max = [&](floatx16 (&sc)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mt = sc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[qb][kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      set_m(qb, mt);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[qb][kb][r] -= mref[qb];
    }
  };
  // Probabilities of a tile against the reference max, as packed bf16 B
  // operands: step st takes entries r = 8*(st%2) + 0..7 of block st/2 (keys
  // 16st + 8*lhi + 0..7).  Returns true if some lane's probabilities sum past
  // the lazy bound (or overflow), i.e. the reference max must be raised.
  // The row sum adds the fp32 exponentials in four independent chains (a
  // single chain of v_dot2 over the bf16 pairs measured ~5% slower per
  // launch on SDXL Down1: the dot products are slow and serialised); the
  // bf16 rounding of the probabilities that the P.V product uses is
  // unbiased, so the two sums agree to ~2^-9 / sqrt(keys).
  auto exponentiate = [&](const floatx16 (&sc)[QB][2], uint4 (&pb)[QB][4],
                          float (&ps)[QB]) -> bool {
    bool big = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float pa[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e0 = __builtin_amdgcn_exp2f(sc[qb][st >> 1][8 * (st & 1) + 2 * j]);
          const float e1 = __builtin_amdgcn_exp2f(sc[qb][st >> 1][8 * (st & 1) + 2 * j + 1]);
          bf16x2 pk;
          pk[0] = static_cast<__bf16>(e0);
          pk[1] = static_cast<__bf16>(e1);
          pa[(2 * j) & 3] += e0;
          pa[(2 * j + 1) & 3] += e1;
          w[j] = __builtin_bit_cast(uint32_t, pk);
        }
        pb[qb][st] = make_uint4(w[0], w[1], w[2], w[3]);
      }
      ps[qb] = (pa[0] + pa[1]) + (pa[2] + pa[3]);
      big |= !(ps[qb] <= kLazyBound);
    }
    return big;
  };

  // O^T += V^T P^T.  V^T operand of dim block db, step st: row db*32 + l32,
  // keys 16st + 8*lhi + 0..7 (chunk 2st + lhi): the keys of the P^T operand,
  // in the same order (see perm).
  auto pv = [&](const uint16_t* vbuf, const uint4 (&pb)[QB][4]) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const uint4 a = lds_operand(vbuf, db, st);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = mfma32x32x16(a, pb[qb][st], o[qb][db], bf16_t{});
      }
  };

  // Keys at or beyond Nk in tile t (the last tile when Nk % KT != 0) -> -inf.
  // The bound is hidden from the compiler so that the comparisons stay here
  // instead of being hoisted out of the loop into 32 live masks.
  auto mask_tile = [&](int t, floatx16 (&sc)[QB][2]) {
    int kvalid = p.Nk - t * KT;
    asm volatile("" : "+v"(kvalid));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (perm(kb * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3)) >= kvalid) sc[qb][kb][r] = -INFINITY;
  };

  // Cross-attention with a key padding mask: masked keys of tile t get a
  // finite score far below any real one (-30000 in base-2 units), not -inf,
  // so that a tile with every key masked still has a finite maximum; the
  // lazy-max rescale then scales its contributions to exactly 0 as soon as a
  // real key appears, and a sample with no real key is zeroed at the store.
  uint32_t kbw[4] = {~0u, ~0u, ~0u, 0u};
  bool any_key = true;
  if constexpr (KIND == 1) {
    if (p.key_bits) {
      const uint4 w = *reinterpret_cast<const uint4*>(p.key_bits + 4LL * b);
      kbw[0] = w.x; kbw[1] = w.y; kbw[2] = w.z; kbw[3] = w.w;
      any_key = (w.x | w.y | w.z | w.w) != 0u;
    }
  }
  auto mask_keys = [&](int t, floatx16 (&sc)[QB][2]) {
    if constexpr (KIND == 1) {
      if (!p.key_bits || t > 1) return;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t wd = t == 0 ? kbw[kb] : kbw[2 + kb];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((wd >> perm(8 * (r >> 2) + 4 * lhi + (r & 3))) & 1u)) sc[qb][kb][r] = -30000.f;
        }
    }
  };

  // Software pipeline over key tiles.  Iteration t turns S_t into P_t on the
  // vector units, computes S_{t+1} in the registers that S_t held, then adds
  // P_t V_t.  Tile j of K and of V^T lives in buffer j % 3: iteration t reads
  // K_{t+1} and V_t, K_{t+2} and V_{t+1} are in flight, and it issues the DMA
  // of K_{t+3} and V_{t+2}, so that every tile has two iterations to arrive.
  // The exact max of tile 0 is taken in the prologue and a ragged last tile
  // is masked as soon as its scores exist.
  // Tiles kt0 .. kt1-1 (all of them unless this workgroup is one piece of a
  // split tile); t below counts from kt0.
  const int ragged_last = (p.Nk % KT) ? ntiles_all - 1 : -1;
  const int ntiles = kt1 - kt0;
  floatx16 sc[QB][2];  // S_t
  issue_k(kt0, sK0);
  issue_v(kt0, sV0);
  if (ntiles > 1) { issue_k(kt0 + 1, sK1); issue_v(kt0 + 1, sV1); }
  if (ntiles > 2) issue_k(kt0 + 2, sK2);
  wait_vmcnt_lds<0>();
  stage_barrier();
  qk(sK0, sc);
  mask_keys(kt0, sc);
  if (ragged_last == kt0) mask_tile(kt0, sc);
  first_max(sc);
  stage_barrier();  // every wavefront is done with K_0 before K_3 replaces it

  constexpr int kIssued = 2 * BPW;  // DMA instructions per wavefront per iteration
  // Self-attention with four wavefronts per workgroup (three per SIMD): the
  // K operands of score block 0 are read before the exponentials, those of
  // block 1 after them, and the blocks alternate (same box, SDXL Down1: 95
  // -> 91.5 us per launch; SD2.1 Down0 448 -> 437 us).  The two-wavefront
  // kernel keeps the reads next to their MFMAs (19.6 vs 20.5 us the other
  // way at 1024 tokens), and so does the 77-key kernel (two key tiles; the
  // read-ahead would spill its key-mask words inside the loop).
  constexpr bool kReadAhead = NW >= 4 && KIND == 0;
  auto iter = [&](int t, const uint16_t* kn, const uint16_t* vc, uint16_t* kw, uint16_t* vw) {
    if (t + 3 < ntiles) issue_k(kt0 + t + 3, kw);
    if (t + 2 < ntiles) issue_v(kt0 + t + 2, vw);
    uint4 ka[2][4];
    if constexpr (kReadAhead) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) ka[0][s4] = lds_operand(kn, 0, s4);
    }
    uint4 pb[QB][4];
    float ps[QB];
    if (__any(exponentiate(sc, pb, ps))) {  // rare
      exact_max(sc);
      exponentiate(sc, pb, ps);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lsum[qb] += ps[qb];
    // S_{t+1} (unused past the last tile: its LDS buffer then holds stale,
    // finite data)
    if constexpr (kReadAhead) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) ka[1][s4] = lds_operand(kn, 1, s4);
      qk_ops(ka, sc);
    } else {
      qk(kn, sc);
    }
    mask_keys(kt0 + t + 1, sc);
    if (kt0 + t + 1 == ragged_last) mask_tile(kt0 + t + 1, sc);
    pv(vc, pb);
    // K_{t+2} and V_{t+1} have landed (loads complete in order, so at most
    // this iteration's own DMA is still in flight)
    if (t + 3 < ntiles) wait_vmcnt_lds<kIssued>();
    else wait_vmcnt_lds<0>();
    stage_barrier();
  };
  // Unrolled by the buffer period, so that every buffer is a distinct LDS
  // object at each use; whole periods first, then up to two tail tiles.
  int t = 0;
  for (; t + 3 <= ntiles; t += 3) {
    iter(t, sK1, sV0, sK0, sV2);
    iter(t + 1, sK2, sV1, sK1, sV0);
    iter(t + 2, sK0, sV2, sK2, sV1);
  }
  if (t < ntiles) {
    iter(t, sK1, sV0, sK0, sV2);
    if (t + 1 < ntiles) iter(t + 1, sK2, sV1, sK1, sV0);
  }
  wait_vmcnt_lds<0>();  // no DMA may still write LDS when the workgroup ends

  // Row sums over both lane halves.  Lane l holds O^T entries of query
  // q0 + 32qb + l32, dims db*32 + 8g + 4*lhi + 0..3 (g = r / 4).
  float l_tot[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) l_tot[qb] = lsum[qb] + __shfl_xor(lsum[qb], 32, 64);

  if (piece >= 0) {
    // One piece of a split tile: store the partial result (unnormalised O,
    // reference max, row sum) for the merge pass.
    constexpr int PF = QT * 66;  // per piece: O [QT][64], max [QT], sum [QT]
    float* mine = p.part + (static_cast<long long>(tile - p.n_full) * nsplit + piece) * PF;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wave * QW + qb * 32 + l32;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(mine + row * 64 + db * 32 + 8 * g + 4 * lhi) =
              make_float4(o[qb][db][4 * g], o[qb][db][4 * g + 1], o[qb][db][4 * g + 2], o[qb][db][4 * g + 3]);
      if (lhi == 0) {
        mine[QT * 64 + row] = mref[qb];
        mine[QT * 65 + row] = l_tot[qb];
      }
    }
    return;  // attn_merge_kernel combines the pieces
  }

  // Whole tile: normalise, store O[token][head*64 + d].
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = any_key ? 1.0f / l_tot[qb] : 0.f;
    const int qrow = q0 + qb * 32 + l32;
    if (qrow < p.Nq) {
      uint16_t* orow = static_cast<uint16_t*>(p.o) +
                       (static_cast<long long>(b) * p.Nq + qrow) * p.C + head * 64;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * lhi;
          const uint2 pk = make_uint2(pack2bf(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv),
                                      pack2bf(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv));
          *reinterpret_cast<uint2*>(orow + d) = pk;
        }
    }
  }
}

// Self-attention over long sequences, with the softmax of each key tile
// overlapped with matrix work inside the wavefront.  Same tiles, LDS ring,
// operand layouts and reference-max scheme as attn_bf16_kernel (128 queries
// per workgroup, four wavefronts of 32), but the scores of two consecutive
// tiles live in two register sets and P.V lags one tile behind, so that each
// half of an iteration pairs MFMAs with vector work that does not depend on
// them.  Iteration t:
//   phase 1: O += V_{t-1} P_{t-1} (8 MFMAs) beside the row sums of the
//            fp32 exponentials of tile t-1 and the row max of S_t; the
//            K_{t+1} operands are read from LDS;
//   (rare)   a probability of tile t would exceed 2^8: the exact max is
//            taken, O and the row sums are rescaled and S_t shifted;
//   phase 2: S_{t+1} = K_{t+1} Q^T - m (9 MFMAs: the two blocks share the
//            -m step) beside exp2 of S_t in place and P_t = bf16 of it (32
//            exp2, 16 packs); the V_t operands are read.
// (Dot products of the probabilities with ones would give the row sums in
// half the instructions, but v_dot2 does not issue beside an MFMA on gfx950:
// a register-only probe of 16 MFMAs with two exp2, a pack and two dot
// products each ran at 860 clocks per wavefront against 628 with fp32 adds.)
// Each phase is issued as chunks of one MFMA and its share of the vector and
// LDS instructions (sched_barrier between chunks), so the matrix pipe works
// while the same wavefront's vector instructions issue: with the DMA, the
// LDS reads and the barrier taken out, the loop runs at ~610 clocks per
// tile and wavefront-pair of a SIMD, close to the 598 of a register-only
// probe of the same instruction mix.  Up to 256 VGPRs per lane: two
// workgroups per CU, whole query tiles only (the dispatch in
// attention_bf16 says why).
constexpr float kLazyExp = 8.f;
// max(a, b, c) as one v_max3_f32 (fmaxf chains add canonicalising moves)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}  // base-2 exponent bound of one probability

template <int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_sa_kernel(AttnParams p) {
  constexpr int QT = 32 * NW;
  constexpr int BPW = 8 / NW;
  __shared__ __attribute__((aligned(16))) uint16_t sK0[KT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[KT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sK2[KT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[64 * KT];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[64 * KT];
  __shared__ __attribute__((aligned(16))) uint16_t sV2[64 * KT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lhi = lane >> 5;

  // Whole tiles only (no key split).  Persistent workgroups, at most two
  // per CU so that all are resident from the start: workgroup w computes
  // tiles w, w + G, ... (G = grid size), in XCD-aware order (as
  // attn_bf16_kernel; with G a multiple of 8 the tiles of one workgroup
  // stay in its XCD's share).
  const int ntiles_all = (p.Nk + KT - 1) / KT;
  const int qtiles = (p.Nq + QT - 1) / QT;
  const int tiles_total = p.B * p.heads * qtiles;
  const int G = gridDim.x;
  auto xcd_order = [](int h, int n) { return (n & 7) ? h : (h & 7) * (n >> 3) + (h >> 3); };
  for (int h = blockIdx.x; h < tiles_total; h += G) {
  const int tile = xcd_order(h, tiles_total);
  const int kt0 = 0, kt1 = ntiles_all;
  const int bh = tile / qtiles;
  const int qt = tile - bh * qtiles;
  const int b = bh / p.heads;
  const int head = bh - b * p.heads;
  const int q0 = qt * QT + wave * 32;

  const uint16_t* Q = static_cast<const uint16_t*>(p.q) + static_cast<long long>(bh) * p.q_pad * 64;
  const uint16_t* K = static_cast<const uint16_t*>(p.k) + static_cast<long long>(bh) * p.kv_pad * 64;
  const uint16_t* VT = static_cast<const uint16_t*>(p.vt) + static_cast<long long>(bh) * 64 * p.kv_pad;

  // Q^T as the B operand: step s -> query q0 + l32, dims 16s + 8*lhi + 0..7.
  uint4 qf[4];
  {
    const int qrow = min(q0 + l32, p.q_pad - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[s] = *reinterpret_cast<const uint4*>(Q + static_cast<long long>(qrow) * 64 + 16 * s + 8 * lhi);
  }

  const int kv_bytes = p.kv_pad * 128;
  unsigned koff[BPW], voff[BPW];
#pragma unroll
  for (int j2 = 0; j2 < BPW; ++j2) {
    const int r = 8 * (wave * BPW + j2) + (lane >> 3);
    const int cl = (lane & 7) ^ ((r >> 1) & 7);
    koff[j2] = static_cast<unsigned>(perm(r) * 64 + cl * 8) * 2u;
    voff[j2] = static_cast<unsigned>(r * p.kv_pad + cl * 8) * 2u;
  }
  auto issue_k = [&](int t, uint16_t* dst) {
#pragma unroll
    for (int j2 = 0; j2 < BPW; ++j2)
      tile_dma(K, kv_bytes, dst + (wave * BPW + j2) * 512, koff[j2], t * KT * 128);
  };
  auto issue_v = [&](int t, uint16_t* dst) {
#pragma unroll
    for (int j2 = 0; j2 < BPW; ++j2)
      tile_dma(VT, kv_bytes, dst + (wave * BPW + j2) * 512, voff[j2], t * KT * 2);
  };

  floatx16 o[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
  float mref = 0.f;
  float ls[4] = {0.f, 0.f, 0.f, 0.f};  // row-sum chains of this lane's keys
  const uint4 ones_col = lhi == 0 ? make_uint4(0x3F803F80u, 0u, 0u, 0u) : make_uint4(0u, 0u, 0u, 0u);
  uint4 negm = make_uint4(0u, 0u, 0u, 0u);
  auto set_m = [&](float x) {
    const uint32_t hi = f2bf(x);
    const uint32_t lo2 = f2bf(x - bf2f(hi));
    mref = bf2f(hi) + bf2f(lo2);
    negm.x = lhi == 0 ? ((hi ^ 0x8000u) | ((lo2 ^ 0x8000u) << 16)) : 0u;
  };
  unsigned lo[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    lo[s4] = static_cast<unsigned>(swz(l32, 2 * s4 + lhi)) * 2u;
    asm volatile("" : "+v"(lo[s4]));
  }
  auto lds_operand = [&](const uint16_t* buf, int half, int s4) -> uint4 {
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(buf) + half * 4096 + lo[s4]);
  };
  auto mask_tile = [&](int t, floatx16 (&sc)[2]) {
    int kvalid = p.Nk - t * KT;
    asm volatile("" : "+v"(kvalid));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (perm(kb * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3)) >= kvalid) sc[kb][r] = -INFINITY;
  };

  uint4 ka[8];  // K_{t+1} operands, MFMA order: ka[2s + kb] = block kb, step s
  uint4 va[8];  // V operands of the lagging P.V: va[2st + db]
  uint4 pb[4];  // P of the lagging tile as B operands (step st)

  // Prologue: K_0, V_0, K_1, V_1, K_2 in flight; S_0 with its exact max.
  const int ragged_last = (p.Nk % KT) ? ntiles_all - 1 : -1;
  const int ntiles = kt1 - kt0;
  floatx16 sA[2], sB[2];
  issue_k(kt0, sK0);
  issue_v(kt0, sV0);
  if (ntiles > 1) { issue_k(kt0 + 1, sK1); issue_v(kt0 + 1, sV1); }
  if (ntiles > 2) issue_k(kt0 + 2, sK2);
  wait_vmcnt_lds<0>();
  stage_barrier();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sA[kb][r] = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sA[kb] = mfma32x32x16(lds_operand(sK0, kb, s), qf[s], sA[kb], bf16_t{});
  if (ragged_last == kt0) mask_tile(kt0, sA);
  {
    float mt = sA[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sA[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    set_m(mt);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sA[kb][r] -= mref;
  }
  stage_barrier();  // every wavefront is done with K_0 before K_3 replaces it

  constexpr int kIssued = 2 * BPW;
  // FIRST: iteration 0 (no lagging P.V, S_0 already exact).
  auto iter = [&](int t, auto first_tag, floatx16 (&cur)[2], floatx16 (&nxt)[2], const uint16_t* kn,
                  const uint16_t* vc, uint16_t* kw, uint16_t* vw) {
    constexpr bool FIRST = decltype(first_tag)::value;
    // this iteration's DMA (K_{t+3}, V_{t+2}) is issued one instruction per
    // chunk of phase 2 (spread out: 95.6 -> 91.8 us on SDXL Down1 against
    // all four at the top of the iteration); past the last tile it reloads
    // that tile, so the DMA is unconditional and the offsets stay in range
    // phase 1 (nxt still holds the exponentials of tile t-1)
    // (two independent max chains: one wavefront per SIMD, as in the last
    // round of a persistent grid, cannot hide a dependent pair per chunk)
    float mt0 = cur[0][0], mt1 = cur[0][1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (!FIRST) {
        o[i & 1] = mfma32x32x16(va[i], pb[i >> 1], o[i & 1], bf16_t{});
#pragma unroll
        for (int j = 0; j < 4; ++j) ls[j] += nxt[i >> 2][4 * (i & 3) + j];
        const int kb = i >> 2, r0 = 4 * (i & 3);
        mt0 = max3f(mt0, cur[kb][r0], cur[kb][r0 + 1]);
        mt1 = max3f(mt1, cur[kb][r0 + 2], cur[kb][r0 + 3]);
      }
      ka[i] = lds_operand(kn, i & 1, i >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    float mt = fmaxf(mt0, mt1);
    if constexpr (!FIRST) {
      if (__any(mt > kLazyExp)) {  // rare
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_old = mref;
        set_m(m_old + fmaxf(mt, 0.f));
        const float delta = mref - m_old;
        const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
        for (int c = 0; c < 4; ++c) ls[c] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) cur[kb][r] -= delta;
      }
    }
    // phase 2: chunk i takes MFMA i of S_{t+1} (two -m steps, then the eight
    // K steps), exponentials [32i/10, 32(i+1)/10) of S_t with the packs of
    // completed pairs, and the read of va[i].
    uint32_t pw[16];
    auto pack_pairs = [&](int k0, int k1) {
#pragma unroll
      for (int k = k0; k < k1; ++k)
        if (k & 1) {
          pw[k >> 1] = pack2bf(cur[(k - 1) >> 4][(k - 1) & 15], cur[k >> 4][k & 15]);
          asm volatile("" : "+v"(pw[k >> 1]));
        }
    };
    const int kdma = min(kt0 + t + 3, kt1 - 1), vdma = min(kt0 + t + 2, kt1 - 1);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      if (i < 2) {
        floatx16 z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.f;
        nxt[i] = mfma32x32x16(ones_col, negm, z, bf16_t{});
      } else {
        const int j = i - 2;
        nxt[j & 1] = mfma32x32x16(ka[j], qf[j >> 1], nxt[j & 1], bf16_t{});
      }
#pragma unroll
      for (int k = (32 * i) / 10; k < (32 * (i + 1)) / 10; ++k) {
        cur[k >> 4][k & 15] = __builtin_amdgcn_exp2f(cur[k >> 4][k & 15]);
        // pin the exponential to this chunk (otherwise it sinks to its
        // first use in the next iteration)
        asm volatile("" : "+v"(cur[k >> 4][k & 15]));
      }
      // packs of the pairs completed in the previous chunk, one chunk after
      // their exponentials (a pack right behind its exp2 waits for it)
      if (i > 0) pack_pairs((32 * (i - 1)) / 10, (32 * i) / 10);
      if (i < 8) va[i] = lds_operand(vc, i & 1, i >> 1);
      if (i >= 1 && i <= BPW) tile_dma(K, kv_bytes, kw + (wave * BPW + i - 1) * 512, koff[i - 1], kdma * KT * 128);
      if (i > BPW && i <= 2 * BPW)
        tile_dma(VT, kv_bytes, vw + (wave * BPW + i - 1 - BPW) * 512, voff[i - 1 - BPW], vdma * KT * 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    pack_pairs(28, 32);
#pragma unroll
    for (int st = 0; st < 4; ++st) pb[st] = make_uint4(pw[4 * st], pw[4 * st + 1], pw[4 * st + 2], pw[4 * st + 3]);
    if (kt0 + t + 1 == ragged_last) mask_tile(kt0 + t + 1, nxt);
    wait_vmcnt_lds<kIssued>();
    stage_barrier();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Tile j of K and V^T lives in buffer j % 3 and S_t in sA (t even) or sB;
  // iteration t reads K_{t+1} and V_t and refills the buffers of K_t and
  // V_{t-1}.  After iteration 0 the loop runs in periods of six.
  iter(0, T_{}, sA, sB, sK1, sV0, sK0, sV2);
  int t = 1;
  for (; t + 6 <= ntiles; t += 6) {
    iter(t, F_{}, sB, sA, sK2, sV1, sK1, sV0);
    iter(t + 1, F_{}, sA, sB, sK0, sV2, sK2, sV1);
    iter(t + 2, F_{}, sB, sA, sK1, sV0, sK0, sV2);
    iter(t + 3, F_{}, sA, sB, sK2, sV1, sK1, sV0);
    iter(t + 4, F_{}, sB, sA, sK0, sV2, sK2, sV1);
    iter(t + 5, F_{}, sA, sB, sK1, sV0, sK0, sV2);
  }
  if (t < ntiles) iter(t, F_{}, sB, sA, sK2, sV1, sK1, sV0);
  if (t + 1 < ntiles) iter(t + 1, F_{}, sA, sB, sK0, sV2, sK2, sV1);
  if (t + 2 < ntiles) iter(t + 2, F_{}, sB, sA, sK1, sV0, sK0, sV2);
  if (t + 3 < ntiles) iter(t + 3, F_{}, sA, sB, sK2, sV1, sK1, sV0);
  if (t + 4 < ntiles) iter(t + 4, F_{}, sB, sA, sK0, sV2, sK2, sV1);
  // the lagging P.V of the last tile
  // exponentials of the last tile: in sA when it had an even index
  const bool last_odd = (ntiles - 1) & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o[i & 1] = mfma32x32x16(va[i], pb[i >> 1], o[i & 1], bf16_t{});
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ls[j] += last_odd ? sB[i >> 2][4 * (i & 3) + j] : sA[i >> 2][4 * (i & 3) + j];
  }
  wait_vmcnt_lds<0>();  // no DMA may still write LDS when the workgroup ends

  float l_tot = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  l_tot += __shfl_xor(l_tot, 32, 64);

  {
  const float inv = 1.0f / l_tot;
  const int qrow = q0 + l32;
  if (qrow < p.Nq) {
    uint16_t* orow = static_cast<uint16_t*>(p.o) + (static_cast<long long>(b) * p.Nq + qrow) * p.C + head * 64;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * lhi;
        const uint2 pk = make_uint2(pack2bf(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                    pack2bf(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(orow + d) = pk;
      }
  }
  }
  // every wavefront's DMA has landed and its reads are done before the next
  // item's prologue refills the buffers
  stage_barrier();
  }
}

// Second pass of the key split: for each split query tile, the pieces'
// partial results are merged in piece order (bitwise reproducible):
// O = sum_i w_i O_i / sum_i w_i l_i with w_i = 2^(m_i - max_i m_i) (the
// references m_i are base-2 exponents).  Eight threads per query row, 8
// dims each, 32 rows per workgroup; every piece's loads are issued before
// the first sum.
constexpr int kMaxPieces = 8;  // attention_bf16_plan splits a tile at most 8 ways
template <int QT>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  constexpr int PF = QT * 66;
  constexpr int kBlocksPerTile = QT / 32;
  const int j = blockIdx.x / kBlocksPerTile;  // split tile index
  const int row = (blockIdx.x - j * kBlocksPerTile) * 32 + (threadIdx.x >> 3);
  const int g = threadIdx.x & 7;  // dims 8g .. 8g+7
  const int tile = p.n_full + j;
  const int qtiles = (p.Nq + QT - 1) / QT;
  const int bh = tile / qtiles;
  const int qrow = (tile - bh * qtiles) * QT + row;
  if (qrow >= p.Nq) return;
  const int b = bh / p.heads, head = bh - b * p.heads;
  const float* tp = p.part + static_cast<long long>(j) * p.nsplit * PF;
  float m[kMaxPieces], l[kMaxPieces];
  float4 v[kMaxPieces][2];
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) {
    if (i < p.nsplit) {
      const float* pi = tp + i * PF;
      m[i] = pi[QT * 64 + row];
      l[i] = pi[QT * 65 + row];
      const float4* src = reinterpret_cast<const float4*>(pi + row * 64 + 8 * g);
      v[i][0] = src[0];
      v[i][1] = src[1];
    }
  }
  float mmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i)
    if (i < p.nsplit) mmax = fmaxf(mmax, m[i]);
  float acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.f;
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) {
    if (i < p.nsplit) {
      const float w = __builtin_amdgcn_exp2f(m[i] - mmax);
      den += l[i] * w;
      acc[0] += v[i][0].x * w; acc[1] += v[i][0].y * w;
      acc[2] += v[i][0].z * w; acc[3] += v[i][0].w * w;
      acc[4] += v[i][1].x * w; acc[5] += v[i][1].y * w;
      acc[6] += v[i][1].z * w; acc[7] += v[i][1].w * w;
    }
  }
  const float inv = 1.0f / den;
  uint16_t* orow = static_cast<uint16_t*>(p.o) +
                   (static_cast<long long>(b) * p.Nq + qrow) * p.C + head * 64 + 8 * g;
  *reinterpret_cast<uint4*>(orow) =
      make_uint4(pack2bf(acc[0] * inv, acc[1] * inv), pack2bf(acc[2] * inv, acc[3] * inv),
                 pack2bf(acc[4] * inv, acc[5] * inv), pack2bf(acc[6] * inv, acc[7] * inv));
}

#ifndef ST_ATTN_QB
#define ST_ATTN_QB 1
#endif
#ifndef ST_ATTN_NW
#define ST_ATTN_NW 4
#endif
constexpr int kQB = ST_ATTN_QB, kNW = ST_ATTN_NW;
constexpr int kQT = 32 * kQB * kNW;

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
      if (p.key_bits && !((p.key_bits[4 * b + ((k0 + j) >> 5)] >> ((k0 + j) & 31)) & 1u)) continue;
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
    const float inv = l > 0.f ? 1.f / l : 0.f;  // every key masked: O = 0
    for (int d = 0; d < 64; ++d) orow[d] = o[d] * inv;
  }
}

}  // namespace

int attention_bf16_q_tile() { return kQT; }
int attention_bf16_kv_tile() { return KT; }
float attention_bf16_q_scale() { return 0.125f * kLog2e; }
int attention_bf16_part_floats() { return kQT * 66; }

void attention_bf16_plan(int B, int heads, int Nq, int Nk, int cus, int& n_full, int& nsplit) {
  const int tiles = B * heads * ((Nq + kQT - 1) / kQT);
  const int ktiles = (Nk + KT - 1) / KT;
  n_full = tiles;
  nsplit = 1;
  if (cus <= 0) return;
  const int full = (tiles / cus) * cus;  // a whole number of tiles per CU
  const int rest = tiles - full;
  if (rest == 0) return;
  // about one piece per CU, each of at least 16 key tiles: shorter pieces
  // (and the merge pass) cost more than the balance gains (measured: 23 ->
  // 26-31 us with 4-tile pieces at 1024 keys; 108 -> 105 us with 32-tile
  // pieces at 4096 keys)
  int sp = (cus + rest / 2) / rest;
  sp = sp < 8 ? sp : 8;
  while (sp > 1 && ktiles / sp < 16) --sp;
  if (sp <= 1) return;
  n_full = full;
  nsplit = sp;
}

// Compute units of the current device (cached per device; host threads may
// race to fill an entry, with the same value).
static int attn_cu_count() {
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

hipError_t attention_bf16(const AttnParams& p, hipStream_t s) {
  const int qtiles = (p.Nq + kQT - 1) / kQT;
  const int tiles = p.B * p.heads * qtiles;
  // Query rows past q_pad are never read (the kernels clamp the row they
  // load); the K and V^T buffers must cover every key tile.
  if (p.q_pad < p.Nq || p.kv_pad < ((p.Nk + KT - 1) / KT) * KT)
    return hipErrorInvalidValue;
  int grid = tiles;
  if (p.key_bits && (p.Nk > 96 || p.nsplit > 1)) return hipErrorInvalidValue;
  if (p.nsplit > 1) {
    if (!p.part || p.n_full < 0 || p.n_full >= tiles || (p.Nk + KT - 1) / KT < p.nsplit)
      return hipErrorInvalidValue;
    grid = p.n_full + (tiles - p.n_full) * p.nsplit;
  }
  // Few query tiles (short sequences, no key split): workgroups of two
  // wavefronts (64 queries) instead, twice as many, so that more CUs and
  // more wavefronts per SIMD take part.
  if (p.nsplit <= 1 && p.B * p.heads * ((p.Nq + 127) / 128) < 2 * attn_cu_count()) {
    const int grid64 = p.B * p.heads * ((p.Nq + 63) / 64);
    if (p.Nk == kCtxLen)
      attn_bf16_kernel<1, 1, 2><<<grid64, 128, 0, s>>>(p);
    else
      attn_bf16_kernel<0, 1, 2><<<grid64, 128, 0, s>>>(p);
    return hipGetLastError();
  }
  // Self-attention without a key split runs the overlapped kernel
  // (attn_sa_kernel: two workgroups per CU); the split plan puts two whole
  // tiles and one piece on every CU, which needs the three resident
  // workgroups per CU of attn_bf16_kernel.  Measured, same box: 9216 tokens
  // (SD2.1 Down0, no split) 230 -> 222 us per launch with the overlapped
  // kernel; 4096 tokens (SDXL Down1, split) 88 -> 92-97 us with it.
  if (p.Nk == kCtxLen)
    attn_bf16_kernel<1, kQB, kNW><<<grid, 64 * kNW, 0, s>>>(p);
  else if (p.nsplit <= 1) {
    const int g = 2 * attn_cu_count() < tiles ? 2 * attn_cu_count() : tiles;
    attn_sa_kernel<kNW><<<g, 64 * kNW, 0, s>>>(p);
    return hipGetLastError();
  } else
    attn_bf16_kernel<0, kQB, kNW><<<grid, 64 * kNW, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit <= 1) return e;
  if (p.nsplit > kMaxPieces) return hipErrorInvalidValue;
  attn_merge_kernel<kQT><<<(tiles - p.n_full) * (kQT / 32), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t attention_f32(const AttnParams& p, hipStream_t s) {
  const int qtiles = (p.Nq + FQ - 1) / FQ;
  attn_f32_kernel<<<p.B * p.heads * qtiles, FQ, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace stb
