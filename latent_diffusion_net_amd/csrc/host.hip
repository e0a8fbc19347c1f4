// C ABI of the Spatial-Transformer block: argument validation, weight
// repacking into library-owned device memory, workspace planning and the
// launch schedule of one forward.  Declared in include/st_block.h.
//
// Launch schedule of one forward (bf16 storage):
//   GroupNorm statistics            x                     -> partial sums [B*32][split]
//   GroupNorm apply + to tokens     x, partial sums       -> u [T][C] fp16
//   proj_in GEMM                    u, W_in               -> h [T][C] fp32
//   context K/V GEMM (all layers)   ctx, [Wk2;Wv2]*depth  -> Kc, Vc^T per layer
//   per layer:
//     Q/K/V GEMM, LayerNorm 1 folded  h16, [Wq1;Wk1;Wv1]*g1 -> Q, K, V^T (per head)
//     self-attention                Q, K, V^T             -> O [T][C] bf16
//     out-projection GEMM           O, Wo1                -> h += .
//     cross Q GEMM, LayerNorm 2 folded, with the cross-attention in its
//       epilogue when H*W % 64 == 0   h16, Wq2*g2, Kc, Vc^T -> O
//       (else: cross Q GEMM -> Q, then the attention kernel -> O)
//     out-projection GEMM           O, Wo2                -> h += .
//     FF1 GEMM+GEGLU, LayerNorm 3 folded  h16, W1*g3      -> f [T][F] fp16
//     FF2 GEMM                      f, W2                 -> h += .
//       (with few [T][C] output tiles: K slices, then their ordered sum)
//   proj_out GEMM, transposed       W_out, h16            -> y = NCHW(.) + x
// The residual stream h lives in fp16 (h16).  Every GEMM that writes it
// (proj_in and the three residual products) also writes, per row and 64
// channels, the sum and the sum of squared deviations of the stored values;
// a product behind a LayerNorm reads h16 with gamma folded into its weights
// and beta into its bias, and corrects each output by the row's mean and
// 1/std combined from those sums:
//   LN(h) W^T = rstd * (h (W*gamma)^T - mean * rowsum(W*gamma)) + W beta.
// The fp32 debug path keeps h in fp32 and runs LayerNorm as its own pass on
// fp32 buffers, and GEGLU as its own pass.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/st_block.h"
#include "kernels.h"
#include "parts.h"

#define ST_API extern "C" __attribute__((visibility("default")))

using namespace stb;

namespace {

thread_local std::string g_err;

st_status fail(st_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

st_status hip_fail(hipError_t e, const char* what) {
  return fail(ST_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline long long round_up(long long v, long long m) { return (v + m - 1) / m * m; }

struct LayerDev {
  float* ln_w[3];
  float* ln_b[3];
  // bf16 path: LayerNorm i is folded into the product that follows it (Q/K/V,
  // cross Q, FF1): those weights hold W * gamma in fp16, their biases gain
  // W beta, and ln_g[i] holds the row sums of the folded weights.
  float* ln_g[3];
  void* wqkv;  // [3C][C]: Wq1, Wk1, Wv1
  float* bqkv;
  void* wo1;
  float* bo1;
  void* wq2;
  float* bq2;
  void* wo2;
  float* bo2;
  void* w1;  // bf16: rows repacked in 64-row groups (32 value, 32 gate); fp32: as given
  float* b1;  // [2F], original order
  void* w2;
  float* b2;
};

struct PendingTiming {
  int kind;
  hipEvent_t e0, e1;
};

}  // namespace

struct st_block {
  int B, C, H, W, heads, D, depth;
  st_dtype dtype;
  bool bf16;
  int N, T, F, npad, cpad;
  size_t esz;
  int device;
  std::vector<void*> allocs;
  size_t bytes_planned;
  size_t bytes_cap;

  float *gn_w, *gn_b;
  void *w_in, *w_out;
  float *b_in, *b_out;
  std::vector<LayerDev> L;
  void* wkv;  // [depth*2C][D]: per layer Wk2 rows then Wv2 rows
  float* bkv;

  // buffers rewritten by every forward (ScratchPlan); bound to an arena of
  // the handle's own, or to one shared with the other parts of a U-Net
  ScratchPlan scratch;
  void* scratch_own;
  bool scratch_bound;
  DevArena* persist;  // arena of the persistent allocations during create, or NULL

  float2* gn_part;
  int gn_max_split;
  void* u;
  float* h;      // fp32 path: residual stream [T][C]
  void* hcopy;  // bf16 path: residual stream [T][C] in fp16 (h16)
  float2* hstats;  // bf16 path: [T][C/64] sums and squared deviations of h
  void *q, *k, *vt, *o, *f;
  float* z;  // fp32 path: FF1 output before GEGLU
  void *kc, *vct;
  long long ctx_layer_stride;
  int attn_n_full, attn_nsplit;  // bf16 self-attention load-balance plan
  float* attn_part;
  int ctx_ksplit;   // bf16 path: K slices of the context K/V GEMM (1 = none)
  float* ctx_ws;    // [ctx_ksplit][B*77][depth*2C] fp32 partial products
  // bf16 path: K slices of the out-projections (K = C) and of FF2 (K = F)
  // when the [T][C] product has fewer output tiles than the GPU has CUs,
  // and their fp32 partial products [slices][T][C]
  int out_ksplit, ff2_ksplit;
  float* res_ws;
  // bf16 path: set to 1 by a kernel that stores a non-finite fp16 value
  // (the residual stream, the GEGLU output or the normalised input); read
  // and cleared by st_block_check_range
  int* range_flag;
  // context key padding mask of the current forward as bits, [B][4] words
  uint32_t* key_bits;

  unsigned timing_mask;
  // per-layer kinds are timed only in layers below timing_layers (0 = all);
  // timing_layer: the layer being launched (-1 outside the layer loop)
  int timing_layers, timing_layer;
  std::vector<PendingTiming> pending;
  std::vector<hipEvent_t> spare_events;
};

namespace {

void* dalloc(st_block* b, size_t bytes) {
  if (bytes == 0) bytes = 16;
  bytes = static_cast<size_t>(round_up(static_cast<long long>(bytes), 256));
  if (b->bytes_cap && b->bytes_planned + bytes > b->bytes_cap) return nullptr;
  if (b->persist && b->persist->base) {
    void* p = b->persist->take(bytes);
    if (p) b->bytes_planned += bytes;
    return p;
  }
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (b->persist) b->persist->count(bytes);
  b->bytes_planned += bytes;
  b->allocs.push_back(p);
  return p;
}

void free_all(st_block* b) {
  for (void* p : b->allocs) (void)hipFree(p);
  b->allocs.clear();
  for (auto& t : b->pending) {
    (void)hipEventDestroy(t.e0);
    (void)hipEventDestroy(t.e1);
  }
  b->pending.clear();
  for (auto e : b->spare_events) (void)hipEventDestroy(e);
  b->spare_events.clear();
}

// ------------------------------------------------------------ create helpers
struct Creator {
  st_block* b;
  hipStream_t s;
  st_status st = ST_OK;
  std::string msg{};

  bool ok() const { return st == ST_OK; }
  void oom(const char* what) {
    if (ok()) { st = ST_ERR_OUT_OF_MEMORY; msg = std::string("out of device memory allocating ") + what; }
  }
  void dev(hipError_t e, const char* what) {
    if (ok() && e != hipSuccess) { st = ST_ERR_DEVICE; msg = std::string(what) + ": " + hipGetErrorString(e); }
  }
  void* alloc(size_t bytes, const char* what) {
    if (!ok()) return nullptr;
    void* p = dalloc(b, bytes);
    if (!p) oom(what);
    return p;
  }
  // a buffer of the scratch arena (bound after create)
  template <typename T>
  void scr(T** field, size_t bytes) {
    if (ok()) b->scratch.add(field, bytes);
  }
  // fp32 copy of a [n] vector given in the handle's dtype (NULL -> fill)
  float* vec(const void* src, long long n, float fill, const char* what) {
    float* d = static_cast<float*>(alloc(n * sizeof(float), what));
    if (d) dev(to_f32(src, b->bf16, d, n, fill, s), what);
    return d;
  }
  void vec_into(float* dst, const void* src, long long n, float fill, const char* what) {
    if (ok()) dev(to_f32(src, b->bf16, dst, n, fill, s), what);
  }
  void copy(void* dst, const void* src, size_t bytes, const char* what) {
    if (ok()) dev(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s), what);
  }
  void* mat(const void* src, long long rows, long long cols, const char* what) {
    void* d = alloc(rows * cols * b->esz, what);
    copy(d, src, rows * cols * b->esz, what);
    return d;
  }
  // bf16 path: weights that meet fp16 activations are kept as fp16 (exact
  // within the fp16 range; larger magnitudes raise *overflow).
  int* overflow = nullptr;
  void to_f16(void* d, long long n, const char* what) {
    if (ok() && b->bf16 && d) dev(bf16_to_f16_inplace(d, n, overflow, s), what);
  }
  // bf16 path: LayerNorm (gamma, beta) folded into the rows x C weights w
  // that follow it (fp16 on return), their bias and the row sums *g.
  void fold_ln(void* w, int rows, int cols, const float* gamma, const float* beta,
               float* bias, const int* map, float*& g, const char* what) {
    g = nullptr;
    if (!ok() || !b->bf16) return;
    g = static_cast<float*>(alloc(sizeof(float) * rows, what));
    if (ok()) dev(weight_fold_layernorm(w, rows, cols, gamma, beta, bias, map, g, overflow, s), what);
  }
};

}  // namespace

// Error text of this host thread, shared with the other ABI sources.
st_status st_set_error(st_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// ======================================================================= ABI

ST_API const char* st_last_error(void) { return g_err.c_str(); }

ST_API st_status st_block_create(int B, int C, int H, int W, int heads,
                                 int D_ctx, int depth, st_dtype dtype,
                                 const st_block_weights* w, void* stream,
                                 st_block** out) {
  return stb_block_create(B, C, H, W, heads, D_ctx, depth, dtype, w, stream, false, nullptr, out);
}

size_t stb_block_scratch_bytes(const st_block* b) { return b->scratch.bytes; }

void stb_block_bind_scratch(st_block* b, void* base) {
  b->scratch.bind(base);
  b->scratch_bound = true;
}

st_status stb_block_create(int B, int C, int H, int W, int heads, int D_ctx, int depth, st_dtype dtype,
                           const st_block_weights* w, void* stream, bool external_scratch,
                           DevArena* persist, st_block** out) {
  g_err.clear();
  if (!out) return fail(ST_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (B < 1 || H < 1 || W < 1) return fail(ST_ERR_INVALID, "B, H and W must be >= 1");
  if (C < 64 || C % 64) return fail(ST_ERR_INVALID, "C must be a positive multiple of 64");
  if (heads * 64 != C) return fail(ST_ERR_INVALID, "heads * 64 must equal C");
  if (D_ctx < 64 || D_ctx % 64) return fail(ST_ERR_INVALID, "D_ctx must be a positive multiple of 64");
  if (depth < 1) return fail(ST_ERR_INVALID, "depth must be >= 1");
  if (dtype != ST_DTYPE_BF16 && dtype != ST_DTYPE_F32) return fail(ST_ERR_INVALID, "unknown dtype");
  const long long N = static_cast<long long>(H) * W;
  const long long T = N * B;
  // The GEMMs address each operand through a buffer resource with 32-bit
  // byte offsets: every operand must stay below 2^31 bytes.  The largest
  // are the GEGLU output [T][4C] (FF2's A operand), the FF1 weights
  // [8C][C] and the context K/V weights of all layers [2C*depth][D_ctx]
  // (16-bit on the bf16 path; the fp32 path shares the limits).
  if (N > (1LL << 24) || T * 4LL * C * 2 >= (1LL << 31))
    return fail(ST_ERR_UNSUPPORTED, "B*H*W*4*C must stay below 2^30 (FF2 operand of 2^31 bytes)");
  if (16LL * C * C >= (1LL << 31))
    return fail(ST_ERR_UNSUPPORTED, "C too large: the FF1 weights [8C][C] reach 2^31 bytes");
  if (4LL * C * depth * D_ctx >= (1LL << 31) || 2LL * B * ST_CTX_LEN * D_ctx >= (1LL << 31))
    return fail(ST_ERR_UNSUPPORTED,
                "C*depth*D_ctx too large: the context K/V weights [2C*depth][D_ctx] reach 2^31 bytes");
  if (!w) return fail(ST_ERR_INVALID, "weights are NULL");
  if (!w->layers) return fail(ST_ERR_INVALID, "weights.layers is NULL");
  auto need = [](const void* p) { return p != nullptr && aligned16(p); };
  if (!need(w->proj_in_w) || !need(w->proj_out_w))
    return fail(ST_ERR_INVALID, "proj_in_w / proj_out_w must be non-NULL and 16-byte aligned");
  for (int l = 0; l < depth; ++l) {
    const st_layer_weights& lw = w->layers[l];
    const void* req[] = {lw.q1_w, lw.k1_w, lw.v1_w, lw.o1_w, lw.q2_w,
                         lw.k2_w, lw.v2_w, lw.o2_w, lw.ff1_w, lw.ff2_w};
    for (const void* p : req)
      if (!need(p))
        return fail(ST_ERR_INVALID, "layer " + std::to_string(l) +
                                        ": every Linear weight must be non-NULL and 16-byte aligned");
  }

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_fail(e, "hipGetDevice");
  }

  st_block* b = new (std::nothrow) st_block();
  if (!b) return fail(ST_ERR_OUT_OF_MEMORY, "host allocation failed");
  b->B = B; b->C = C; b->H = H; b->W = W; b->heads = heads; b->D = D_ctx; b->depth = depth;
  b->dtype = dtype;
  b->bf16 = dtype == ST_DTYPE_BF16;
  b->N = static_cast<int>(N);
  b->T = static_cast<int>(T);
  b->F = 4 * C;
  b->npad = static_cast<int>(round_up(N, 128));
  b->cpad = 128;
  b->esz = b->bf16 ? 2 : 4;
  b->device = dev;
  b->bytes_planned = 0;
  b->bytes_cap = 0;
  if (const char* cap = std::getenv("ST_MAX_DEVICE_BYTES")) b->bytes_cap = std::strtoull(cap, nullptr, 10);
  b->timing_mask = 0;
  b->timing_layers = 0;
  b->timing_layer = -1;
  b->range_flag = nullptr;
  b->key_bits = nullptr;
  b->scratch_own = nullptr;
  b->scratch_bound = false;
  b->persist = persist;

  hipStream_t s = static_cast<hipStream_t>(stream);
  Creator cr{b, s};
  const long long CC = static_cast<long long>(C) * C;
  const size_t es = b->esz;

  // Block-level weights.
  b->gn_w = cr.vec(w->gn_w, C, 1.f, "gn_w");
  b->gn_b = cr.vec(w->gn_b, C, 0.f, "gn_b");
  if (b->bf16) {
    cr.overflow = static_cast<int*>(cr.alloc(sizeof(int), "overflow flag"));
    if (cr.overflow) cr.dev(hipMemsetAsync(cr.overflow, 0, sizeof(int), s), "overflow flag");
    b->range_flag = static_cast<int*>(cr.alloc(sizeof(int), "range flag"));
    if (b->range_flag) cr.dev(hipMemsetAsync(b->range_flag, 0, sizeof(int), s), "range flag");
  }
  b->w_in = cr.mat(w->proj_in_w, C, C, "proj_in_w");
  cr.to_f16(b->w_in, CC, "proj_in_w to fp16");
  b->b_in = cr.vec(w->proj_in_b, C, 0.f, "proj_in_b");
  b->w_out = cr.mat(w->proj_out_w, C, C, "proj_out_w");
  cr.to_f16(b->w_out, CC, "proj_out_w to fp16");
  b->b_out = cr.vec(w->proj_out_b, C, 0.f, "proj_out_b");

  // Context K/V weights of every layer in one matrix.
  const long long kvrows = 2LL * C * depth;
  b->wkv = cr.alloc(kvrows * D_ctx * es, "context K/V weights");
  b->bkv = static_cast<float*>(cr.alloc(kvrows * sizeof(float), "context K/V biases"));

  // GEGLU row map for the bf16 path (value/gate pairs in 64-row groups).
  const int F = b->F;
  int* d_map = nullptr;
  if (b->bf16 && cr.ok()) {
    std::vector<int> map(2 * F);
    for (int p = 0; p < 2 * F; ++p) {
      const int grp = p / 64, wi = p % 64;
      map[p] = wi < 32 ? grp * 32 + wi : F + grp * 32 + (wi - 32);
    }
    d_map = static_cast<int*>(cr.alloc(map.size() * sizeof(int), "GEGLU row map"));
    if (d_map) cr.dev(hipMemcpyAsync(d_map, map.data(), map.size() * sizeof(int),
                                     hipMemcpyHostToDevice, s), "GEGLU row map");
    if (cr.ok()) cr.dev(hipStreamSynchronize(s), "GEGLU row map");
  }

  b->L.resize(depth);
  for (int l = 0; l < depth && cr.ok(); ++l) {
    const st_layer_weights& lw = w->layers[l];
    LayerDev& d = b->L[l];
    const void* lnw[3] = {lw.ln1_w, lw.ln2_w, lw.ln3_w};
    const void* lnb[3] = {lw.ln1_b, lw.ln2_b, lw.ln3_b};
    for (int i = 0; i < 3; ++i) {
      d.ln_w[i] = cr.vec(lnw[i], C, 1.f, "LayerNorm gamma");
      d.ln_b[i] = cr.vec(lnb[i], C, 0.f, "LayerNorm beta");
    }
    d.wqkv = cr.alloc(3 * CC * es, "Q/K/V weights");
    if (d.wqkv) {
      cr.copy(d.wqkv, lw.q1_w, CC * es, "q1_w");
      cr.copy(static_cast<char*>(d.wqkv) + CC * es, lw.k1_w, CC * es, "k1_w");
      cr.copy(static_cast<char*>(d.wqkv) + 2 * CC * es, lw.v1_w, CC * es, "v1_w");
    }
    d.bqkv = static_cast<float*>(cr.alloc(3LL * C * sizeof(float), "Q/K/V biases"));
    if (d.bqkv) {
      cr.vec_into(d.bqkv, lw.q1_b, C, 0.f, "q1_b");
      cr.vec_into(d.bqkv + C, lw.k1_b, C, 0.f, "k1_b");
      cr.vec_into(d.bqkv + 2 * C, lw.v1_b, C, 0.f, "v1_b");
    }
    cr.fold_ln(d.wqkv, 3 * C, C, d.ln_w[0], d.ln_b[0], d.bqkv, nullptr, d.ln_g[0], "fold LayerNorm 1");
    d.wo1 = cr.mat(lw.o1_w, C, C, "o1_w");
    d.bo1 = cr.vec(lw.o1_b, C, 0.f, "o1_b");
    d.wq2 = cr.mat(lw.q2_w, C, C, "q2_w");
    d.bq2 = cr.vec(lw.q2_b, C, 0.f, "q2_b");
    cr.fold_ln(d.wq2, C, C, d.ln_w[1], d.ln_b[1], d.bq2, nullptr, d.ln_g[1], "fold LayerNorm 2");
    d.wo2 = cr.mat(lw.o2_w, C, C, "o2_w");
    d.bo2 = cr.vec(lw.o2_b, C, 0.f, "o2_b");
    if (b->wkv && b->bkv) {
      const long long r0 = 2LL * C * l;
      const long long CD = static_cast<long long>(C) * D_ctx;
      cr.copy(static_cast<char*>(b->wkv) + r0 * D_ctx * es, lw.k2_w, CD * es, "k2_w");
      cr.copy(static_cast<char*>(b->wkv) + (r0 + C) * D_ctx * es, lw.v2_w, CD * es, "v2_w");
      cr.vec_into(b->bkv + r0, lw.k2_b, C, 0.f, "k2_b");
      cr.vec_into(b->bkv + r0 + C, lw.v2_b, C, 0.f, "v2_b");
    }
    d.w1 = cr.alloc(2LL * F * C * es, "ff1_w");
    if (d.w1 && cr.ok()) {
      if (b->bf16)
        cr.dev(gather_rows(lw.ff1_w, d.w1, d_map, 2 * F, static_cast<long long>(C) * es, s), "ff1_w repack");
      else
        cr.copy(d.w1, lw.ff1_w, 2LL * F * C * es, "ff1_w");
    }
    d.b1 = cr.vec(lw.ff1_b, 2LL * F, 0.f, "ff1_b");
    // rows repacked, biases in the original order
    cr.fold_ln(d.w1, 2 * F, C, d.ln_w[2], d.ln_b[2], d.b1, d_map, d.ln_g[2], "fold LayerNorm 3");
    d.w2 = cr.mat(lw.ff2_w, C, F, "ff2_w");
    cr.to_f16(d.w2, static_cast<long long>(C) * F, "ff2_w to fp16");
    d.b2 = cr.vec(lw.ff2_b, C, 0.f, "ff2_b");
  }

  // Workspace.
  b->gn_max_split = 64;
  b->gn_part = nullptr; b->u = nullptr; b->h = nullptr; b->hcopy = nullptr; b->hstats = nullptr;
  b->z = nullptr;
  cr.scr(&b->gn_part, sizeof(float2) * B * ST_GN_GROUPS * b->gn_max_split);
  cr.scr(&b->u, T * C * es);
  // the residual stream: fp32 on the fp32 path, fp16 (hcopy) on the bf16 path
  if (b->bf16) {
    cr.scr(&b->hcopy, T * static_cast<long long>(C) * es);
    cr.scr(&b->hstats, T * static_cast<long long>(C / 64) * sizeof(float2));
  } else {
    cr.scr(&b->h, T * C * sizeof(float));
  }
  // Per-head Q / K / V^T: padding rows (N not a multiple of 128) are read by
  // the attention kernels and must stay finite, so those buffers are the
  // handle's own and cleared once; without padding rows they are scratch.
  const long long headbuf = static_cast<long long>(B) * heads * b->npad * 64 * es;
  const bool head_pad = b->npad != b->N;
  if (head_pad) {
    b->q = cr.alloc(headbuf, "Q");
    b->k = cr.alloc(headbuf, "K");
    b->vt = cr.alloc(headbuf, "V^T");
  } else {
    cr.scr(&b->q, headbuf);
    cr.scr(&b->k, headbuf);
    cr.scr(&b->vt, headbuf);
  }
  cr.scr(&b->o, T * C * es);
  cr.scr(&b->f, T * F * es);
  if (!b->bf16) cr.scr(&b->z, T * 2LL * F * sizeof(float));
  b->ctx_layer_stride = static_cast<long long>(B) * heads * b->cpad * 64;
  // The context K/V GEMM has only B*77 rows: with few output tiles it
  // splits K so that enough workgroups stream the weights.
  {
    const int ctx_rows = B * ST_CTX_LEN;
    const long long tiles = ((ctx_rows + 127) / 128) * ((kvrows + 127) / 128);
    b->ctx_ksplit = 1;
    int cus = 0;
    if (b->bf16 && tiles < 128) {
      cr.dev(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "CU count");
      // the most slices (up to 8) whose workgroups all fit one per CU
      for (int sp = 8; sp > 1; sp /= 2)
        if (D_ctx % (sp * 64) == 0 && tiles * sp <= cus) { b->ctx_ksplit = sp; break; }
    }
    b->ctx_ws = nullptr;
    if (b->ctx_ksplit > 1) cr.scr(&b->ctx_ws, sizeof(float) * b->ctx_ksplit * ctx_rows * kvrows);
  }
  // Self-attention load balance: with more query tiles than fit a whole
  // number per CU, the remainder is split over keys (ST_ATTN_CUS overrides
  // the CU count the plan assumes; it changes only the work split).
  b->attn_n_full = 0;
  b->attn_nsplit = 1;
  b->attn_part = nullptr;
  b->out_ksplit = b->ff2_ksplit = 1;
  b->res_ws = nullptr;
  if (b->bf16 && cr.ok()) {
    int cus = 0;
    cr.dev(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "CU count");
    // The residual products write [T][C] in 128x128 tiles.  With fewer
    // tiles than CUs (short sequences) each tile has a CU to itself on the
    // three-stage ring, and K is split into the most slices that keep every
    // slice at least 640 deep and still give each slice a CU of its own;
    // the slices are summed in order by a second pass.  (640 rather than
    // 1024 splits the 1280-deep out-projections of 1024-token levels in
    // two: SDXL-Inpaint timestep 17.75 -> 17.49 ms, SD2.1-base at batch 1
    // 6.52 -> 6.49 ms, the block workloads unchanged, same box.)
    {
      const long long tiles = ((T + 127) / 128) * ((C + 127) / 128);
      auto slices = [&](int K) {
        if (tiles >= cus) return 1;
        for (int sp = 8; sp > 1; --sp)
          if (K % (64 * sp) == 0 && K / sp >= 640 && sp * tiles <= cus) return sp;
        return 1;
      };
      b->out_ksplit = slices(C);
      b->ff2_ksplit = slices(b->F);
      const int most = b->out_ksplit > b->ff2_ksplit ? b->out_ksplit : b->ff2_ksplit;
      if (most > 1) cr.scr(&b->res_ws, sizeof(float) * most * T * C);
    }
    if (const char* e = std::getenv("ST_ATTN_CUS")) cus = std::atoi(e);
    attention_bf16_plan(B, heads, b->N, b->N, cus, b->attn_n_full, b->attn_nsplit);
    if (b->attn_nsplit > 1) {
      const long long split_tiles =
          static_cast<long long>(B) * heads * ((b->N + attention_bf16_q_tile() - 1) / attention_bf16_q_tile()) -
          b->attn_n_full;
      cr.scr(&b->attn_part, sizeof(float) * split_tiles * b->attn_nsplit * attention_bf16_part_floats());
    }
  }
  b->key_bits = static_cast<uint32_t*>(cr.alloc(sizeof(uint32_t) * 4 * B, "context key mask"));
  b->kc = cr.alloc(b->ctx_layer_stride * depth * es, "context K");
  b->vct = cr.alloc(b->ctx_layer_stride * depth * es, "context V^T");
  // Padding rows of the per-head buffers are read by the attention kernels
  // and must hold finite values; no kernel ever writes them.
  if (cr.ok() && head_pad) {
    cr.dev(hipMemsetAsync(b->q, 0, headbuf, s), "clear Q");
    cr.dev(hipMemsetAsync(b->k, 0, headbuf, s), "clear K");
    cr.dev(hipMemsetAsync(b->vt, 0, headbuf, s), "clear V^T");
  }
  if (!external_scratch && cr.ok()) {
    void* arena = cr.alloc(b->scratch.bytes, "workspace");
    if (arena) {
      b->scratch_own = arena;
      stb_block_bind_scratch(b, arena);
    }
  }
  if (cr.ok()) {
    cr.dev(hipMemsetAsync(b->kc, 0, b->ctx_layer_stride * depth * es, s), "clear context K");
    cr.dev(hipMemsetAsync(b->vct, 0, b->ctx_layer_stride * depth * es, s), "clear context V^T");
  }
  if (cr.ok()) cr.dev(hipStreamSynchronize(s), "create: synchronise");
  if (cr.ok() && cr.overflow) {
    int flag = 0;
    cr.dev(hipMemcpy(&flag, cr.overflow, sizeof(int), hipMemcpyDeviceToHost), "overflow flag");
    if (cr.ok() && flag) {
      cr.st = ST_ERR_UNSUPPORTED;
      cr.msg = "a projection weight exceeds the fp16 range (|w| > 65504)";
    }
  }
  if (!cr.ok()) {
    (void)hipStreamSynchronize(s);
    (void)hipGetLastError();
    free_all(b);
    delete b;
    return fail(cr.st, cr.msg);
  }
  b->persist = nullptr;  // create is over: nothing more is taken from it
  *out = b;
  return ST_OK;
}

namespace {

hipEvent_t take_event(st_block* b) {
  if (!b->spare_events.empty()) {
    hipEvent_t e = b->spare_events.back();
    b->spare_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // Timing only: without the system-scope fence, recording an event does not
  // write back and invalidate the caches (a gap of several microseconds
  // between kernels on a multi-XCD GPU otherwise); the caller synchronises
  // its stream before the times are read.
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}

// Runs `launch` and, if its kind is selected (and, inside the layer loop,
// its layer is below the timing_layers limit), brackets it with events.
template <class Fn>
hipError_t run(st_block* b, int kind, hipStream_t s, Fn&& launch) {
  if (!((b->timing_mask >> kind) & 1u)) return launch();
  if (b->timing_layers > 0 && b->timing_layer >= b->timing_layers) return launch();
  hipEvent_t e0 = take_event(b), e1 = take_event(b);
  if (!e0 || !e1) {
    if (e0) b->spare_events.push_back(e0);
    if (e1) b->spare_events.push_back(e1);
    return launch();
  }
  hipError_t r = hipEventRecord(e0, s);
  if (r != hipSuccess) return r;
  r = launch();
  if (r != hipSuccess) return r;
  r = hipEventRecord(e1, s);
  b->pending.push_back({kind, e0, e1});
  return r;
}

// LayerNorm's epsilon (the default of the pages' Transformer blocks).
constexpr float kLayerNormEps = 1e-5f;

GemmParams gemm(const void* A, long long lda, const void* Bm, long long ldb,
                int M, int N, int K, int kind) {
  GemmParams p{};
  p.A = A; p.lda = lda; p.B = Bm; p.ldb = ldb;
  p.M = M; p.N = N; p.K = K;
  p.epi.kind = kind;
  for (float& v : p.epi.hs.scale) v = 1.f;
  return p;
}

#define ST_TRY(expr, what)                         \
  do {                                             \
    hipError_t e_ = (expr);                        \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

st_status forward_impl(st_block* b, const void* x, const void* ctx, const uint8_t* ctx_mask,
                       void* y, int stop_stage, float* h_out, hipStream_t s) {
  if (!b->scratch_bound) return fail(ST_ERR_INVALID, "the handle's workspace is not bound");
  const bool bf = b->bf16;
  const int B = b->B, C = b->C, N = b->N, T = b->T, F = b->F, D = b->D;
  // 16-bit path operand types: fp16 where an activation produced by a norm
  // or by GEGLU meets a weight, bf16 for attention outputs and the context.
  const int act = bf ? ACT_F16 : ACT_F32;
  auto G = [&](const GemmParams& p, int op) {
    return bf ? gemm_mfma(p, op, s) : gemm_f32(p, s);
  };
  // bf16 path: the residual stream is kept in fp16 (h16); every product
  // that writes it also leaves its per-row statistics, and the products
  // behind a LayerNorm read it with the norm folded into their weights (no
  // LayerNorm launch).
  auto keep_h = [&](GemmParams& p) {
    if (!bf) return;
    p.epi.kind = p.epi.kind == EPI_STORE_F32 ? EPI_STORE_H16 : EPI_RESID_H16;
    p.epi.out_f32 = nullptr;
    p.epi.out_act = b->hcopy;
    p.epi.row_stats = b->hstats;
    p.epi.range_flag = b->range_flag;
  };
  // K slices of a residual product (bf16 path; set at create)
  auto split_k = [&](GemmParams& p, int slices) {
    if (!bf || slices <= 1) return;
    p.ksplit = slices;
    p.ws = b->res_ws;
  };
  // h of the stage dump as fp32
  auto dump_h = [&]() {
    return bf ? f16_to_f32(b->hcopy, h_out, static_cast<long long>(T) * C, s)
              : hipMemcpyAsync(h_out, b->h, static_cast<size_t>(T) * C * sizeof(float),
                               hipMemcpyDeviceToDevice, s);
  };
  // bf16 path with whole 64-token blocks per sample: the cross-attention
  // runs in the epilogue of its Q projection (77 context keys)
  const bool cross_fused = bf && N % 64 == 0;
  auto normed = [&](GemmParams& p, const LayerDev& L, int i) {
    if (!bf) return;
    p.A = b->hcopy;
    p.epi.ln_stats = b->hstats; p.epi.ln_g = L.ln_g[i];
    p.epi.ln_blocks = C / 64; p.epi.ln_eps = kLayerNormEps;
  };

  // the context's key padding mask as bits (read by every cross-attention)
  const uint32_t* key_bits = nullptr;
  if (ctx_mask) {
    ST_TRY(mask_to_bits(ctx_mask, b->key_bits, B, ST_CTX_LEN, s), "context key mask");
    key_bits = b->key_bits;
  }
  ST_TRY(run(b, ST_K_GN_STATS, s, [&] {
           return gn_stats(x, bf, B, C, N, b->gn_part, b->gn_max_split, s);
         }), "GroupNorm statistics");
  ST_TRY(run(b, ST_K_PROJ_IN, s, [&] {
           hipError_t e = gn_apply_tokens(x, bf, b->gn_part, b->gn_max_split, b->gn_w, b->gn_b,
                                          b->u, act, B, C, N, b->range_flag, s);
           if (e != hipSuccess) return e;
           GemmParams p = gemm(b->u, C, b->w_in, C, T, C, C, EPI_STORE_F32);
           p.epi.bias = b->b_in; p.epi.out_f32 = b->h; p.epi.ldo = C;
           keep_h(p);
           return G(p, ACT_F16);
         }), "proj_in");
  int stage = 0;
  auto dump = [&]() -> bool { return stop_stage >= 0 && stage == stop_stage; };
  if (dump()) {
    ST_TRY(dump_h(), "stage copy");
    return ST_OK;
  }

  ST_TRY(run(b, ST_K_CTX_KV, s, [&] {
           GemmParams p = gemm(ctx, D, b->wkv, D, B * ST_CTX_LEN, 2 * C * b->depth, D, EPI_HEADS);
           p.epi.bias = b->bkv;
           p.epi.hs.dst[0] = b->kc; p.epi.hs.dst[1] = b->vct; p.epi.hs.dst[2] = nullptr;
           p.epi.hs.transposed_mask = 2; p.epi.hs.nsplit = 2;
           p.epi.hs.layer_stride = b->ctx_layer_stride;
           p.epi.hs.rows_per_batch = ST_CTX_LEN; p.epi.hs.npad = b->cpad;
           p.epi.hs.heads = b->heads; p.epi.hs.C = C;
           p.ksplit = b->ctx_ksplit; p.ws = b->ctx_ws;
           return G(p, ACT_BF16);
         }), "context K/V projection");

  for (int l = 0; l < b->depth; ++l) {
    const LayerDev& L = b->L[l];
    b->timing_layer = l;
    // ---- self-attention sublayer
    if (!bf)
      ST_TRY(run(b, ST_K_LAYERNORM, s, [&] {
               return layernorm(b->h, L.ln_w[0], L.ln_b[0], b->u, act, T, C, s);
             }), "LayerNorm 1");
    ST_TRY(run(b, ST_K_QKV, s, [&] {
             GemmParams p = gemm(b->u, C, L.wqkv, C, T, 3 * C, C, EPI_HEADS);
             normed(p, L, 0);
             p.epi.bias = L.bqkv;
             p.epi.hs.dst[0] = b->q; p.epi.hs.dst[1] = b->k; p.epi.hs.dst[2] = b->vt;
             if (bf) p.epi.hs.scale[0] = attention_bf16_q_scale();
             p.epi.hs.transposed_mask = 4; p.epi.hs.nsplit = 3; p.epi.hs.layer_stride = 0;
             p.epi.hs.rows_per_batch = N; p.epi.hs.npad = b->npad;
             p.epi.hs.heads = b->heads; p.epi.hs.C = C;
             return G(p, ACT_F16);
           }), "Q/K/V projection");
    ST_TRY(run(b, ST_K_SELF_ATTN, s, [&] {
             AttnParams a{};
             a.q = b->q; a.k = b->k; a.vt = b->vt; a.o = b->o;
             a.B = B; a.heads = b->heads; a.C = C; a.Nq = N; a.Nk = N;
             a.q_pad = b->npad; a.kv_pad = b->npad;
             a.n_full = b->attn_n_full; a.nsplit = b->attn_nsplit;
             a.part = b->attn_part;
             return bf ? attention_bf16(a, s) : attention_f32(a, s);
           }), "self-attention");
    ST_TRY(run(b, ST_K_ATTN_OUT, s, [&] {
             GemmParams p = gemm(b->o, C, L.wo1, C, T, C, C, EPI_RESID_F32);
             p.epi.bias = L.bo1; p.epi.out_f32 = b->h; p.epi.ldo = C;
             keep_h(p);
             split_k(p, b->out_ksplit);
             return G(p, ACT_BF16);
           }), "self-attention out-projection");
    ++stage;
    if (dump()) break;
    // ---- cross-attention sublayer
    if (!bf)
      ST_TRY(run(b, ST_K_LAYERNORM, s, [&] {
               return layernorm(b->h, L.ln_w[1], L.ln_b[1], b->u, act, T, C, s);
             }), "LayerNorm 2");
    const void* kc_l = static_cast<const char*>(b->kc) + l * b->ctx_layer_stride * b->esz;
    const void* vct_l = static_cast<const char*>(b->vct) + l * b->ctx_layer_stride * b->esz;
    ST_TRY(run(b, ST_K_CROSS_Q, s, [&] {
             GemmParams p = gemm(b->u, C, L.wq2, C, T, C, C, cross_fused ? EPI_CROSS_ATTN : EPI_HEADS);
             normed(p, L, 1);
             p.epi.bias = L.bq2;
             if (cross_fused) {
               // the cross-attention runs in this product's epilogue
               p.epi.out_act = b->o; p.epi.ldo = C;
               p.epi.ca.k = kc_l; p.epi.ca.vt = vct_l;
               p.epi.ca.kv_pad = b->cpad; p.epi.ca.nk = ST_CTX_LEN;
               p.epi.ca.rows_per_batch = N; p.epi.ca.heads = b->heads;
               p.epi.ca.scale = attention_bf16_q_scale();
               p.epi.ca.key_bits = key_bits;
               return G(p, ACT_F16);
             }
             p.epi.hs.dst[0] = b->q; p.epi.hs.dst[1] = nullptr; p.epi.hs.dst[2] = nullptr;
             if (bf) p.epi.hs.scale[0] = attention_bf16_q_scale();
             p.epi.hs.transposed_mask = 0; p.epi.hs.nsplit = 1; p.epi.hs.layer_stride = 0;
             p.epi.hs.rows_per_batch = N; p.epi.hs.npad = b->npad;
             p.epi.hs.heads = b->heads; p.epi.hs.C = C;
             return G(p, ACT_F16);
           }), "cross-attention Q projection");
    if (!cross_fused) ST_TRY(run(b, ST_K_CROSS_ATTN, s, [&] {
             AttnParams a{};
             a.q = b->q;
             a.k = kc_l;
             a.vt = vct_l;
             a.o = b->o;
             a.B = B; a.heads = b->heads; a.C = C; a.Nq = N; a.Nk = ST_CTX_LEN;
             a.q_pad = b->npad; a.kv_pad = b->cpad;
             a.key_bits = key_bits;
             return bf ? attention_bf16(a, s) : attention_f32(a, s);
           }), "cross-attention");
    ST_TRY(run(b, ST_K_ATTN_OUT, s, [&] {
             GemmParams p = gemm(b->o, C, L.wo2, C, T, C, C, EPI_RESID_F32);
             p.epi.bias = L.bo2; p.epi.out_f32 = b->h; p.epi.ldo = C;
             keep_h(p);
             split_k(p, b->out_ksplit);
             return G(p, ACT_BF16);
           }), "cross-attention out-projection");
    ++stage;
    if (dump()) break;
    // ---- feed-forward sublayer
    if (!bf)
      ST_TRY(run(b, ST_K_LAYERNORM, s, [&] {
               return layernorm(b->h, L.ln_w[2], L.ln_b[2], b->u, act, T, C, s);
             }), "LayerNorm 3");
    ST_TRY(run(b, ST_K_FF1_GEGLU, s, [&] {
             if (bf) {
               GemmParams p = gemm(b->u, C, L.w1, C, T, 2 * F, C, EPI_GEGLU);
               normed(p, L, 2);
               p.epi.bias = L.b1; p.epi.out_act = b->f; p.epi.F = F;
               p.epi.range_flag = b->range_flag;
               return gemm_mfma(p, ACT_F16, s);
             }
             GemmParams p = gemm(b->u, C, L.w1, C, T, 2 * F, C, EPI_STORE_F32);
             p.epi.bias = L.b1; p.epi.out_f32 = b->z; p.epi.ldo = 2 * F;
             hipError_t e = gemm_f32(p, s);
             if (e != hipSuccess) return e;
             return geglu_f32(b->z, static_cast<float*>(b->f), T, F, s);
           }), "feed-forward 1 + GEGLU");
    ST_TRY(run(b, ST_K_FF2, s, [&] {
             GemmParams p = gemm(b->f, F, L.w2, F, T, C, F, EPI_RESID_F32);
             p.epi.bias = L.b2; p.epi.out_f32 = b->h; p.epi.ldo = C;
             keep_h(p);
             split_k(p, b->ff2_ksplit);
             return G(p, ACT_F16);
           }), "feed-forward 2");
    ++stage;
    if (dump()) break;
  }
  b->timing_layer = -1;
  if (stop_stage >= 0) {
    if (stage != stop_stage) return fail(ST_ERR_INVALID, "stage out of range");
    ST_TRY(dump_h(), "stage copy");
    return ST_OK;
  }
  ST_TRY(run(b, ST_K_PROJ_OUT, s, [&] {
           // y^T orientation: rows = channels, columns = tokens, so the NCHW
           // store is contiguous along tokens; bf16 path: fp16 operands.
           GemmParams p = bf ? gemm(b->w_out, C, b->hcopy, C, C, T, C, EPI_NCHW)
                             : gemm(b->w_out, C, b->h, C, C, T, C, EPI_NCHW);
           p.epi.bias = b->b_out; p.epi.out_act = y; p.epi.resid_act = x;
           p.epi.ntok = N; p.epi.ldo = C;
           return G(p, ACT_F16);
         }), "proj_out");
  return ST_OK;
}

bool overlaps(const void* a, size_t an, const void* c, size_t cn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), c0 = reinterpret_cast<uintptr_t>(c);
  return a0 < c0 + cn && c0 < a0 + an;
}

st_status check_forward_args(st_block* b, const void* x, const void* ctx,
                             const void* y) {
  if (!b) return fail(ST_ERR_INVALID, "handle is NULL");
  if (!x || !ctx || !y) return fail(ST_ERR_INVALID, "x, ctx and y must be non-NULL");
  if (!aligned16(x) || !aligned16(ctx) || !aligned16(y))
    return fail(ST_ERR_INVALID, "x, ctx and y must be 16-byte aligned");
  const size_t xbytes = static_cast<size_t>(b->T) * b->C * b->esz;
  const size_t cbytes = static_cast<size_t>(b->B) * ST_CTX_LEN * b->D * b->esz;
  if (overlaps(y, xbytes, x, xbytes) || overlaps(y, xbytes, ctx, cbytes))
    return fail(ST_ERR_INVALID, "y overlaps x or ctx");
  return ST_OK;
}

struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) {
      err = hipSetDevice(dev);
      changed = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

}  // namespace

ST_API st_status st_block_forward(st_block* b, const void* x, const void* ctx,
                                  void* y, void* stream) {
  g_err.clear();
  st_status st = check_forward_args(b, x, ctx, y);
  if (st != ST_OK) return st;
  DeviceGuard g(b->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "select device");
  return forward_impl(b, x, ctx, nullptr, y, -1, nullptr, static_cast<hipStream_t>(stream));
}

ST_API st_status st_block_forward_masked(st_block* b, const void* x, const void* ctx,
                                         const unsigned char* ctx_mask, void* y, void* stream) {
  g_err.clear();
  st_status st = check_forward_args(b, x, ctx, y);
  if (st != ST_OK) return st;
  if (ctx_mask && overlaps(y, static_cast<size_t>(b->T) * b->C * b->esz, ctx_mask,
                           static_cast<size_t>(b->B) * ST_CTX_LEN))
    return fail(ST_ERR_INVALID, "y overlaps ctx_mask");
  DeviceGuard g(b->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "select device");
  return forward_impl(b, x, ctx, reinterpret_cast<const uint8_t*>(ctx_mask), y, -1, nullptr,
                      static_cast<hipStream_t>(stream));
}

ST_API st_status st_block_forward_stage(st_block* b, const void* x,
                                        const void* ctx, int stage,
                                        float* h_out, void* stream) {
  g_err.clear();
  if (!b) return fail(ST_ERR_INVALID, "handle is NULL");
  if (!x || !ctx || !h_out) return fail(ST_ERR_INVALID, "x, ctx and h_out must be non-NULL");
  if (!aligned16(x) || !aligned16(ctx) || !aligned16(h_out))
    return fail(ST_ERR_INVALID, "x, ctx and h_out must be 16-byte aligned");
  if (stage < 0 || stage > 3 * b->depth) return fail(ST_ERR_INVALID, "stage out of range");
  DeviceGuard g(b->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "select device");
  return forward_impl(b, x, ctx, nullptr, nullptr, stage, h_out, static_cast<hipStream_t>(stream));
}

ST_API void st_block_destroy(st_block* b) {
  if (!b) return;
  DeviceGuard g(b->device);
  // Forwards may have been enqueued on any number of streams (some perhaps
  // destroyed by now): waiting for the whole device covers every one.
  (void)hipDeviceSynchronize();
  (void)hipGetLastError();
  free_all(b);
  delete b;
}

ST_API st_status st_block_check_range(st_block* b, void* stream) {
  g_err.clear();
  if (!b) return fail(ST_ERR_INVALID, "handle is NULL");
  if (!b->range_flag) return ST_OK;  // fp32 storage keeps no fp16 intermediates
  DeviceGuard g(b->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "select device");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, b->range_flag, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "read the range flag");
  if (!flag) return ST_OK;
  e = hipMemsetAsync(b->range_flag, 0, sizeof(int), s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "clear the range flag");
  return fail(ST_ERR_RANGE,
              "an fp16 intermediate (residual stream, GEGLU output or normalised input) "
              "left the fp16 range (|value| >= 65520 or NaN): outputs of the forwards since "
              "the last check are not valid");
}

ST_API st_status st_block_set_timing(st_block* b, unsigned kind_mask) {
  g_err.clear();
  if (!b) return fail(ST_ERR_INVALID, "handle is NULL");
  b->timing_mask = kind_mask & ((1u << ST_K_COUNT) - 1u);
  return ST_OK;
}

ST_API st_status st_block_set_timing_layers(st_block* b, int layers) {
  g_err.clear();
  if (!b) return fail(ST_ERR_INVALID, "handle is NULL");
  if (layers < 0) return fail(ST_ERR_INVALID, "layers must be >= 0");
  b->timing_layers = layers;
  return ST_OK;
}

ST_API st_status st_block_read_timing_launches(st_block* b, int* kinds, double* ms,
                                              long long capacity, long long* count) {
  g_err.clear();
  if (!b || !count || (capacity > 0 && (!kinds || !ms)))
    return fail(ST_ERR_INVALID, "handle, count, kinds or ms is NULL");
  st_status st = ST_OK;
  long long n = 0;
  for (auto& t : b->pending) {
    float v = 0.f;
    hipError_t e = hipEventElapsedTime(&v, t.e0, t.e1);
    if (e != hipSuccess && st == ST_OK) st = hip_fail(e, "hipEventElapsedTime (stream not synchronised?)");
    if (n < capacity) {
      kinds[n] = t.kind;
      ms[n] = v;
    }
    ++n;
    b->spare_events.push_back(t.e0);
    b->spare_events.push_back(t.e1);
  }
  b->pending.clear();
  *count = n;
  return st;
}

ST_API st_status st_measure_mfma_bf16(int iters, void* stream, double* tflops,
                                      double* sclk_mhz) {
  g_err.clear();
  if (!tflops || !sclk_mhz || iters < 1) return fail(ST_ERR_INVALID, "bad arguments");
  int dev = 0, cus = 0, wall_khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return hip_fail(e, "device attributes");
  const int grid = mfma_probe_grid(cus);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* out = nullptr;
  long long* clocks = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  std::vector<long long> host(2 * static_cast<size_t>(grid));
  float ms = 0.f;
  e = hipMalloc(&out, sizeof(float) * 256 * grid);
  if (e == hipSuccess) e = hipMalloc(&clocks, sizeof(long long) * 2 * grid);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = mfma_probe(grid, iters, out, clocks, s);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) e = mfma_probe(grid, iters, out, clocks, s);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e == hipSuccess)
    e = hipMemcpy(host.data(), clocks, sizeof(long long) * 2 * grid, hipMemcpyDeviceToHost);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (clocks) (void)hipFree(clocks);
  if (e != hipSuccess) return hip_fail(e, "MFMA probe");
  double cyc = 0.0, ticks = 0.0;
  for (int i = 0; i < grid; ++i) {
    cyc += static_cast<double>(host[2 * i]);
    ticks += static_cast<double>(host[2 * i + 1]);
  }
  *tflops = static_cast<double>(mfma_probe_flops(grid, iters)) / (ms * 1e-3) / 1e12;
  *sclk_mhz = ticks > 0.0 ? cyc / ticks * (wall_khz / 1000.0) : 0.0;
  return ST_OK;
}

ST_API st_status st_block_read_timing(st_block* b, st_timing* out) {
  g_err.clear();
  if (!b || !out) return fail(ST_ERR_INVALID, "handle or out is NULL");
  std::memset(out, 0, sizeof(*out));
  st_status st = ST_OK;
  for (auto& t : b->pending) {
    float ms = 0.f;
    hipError_t e = hipEventElapsedTime(&ms, t.e0, t.e1);
    if (e != hipSuccess && st == ST_OK) st = hip_fail(e, "hipEventElapsedTime (stream not synchronised?)");
    out->ms[t.kind] += ms;
    out->launches[t.kind] += 1;
    b->spare_events.push_back(t.e0);
    b->spare_events.push_back(t.e1);
  }
  b->pending.clear();
  return st;
}
