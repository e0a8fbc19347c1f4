// C ABI of one U-Net denoiser timestep (include/st_unet.h): the parts are
// the library's ResnetBlock2D and Spatial-Transformer handles; the U-Net
// adds the embedding MLPs, conv_in, the DownSample / UpSample convolutions,
// the skip concatenations and the output GroupNorm + SiLU + conv_out.
//
// Every 3x3 convolution of the U-Net runs on the implicit-GEMM path of the
// ResNets: its input is written into a zero-haloed NHWC fp16 buffer (channels
// padded to a multiple of 64 for conv_in; nearest 2x upsampling done by the
// same pass for UpSample; GroupNorm + SiLU for conv_out), and the GEMM reads
// the nine taps as row offsets of that buffer (stride 2: every other pixel
// row, the DownSample).  Skip tensors stay resident in HBM (bf16 NCHW) from
// the down path to the up path; a skip concatenation is two strided copies.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <new>
#include <string>
#include <vector>

#include "../../include/st_unet.h"
#include "kernels.h"
#include "parts.h"

#define ST_API extern "C" __attribute__((visibility("default")))

using namespace stb;

st_status st_set_error(st_status s, const std::string& msg);

namespace {

constexpr int kMaxSplit = 64;

// One 3x3 convolution of the U-Net (conv_in, DownSample, UpSample, conv_out).
struct Conv {
  int Cin, Cp, Cout, stride, up, gn;
  int Hi, Wi;          // input map
  int Hg, Wg;          // operand grid (Hi, Wi, or twice that with up)
  int Ho, Wo, Wp;
  long long prows;
  void* w;             // fp16 [Cout][9 Cp]
  float* cadd;         // [B][Cout]
  void* P;             // operand buffer, zero halo (scratch)
  float *gn_w, *gn_b;  // conv_out's GroupNorm
  int ksplit;          // K slices (1 = none), partial products in st_unet::ws
};

}  // namespace

struct st_unet {
  st_unet_config cfg;
  int B, H, W, device;
  std::vector<void*> allocs;
  std::vector<st_resnet*> res;
  std::vector<st_block*> blk;
  std::vector<Conv> convs;  // conv_in, down[levels-1], up[levels-1], conv_out
  // embedding MLPs
  void *t1w, *t2w, *a1w, *a2w;
  float *t1b, *t2b, *a1b, *a2b;
  float *emb, *mid1, *temb, *amid;
  void* temb16;
  float2* part;
  // activations
  std::vector<void*> skips;       // down-path outputs, in push order
  std::vector<long long> skip_c;  // their channels
  std::vector<int> skip_h, skip_w;
  void *ta, *tb, *cat;            // work maps and the concatenation (bf16 NCHW)
  int* range_flag;
  float* ws;                      // split-K partial products of the convolutions
  // The parts run one after another on one stream, so the buffers that each
  // rewrites in every forward (its ScratchPlan) and the U-Net's own (the
  // convolutions' GroupNorm partials and split-K products) share one arena
  // of the largest plan's size.
  ScratchPlan scratch;
  void* arena;
  DevArena* persist;  // arena of the persistent allocations during create
  unsigned long long bytes;
};

namespace {

st_status fail(st_status s, const std::string& msg) { return st_set_error(s, msg); }
st_status hip_fail(hipError_t e, const char* what) {
  return fail(ST_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void free_all(st_unet* u) {
  for (st_resnet* r : u->res) st_resnet_destroy(r);
  u->res.clear();
  for (st_block* b : u->blk) st_block_destroy(b);
  u->blk.clear();
  for (void* p : u->allocs) (void)hipFree(p);
  u->allocs.clear();
}

struct Maker {
  st_unet* u;
  hipStream_t s;
  st_status st = ST_OK;
  std::string msg{};
  bool ok() const { return st == ST_OK; }
  void dev(hipError_t e, const char* what) {
    if (ok() && e != hipSuccess) { st = ST_ERR_DEVICE; msg = std::string(what) + ": " + hipGetErrorString(e); }
  }
  void part(st_status r, const char* what) {
    if (ok() && r != ST_OK) { st = r; msg = std::string(what) + ": " + st_last_error(); }
  }
  void* alloc(size_t bytes, const char* what) {
    if (!ok()) return nullptr;
    if (!bytes) bytes = 16;
    void* p = nullptr;
    if (u->persist && u->persist->base) {
      p = u->persist->take(bytes);
    } else if (hipMalloc(&p, bytes) == hipSuccess) {
      u->allocs.push_back(p);
      if (u->persist) u->persist->count(bytes);
    } else {
      (void)hipGetLastError();
      p = nullptr;
    }
    if (!p) {
      st = ST_ERR_OUT_OF_MEMORY;
      msg = std::string("out of device memory allocating ") + what;
    }
    return p;
  }
  float* vec(const void* src, long long n, float fill, const char* what) {
    float* d = static_cast<float*>(alloc(n * sizeof(float), what));
    if (d) dev(to_f32(src, true, d, n, fill, s), what);
    return d;
  }
  void* copy(const void* src, size_t bytes, const char* what) {
    void* d = alloc(bytes, what);
    if (d) dev(hipMemcpyAsync(d, src, bytes, hipMemcpyDeviceToDevice, s), what);
    return d;
  }
  // a convolution layer: weights packed (its operand map is scratch,
  // placed once the list of layers is complete)
  Conv conv(const void* w, const void* b, int Cin, int Cout, int Hi, int Wi, int stride, int up,
            int gn, const void* gn_w, const void* gn_b, int* overflow, const char* what) {
    Conv c{};
    c.Cin = Cin; c.Cp = (Cin + 63) / 64 * 64; c.Cout = Cout; c.stride = stride; c.up = up; c.gn = gn;
    c.Hi = Hi; c.Wi = Wi;
    c.Hg = up ? 2 * Hi : Hi; c.Wg = up ? 2 * Wi : Wi;
    c.Ho = stride == 2 ? c.Hg / 2 : c.Hg; c.Wo = stride == 2 ? c.Wg / 2 : c.Wg;
    c.Wp = (c.Wg + 2 + 3) / 4 * 4;
    c.prows = static_cast<long long>(u->B) * (c.Hg + 2) * c.Wp + 2LL * c.Wp + 8;
    c.w = alloc(static_cast<size_t>(Cout) * 9 * c.Cp * 2, what);
    if (c.w) dev(conv_weight_pack_padded(w, nullptr, c.w, Cout, Cin, c.Cp, 0, overflow, s), what);
    c.cadd = static_cast<float*>(alloc(sizeof(float) * u->B * Cout, what));
    if (c.cadd) {
      float* bias = vec(b, Cout, 0.f, what);
      for (int i = 0; i < u->B && ok(); ++i)
        dev(hipMemcpyAsync(c.cadd + static_cast<long long>(i) * Cout, bias, sizeof(float) * Cout,
                           hipMemcpyDeviceToDevice, s), what);
    }
    c.P = nullptr;
    if (gn) {
      c.gn_w = vec(gn_w, Cin, 1.f, what);
      c.gn_b = vec(gn_b, Cin, 0.f, what);
    }
    return c;
  }
};

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

hipError_t run_conv(st_unet* u, const Conv& c, const void* x, void* y, hipStream_t s) {
  hipError_t e;
  if (c.gn) {
    e = gn_stats(x, true, u->B, c.Cin, c.Hi * c.Wi, u->part, kMaxSplit, s);
    if (e == hipSuccess)
      e = gn_apply_pad(x, u->part, kMaxSplit, c.gn_w, c.gn_b, c.P, u->B, c.Cin, c.Hi, c.Wi, c.Wp, c.Cp,
                       1e-5f, nullptr, 0, 0, u->range_flag, s);
  } else {
    e = nchw_to_pad(x, c.P, u->B, c.Cin, c.Hi, c.Wi, c.Wp, c.Cp, c.up != 0, u->range_flag, s);
  }
  if (e != hipSuccess) return e;
  GemmParams p{};
  p.A = c.w; p.lda = 9 * c.Cp;
  p.B = c.P; p.ldb = static_cast<long long>(c.stride) * c.Cp;
  p.M = c.Cout;
  p.K = 9 * c.Cp;
  p.epi.kind = EPI_CONV;
  p.conv.L = c.Cp; p.conv.Wp = c.Wp;
  p.conv.Hq = c.stride == 2 ? (c.Hg + 2) / 2 : c.Hg + 2;
  p.conv.Ho = c.Ho; p.conv.Wo = c.Wo;
  p.N = u->B * p.conv.Hq * c.Wp;
  p.conv.spt = c.Cp / 64; p.conv.sc_spt = 0; p.conv.sc_cbase = 0; p.conv.sc_roff = c.Wp + 1;
  p.conv.b_bytes = c.prows * c.Cp * 2;
  p.conv.cadd = c.cadd; p.conv.resid = nullptr; p.conv.out = y;
  if (c.ksplit > 1) {
    p.ksplit = c.ksplit;
    p.ws = u->ws;
  }
  return gemm_mfma(p, ACT_F16, s);
}

st_status unet_build(const st_unet_config* cfg, int B, int H, int W, const st_unet_weights* w,
                     hipStream_t s, int dev, DevArena* persist, st_unet** out);

// dst [B][C1 + C2][HW] = concat(a [B][C1][HW], b [B][C2][HW]) along channels
hipError_t concat(void* dst, const void* a, long long C1, const void* b, long long C2, long long HW,
                  int B, hipStream_t s) {
  const size_t pa = C1 * HW * 2, pb = C2 * HW * 2, pd = pa + pb;
  hipError_t e = hipMemcpy2DAsync(dst, pd, a, pa, pa, B, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return e;
  return hipMemcpy2DAsync(static_cast<char*>(dst) + pa, pd, b, pb, pb, B, hipMemcpyDeviceToDevice, s);
}

}  // namespace

ST_API st_status st_unet_create(const st_unet_config* cfg, int B, int H, int W,
                                const st_unet_weights* w, void* stream, st_unet** out) {
  st_set_error(ST_OK, "");
  if (!out) return fail(ST_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!cfg || !w) return fail(ST_ERR_INVALID, "config and weights must be non-NULL");
  const int L = cfg->levels;
  if (L < 1 || L > 4) return fail(ST_ERR_INVALID, "levels must be 1 .. 4");
  if (B < 1 || B > 4) return fail(ST_ERR_UNSUPPORTED, "B must be 1 .. 4");
  if (cfg->in_channels < 1 || cfg->in_channels > 64 || cfg->out_channels < 1 || cfg->out_channels > 64)
    return fail(ST_ERR_INVALID, "in_channels and out_channels must be 1 .. 64");
  if (cfg->layers_per_block < 1 || cfg->mid_depth < 0 || cfg->add_in < 0)
    return fail(ST_ERR_INVALID, "layers_per_block >= 1, mid_depth >= 0, add_in >= 0");
  if (cfg->ctx_dim < 64 || cfg->ctx_dim % 64) return fail(ST_ERR_INVALID, "ctx_dim must be a multiple of 64");
  for (int l = 0; l < L; ++l)
    if (cfg->channels[l] < 64 || cfg->channels[l] % 64 || cfg->depths[l] < 0)
      return fail(ST_ERR_INVALID, "channels must be multiples of 64, depths >= 0");
  const int f = 1 << (L - 1);
  if (H < 1 || W < 1 || H % f || (W / f) % 4 || W % f)
    return fail(ST_ERR_UNSUPPORTED, "H must be a multiple of 2^(levels-1) and W / 2^(levels-1) of 4");
  if (!w->resnets || !w->conv_in_w || !w->conv_out_w || !w->time1_w || !w->time2_w ||
      (L > 1 && (!w->down_w || !w->up_w)) || (cfg->add_in && (!w->add1_w || !w->add2_w)))
    return fail(ST_ERR_INVALID, "a required weight is NULL");
  int nblk = cfg->mid_depth ? 1 : 0;
  for (int l = 0; l < L; ++l)
    if (cfg->depths[l]) nblk += cfg->layers_per_block + (cfg->layers_per_block + 1);
  if (nblk && !w->blocks) return fail(ST_ERR_INVALID, "blocks is NULL");
  const int C0 = cfg->channels[0], Td = 4 * C0;
  if (!temb_proj_supported(B, C0) || !temb_proj_supported(B, Td) ||
      (cfg->add_in && !temb_proj_supported(B, cfg->add_in)))
    return fail(ST_ERR_UNSUPPORTED, "embedding widths must be multiples of 8 with B * width <= 16384");

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_fail(e, "hipGetDevice");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // First build: every allocation from the runtime, sizes counted; then the
  // handle again, packed into one block of the counted size (DevArena).
  DevArena count;
  st_unet* u = nullptr;
  st_status st = unet_build(cfg, B, H, W, w, s, dev, &count, &u);
  if (st != ST_OK) return st;
  free_all(u);
  delete u;
  u = nullptr;
  size_t free0 = 0, total = 0;
  (void)hipMemGetInfo(&free0, &total);
  void* block = nullptr;
  if (hipMalloc(&block, count.counted) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ST_ERR_OUT_OF_MEMORY, "out of device memory allocating the U-Net's block");
  }
  DevArena packed;
  packed.base = static_cast<char*>(block);
  packed.cap = count.counted;
  st = unet_build(cfg, B, H, W, w, s, dev, &packed, &u);
  if (st != ST_OK) {
    (void)hipFree(block);
    return st;
  }
  u->allocs.push_back(block);
  size_t free1 = 0;
  (void)hipMemGetInfo(&free1, &total);
  u->bytes = free0 > free1 ? static_cast<unsigned long long>(free0 - free1) : 0ull;
  *out = u;
  return ST_OK;
}

namespace {

// One build of the handle (validated arguments); on failure nothing is kept.
st_status unet_build(const st_unet_config* cfg, int B, int H, int W, const st_unet_weights* w,
                     hipStream_t s, int dev, DevArena* persist, st_unet** out) {
  const int L = cfg->levels;
  const int C0 = cfg->channels[0], Td = 4 * C0;
  st_unet* u = new (std::nothrow) st_unet();
  if (!u) return fail(ST_ERR_OUT_OF_MEMORY, "host allocation failed");
  u->cfg = *cfg; u->B = B; u->H = H; u->W = W; u->device = dev;
  u->persist = persist;
  Maker mk{u, s};
  int* overflow = static_cast<int*>(mk.alloc(sizeof(int), "overflow flag"));
  if (overflow) mk.dev(hipMemsetAsync(overflow, 0, sizeof(int), s), "overflow flag");
  u->range_flag = static_cast<int*>(mk.alloc(sizeof(int), "range flag"));
  if (u->range_flag) mk.dev(hipMemsetAsync(u->range_flag, 0, sizeof(int), s), "range flag");
  // embedding MLPs
  u->t1w = mk.copy(w->time1_w, static_cast<size_t>(Td) * C0 * 2, "time1_w");
  u->t1b = mk.vec(w->time1_b, Td, 0.f, "time1_b");
  u->t2w = mk.copy(w->time2_w, static_cast<size_t>(Td) * Td * 2, "time2_w");
  u->t2b = mk.vec(w->time2_b, Td, 0.f, "time2_b");
  if (cfg->add_in) {
    u->a1w = mk.copy(w->add1_w, static_cast<size_t>(Td) * cfg->add_in * 2, "add1_w");
    u->a1b = mk.vec(w->add1_b, Td, 0.f, "add1_b");
    u->a2w = mk.copy(w->add2_w, static_cast<size_t>(Td) * Td * 2, "add2_w");
    u->a2b = mk.vec(w->add2_b, Td, 0.f, "add2_b");
  }
  u->emb = static_cast<float*>(mk.alloc(sizeof(float) * B * C0, "embedding"));
  u->mid1 = static_cast<float*>(mk.alloc(sizeof(float) * B * Td, "embedding MLP"));
  u->amid = static_cast<float*>(mk.alloc(sizeof(float) * B * Td, "embedding MLP"));
  u->temb = static_cast<float*>(mk.alloc(sizeof(float) * B * Td, "time embedding"));
  u->temb16 = mk.alloc(2ull * B * Td, "time embedding (bf16)");
  u->scratch.add(&u->part, sizeof(float2) * B * ST_GN_GROUPS * kMaxSplit);

  // parts, in execution order; the largest output held by a work map (a
  // ResNet's, a transformer block's or an UpSample's) and the largest
  // concatenation sized for the buffers
  long long maxwork = 0;
  long long maxcat = 0;
  int ri = 0, bi = 0;
  auto add_res = [&](int Ci, int Co, int h, int wd) {
    st_resnet* r = nullptr;
    if (mk.ok()) mk.part(stb_resnet_create(B, Ci, Co, h, wd, Td, 1e-5f, ST_DTYPE_BF16, &w->resnets[ri], s,
                                           true, persist, &r),
                         "ResnetBlock2D");
    ++ri;
    if (r) u->res.push_back(r);
    maxwork = std::max(maxwork, static_cast<long long>(B) * Co * h * wd);
  };
  auto add_blk = [&](int C, int depth, int h, int wd) {
    st_block* b = nullptr;
    if (mk.ok()) mk.part(stb_block_create(B, C, h, wd, C / 64, cfg->ctx_dim, depth, ST_DTYPE_BF16,
                                          &w->blocks[bi], s, true, persist, &b), "Spatial-Transformer block");
    ++bi;
    if (b) u->blk.push_back(b);
  };
  u->convs.push_back(mk.conv(w->conv_in_w, w->conv_in_b, cfg->in_channels, C0, H, W, 1, 0, 0, nullptr, nullptr,
                             overflow, "conv_in"));
  std::vector<long long> sk = {C0};
  std::vector<int> skh = {H}, skw = {W};
  int ch = C0, h = H, wd = W;
  for (int l = 0; l < L && mk.ok(); ++l) {
    const int c = cfg->channels[l];
    for (int r = 0; r < cfg->layers_per_block; ++r) {
      add_res(ch, c, h, wd);
      ch = c;
      if (cfg->depths[l]) add_blk(c, cfg->depths[l], h, wd);
      sk.push_back(c); skh.push_back(h); skw.push_back(wd);
    }
    if (l < L - 1) {
      u->convs.push_back(mk.conv(w->down_w[l], w->down_b ? w->down_b[l] : nullptr, c, c, h, wd, 2, 0, 0,
                                 nullptr, nullptr, overflow, "DownSample"));
      h /= 2; wd /= 2;
      sk.push_back(c); skh.push_back(h); skw.push_back(wd);
    }
  }
  add_res(ch, ch, h, wd);
  if (cfg->mid_depth) add_blk(ch, cfg->mid_depth, h, wd);
  add_res(ch, ch, h, wd);
  std::vector<long long> pop = sk;
  for (int lv = L - 1; lv >= 0 && mk.ok(); --lv) {
    const int c = cfg->channels[lv];
    for (int r = 0; r < cfg->layers_per_block + 1; ++r) {
      const long long s2 = pop.back();
      pop.pop_back();
      maxcat = std::max(maxcat, static_cast<long long>(B) * (ch + s2) * h * wd);
      add_res(static_cast<int>(ch + s2), c, h, wd);
      ch = c;
      if (cfg->depths[lv]) add_blk(c, cfg->depths[lv], h, wd);
    }
    if (lv > 0) {
      u->convs.push_back(mk.conv(w->up_w[L - 1 - lv], w->up_b ? w->up_b[L - 1 - lv] : nullptr, c, c, h, wd, 1,
                                 1, 0, nullptr, nullptr, overflow, "UpSample"));
      h *= 2; wd *= 2;
      maxwork = std::max(maxwork, static_cast<long long>(B) * c * h * wd);
    }
  }
  u->convs.push_back(mk.conv(w->conv_out_w, w->conv_out_b, C0, cfg->out_channels, H, W, 1, 0, 1, w->norm_out_w,
                             w->norm_out_b, overflow, "conv_out"));
  // skips (resident from the down path to the up path) and work maps
  for (size_t i = 0; i < sk.size() && mk.ok(); ++i) {
    u->skips.push_back(mk.alloc(2ull * B * sk[i] * skh[i] * skw[i], "skip"));
    u->skip_c.push_back(sk[i]);
    u->skip_h.push_back(skh[i]);
    u->skip_w.push_back(skw[i]);
  }
  u->ta = mk.alloc(2ull * maxwork, "work map");
  u->tb = mk.alloc(2ull * maxwork, "work map");
  u->cat = mk.alloc(2ull * maxcat, "concatenation");
  // K slices of the convolutions with few output tiles, one workspace
  {
    int cus = 0;
    mk.dev(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "CU count");
    long long wsf = 0;
    for (Conv& cv : u->convs) {
      const int Hq = cv.stride == 2 ? (cv.Hg + 2) / 2 : cv.Hg + 2;
      const int N = B * Hq * cv.Wp;
      cv.ksplit = conv_ksplit(cv.Cout, N, 9 * cv.Cp, cus);
      if (cv.ksplit > 1)
        wsf = std::max(wsf, static_cast<long long>(cv.ksplit) * cv.Cout * ((N + 63) / 64 * 64));
    }
    u->ws = nullptr;
    if (wsf) u->scratch.add(&u->ws, sizeof(float) * wsf);
  }
  // operand maps of the convolutions (their padding passes write the halo):
  // one at a time, so all of them start at the same offset
  size_t pmax = 0;
  for (const Conv& cv : u->convs) pmax = std::max(pmax, static_cast<size_t>(cv.prows) * cv.Cp * 2);
  const size_t pmap_off = u->scratch.reserve(pmax);
  // the shared arena
  if (mk.ok()) {
    size_t arena = u->scratch.bytes;
    for (st_resnet* r : u->res) arena = std::max(arena, stb_resnet_scratch_bytes(r));
    for (st_block* b : u->blk) arena = std::max(arena, stb_block_scratch_bytes(b));
    u->arena = mk.alloc(arena, "shared workspace");
    if (u->arena) {
      u->scratch.bind(u->arena);
      for (Conv& cv : u->convs) cv.P = static_cast<char*>(u->arena) + pmap_off;
      for (st_resnet* r : u->res) stb_resnet_bind_scratch(r, u->arena);
      for (st_block* b : u->blk) stb_block_bind_scratch(b, u->arena);
    }
  }
  if (mk.ok()) mk.dev(hipStreamSynchronize(s), "create: synchronise");
  if (mk.ok() && overflow) {
    int flag = 0;
    mk.dev(hipMemcpy(&flag, overflow, sizeof(int), hipMemcpyDeviceToHost), "overflow flag");
    if (mk.ok() && flag) {
      mk.st = ST_ERR_UNSUPPORTED;
      mk.msg = "a convolution weight exceeds the fp16 range (|w| > 65504)";
    }
  }
  if (!mk.ok()) {
    (void)hipStreamSynchronize(s);
    (void)hipGetLastError();
    free_all(u);
    delete u;
    return fail(mk.st, mk.msg);
  }
  u->persist = nullptr;
  *out = u;
  return ST_OK;
}

}  // namespace

#define UN_TRY(expr, what)                           \
  do {                                               \
    hipError_t e_ = (expr);                          \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)
#define UN_PART(expr)                      \
  do {                                     \
    st_status s_ = (expr);                 \
    if (s_ != ST_OK) return s_;            \
  } while (0)

ST_API st_status st_unet_forward(st_unet* u, const void* x, const float* t, const void* ctx,
                                 const void* add, void* y, void* stream) {
  st_set_error(ST_OK, "");
  if (!u) return fail(ST_ERR_INVALID, "handle is NULL");
  const st_unet_config& c = u->cfg;
  if (!x || !t || !ctx || !y || (c.add_in && !add))
    return fail(ST_ERR_INVALID, "x, t, ctx, y (and add) must be non-NULL");
  if (!aligned16(x) || !aligned16(t) || !aligned16(ctx) || !aligned16(y) || (add && !aligned16(add)))
    return fail(ST_ERR_INVALID, "buffers must be 16-byte aligned");
  DeviceGuard g(u->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "select device");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int B = u->B, L = c.levels, C0 = c.channels[0], Td = 4 * C0;
  // time embedding (+ the extra embedding), bf16 copy for the ResNets
  UN_TRY(timestep_embed(t, u->emb, B, C0, s), "timestep embedding");
  UN_TRY(mlp_linear(u->emb, false, false, u->t1w, u->t1b, u->mid1, nullptr, false, B, C0, Td, s), "time MLP");
  UN_TRY(mlp_linear(u->mid1, false, true, u->t2w, u->t2b, u->temb, c.add_in ? nullptr : u->temb16, false, B, Td,
                    Td, s), "time MLP");
  if (c.add_in) {
    UN_TRY(mlp_linear(add, true, false, u->a1w, u->a1b, u->amid, nullptr, false, B, c.add_in, Td, s), "add MLP");
    UN_TRY(mlp_linear(u->amid, false, true, u->a2w, u->a2b, u->temb, u->temb16, true, B, Td, Td, s), "add MLP");
  }
  size_t ci = 0, ri = 0, bi = 0, si = 0;
  UN_TRY(run_conv(u, u->convs[ci++], x, u->skips[si++], s), "conv_in");
  const void* h = u->skips[0];
  // down path: every output goes straight into its skip buffer
  for (int l = 0; l < L; ++l) {
    for (int r = 0; r < c.layers_per_block; ++r) {
      void* dst = u->skips[si++];
      if (c.depths[l]) {
        UN_PART(st_resnet_forward(u->res[ri++], h, u->temb16, u->ta, s));
        UN_PART(st_block_forward(u->blk[bi++], u->ta, ctx, dst, s));
      } else {
        UN_PART(st_resnet_forward(u->res[ri++], h, u->temb16, dst, s));
      }
      h = dst;
    }
    if (l < L - 1) {
      void* dst = u->skips[si++];
      UN_TRY(run_conv(u, u->convs[ci++], h, dst, s), "DownSample");
      h = dst;
    }
  }
  // middle block
  UN_PART(st_resnet_forward(u->res[ri++], h, u->temb16, u->ta, s));
  const void* hm = u->ta;
  if (c.mid_depth) {
    UN_PART(st_block_forward(u->blk[bi++], u->ta, ctx, u->tb, s));
    hm = u->tb;
  }
  void* hout = hm == u->ta ? u->tb : u->ta;
  UN_PART(st_resnet_forward(u->res[ri++], hm, u->temb16, hout, s));
  h = hout;
  long long ch = c.channels[L - 1];
  // up path: concat(h, skip) -> ResNet (-> transformer), ping-pong over
  // ta / tb: the concatenation consumes h, so each part writes the map its
  // input is not in
  auto other = [&](const void* m) { return m == u->ta ? u->tb : u->ta; };
  for (int lv = L - 1; lv >= 0; --lv) {
    for (int r = 0; r < c.layers_per_block + 1; ++r) {
      --si;
      const long long hw = static_cast<long long>(u->skip_h[si]) * u->skip_w[si];
      UN_TRY(concat(u->cat, h, ch, u->skips[si], u->skip_c[si], hw, B, s), "skip concatenation");
      void* r_out = other(h);
      UN_PART(st_resnet_forward(u->res[ri++], u->cat, u->temb16, r_out, s));
      h = r_out;
      ch = c.channels[lv];
      if (c.depths[lv]) {
        void* b_out = other(h);
        UN_PART(st_block_forward(u->blk[bi++], h, ctx, b_out, s));
        h = b_out;
      }
    }
    if (lv > 0) {
      void* dst = other(h);
      UN_TRY(run_conv(u, u->convs[ci++], h, dst, s), "UpSample");
      h = dst;
    }
  }
  UN_TRY(run_conv(u, u->convs[ci++], h, y, s), "conv_out");
  return ST_OK;
}

ST_API st_status st_unet_device_bytes(st_unet* u, unsigned long long* bytes) {
  st_set_error(ST_OK, "");
  if (!u || !bytes) return fail(ST_ERR_INVALID, "handle or bytes is NULL");
  *bytes = u->bytes;
  return ST_OK;
}

ST_API st_status st_unet_check_range(st_unet* u, void* stream) {
  st_set_error(ST_OK, "");
  if (!u) return fail(ST_ERR_INVALID, "handle is NULL");
  for (st_resnet* r : u->res) UN_PART(st_resnet_check_range(r, stream));
  for (st_block* b : u->blk) UN_PART(st_block_check_range(b, stream));
  DeviceGuard g(u->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, u->range_flag, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "read the range flag");
  if (!flag) return ST_OK;
  e = hipMemsetAsync(u->range_flag, 0, sizeof(int), s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "clear the range flag");
  return fail(ST_ERR_RANGE, "an fp16 convolution operand of the U-Net left the fp16 range");
}

ST_API void st_unet_destroy(st_unet* u) {
  if (!u) return;
  DeviceGuard g(u->device);
  (void)hipDeviceSynchronize();
  (void)hipGetLastError();
  free_all(u);
  delete u;
}
