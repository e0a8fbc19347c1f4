// C ABI of the ResnetBlock2D (include/st_resnet.h): validation, weight
// repacking, workspace and the launch schedule of one forward.
//
// Launch schedule (x [B][Cin][H][W] bf16):
//   GroupNorm statistics        x                      -> partial sums
//   GroupNorm1 + SiLU, to NHWC  x, partial sums        -> P1 (zero halo), and
//                                                         x itself into P2's
//                                                         shortcut channels
//   time embedding              temb, temb_w           -> cadd1 [B][Cout]
//   conv1 (implicit GEMM)       W1 [Cout][9 Cin], P1   -> h [B][Cout][H][W] bf16
//   GroupNorm statistics        h                      -> partial sums
//   GroupNorm2 + SiLU, to NHWC  h, partial sums        -> P2 channels [0, Cout)
//   conv2 (+ 1x1 shortcut as    W2 [Cout][9 Cout + Csc], P2
//     a tenth tap, or + x)                              -> y [B][Cout][H][W] bf16
// P1 and P2 hold each pixel's channels contiguously (NHWC) with a zero
// border of one pixel and Wp = W + 2 rounded up to 4 columns, so that every
// tap of the 3x3 convolution is the same GEMM operand shifted by a whole
// number of rows (the GEMM computes the padding columns too and discards
// them in its epilogue); the GroupNorm passes write the border's zeros too,
// so the maps live in the scratch arena.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <new>
#include <string>
#include <vector>

#include "../../include/st_resnet.h"
#include "kernels.h"
#include "parts.h"

#define ST_API extern "C" __attribute__((visibility("default")))

using namespace stb;

st_status st_set_error(st_status s, const std::string& msg);

struct st_resnet {
  int B, Cin, Cout, H, W, Dt, Csc;
  float eps;
  int device;
  int Wp;            // padded width of P1 / P2 (pixels)
  long long prows;   // pixel rows of P1 / P2
  int L2;            // elements per P2 row (Cout + Csc)
  std::vector<void*> allocs;
  float *gn1_w, *gn1_b, *gn2_w, *gn2_b, *temb_b, *conv1_b;
  void* temb_w;      // bf16 [Cout][Dt]
  void *w1, *w2;     // fp16 GEMM operands
  float *cadd1, *cadd2;
  float2* part;
  void *p1, *p2, *h;
  int* range_flag;
  int ks1, ks2;      // K slices of conv1 / conv2 (1 = none)
  float* ws;         // their fp32 partial products
  // part, h, cadd1, p1, p2 and ws are rewritten by every forward (ScratchPlan)
  ScratchPlan scratch;
  void* scratch_own;
  bool scratch_bound;
  DevArena* persist;  // arena of the persistent allocations during create, or NULL
};

namespace {

constexpr int kMaxSplit = 64;

st_status fail(st_status s, const std::string& msg) { return st_set_error(s, msg); }
st_status hip_fail(hipError_t e, const char* what) {
  return fail(ST_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void free_all(st_resnet* r) {
  for (void* p : r->allocs) (void)hipFree(p);
  r->allocs.clear();
}

struct Maker {
  st_resnet* r;
  hipStream_t s;
  st_status st = ST_OK;
  std::string msg{};
  bool ok() const { return st == ST_OK; }
  void dev(hipError_t e, const char* what) {
    if (ok() && e != hipSuccess) { st = ST_ERR_DEVICE; msg = std::string(what) + ": " + hipGetErrorString(e); }
  }
  void* alloc(size_t bytes, const char* what) {
    if (!ok()) return nullptr;
    if (!bytes) bytes = 16;
    void* p = nullptr;
    if (r->persist && r->persist->base) {
      p = r->persist->take(bytes);
    } else if (hipMalloc(&p, bytes) == hipSuccess) {
      r->allocs.push_back(p);
      if (r->persist) r->persist->count(bytes);
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

bool overlaps(const void* a, size_t an, const void* c, size_t cn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), c0 = reinterpret_cast<uintptr_t>(c);
  return a0 < c0 + cn && c0 < a0 + an;
}

// The implicit-GEMM convolution over P (L elements per pixel row): A = the
// packed weights, B = P shifted per tap (see ConvGemm).
GemmParams conv_gemm(const st_resnet* r, const void* w, int K, const void* P, int L, int spt,
                     int sc_spt, int sc_cbase, const float* cadd, const void* resid, void* out,
                     int ksplit) {
  GemmParams p{};
  p.A = w; p.lda = K;
  p.B = P; p.ldb = L;
  p.M = r->Cout;
  p.N = r->B * (r->H + 2) * r->Wp;
  p.K = K;
  p.epi.kind = EPI_CONV;
  p.conv.L = L; p.conv.Wp = r->Wp; p.conv.Hq = r->H + 2; p.conv.Ho = r->H; p.conv.Wo = r->W;
  p.conv.spt = spt; p.conv.sc_spt = sc_spt; p.conv.sc_cbase = sc_cbase; p.conv.sc_roff = r->Wp + 1;
  p.conv.b_bytes = r->prows * L * 2;
  p.conv.cadd = cadd; p.conv.resid = resid; p.conv.out = out;
  if (ksplit > 1) {
    p.ksplit = ksplit;
    p.ws = r->ws;
  }
  return p;
}

}  // namespace

ST_API st_status st_resnet_create(int B, int Cin, int Cout, int H, int W, int Dt, float eps,
                                  st_dtype dtype, const st_resnet_weights* w, void* stream,
                                  st_resnet** out) {
  return stb_resnet_create(B, Cin, Cout, H, W, Dt, eps, dtype, w, stream, false, nullptr, out);
}

size_t stb_resnet_scratch_bytes(const st_resnet* r) { return r->scratch.bytes; }

void stb_resnet_bind_scratch(st_resnet* r, void* base) {
  r->scratch.bind(base);
  r->scratch_bound = true;
}

st_status stb_resnet_create(int B, int Cin, int Cout, int H, int W, int Dt, float eps, st_dtype dtype,
                            const st_resnet_weights* w, void* stream, bool external_scratch,
                            DevArena* persist, st_resnet** out) {
  st_set_error(ST_OK, "");
  if (!out) return fail(ST_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (B < 1 || H < 1 || W < 1 || Dt < 1) return fail(ST_ERR_INVALID, "B, H, W and Dt must be >= 1");
  if (Cin < 64 || Cin % 64 || Cout < 64 || Cout % 64)
    return fail(ST_ERR_INVALID, "Cin and Cout must be positive multiples of 64");
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(ST_ERR_INVALID, "eps must be positive");
  if (dtype != ST_DTYPE_BF16 && dtype != ST_DTYPE_F32) return fail(ST_ERR_INVALID, "unknown dtype");
  if (dtype != ST_DTYPE_BF16) return fail(ST_ERR_UNSUPPORTED, "the ResnetBlock2D runs with bf16 storage only");
  if (B > 16) return fail(ST_ERR_UNSUPPORTED, "B must be <= 16");
  if (!temb_proj_supported(B, Dt))
    return fail(ST_ERR_UNSUPPORTED, "the time embedding needs Dt % 8 == 0 and B * Dt <= 16384");
  if (W % 4) return fail(ST_ERR_UNSUPPORTED, "W must be a multiple of 4");
  if (!w) return fail(ST_ERR_INVALID, "weights are NULL");
  auto need = [](const void* p) { return p != nullptr && aligned16(p); };
  const int Csc = Cin != Cout ? Cin : 0;
  if (!need(w->conv1_w) || !need(w->conv2_w) || !need(w->temb_w) || (Csc && !need(w->sc_w)))
    return fail(ST_ERR_INVALID, "conv1_w, conv2_w, temb_w (and sc_w when Cin != Cout) must be "
                                "non-NULL and 16-byte aligned");
  const int Wp = (W + 2 + 3) / 4 * 4;
  const long long prows = static_cast<long long>(B) * (H + 2) * Wp + 2LL * Wp + 8;
  const long long L2 = Cout + Csc;
  // 32-bit byte offsets of the GEMM operands and of the NCHW maps
  if (prows * (L2 > Cin ? L2 : Cin) * 2 >= (1LL << 31) ||
      static_cast<long long>(B) * (Cin > Cout ? Cin : Cout) * H * W * 2 >= (1LL << 31) ||
      static_cast<long long>(Cout) * (9 * Cout + Csc) * 2 >= (1LL << 31))
    return fail(ST_ERR_UNSUPPORTED, "feature map too large: an operand reaches 2^31 bytes");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_fail(e, "hipGetDevice");
  }
  st_resnet* r = new (std::nothrow) st_resnet();
  if (!r) return fail(ST_ERR_OUT_OF_MEMORY, "host allocation failed");
  r->B = B; r->Cin = Cin; r->Cout = Cout; r->H = H; r->W = W; r->Dt = Dt; r->Csc = Csc;
  r->eps = eps; r->device = dev; r->Wp = Wp; r->prows = prows; r->L2 = static_cast<int>(L2);
  r->scratch_own = nullptr;
  r->scratch_bound = false;
  r->persist = persist;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Maker mk{r, s};
  r->gn1_w = mk.vec(w->gn1_w, Cin, 1.f, "gn1_w");
  r->gn1_b = mk.vec(w->gn1_b, Cin, 0.f, "gn1_b");
  r->gn2_w = mk.vec(w->gn2_w, Cout, 1.f, "gn2_w");
  r->gn2_b = mk.vec(w->gn2_b, Cout, 0.f, "gn2_b");
  r->temb_b = mk.vec(w->temb_b, Cout, 0.f, "temb_b");
  r->conv1_b = mk.vec(w->conv1_b, Cout, 0.f, "conv1_b");
  float* conv2_b = mk.vec(w->conv2_b, Cout, 0.f, "conv2_b");
  float* sc_b = Csc ? mk.vec(w->sc_b, Cout, 0.f, "sc_b") : nullptr;
  r->temb_w = mk.alloc(static_cast<size_t>(Cout) * Dt * 2, "temb_w");
  if (mk.ok()) mk.dev(hipMemcpyAsync(r->temb_w, w->temb_w, static_cast<size_t>(Cout) * Dt * 2,
                                     hipMemcpyDeviceToDevice, s), "temb_w");
  int* overflow = static_cast<int*>(mk.alloc(sizeof(int), "overflow flag"));
  if (overflow) mk.dev(hipMemsetAsync(overflow, 0, sizeof(int), s), "overflow flag");
  r->w1 = mk.alloc(static_cast<size_t>(Cout) * 9 * Cin * 2, "conv1 operand");
  r->w2 = mk.alloc(static_cast<size_t>(Cout) * (9 * Cout + Csc) * 2, "conv2 operand");
  if (mk.ok()) mk.dev(conv_weight_pack(w->conv1_w, nullptr, r->w1, Cout, Cin, 0, overflow, s), "pack conv1");
  if (mk.ok()) mk.dev(conv_weight_pack(w->conv2_w, Csc ? w->sc_w : nullptr, r->w2, Cout, Cout, Csc, overflow, s),
                      "pack conv2");
  // conv2 adds its bias and the shortcut's, the same for every sample
  r->scratch.add(&r->cadd1, sizeof(float) * B * Cout);  // written by every forward
  r->cadd2 = static_cast<float*>(mk.alloc(sizeof(float) * B * Cout, "cadd2"));
  if (mk.ok()) {
    for (int b = 0; b < B && mk.ok(); ++b) {
      mk.dev(hipMemcpyAsync(r->cadd2 + static_cast<long long>(b) * Cout, conv2_b, sizeof(float) * Cout,
                            hipMemcpyDeviceToDevice, s), "cadd2");
    }
  }
  if (mk.ok() && sc_b) {
    // cadd2 += sc_b, through a tiny temporary on the host (create only)
    std::vector<float> a(static_cast<size_t>(B) * Cout), c(Cout);
    mk.dev(hipMemcpyAsync(a.data(), r->cadd2, sizeof(float) * B * Cout, hipMemcpyDeviceToHost, s), "cadd2");
    mk.dev(hipMemcpyAsync(c.data(), sc_b, sizeof(float) * Cout, hipMemcpyDeviceToHost, s), "sc_b");
    if (mk.ok()) mk.dev(hipStreamSynchronize(s), "cadd2");
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < Cout; ++i) a[static_cast<size_t>(b) * Cout + i] += c[i];
    if (mk.ok()) mk.dev(hipMemcpyAsync(r->cadd2, a.data(), sizeof(float) * B * Cout, hipMemcpyHostToDevice, s),
                        "cadd2");
    if (mk.ok()) mk.dev(hipStreamSynchronize(s), "cadd2");
  }
  r->scratch.add(&r->part, sizeof(float2) * B * ST_GN_GROUPS * kMaxSplit);
  // the operand maps: every forward writes their pixels and their halo
  r->scratch.add(&r->p1, static_cast<size_t>(prows) * Cin * 2);
  r->scratch.add(&r->p2, static_cast<size_t>(prows) * L2 * 2);
  r->scratch.add(&r->h, static_cast<size_t>(B) * Cout * H * W * 2);
  r->range_flag = static_cast<int*>(mk.alloc(sizeof(int), "range flag"));
  // convolutions with few output tiles split K (one slice per CU)
  {
    int cus = 0;
    mk.dev(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "CU count");
    const int N = B * (H + 2) * Wp;
    r->ks1 = conv_ksplit(Cout, N, 9 * Cin, cus);
    r->ks2 = conv_ksplit(Cout, N, 9 * Cout + Csc, cus);
    const int most = r->ks1 > r->ks2 ? r->ks1 : r->ks2;
    r->ws = nullptr;
    if (most > 1) r->scratch.add(&r->ws, sizeof(float) * most * Cout * ((N + 63) / 64 * 64));
  }
  if (!external_scratch && mk.ok()) {
    void* arena = mk.alloc(r->scratch.bytes, "workspace");
    if (arena) {
      r->scratch_own = arena;
      stb_resnet_bind_scratch(r, arena);
    }
  }
  if (mk.ok()) mk.dev(hipMemsetAsync(r->range_flag, 0, sizeof(int), s), "range flag");
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
    free_all(r);
    delete r;
    return fail(mk.st, mk.msg);
  }
  r->persist = nullptr;  // create is over: nothing more is taken from it
  *out = r;
  return ST_OK;
}

#define RS_TRY(expr, what)                            \
  do {                                                \
    hipError_t e_ = (expr);                           \
    if (e_ != hipSuccess) return hip_fail(e_, what);  \
  } while (0)

ST_API st_status st_resnet_forward(st_resnet* r, const void* x, const void* temb, void* y,
                                   void* stream) {
  st_set_error(ST_OK, "");
  if (!r) return fail(ST_ERR_INVALID, "handle is NULL");
  if (!x || !temb || !y) return fail(ST_ERR_INVALID, "x, temb and y must be non-NULL");
  if (!aligned16(x) || !aligned16(temb) || !aligned16(y))
    return fail(ST_ERR_INVALID, "x, temb and y must be 16-byte aligned");
  const size_t xb = static_cast<size_t>(r->B) * r->Cin * r->H * r->W * 2;
  const size_t yb = static_cast<size_t>(r->B) * r->Cout * r->H * r->W * 2;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, temb, static_cast<size_t>(r->B) * r->Dt * 2))
    return fail(ST_ERR_INVALID, "y overlaps x or temb");
  if (!r->scratch_bound) return fail(ST_ERR_INVALID, "the handle's workspace is not bound");
  DeviceGuard g(r->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "select device");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int B = r->B, Cin = r->Cin, Cout = r->Cout, H = r->H, W = r->W, N = H * W;
  RS_TRY(gn_stats(x, true, B, Cin, N, r->part, kMaxSplit, s), "GroupNorm 1 statistics");
  RS_TRY(gn_apply_pad(x, r->part, kMaxSplit, r->gn1_w, r->gn1_b, r->p1, B, Cin, H, W, r->Wp, Cin,
                      r->eps, r->Csc ? r->p2 : nullptr, r->L2, Cout, r->range_flag, s),
         "GroupNorm 1 + SiLU");
  RS_TRY(temb_proj(temb, r->temb_w, r->temb_b, r->conv1_b, r->cadd1, B, r->Dt, Cout, s),
         "time embedding");
  RS_TRY(gemm_mfma(conv_gemm(r, r->w1, 9 * Cin, r->p1, Cin, Cin / 64, 0, 0, r->cadd1, nullptr, r->h,
                             r->ks1),
                   ACT_F16, s),
         "conv1");
  RS_TRY(gn_stats(r->h, true, B, Cout, N, r->part, kMaxSplit, s), "GroupNorm 2 statistics");
  RS_TRY(gn_apply_pad(r->h, r->part, kMaxSplit, r->gn2_w, r->gn2_b, r->p2, B, Cout, H, W, r->Wp, r->L2,
                      r->eps, nullptr, 0, 0, r->range_flag, s),
         "GroupNorm 2 + SiLU");
  RS_TRY(gemm_mfma(conv_gemm(r, r->w2, 9 * Cout + r->Csc, r->p2, r->L2, Cout / 64, r->Csc / 64, Cout,
                             r->cadd2, r->Csc ? nullptr : x, y, r->ks2),
                   ACT_F16, s),
         "conv2");
  return ST_OK;
}

ST_API st_status st_resnet_check_range(st_resnet* r, void* stream) {
  st_set_error(ST_OK, "");
  if (!r) return fail(ST_ERR_INVALID, "handle is NULL");
  DeviceGuard g(r->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "select device");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, r->range_flag, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "read the range flag");
  if (!flag) return ST_OK;
  e = hipMemsetAsync(r->range_flag, 0, sizeof(int), s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "clear the range flag");
  return fail(ST_ERR_RANGE, "an fp16 convolution operand left the fp16 range: outputs of the "
                            "forwards since the last check are not valid");
}

ST_API void st_resnet_destroy(st_resnet* r) {
  if (!r) return;
  DeviceGuard g(r->device);
  (void)hipDeviceSynchronize();
  (void)hipGetLastError();
  free_all(r);
  delete r;
}
