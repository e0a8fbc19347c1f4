// C ABI of the standalone operations declared in include/st_ops.h:
// GroupNorm (+ SiLU) on NCHW maps and the guided DDPM step.  Argument
// validation and launch only; the kernels are in k_norm.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>

#include "../../include/st_ops.h"
#include "kernels.h"

#define ST_API extern "C" __attribute__((visibility("default")))

using namespace stb;

// Defined in host.hip: the per-thread error text behind st_last_error().
st_status st_set_error(st_status s, const std::string& msg);

namespace {

// Partial-sum slices per (sample, group) of the GroupNorm statistics.
constexpr int kGnMaxSplit = 64;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

st_status fail(st_status s, const std::string& msg) { return st_set_error(s, msg); }

st_status check_gn(const void* x, const void* y, int B, int C, int H, int W, float eps,
                   st_dtype dtype) {
  if (!x || !y) return fail(ST_ERR_INVALID, "x and y must be non-NULL");
  if (B < 1 || H < 1 || W < 1) return fail(ST_ERR_INVALID, "B, H and W must be >= 1");
  if (C < ST_GN_GROUPS || C % ST_GN_GROUPS) return fail(ST_ERR_INVALID, "C must be a positive multiple of 32");
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(ST_ERR_INVALID, "eps must be positive");
  if (dtype != ST_DTYPE_BF16 && dtype != ST_DTYPE_F32) return fail(ST_ERR_INVALID, "unknown dtype");
  if (!aligned16(x) || !aligned16(y)) return fail(ST_ERR_INVALID, "x and y must be 16-byte aligned");
  const long long n = static_cast<long long>(B) * C * H * W;
  if (static_cast<long long>(H) * W > (1LL << 30) || n > (1LL << 40))
    return fail(ST_ERR_UNSUPPORTED, "feature map too large");
  // the apply pass reads each group's first element of x as the shift of
  // its sums: y may not overwrite x
  const size_t es = dtype == ST_DTYPE_BF16 ? 2 : 4;
  const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
  const uintptr_t len = static_cast<uintptr_t>(n) * es;
  if (a < b + len && b < a + len) return fail(ST_ERR_INVALID, "y overlaps x");
  return ST_OK;
}

st_status run_gn(const void* x, const void* gamma, const void* beta, void* y, int B, int C,
                 int H, int W, float eps, int silu, st_dtype dtype, float2* partial,
                 hipStream_t s) {
  const bool bf = dtype == ST_DTYPE_BF16;
  const int N = H * W;
  hipError_t e = gn_stats(x, bf, B, C, N, partial, kGnMaxSplit, s);
  if (e == hipSuccess) e = gn_apply_nchw(x, bf, partial, kGnMaxSplit, gamma, beta, y, B, C, N, eps, silu != 0, s);
  if (e != hipSuccess) return fail(ST_ERR_DEVICE, std::string("GroupNorm: ") + hipGetErrorString(e));
  return ST_OK;
}

// Allocation-free GroupNorm: the partial sums live in this file-scope
// device array (one copy per GPU, held until the process ends) instead of
// a caller workspace.  1 MiB: B <= 64 samples of 32 groups x 64 slices.
// Host code never passes the array's name to a kernel (on the host it is
// only a stand-in for the symbol): it passes the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept in g_scratch_dev.
constexpr int kScratchMaxBatch = 64;
constexpr int kScratchPartials = kScratchMaxBatch * ST_GN_GROUPS * kGnMaxSplit;
static __device__ __align__(256) float2 scratch[kScratchPartials];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float2* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device.
st_status scratch_on_current_device(float2** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ST_ERR_DEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(ST_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ST_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_dev[dev] = static_cast<float2*>(p);
  }
  *out = g_scratch_dev[dev];
  return ST_OK;
}

}  // namespace

ST_API st_status st_group_norm_noalloc(const void* x, const void* gamma, const void* beta,
                                       void* y, int B, int C, int H, int W, float eps, int silu,
                                       st_dtype dtype, void* stream) {
  st_set_error(ST_OK, "");
  st_status st = check_gn(x, y, B, C, H, W, eps, dtype);
  if (st != ST_OK) return st;
  if (B > kScratchMaxBatch)
    return fail(ST_ERR_UNSUPPORTED, "st_group_norm_noalloc: B must be <= 64 (static scratch of 1 MiB)");
  float2* part = nullptr;
  st = scratch_on_current_device(&part);
  if (st != ST_OK) return st;
  // every slot the statistics pass writes is read back by the apply pass of
  // the same call: nothing needs clearing
  return run_gn(x, gamma, beta, y, B, C, H, W, eps, silu, dtype, part, static_cast<hipStream_t>(stream));
}

ST_API size_t st_group_norm_workspace_bytes(int B) {
  return B > 0 ? static_cast<size_t>(B) * ST_GN_GROUPS * kGnMaxSplit * sizeof(float2) : 0;
}

ST_API st_status st_group_norm(const void* x, const void* gamma, const void* beta, void* y,
                               int B, int C, int H, int W, float eps, int silu,
                               st_dtype dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  st_set_error(ST_OK, "");
  st_status st = check_gn(x, y, B, C, H, W, eps, dtype);
  if (st != ST_OK) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < st_group_norm_workspace_bytes(B))
    return fail(ST_ERR_INVALID, "workspace must be 16-byte aligned and at least st_group_norm_workspace_bytes(B)");
  return run_gn(x, gamma, beta, y, B, C, H, W, eps, silu, dtype, static_cast<float2*>(workspace),
                static_cast<hipStream_t>(stream));
}

ST_API st_status st_guided_ddpm_step(const void* eps_pair, st_dtype eps_dtype,
                                     const float* x_t, const float* noise, float* x_prev,
                                     long long n, float guidance_scale, int t, int T,
                                     double beta_start, double beta_end, void* stream) {
  st_set_error(ST_OK, "");
  if (n < 0) return fail(ST_ERR_INVALID, "n must be >= 0");
  if (T < 1 || t < 1 || t > T) return fail(ST_ERR_INVALID, "need 1 <= t <= T");
  if (!(beta_start > 0.0 && beta_start < 1.0 && beta_end > 0.0 && beta_end < 1.0))
    return fail(ST_ERR_INVALID, "beta_start and beta_end must lie in (0, 1)");
  if (!std::isfinite(guidance_scale)) return fail(ST_ERR_INVALID, "guidance_scale must be finite");
  if (eps_dtype != ST_DTYPE_BF16 && eps_dtype != ST_DTYPE_F32) return fail(ST_ERR_INVALID, "unknown dtype");
  if (n == 0) return ST_OK;
  if (!eps_pair || !x_t || !x_prev) return fail(ST_ERR_INVALID, "eps_pair, x_t and x_prev must be non-NULL");
  // the linear schedule, alphabar_t as a product in fp64
  auto beta_at = [&](int s) {
    return T == 1 ? beta_start : beta_start + (s - 1) * (beta_end - beta_start) / (T - 1);
  };
  double alphabar = 1.0;
  for (int s = 1; s <= t; ++s) alphabar *= 1.0 - beta_at(s);
  const double bt = beta_at(t), at = 1.0 - bt;
  const float c1 = static_cast<float>(1.0 / std::sqrt(at));
  const float c2 = static_cast<float>(bt / std::sqrt(1.0 - alphabar));
  const float sigma = static_cast<float>(std::sqrt(bt));
  hipError_t e = guided_ddpm(eps_pair, eps_dtype == ST_DTYPE_BF16, x_t, noise, x_prev, n,
                             guidance_scale, c1, c2, sigma, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ST_ERR_DEVICE, std::string("guided DDPM step: ") + hipGetErrorString(e));
  return ST_OK;
}
