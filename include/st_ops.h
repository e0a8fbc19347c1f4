/*
 * st_ops.h -- C ABI of the standalone operations around the
 * Spatial-Transformer block for AMD Instinct MI355X (gfx950): GroupNorm
 * (optionally with SiLU) on NCHW feature maps, and the guided DDPM sampling
 * step.  Same library (libst_block.so) and status codes as st_block.h.
 *
 * Pages cited by title and section:
 *   - "Stable Diffusion XL Inpainting 宏观架构" §4 and "Stable Diffusion 2.1
 *     Base 宏观架构" §4: the ResnetBlock2D's GroupNorm + SiLU + Conv.
 *   - DDPM / SD / SDXL tutorial page: GSC (GroupNorm + SiLU + Conv); the
 *     DDPM reverse step x_{t-1} = 1/sqrt(alpha_t) (x_t - beta_t /
 *     sqrt(1 - alphabar_t) eps) + sqrt(beta_t) z with alpha_t = 1 - beta_t,
 *     alphabar_t = alpha_1 ... alpha_t and beta linear in t.
 *   - "企业官网建设流程全解析" (SD1.5 anatomy article) §1, §5: the CFG scale
 *     applied to the U-Net's noise prediction.
 *
 * Every call validates its arguments before enqueuing anything (on an
 * error nothing is enqueued), only enqueues work on `stream` (hipStream_t,
 * NULL = default stream) and returns before it completes; buffers are
 * borrowed and must stay valid until the stream reaches the work.
 */
#ifndef ST_OPS_H
#define ST_OPS_H

#include <stddef.h>

#include "st_block.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * GroupNorm over NCHW with 32 contiguous channel groups and population
 * variance, then, when `silu` is nonzero, SiLU(v) = v / (1 + exp(-v)):
 *   y[b][c][i][j] = act((x[b][c][i][j] - mean_bg) / sqrt(var_bg + eps)
 *                       * gamma[c] + beta[c]),  g = c / (C / 32).
 *   x, y    [B][C][H][W], device, `dtype`, 16-byte aligned; y must not
 *           overlap x.
 *   gamma, beta  [C] device, `dtype`; NULL = ones / zeros.
 *   B, H, W >= 1; C >= 32, C % 32 == 0; eps > 0.
 *   workspace: device memory of at least st_group_norm_workspace_bytes(B)
 *           bytes (16-byte aligned), used for the per-(sample, group)
 *           partial sums; it must not be used by anything else until the
 *           stream has finished the call.
 * Errors: ST_ERR_INVALID (nothing enqueued), ST_ERR_DEVICE.
 */
size_t st_group_norm_workspace_bytes(int B);
st_status st_group_norm(const void *x, const void *gamma, const void *beta, void *y,
                        int B, int C, int H, int W, float eps, int silu,
                        st_dtype dtype, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation as st_group_norm, with the partial sums in a static 1 MiB
 * device array of the library (one per GPU, held until the process ends)
 * instead of a caller workspace.  It calls no allocating routine.  B <= 64
 * (larger: ST_ERR_UNSUPPORTED, nothing enqueued).  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race on it, so they must be serialised; sequential
 * calls need no clearing (each call writes every slot it reads).
 */
st_status st_group_norm_noalloc(const void *x, const void *gamma, const void *beta,
                                void *y, int B, int C, int H, int W, float eps, int silu,
                                st_dtype dtype, void *stream);

/*
 * Guided DDPM step for one classifier-free-guidance pair:
 *   eps      = eps_u + guidance_scale * (eps_c - eps_u)
 *   x_prev   = 1/sqrt(alpha_t) * (x_t - beta_t / sqrt(1 - alphabar_t) * eps)
 *              + sqrt(beta_t) * noise
 * with beta_s = beta_start + (s - 1) (beta_end - beta_start) / (T - 1)
 * (beta_start when T == 1), alpha_s = 1 - beta_s, alphabar_t the product of
 * alpha_1 .. alpha_t, evaluated on the host in fp64; the elementwise update
 * runs in fp32.
 *   eps_pair [2][n] device, `eps_dtype` (bf16 or fp32): the U-Net's output
 *            for the pair, the unconditional half first.
 *   x_t, x_prev [n] device fp32 (latents); x_prev may equal x_t.
 *   noise    [n] device fp32, or NULL for no noise term (z = 0).
 *   n >= 0 (0 enqueues nothing); 1 <= t <= T; 0 < beta_start, beta_end < 1.
 * Errors: ST_ERR_INVALID (nothing enqueued), ST_ERR_DEVICE.
 */
st_status st_guided_ddpm_step(const void *eps_pair, st_dtype eps_dtype,
                              const float *x_t, const float *noise, float *x_prev,
                              long long n, float guidance_scale, int t, int T,
                              double beta_start, double beta_end, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* ST_OPS_H */
