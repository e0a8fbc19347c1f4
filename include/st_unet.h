/*
 * st_unet.h -- C ABI of one U-Net denoiser timestep for AMD Instinct MI355X
 * (gfx950), composed of the library's ResnetBlock2D (st_resnet.h) and
 * Spatial-Transformer blocks (st_block.h) and its implicit-GEMM 3x3
 * convolutions.  Same library and status codes as st_block.h.
 *
 * Topology (the architecture pages' §3 "完整 U-Net 多尺度拓扑", "Stable
 * Diffusion XL Inpainting 宏观架构" and "Stable Diffusion 2.1 Base 宏观架构";
 * the DDPM / SD / SDXL tutorial page's DownSample (Conv 3x3, stride 2,
 * padding 1) and UpSample (nearest interpolation + Conv) modules and
 * CrossAttnDown/Up/Mid blocks):
 *   temb = Linear2(SiLU(Linear1(sinusoidal(t))))  [+ the same MLP on `add`]
 *   h = conv_in(x);                      skips = [h]
 *   per level l: layers_per_block x (h = ResNet(h, temb); if depths[l]:
 *                h = SpatialTransformer(h, ctx); skips += [h]);
 *                if not the last level: h = DownSample(h); skips += [h]
 *   mid:         h = ResNet; if mid_depth: SpatialTransformer; ResNet
 *   per level, deepest first: (layers_per_block + 1) x (h = ResNet(
 *                concat(h, skips.pop()), temb); if depths[l]:
 *                SpatialTransformer); if not the shallowest: UpSample
 *   y = conv_out(SiLU(GroupNorm(h)))
 * The sinusoidal embedding has channels[0] entries: half frequencies
 * 10000^(-i/half), cosines first; the time MLP is channels[0] -> 4
 * channels[0] -> 4 channels[0].  ResNet and output GroupNorms use eps 1e-5,
 * the transformer blocks heads = C / 64.
 *
 * Precision: bf16 storage everywhere (weights, activations, skips, y),
 * fp16 / bf16 operands with fp32 accumulation inside each part (see
 * st_block.h and st_resnet.h); the embedding MLPs run in fp32 on bf16
 * weights and hand the ResNets a bf16 time embedding.
 */
#ifndef ST_UNET_H
#define ST_UNET_H

#include "st_block.h"
#include "st_resnet.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct st_unet st_unet; /* opaque handle */

typedef struct {
  int in_channels, out_channels; /* 4 or 9 in (SD2.1 / SDXL-Inpaint), 4 out; <= 64 */
  int levels;                    /* 1 .. 4 resolution levels */
  int channels[4];               /* per level, multiples of 64 */
  int depths[4];                 /* Spatial-Transformer depth per level, 0 = ResNet only */
  int mid_depth;                 /* 0 = no transformer in the middle block */
  int layers_per_block;          /* ResNets per down level (up levels: one more) */
  int ctx_dim;                   /* context width D_ctx (multiple of 64) */
  int add_in;                    /* width of the extra embedding added to the time
                                    embedding (SDXL: 2816), 0 = none */
} st_unet_config;

/*
 * Weights, device pointers (bf16), biases nullable, in execution order.
 * resnets: HOST array of every ResNet: the down levels' in order, the two
 *   of the middle block, then the up levels', deepest level first.
 * blocks: HOST array of every Spatial-Transformer block in the same order
 *   (levels with depth 0 have none; the middle block's between its ResNets).
 * down_w / down_b: HOST arrays of levels-1 DownSample convolutions
 *   [C_l][C_l][3][3]; up_w / up_b: HOST arrays of levels-1 UpSample
 *   convolutions, deepest up level first.
 */
typedef struct {
  const void *time1_w, *time1_b;  /* [4 C0][C0], [4 C0] */
  const void *time2_w, *time2_b;  /* [4 C0][4 C0], [4 C0] */
  const void *add1_w, *add1_b;    /* [4 C0][add_in], [4 C0] (add_in > 0) */
  const void *add2_w, *add2_b;    /* [4 C0][4 C0], [4 C0] (add_in > 0) */
  const void *conv_in_w, *conv_in_b;          /* [C0][in][3][3], [C0] */
  const st_resnet_weights *resnets;
  const st_block_weights *blocks;
  const void *const *down_w, *const *down_b;
  const void *const *up_w, *const *up_b;
  const void *norm_out_w, *norm_out_b;        /* [C0] */
  const void *conv_out_w, *conv_out_b;        /* [out][C0][3][3], [out] */
} st_unet_weights;

/*
 * Create the U-Net for batch B (1 <= B <= 4) at latent size H x W (both
 * multiples of 8 * 2^(levels-1) / 2 so that every DownSample halves an even
 * size and every level's width stays a multiple of 4: H % 2^(levels-1) ==
 * 0 and (W >> (levels-1)) % 4 == 0).  Weights are copied (through the
 * parts' own create calls); `stream` is synchronised before returning.
 * Memory: the handle's persistent memory (weights, skips, work maps) is one
 * block of exactly its size (create builds the handle twice: once to count
 * the sizes, which briefly holds more memory, then into the block), and
 * the parts' per-forward buffers share one arena of the largest part's
 * size, since the parts run one after another on `stream`.
 * Errors: ST_ERR_INVALID / ST_ERR_UNSUPPORTED / ST_ERR_OUT_OF_MEMORY /
 * ST_ERR_DEVICE, nothing kept.
 */
st_status st_unet_create(const st_unet_config *cfg, int B, int H, int W,
                         const st_unet_weights *w, void *stream, st_unet **out);

/*
 * Enqueue one denoiser timestep: y = UNet(x, t, ctx, add).
 *   x [B][in][H][W] bf16, t [B] fp32 (timesteps), ctx [B][77][ctx_dim] bf16,
 *   add [B][add_in] bf16 (NULL when add_in == 0), y [B][out][H][W] bf16; all
 *   device, 16-byte aligned, y not overlapping the inputs.  Allocates
 *   nothing; validates before the first launch.
 */
st_status st_unet_forward(st_unet *u, const void *x, const float *t, const void *ctx,
                          const void *add, void *y, void *stream);

/* Device bytes the handle holds (its parts included): the drop of the
 * device's free memory across the final build in create. */
st_status st_unet_device_bytes(st_unet *u, unsigned long long *bytes);

/* Range check of every part's fp16 intermediates (st_block_check_range). */
st_status st_unet_check_range(st_unet *u, void *stream);

/* Wait for the device to go idle, then free everything.  NULL-safe. */
void st_unet_destroy(st_unet *u);

#ifdef __cplusplus
}
#endif
#endif /* ST_UNET_H */
