/*
 * st_resnet.h -- C ABI of the ResnetBlock2D for AMD Instinct MI355X
 * (gfx950).  Same library (libst_block.so) and status codes as st_block.h.
 *
 * What it computes (pages cited by title and section):
 *   - "Stable Diffusion XL Inpainting 宏观架构" §4 "核心算子与任务差异" and
 *     "Stable Diffusion 2.1 Base 宏观架构" §4: ResnetBlock2D = GroupNorm +
 *     SiLU + Conv, add the time embedding, GroupNorm + Dropout + Conv,
 *     residual / shortcut add.
 *   - DDPM / SD / SDXL tutorial page, "（1）ResNetBlock模块" and its
 *     image-decoder passage: GSC (GroupNorm + SiLU + Conv) on the feature,
 *     added to the time embedding after SiLU + a fully connected layer, a
 *     second GSC, added to the skip connection.
 * Concretely, x [B][Cin][H][W], temb [B][Dt] -> y [B][Cout][H][W]:
 *   h = Conv3x3(SiLU(GroupNorm1(x))) + conv1_b
 *   h = h + (temb_w SiLU(temb) + temb_b)          per (sample, channel)
 *   h = Conv3x3(SiLU(GroupNorm2(h))) + conv2_b     (Dropout = identity)
 *   y = shortcut(x) + h,  shortcut = x (Cin == Cout) or a 1x1 Conv (sc_w, sc_b)
 * GroupNorm: 32 contiguous channel groups, population variance, epsilon
 * `eps`; Conv3x3: stride 1, zero padding 1, cross-correlation (the kernel is
 * applied unflipped, weight [Cout][Cin][3][3]).
 *
 * Precision (ST_DTYPE_BF16, the only storage type): x, temb, weights and y
 * are bf16; the convolutions run as implicit GEMMs on fp16 operands (the
 * GroupNorm + SiLU output, bf16 weights converted exactly) with fp32
 * accumulation; the intermediate h is stored in bf16; statistics in
 * fp32/fp64.  fp16 operands are range-checked where they are stored
 * (st_resnet_check_range).
 *
 * Threading: as st_block.h (one forward at a time per handle).
 */
#ifndef ST_RESNET_H
#define ST_RESNET_H

#include "st_block.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct st_resnet st_resnet; /* opaque handle */

/* Device pointers, bf16, row-major; every bias may be NULL (= 0), GroupNorm
 * gammas NULL = ones, betas NULL = zeros. */
typedef struct {
  const void *gn1_w, *gn1_b;      /* [Cin] */
  const void *conv1_w, *conv1_b;  /* [Cout][Cin][3][3], [Cout] */
  const void *temb_w, *temb_b;    /* [Cout][Dt], [Cout] */
  const void *gn2_w, *gn2_b;      /* [Cout] */
  const void *conv2_w, *conv2_b;  /* [Cout][Cout][3][3], [Cout] */
  const void *sc_w, *sc_b;        /* [Cout][Cin], [Cout]: required when Cin != Cout,
                                     ignored when Cin == Cout */
} st_resnet_weights;

/*
 * Create a ResnetBlock2D handle on the current HIP device.
 *   1 <= B <= 16; Cin, Cout positive multiples of 64; H >= 1; W >= 4 and
 *   W % 4 == 0 (other widths: ST_ERR_UNSUPPORTED); Dt >= 1, with Dt % 8 ==
 *   0 and B * Dt <= 16384 (else ST_ERR_UNSUPPORTED); eps > 0;
 *   dtype ST_DTYPE_BF16 (ST_DTYPE_F32: ST_ERR_UNSUPPORTED).
 *   w: device pointers as above, weights non-NULL and 16-byte aligned.  The
 *      weights are COPIED and repacked (tap-major fp16 convolution operands;
 *      a weight beyond the fp16 range gives ST_ERR_UNSUPPORTED); the caller
 *      may free them once create returns.
 *   stream: used for the copies; synchronised before create returns.
 * Returns ST_OK or an error with nothing allocated and *out = NULL.
 */
st_status st_resnet_create(int B, int Cin, int Cout, int H, int W, int Dt, float eps,
                           st_dtype dtype, const st_resnet_weights *w, void *stream,
                           st_resnet **out);

/*
 * Enqueue y = ResnetBlock2D(x, temb) on `stream`.
 *   x [B][Cin][H][W], temb [B][Dt], y [B][Cout][H][W]: device bf16, 16-byte
 *   aligned; y must not overlap x or temb.  Allocates nothing; validates
 *   every argument before the first launch (ST_ERR_INVALID: nothing
 *   enqueued).  Buffers must stay valid until the stream reaches the work.
 */
st_status st_resnet_forward(st_resnet *blk, const void *x, const void *temb, void *y,
                            void *stream);

/* As st_block_check_range, for the fp16 convolution operands. */
st_status st_resnet_check_range(st_resnet *blk, void *stream);

/* Wait for the device to go idle, then free everything.  NULL-safe. */
void st_resnet_destroy(st_resnet *blk);

#ifdef __cplusplus
}
#endif
#endif /* ST_RESNET_H */
