/*
 * st_block.h -- C ABI of the Spatial-Transformer (Transformer2DModel) block
 * for AMD Instinct MI355X (gfx950).
 *
 * What the block computes (pages cited by title and section):
 *   - "Stable Diffusion XL Inpainting 宏观架构", §4 核心算子: Transformer2DModel
 *     = Norm -> self-attention (Q=K=V=image tokens), Norm -> cross-attention
 *     (K=V=context [B,77,D_ctx]), Norm -> GEGLU feed-forward, a residual after
 *     every sublayer.
 *   - "Stable Diffusion 2.1 Base 宏观架构", §4: input and output shapes are
 *     equal; spatial attention flattens H x W into a token sequence.
 *   - DDPM/SD/SDXL tutorial page, "（4）Spatial Transformer模块" and the SDXL
 *     U-Net part: GroupNorm + Linear (1x1 Conv) + X BasicTransformer blocks
 *     + Linear, with an outer residual; "BasicTransformer Block" = LayerNorm
 *     + SelfAttention + CrossAttention + FeedForward(GeGLU + Dropout +
 *     Linear), each residual.
 *   - "企业官网建设流程全解析" (SD1.5 anatomy article) §3.2 and §3.4: K/V of
 *     the cross-attention are Linear maps of the context width to C;
 *     attention = Softmax(Q K^T / sqrt(d)) V, per head [batch, heads, tokens,
 *     dim].
 *
 * Concretely, with N = H*W, T = B*N, F = 4*C, d = 64, heads = C/64:
 *   z  = GroupNorm(x; 32 contiguous channel groups, eps 1e-6, gn_w, gn_b)
 *   h  = tokens(z) W_in^T + b_in          token n = i*W + j, h is [T, C]
 *   for each layer:
 *     h += MHA(LN1(h) Wq1^T+bq1, LN1(h) Wk1^T+bk1, LN1(h) Wv1^T+bv1) Wo1^T + bo1
 *     h += MHA(LN2(h) Wq2^T+bq2, ctx Wk2^T+bk2, ctx Wv2^T+bv2) Wo2^T + bo2
 *     h += GEGLU(LN3(h) W1^T + b1) W2^T + b2
 *           GEGLU(z) = z[:, :F] * GELU_erf(z[:, F:]);  LN eps 1e-5
 *   y  = NCHW(h W_out^T + b_out) + x
 * The softmax scale is 1/sqrt(64); there is no mask and no positional
 * encoding; dropout is the identity.
 *
 * Precision.  ST_DTYPE_BF16: inputs, weights and output are bf16; GEMM and
 * attention operands are 16-bit (fp16 where a normalised activation or the
 * GEGLU output meets a weight, bf16 for attention and the context) with fp32
 * accumulation; norm statistics and the softmax are fp32; the residual
 * stream h is kept in fp16.  Every fp16 intermediate (h, the GEGLU output,
 * the GroupNorm output) is range-checked where it is stored: a value that
 * leaves the fp16 range (|v| >= 65520, or NaN) sets a flag of the handle,
 * which st_block_check_range() reports -- a forward never hides such an
 * overflow.  ST_DTYPE_F32: every buffer and every operation is fp32 (a
 * debug path for tight parity checks).
 *
 * Threading.  Distinct handles are independent.  One handle runs one forward
 * at a time: forwards (and forward_stage calls) on one handle must be
 * serialised by the caller -- two that overlap on the device race on the
 * handle's workspace (and its range flag), e.g. when enqueued on two
 * streams without an event between them.  st_last_error() is per host
 * thread.
 */
#ifndef ST_BLOCK_H
#define ST_BLOCK_H

#ifdef __cplusplus
extern "C" {
#endif

#define ST_CTX_LEN 77   /* context tokens (CLIP token limit) */
#define ST_HEAD_DIM 64  /* channels per attention head */
#define ST_GN_GROUPS 32 /* GroupNorm groups */

typedef struct st_block st_block; /* opaque handle */

typedef enum {
  ST_OK = 0,
  ST_ERR_INVALID = 1,       /* bad argument: NULL, shape, alignment, aliasing */
  ST_ERR_UNSUPPORTED = 2,   /* valid shape the kernels cannot compute */
  ST_ERR_OUT_OF_MEMORY = 3, /* device allocation failed */
  ST_ERR_DEVICE = 4,        /* a HIP call failed; st_last_error() has the text */
  ST_ERR_RANGE = 5          /* an fp16 intermediate left the fp16 range
                               (st_block_check_range) */
} st_status;

typedef enum { ST_DTYPE_BF16 = 0, ST_DTYPE_F32 = 1 } st_dtype;

/*
 * Weights of one BasicTransformer layer.  Device pointers, element type
 * given by the handle's dtype, row-major.  Linear weights are (out, in).
 * Every bias (*_b) and every LayerNorm beta may be NULL (= zeros); LayerNorm
 * gammas may be NULL (= ones).
 */
typedef struct {
  const void *ln1_w, *ln1_b;               /* [C] */
  const void *q1_w, *k1_w, *v1_w;          /* [C][C] */
  const void *q1_b, *k1_b, *v1_b;          /* [C] */
  const void *o1_w, *o1_b;                 /* [C][C], [C] */
  const void *ln2_w, *ln2_b;               /* [C] */
  const void *q2_w, *q2_b;                 /* [C][C], [C] */
  const void *k2_w, *v2_w;                 /* [C][D_ctx] */
  const void *k2_b, *v2_b;                 /* [C] */
  const void *o2_w, *o2_b;                 /* [C][C], [C] */
  const void *ln3_w, *ln3_b;               /* [C] */
  const void *ff1_w, *ff1_b;               /* [2F][C], [2F]; rows [0,F) value, [F,2F) gate */
  const void *ff2_w, *ff2_b;               /* [C][F], [C] */
} st_layer_weights;

typedef struct {
  const void *gn_w, *gn_b;                 /* [C]; NULL = ones / zeros */
  const void *proj_in_w, *proj_in_b;       /* [C][C] (== 1x1 conv [C][C][1][1]), [C] */
  const void *proj_out_w, *proj_out_b;     /* [C][C], [C] */
  const st_layer_weights *layers;          /* HOST array of `depth` entries */
} st_block_weights;

/*
 * Create a block handle on the current HIP device.
 *   B, H, W >= 1; C % 64 == 0 and heads * 64 == C; D_ctx % 64 == 0, D_ctx >= 64;
 *   depth >= 1; dtype one of st_dtype.  Every workspace must fit the device.
 *   The kernels address each GEMM operand with 32-bit byte offsets, so
 *   shapes whose largest operands reach 2^31 bytes are refused with
 *   ST_ERR_UNSUPPORTED: B*H*W*4*C >= 2^30 (the GEGLU output), 16*C*C >= 2^31
 *   (the FF1 weights) or 4*C*depth*D_ctx >= 2^31 (the context K/V weights
 *   of all layers).  A handle that create returns therefore never fails a
 *   forward on its shape.
 *   w:      device pointers as described above; every non-bias weight must be
 *           non-NULL and 16-byte aligned.  The weights are COPIED (and
 *           repacked) into memory the handle owns; the caller may free them
 *           once create returns.
 *   stream: hipStream_t used for the copies (NULL = default stream); create
 *           synchronises it before returning.
 *   out:    receives the handle; set to NULL on any error.
 * Returns ST_OK, or an error with nothing allocated.
 * Environment, read here: ST_MAX_DEVICE_BYTES (decimal) caps the device
 * memory the handle may allocate (beyond it create fails with
 * ST_ERR_OUT_OF_MEMORY); ST_ATTN_CUS overrides the CU count that the bf16
 * self-attention's load-balance plan assumes (it changes only how the work
 * is split over keys, and with it which of the two self-attention kernels
 * runs -- not the result beyond rounding order; for tests).
 */
st_status st_block_create(int B, int C, int H, int W, int heads, int D_ctx,
                          int depth, st_dtype dtype, const st_block_weights *w,
                          void *stream, st_block **out);

/*
 * Enqueue one forward on `stream` (hipStream_t, NULL = default stream).
 *   x   [B][C][H][W]      device, dtype, 16-byte aligned, read only
 *   ctx [B][77][D_ctx]    device, dtype, 16-byte aligned, read only
 *   y   [B][C][H][W]      device, dtype, 16-byte aligned, written
 * y must not overlap x or ctx.  The call only enqueues work and returns before
 * it completes; x, ctx and y must stay valid until the stream reaches it.
 * It allocates nothing.  Every argument is validated before the first
 * launch: on ST_ERR_INVALID nothing is enqueued.  ST_ERR_DEVICE (a launch
 * that the HIP runtime refused) can leave earlier launches of the same call
 * enqueued; y is then undefined.  Forwards on one handle must not overlap
 * (see Threading).
 */
st_status st_block_forward(st_block *blk, const void *x, const void *ctx,
                           void *y, void *stream);

/*
 * st_block_forward with a key padding mask on the context ("企业官网建设流程全解析"
 * §5.5, Cross-Attention mask: the tokenizer's attention_mask, 0 marking a
 * padding token that must take no part in the cross-attention).
 *   ctx_mask [B][77] device bytes, nonzero = a real token (attended), 0 =
 *            padding (excluded from the softmax of every cross-attention);
 *            NULL = no mask (exactly st_block_forward).  A sample whose
 *            every token is masked gets a zero cross-attention output.
 * Other arguments, validation and errors as st_block_forward; ctx_mask is
 * read on the stream and must stay valid until the stream reaches it; y
 * must not overlap it.
 */
st_status st_block_forward_masked(st_block *blk, const void *x, const void *ctx,
                                  const unsigned char *ctx_mask, void *y, void *stream);

/*
 * Debug: run the forward up to `stage` and copy the fp32 residual stream h
 * ([T][C], token n = i*W + j of sample b at row b*N + n) to `h_out` (device,
 * T*C floats).  stage 0 = after proj_in; stage 1 + 3*l + s = after sublayer
 * s of layer l (s = 0 self-attention, 1 cross-attention, 2 feed-forward).
 * The returned values equal the ones the full forward computes at that point.
 */
st_status st_block_forward_stage(st_block *blk, const void *x, const void *ctx,
                                 int stage, float *h_out, void *stream);

/*
 * Wait for the handle's device to go idle (every stream any forward used,
 * including streams the caller may have destroyed since), then free
 * everything.  NULL-safe.
 */
void st_block_destroy(st_block *blk);

/*
 * Range check of the fp16 intermediates (bf16 storage).  Enqueues a read of
 * the handle's range flag on `stream`, waits for it, and returns
 * ST_ERR_RANGE (and clears the flag) if any forward on this handle since the
 * last check stored a value outside the fp16 range -- the residual stream
 * h, the GEGLU output or the GroupNorm output reached |v| >= 65520 or NaN;
 * the y of those forwards is then not valid.  ST_OK otherwise, and always
 * for fp32 storage.  Call it on the stream of the forwards (or after they
 * are complete); like a forward, it must not overlap another call on the
 * same handle.
 */
st_status st_block_check_range(st_block *blk, void *stream);

/* Text of the last error on this host thread; never NULL ("" if none). */
const char *st_last_error(void);

/*
 * Per-kernel timing.  st_block_set_timing(blk, mask) selects kernel kinds by
 * bit (1u << st_kernel_kind; 0 = off).  Every later forward records a pair of
 * HIP events around each launch of a selected kind, on the stream the kernel
 * is launched on (events without the system-scope fence: they time, they
 * do not synchronise).  After the caller has synchronised that stream,
 * st_block_read_timing() adds the elapsed times up by kind (milliseconds
 * summed over every forward since the last read, and launch counts) and
 * clears them.  Selecting fewer kinds perturbs the other kernels less.
 */
typedef enum {
  ST_K_GN_STATS = 0, /* GroupNorm statistics */
  ST_K_PROJ_IN,      /* GroupNorm apply + NCHW->tokens + proj_in GEMM */
  ST_K_LAYERNORM,    /* the three LayerNorms of each layer (fp32 storage
                        only: with bf16 storage they are folded into the
                        GEMMs around them and have no launch) */
  ST_K_QKV,          /* fused Q/K/V projection of the self-attention */
  ST_K_SELF_ATTN,    /* self-attention over the H*W tokens */
  ST_K_ATTN_OUT,     /* output projections of both attentions (+ residual) */
  ST_K_CROSS_Q,      /* Q projection of the cross-attention (bf16 storage
                        with H*W % 64 == 0: with the cross-attention in its
                        epilogue) */
  ST_K_CTX_KV,       /* K/V projections of the context, all layers */
  ST_K_CROSS_ATTN,   /* cross-attention over the 77 context tokens (when
                        it is not fused into ST_K_CROSS_Q) */
  ST_K_FF1_GEGLU,    /* first feed-forward GEMM + GEGLU */
  ST_K_FF2,          /* second feed-forward GEMM (+ residual) */
  ST_K_PROJ_OUT,     /* proj_out GEMM + tokens->NCHW + outer residual */
  ST_K_COUNT
} st_kernel_kind;

typedef struct {
  double ms[ST_K_COUNT];   /* summed elapsed milliseconds */
  long long launches[ST_K_COUNT];
} st_timing;

st_status st_block_set_timing(st_block *blk, unsigned kind_mask);
st_status st_block_read_timing(st_block *blk, st_timing *out);

/*
 * Limits the timing of the per-layer kinds (LayerNorm, Q/K/V, both
 * attentions, their output projections, the cross Q projection, FF1, FF2)
 * to the launches of layers 0 .. layers-1 of each forward; 0 (the
 * default) times every layer, and the other kinds are unaffected.  Each
 * event pair leaves a bubble of a few microseconds between two kernels,
 * so timing one layer of a deep block perturbs it less.  ST_ERR_INVALID
 * for a NULL handle or layers < 0.
 */
st_status st_block_set_timing_layers(st_block *blk, int layers);

/*
 * The same recorded launches one by one, in launch order: kinds[i] (an
 * st_kernel_kind) and ms[i] for the first `capacity` of them; *count
 * receives the number recorded.  Clears them, as st_block_read_timing does.
 */
st_status st_block_read_timing_launches(st_block *blk, int *kinds, double *ms,
                                        long long capacity, long long *count);

/*
 * Measurement helper: the sustained bf16 MFMA rate of the current device.
 * Launches a kernel of two workgroups per CU whose wavefronts each run four
 * independent v_mfma_f32_32x32x16_bf16 chains for `iters` rounds (no memory
 * traffic in the loop), timed by HIP events on `stream` (after one untimed
 * launch), and reads the shader-cycle and real-time counters around each
 * workgroup's loop.  *tflops = dense bf16 TFLOP/s achieved; *sclk_mhz = the
 * mean shader clock during the loop.  Allocates and frees a small buffer;
 * synchronises `stream`.
 */
st_status st_measure_mfma_bf16(int iters, void *stream, double *tflops,
                               double *sclk_mhz);

#ifdef __cplusplus
}
#endif
#endif /* ST_BLOCK_H */
