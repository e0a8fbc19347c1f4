// Host-side launch interface of the Spatial-Transformer block kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stb {

// Element type of an activation buffer.
enum ActType { ACT_F32 = 0, ACT_BF16 = 1, ACT_F16 = 2 };

enum EpiKind {
  EPI_STORE_F32 = 0,  // out_f32[row*ldo + col] = acc + bias[col]
  EPI_RESID_F32 = 1,  // out_f32[row*ldo + col] += acc + bias[col]
  EPI_HEADS = 2,      // scatter into per-head Q/K (row-major) or V^T layouts
  EPI_GEGLU = 3,      // paired value/gate columns -> value * GELU(gate), fp16 out
  EPI_NCHW = 4,       // rows = channels, cols = tokens: y = acc + bias[row] + x
  EPI_STORE_H16 = 5,  // out_act (fp16) [row*ldo + col] = fp16(acc + bias[col])
  EPI_RESID_H16 = 6,  // out_act (fp16) [row*ldo + col] = fp16(that value + acc + bias[col])
  EPI_CROSS_ATTN = 7,  // the product is Q of the cross-attention: attend (CrossAttn)
  EPI_CONV = 8         // implicit-GEMM convolution (ConvGemm): rows = output
                       // channels, cols = output pixels on the padded grid
};

// Implicit-GEMM 3x3 convolution (EPI_CONV).  The activations live in a
// zero-haloed NHWC buffer: pixel row r = (b * Hp + ip) * Wp + jp for the
// padded position (ip, jp) (input pixel (i, j) at (i + 1, j + 1)), L
// elements per pixel row.  The product is C[M = Cout][N] = A[Cout][K] (the
// weights, tap-major: K index t * Cin + ci for tap t = 3 di + dj, then the
// shortcut's Csc channels) times B^T, where B row m (an output pixel of the
// padded grid, m = (b * Hq + i) * Wp + j) for tap (di, dj) is buffer row
// stride * m + di * Wp + dj, channels [0, Cin); the shortcut segment reads
// buffer row stride * m + sc_roff, channels [sc_cbase, sc_cbase + Csc).
// GEMM parameters: B = the buffer, ldb = stride * L, N = B * Hq * Wp; the
// K stages (64 deep) walk the taps in order, spt = Cin / 64 stages per tap,
// sc_spt = Csc / 64 after them.  Output pixel m is valid when i < Ho and
// j < Wo; its value acc + cadd[b * M + row] (+ resid, NCHW, when given)
// is stored to out NCHW [B][M][Ho][Wo] as bf16.
struct ConvGemm {
  int L, Wp, Hq, Ho, Wo;
  int spt, sc_spt, sc_cbase, sc_roff;
  long long b_bytes;        // bytes of the activation buffer (reads past it return 0)
  const float* cadd;        // [B][M] per sample and output channel (bias + time embedding)
  const void* resid;        // NCHW [B][M][Ho][Wo] bf16, or NULL
  void* out;                // NCHW [B][M][Ho][Wo] bf16
};

// Cross-attention in the epilogue of its Q projection (EPI_CROSS_ATTN).
// Column col of the product is dimension col % 64 of head col / 64; row r is
// query n = r % rows_per_batch of sample r / rows_per_batch, and every
// 64-row block of the product must lie in one sample (rows_per_batch % 64 ==
// 0).  Q = (acc + bias) * scale is rounded to bf16 and attends over the nk
// keys (64 < nk <= 96) of k [B*heads][kv_pad][64] and vt [B*heads][64][kv_pad] (bf16,
// kv_pad >= 96, padding finite) with softmax base 2 (scale includes
// log2(e)); O goes to o [M][ldo] bf16, columns as in the product.
// key_bits (may be NULL): the context's key padding mask, 4 words per
// sample, bit k of word w set when key 32 w + k attends; a sample with no
// bit set gets O = 0.
struct CrossAttn {
  const void* k;
  const void* vt;
  int kv_pad, nk;
  int rows_per_batch, heads;
  float scale;
  const uint32_t* key_bits;
};

// Destination of the head-split epilogue.  Column col of the product maps to
// which = col / C, split s = which % nsplit, layer = which / nsplit, head =
// (col % C) / 64, dim = col % 64; row maps to sample b = row / rows_per_batch
// and sequence position n = row % rows_per_batch.  dst[s] + layer*layer_stride
// is a [B*heads][npad][64] array, or [B*heads][64][npad] when bit s of
// transposed_mask is set.  Values of split s (bias included) are multiplied
// by scale[s] before rounding.
struct HeadSplit {
  void* dst[3];
  float scale[3];
  int transposed_mask;
  int nsplit;
  long long layer_stride;
  int rows_per_batch;
  int npad;
  int heads;
  int C;
};

struct EpiParams {
  int kind;
  const float* bias;      // by column; by row for EPI_NCHW; may be NULL
  float* out_f32;         // EPI_STORE_F32 / EPI_RESID_F32
  int ldo;
  void* out_act;          // EPI_GEGLU: [M][F]; EPI_NCHW: y [B][M][ntok];
                          // EPI_RESID_F32 (optional): the new value as fp16
                          // [M][ldo]
  const void* resid_act;  // EPI_NCHW: x [B][M][ntok]
  int F;                  // EPI_GEGLU: value width
  int ntok;               // EPI_NCHW: tokens per sample
  HeadSplit hs;
  // EPI_STORE_* / EPI_RESID_* (optional): per row and 64-column block of the
  // new values (as stored), their sum and their sum of squared deviations
  // from the block's mean, [M][ldo / 64].
  float2* row_stats;
  // LayerNorm folded into the product (EPI_HEADS or EPI_GEGLU, no split-K):
  // A holds h and B the weights times gamma (weight_fold_layernorm), and each
  // product is corrected per row to rstd * (acc - mean * ln_g[col]) before
  // the epilogue, with mean and rstd = 1 / sqrt(var + ln_eps) of the row of
  // h combined from ln_stats (written as row_stats above; K = 64 * ln_blocks).
  const float2* ln_stats;
  const float* ln_g;
  int ln_blocks;
  float ln_eps;
  CrossAttn ca;  // EPI_CROSS_ATTN (output: out_act, row stride ldo)
  // fp16 outputs (EPI_STORE_H16, EPI_RESID_H16, EPI_GEGLU and their split-K
  // pass): set to 1 when a stored value is not finite (an fp32 value at or
  // beyond 65520 in magnitude rounds to infinity); may be NULL
  int* range_flag;
};

// C[M][N] = A[M][K] * B[N][K]^T, then the epilogue.
struct GemmParams {
  const void* A;
  long long lda;
  const void* B;
  long long ldb;
  int M, N, K;
  EpiParams epi;
  // Split-K (gemm_mfma only; EPI_HEADS or EPI_STORE_F32 with bf16 operands
  // and no row sums, or EPI_STORE_H16 / EPI_RESID_H16; no folded LayerNorm):
  // with ksplit > 1, K is cut into ksplit equal slices whose fp32 products
  // land in ws[ksplit][M][N]; a second pass adds the slices in order and
  // applies the epilogue.
  int ksplit;
  float* ws;
  // First output column this launch computes (set by gemm_mfma when it
  // splits a product's columns between two tile shapes; callers leave 0).
  int n_off;
  ConvGemm conv;  // EPI_CONV only
};

// K slices for an implicit-GEMM convolution (M = Cout, N = pixels of the
// padded grid, K = 9 Cin + Csc): with fewer than half as many 128x128
// output tiles as CUs, the most slices (<= 12) that keep each at least 16
// stages deep and give every slice a CU; 1 = no split.  Workspace of a
// split product: ksplit * M * (N rounded up to 64) floats.
int conv_ksplit(int M, int N, int K, int cus);

// MFMA GEMM with 16-bit operands and fp32 accumulation.  `op` is ACT_BF16 or
// ACT_F16 and gives the type of A and B.  Requires K % 64 == 0 and 16-byte
// aligned rows; any M, N.
hipError_t gemm_mfma(const GemmParams& p, int op, hipStream_t s);
// fp32 everything (debug path).  Requires K % 16 == 0.
hipError_t gemm_f32(const GemmParams& p, hipStream_t s);

// Multi-head attention, per (b, head): O = softmax(Q K^T / 8) V.
// q: [B*heads][q_pad][64], k: [B*heads][kv_pad][64], vt: [B*heads][64][kv_pad]
// (padding rows must hold finite values), o: token-major [B*Nq][C].
struct AttnParams {
  const void* q;
  const void* k;
  const void* vt;
  void* o;
  int B, heads, C;
  int Nq, Nk;
  int q_pad, kv_pad;
  // Load balance of the bf16 kernel (attention_bf16_plan): the first n_full
  // query tiles, in (b, head, tile) order, are computed whole; every later
  // tile is split over its key tiles into nsplit pieces whose partial
  // results (unnormalised O, running max and row sum) go to `part`, and a
  // second kernel merges them in piece order.  nsplit <= 1: no split.
  int n_full, nsplit;
  float* part;        // [tiles - n_full][nsplit][attention_bf16_part_floats()]
  // Cross-attention only (Nk <= 96, no split): key padding mask as in
  // CrossAttn::key_bits, or NULL.
  const uint32_t* key_bits;
};
// bf16 path: q holds the queries already multiplied by
// attention_bf16_q_scale() = log2(e) / sqrt(64), so that the kernel's scores
// are base-2 exponents.
hipError_t attention_bf16(const AttnParams& p, hipStream_t s);
float attention_bf16_q_scale();
hipError_t attention_f32(const AttnParams& p, hipStream_t s);
int attention_bf16_q_tile();   // query rows per workgroup of the bf16 kernel
int attention_bf16_kv_tile();  // key rows per LDS tile of the bf16 kernel
int attention_bf16_part_floats();  // partial-result floats per piece
// Split plan for B*heads*ceil(Nq/q_tile) query tiles over `cus` compute
// units: whole tiles fill a whole number per CU, the rest are split so that
// each CU also gets about one piece.  Sets n_full and nsplit.
void attention_bf16_plan(int B, int heads, int Nq, int Nk, int cus, int& n_full, int& nsplit);

// Norms and helpers.  `bf16` flags say whether activations are bf16 (else fp32).
// GroupNorm in two launches: gn_stats writes, per (sample, group), the sums
// of (x - the group's first element) and of its square over gn_split()
// slices into partial[B*32][split]; gn_apply_tokens combines them (fp64),
// normalises, applies gamma/beta and transposes NCHW -> tokens [B*N][C] of
// type `out_type` (ACT_F32 or ACT_F16).
hipError_t gn_stats(const void* x, bool bf16, int B, int C, int N,
                    float2* partial, int max_split, hipStream_t s);
int gn_split(int C, int N, int max_split);
// With an fp16 output, *range_flag (may be NULL) is set to 1 when a stored
// value is not finite.
hipError_t gn_apply_tokens(const void* x, bool bf16, const float2* partial,
                           int max_split, const float* gamma, const float* beta,
                           void* out, int out_type, int B, int C, int N,
                           int* range_flag, hipStream_t s);
// GroupNorm apply NCHW -> NCHW from gn_stats partials, optionally followed
// by SiLU; gamma/beta of the activation type (NULL = ones / zeros).
hipError_t gn_apply_nchw(const void* x, bool bf16, const float2* partial, int max_split,
                         const void* gamma, const void* beta, void* y, int B, int C, int N,
                         float eps, bool silu, hipStream_t s);
// ResnetBlock2D helpers.  gn_apply_pad: GroupNorm apply + SiLU of NCHW
// bf16 x (partials of gn_stats) into the zero-haloed NHWC fp16 operand of a
// 3x3 convolution (row (b (H + 2) + i + 1) Wp + j + 1, L elements per row);
// with `raw`, the raw x also to raw (row length L_raw, channels from
// raw_cbase).  C % 64 == 0.  gamma, beta fp32.
hipError_t gn_apply_pad(const void* x, const float2* partial, int max_split, const float* gamma,
                        const float* beta, void* out, int B, int C, int H, int W, int Wp, int L,
                        float eps, void* raw, int L_raw, int raw_cbase, int* range_flag,
                        hipStream_t s);
// cadd[b][co] = w[co] . SiLU(temb[b]) + temb_b[co] + conv_b[co] (bf16 temb
// and w, fp32 biases, NULL = 0); needs temb_proj_supported(B, Dt): B <= 16,
// Dt % 8 == 0 and B * Dt <= 16384.
hipError_t temb_proj(const void* temb, const void* w, const float* temb_b, const float* conv_b,
                     float* cadd, int B, int Dt, int Cout, hipStream_t s);
bool temb_proj_supported(int B, int Dt);
// 3x3 convolution weights [Cout][Cin][3][3] bf16 (+ 1x1 shortcut [Cout][Csc])
// -> tap-major fp16 GEMM operand [Cout][9 Cin + Csc].
hipError_t conv_weight_pack(const void* w, const void* sc, void* dst, int Cout, int Cin, int Csc,
                            int* overflow, hipStream_t s);
// The same with the input channels padded to Cp (>= Cin, zero weights).
hipError_t conv_weight_pack_padded(const void* w, const void* sc, void* dst, int Cout, int Cin,
                                   int Cp, int Csc, int* overflow, hipStream_t s);
// U-Net helpers.  nchw_to_pad: NCHW bf16 x -> zero-haloed NHWC fp16 operand
// (grid Hg = H or 2H with `up` (nearest 2x), rows (b (Hg + 2) + i + 1) Wp +
// j + 1, L >= C elements per row, channels >= C untouched).
hipError_t nchw_to_pad(const void* x, void* out, int B, int C, int H, int W, int Wp, int L, bool up,
                       int* range_flag, hipStream_t s);
// Sinusoidal embedding of t [B] (fp32) -> out [B][dim] fp32, cosines first.
hipError_t timestep_embed(const float* t, float* out, int B, int dim, hipStream_t s);
// y [B][Dout] (+)= w act(x) + bias for the embedding MLPs (x fp32 or bf16,
// act SiLU or identity, w bf16 [Dout][Din]; y16 (optional) gets a bf16
// copy); needs temb_proj_supported(B, Din).
hipError_t mlp_linear(const void* x, bool x_bf16, bool silu, const void* w, const float* bias,
                      float* y, void* y16, bool accumulate, int B, int Din, int Dout, hipStream_t s);
// Key padding mask [B][nk] bytes (nonzero = attend) -> bits [B][4] words
// (bit k of word w: key 32 w + k; keys >= nk clear); nk <= 96.
hipError_t mask_to_bits(const uint8_t* mask, uint32_t* bits, int B, int nk, hipStream_t s);
// Guided DDPM step: x_prev[i] = c1 * (x_t[i] - c2 * e) + sigma * noise[i]
// (noise NULL: no term), e = eps_u + scale * (eps_c - eps_u), eps_pair =
// [eps_u (n); eps_c (n)] in bf16 or fp32; latents fp32.
hipError_t guided_ddpm(const void* eps_pair, bool eps_bf16, const float* x_t, const float* noise,
                       float* x_prev, long long n, float scale, float c1, float c2, float sigma,
                       hipStream_t s);
// u: [T][C] of type `out_type` (ACT_F32, ACT_BF16 or ACT_F16).
hipError_t layernorm(const float* h, const float* gamma, const float* beta,
                     void* u, int out_type, int T, int C, hipStream_t s);
hipError_t geglu_f32(const float* z, float* f, long long T, int F,
                     hipStream_t s);
// dst[i] = float(src[i]) (src fp16), n elements.
hipError_t f16_to_f32(const void* src, float* dst, long long n, hipStream_t s);
// dst[i] = float(src[i]) (src bf16 or fp32); src NULL -> dst[i] = fill.
hipError_t to_f32(const void* src, bool bf16, float* dst, long long n,
                  float fill, hipStream_t s);
// In place: bf16 values -> fp16 (exact within the fp16 range; magnitudes
// above 65504 set *overflow to 1).
hipError_t bf16_to_f16_inplace(void* buf, long long n, int* overflow,
                               hipStream_t s);
// LayerNorm folded into the Linear layer that follows it, for rows x C
// weights w (bf16 on entry, fp16 on return, in place): w[j][c] <- w[j][c] *
// gamma[c] rounded to fp16, g[j] = sum_c of the rounded w[j][c], and
// bias[map ? map[j] : j] += sum_c beta[c] * w[j][c] (the entry weights);
// sums in fp64.  Magnitudes above 65504 set *overflow to 1.
hipError_t weight_fold_layernorm(void* w, int rows, int C, const float* gamma,
                                 const float* beta, float* bias, const int* map,
                                 float* g, int* overflow, hipStream_t s);
// dst row r = src row map[r], rows of `row_bytes` bytes (multiple of 16).
hipError_t gather_rows(const void* src, void* dst, const int* map, int rows,
                       long long row_bytes, hipStream_t s);

// Matrix-pipe probe (k_probe.hip): `grid` workgroups of four wavefronts,
// each running four independent bf16 32x32x16 MFMA chains for `iters`
// rounds.  out: grid * 256 floats (the sums, kept live); clocks: 2 * grid
// values, per workgroup the shader cycles and the real-time ticks of the
// loop.
int mfma_probe_grid(int cus);
long long mfma_probe_flops(int grid, int iters);
hipError_t mfma_probe(int grid, int iters, float* out, long long* clocks, hipStream_t s);

}  // namespace stb
