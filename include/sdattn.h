/*
 * sdattn.h -- C ABI of libsdattn: fused scaled dot-product attention for the
 * transformer blocks of a diffusion UNet, and the GroupNorm(+SiLU) of its
 * residual blocks, on AMD MI355X (gfx950).
 *
 * Operation.  For every batch b < B, head h < H and query row i < Lq:
 *
 *     O[b,h,i,:] = sum_j softmax_j( scale * <Q[b,h,i,:], K[b,h,j,:]> ) V[b,h,j,:]
 *
 * This is the attention of the page "Diffusion inference engine from
 * scratch: Rust + wgpu" (ybb.press), section 3.2: queries come from the
 * latent feature map (HW tokens), keys and values either from the same map
 * (self-attention) or from the 77-token CLIP text context (cross-attention),
 * and the score matrix Q.K^T is never written to memory -- the softmax is
 * evaluated block by block with a running maximum and running sum, which
 * gives the plain softmax result up to rounding.  The scale is an explicit
 * argument (1/sqrt(d) for the UNet; the pages do not print it).
 *
 * Layout.  q, k, v and out are contiguous row-major [B, H, L, d] device
 * buffers: L = Lq for q and out, L = Lk (or Lctx) for k and v.  Keys and
 * values carry their own batch index (classifier-free guidance concatenates
 * the unconditional and conditional contexts along B; nothing is broadcast).
 *
 * Types (the dtype argument):
 *   SDATTN_DTYPE_F32          fp32 q/k/v, fp32 out; fp32 arithmetic.
 *   SDATTN_DTYPE_BF16         bf16 q/k/v, bf16 out (round to nearest even);
 *                             bf16 matrix products with fp32 accumulation,
 *                             the softmax weights are rounded to bf16 before
 *                             the second product.
 *   SDATTN_DTYPE_BF16_F32OUT  as SDATTN_DTYPE_BF16 but out is fp32.
 *   SDATTN_DTYPE_F16          fp16 q/k/v, fp16 out: the half-precision
 *                             storage the same page's section 5.2 uses for
 *                             weights and activations; fp16 matrix products
 *                             with fp32 accumulation, weights rounded to fp16
 *                             (kept <= 2^8 by the running maximum, well
 *                             inside fp16's range).
 *   SDATTN_DTYPE_F16_F32OUT   as SDATTN_DTYPE_F16 but out is fp32.
 *
 * Ownership and synchronisation.  The caller owns every buffer and the
 * stream.  The library allocates no device memory and needs no workspace.
 * Calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 * stream) and return without synchronising; buffers must stay alive until
 * that work completes.  Inputs are read only; out must not overlap them.
 * Calls are stateless and thread-safe.
 *
 * Errors.  Every function returns an sdattn_status; nothing is printed and
 * no exception crosses the ABI.  Arguments are validated on the host before
 * any HIP call.  A fault inside a kernel surfaces at the caller's next
 * synchronisation of the stream, not as a return code.
 */
#ifndef SDATTN_H
#define SDATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SDATTN_OK = 0,
  SDATTN_ERR_INVALID_ARG = 1,  /* null pointer, B/H/Lq/Lk/d < 1, unknown dtype,
                                  non-finite scale, out overlapping an input,
                                  or a tensor larger than 2^31 - 1 elements */
  SDATTN_ERR_UNSUPPORTED = 2,  /* d % 8 != 0, d > 256, or (cross entry) a
                                  context longer than sdattn_cross_max_ctx */
  SDATTN_ERR_MISALIGNED = 3,   /* a pointer not 16-byte aligned */
  SDATTN_ERR_DEVICE = 4,       /* no HIP device, or the current device is
                                  not gfx950 */
  SDATTN_ERR_LAUNCH = 5        /* the kernel launch reported an error */
} sdattn_status;

typedef enum {
  SDATTN_DTYPE_F32 = 0,
  SDATTN_DTYPE_BF16 = 1,
  SDATTN_DTYPE_BF16_F32OUT = 2,
  SDATTN_DTYPE_F16 = 3,
  SDATTN_DTYPE_F16_F32OUT = 4
} sdattn_dtype;

/* Attention with any key length.  Internally dispatches to the short-key
 * kernel (all keys resident in LDS, single-pass softmax) when
 * Lk <= sdattn_cross_max_ctx(d, dtype), and to a streaming kernel
 * (K/V tiles streamed through several LDS buffers ahead of their use,
 * blockwise softmax) otherwise.
 * Used for UNet self-attention (Lk = Lq = HW). */
int sdattn_fwd(const void *q, const void *k, const void *v, void *out, int B,
               int H, int Lq, int Lk, int d, float scale, int dtype,
               void *stream);

/* Cross-attention to a short context (the text encoder's 77 tokens): always
 * the short-key kernel; returns SDATTN_ERR_UNSUPPORTED when
 * Lctx > sdattn_cross_max_ctx(d, dtype).  For Lctx within the cap the
 * result is bit-identical to sdattn_fwd on the same arguments. */
int sdattn_cross_fwd(const void *q, const void *ctx_k, const void *ctx_v,
                     void *out, int B, int H, int Lq, int Lctx, int d,
                     float scale, int dtype, void *stream);

/* Attention that always takes the streaming (online-softmax) kernel, for
 * any Lk >= 1.  For SDATTN_DTYPE_F32 this is the same kernel sdattn_fwd
 * uses. */
int sdattn_stream_fwd(const void *q, const void *k, const void *v, void *out,
                      int B, int H, int Lq, int Lk, int d, float scale,
                      int dtype, void *stream);

/* The same attention on token-major operands, as the page's section 3.2
 * has them: activations [B, HW, C] with C = H*d and the head split implicit.
 * q is [B, Lq, ldq], k and v are [B, Lk, ldkv], out is [B, Lq, ldo]
 * (row-major; element (b, i, h*d + c) is head h, column c of token i).  A
 * row stride larger than H*d lets q, k and v be column slices of one fused
 * projection, e.g. [B, L, 3C] with k = q + C and v = q + 2C, ld = 3C.
 * Requires every ld >= H*d and ld % 8 == 0 (else SDATTN_ERR_INVALID_ARG);
 * the out rows must not overlap the inputs' spans.  Dispatch, dtypes and
 * results are those of sdattn_fwd on the same values in [B, H, L, d]
 * layout (bit-identical). */
int sdattn_fwd_strided(const void *q, const void *k, const void *v, void *out,
                       int B, int H, int Lq, int Lk, int d, int ldq, int ldkv,
                       int ldo, float scale, int dtype, void *stream);

/* GroupNorm, optionally fused with the SiLU that follows it: the page's
 * section 3.1 normalisation (each group's mean and variance, inverse
 * standard deviation 1/sqrt(var + eps)) with the GroupNorm + SiLU fusion its
 * model-level optimisation list names.  x and y are contiguous [N, C, HW]
 * (NCHW with HW = H*W); the G groups are C/G consecutive channels each; for
 * every sample n and group g with M = (C/G)*HW elements:
 *
 *     mu = mean(x over the group),  var = mean((x - mu)^2)   (population)
 *     y  = (x - mu) / sqrt(var + eps) * gamma[c] + beta[c]
 *     y  = y / (1 + exp(-y))                                  if silu == 1
 *
 * gamma and beta are fp32 device arrays of C values.  dtype (as above)
 * gives x's type and y's: fp32/fp32, bf16/bf16, bf16/fp32, fp16/fp16,
 * fp16/fp32; statistics and arithmetic are fp32.  y == x (in place) is
 * allowed when both have the same element size; any other overlap of y with
 * x, gamma or beta is SDATTN_ERR_INVALID_ARG, as are N, C, HW, G < 1,
 * C % G != 0, a non-finite or negative eps and silu not 0/1.  HW % 8 != 0
 * or more than 8192 channels per group is SDATTN_ERR_UNSUPPORTED; x and y
 * must be 16-byte aligned, gamma and beta 4-byte aligned
 * (SDATTN_ERR_MISALIGNED). */
int sdattn_group_norm(const void *x, const float *gamma, const float *beta, void *y,
                      int N, int C, int HW, int G, float eps, int silu, int dtype,
                      void *stream);

/* Largest context length the short-key path accepts for this head dim and
 * dtype; 0 if (d, dtype) is unsupported. */
int sdattn_cross_max_ctx(int d, int dtype);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *sdattn_strerror(int status);

/* ABI version: major * 10000 + minor * 100 + patch (1.3: fp16 dtypes,
 * sdattn_fwd_strided, sdattn_group_norm). */
int sdattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDATTN_H */
