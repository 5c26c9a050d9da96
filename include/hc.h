/*
 * hc.h -- C ABI of libhc.so, the identity Hyper-Connections residual path on
 * MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [EXPL]  learnaivisually.com, "Tencent open-sources Hy4 Preview at 770B --
 *           Identity Hyper-Connections -- What does it mean?"
 *   [GLOSS] hfviewer.com glossary entry "Hyper-connections (mHC)"
 *   [ATLAS] llm-atlas model card "Tencent Hy4-preview (770B-A49B)"
 *   [MAP]   models.inteligile.com, "Hy4-preview" model techniques map
 *
 * The residual stream is widened to n parallel streams that a block reads
 * from and writes to separately ([EXPL] "Jargon", Hyper-Connections); learned
 * matrices mix them before and after the block ([GLOSS] definition).  Around
 * a user's block the path is therefore two calls: hc_pre_mix before it (the
 * block's input) and hc_post_mix after it (write-back into the streams), plus
 * the producers of per-token mixing weights (hc_weights, hc_sinkhorn).
 *
 * Common conventions
 * ------------------
 *  - Residual state H: [T][n][d] contiguous, token-major; T tokens in flight,
 *    n streams (1..4; Hy4 uses 4 per [EXPL] TL;DR), hidden width d.
 *  - Block input u and block output F: [T][d] contiguous.
 *  - Storage dtype (hc_dtype) applies to H, F, u, H_out and W.  Arithmetic is
 *    fp32; results are rounded once to the storage type (nearest, ties to
 *    even; subnormals kept).  FP8 stores saturate: magnitudes beyond 448
 *    (infinities included) store as +-448; NaN stays NaN.
 *  - Weight record: K = 2n + n^2 fp32 values
 *        [alpha_0..alpha_{n-1} | beta_0..beta_{n-1} | A row-major]
 *    A[i][j] (at 2n + i*n + j) weighs input stream j into output stream i.
 *    Record of token t is at w + t * w_stride; w_stride = 0 shares one record
 *    (static weights), otherwise w_stride >= K.
 *  - Identity weights (alpha = e_0, beta = 1, A = I) on n copies of one
 *    stream reproduce the ordinary residual x + f(x) bitwise ([EXPL]
 *    "Jargon", Identity initialization).
 *  - Every pointer is device memory owned by the caller.  The library
 *    allocates nothing and keeps no state, and calls are thread-safe; the one
 *    exception is hc_post_mix_backward_noalloc, whose scratch is a fixed
 *    array per GPU that overlapping calls on one GPU share.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Work
 *    is enqueued and the call returns without synchronising.
 *  - All arguments are validated before anything is launched; a failed check
 *    returns its code with nothing enqueued.  A launch failure reported by the
 *    HIP runtime returns HC_ERR_HIP.  No exception crosses the ABI and the
 *    library never prints.
 *  - Sizes: 1 <= n <= 4; 1 <= d <= HC_MAX_HIDDEN; d % 16 == 0 for fp8,
 *    d % 8 == 0 for bf16 and d % 4 == 0 for fp32 (16-byte vectors) else
 *    HC_ERR_SHAPE.  T < 0 is
 *    HC_ERR_ARG.  T == 0 (count == 0 for hc_block_tanh) is a no-op returning
 *    HC_OK once the scalar arguments are valid; the data pointers are then
 *    not checked and may be NULL (an empty tensor has no storage).
 *  - Alignment: H, F, u, H_out, W and gamma 16 bytes; weight records and
 *    logits 4 bytes (HC_ERR_ALIGN).
 *  - Aliasing: outputs may not overlap any input or each other
 *    (HC_ERR_ALIAS), except H_out == H exactly in hc_post_mix (in place).
 */
#ifndef HC_H
#define HC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hc_status {
    HC_OK = 0,
    HC_ERR_NULL = 1,   /* a required pointer is NULL                        */
    HC_ERR_SHAPE = 2,  /* n, d or a stride outside the supported set       */
    HC_ERR_DTYPE = 3,  /* unknown hc_dtype, or one the call does not take   */
    HC_ERR_ALIGN = 4,  /* pointer not aligned as required                   */
    HC_ERR_ALIAS = 5,  /* an output overlaps an input or another output     */
    HC_ERR_ARG = 6,    /* T < 0, eps not positive/finite, iters out of range */
    HC_ERR_HIP = 7     /* the HIP runtime reported a launch error           */
} hc_status;

/* Storage dtypes.  HC_FP8 is E4M3 (OCP 8-bit float: 4 exponent bits, bias 7,
 * 3 mantissa bits, no infinities, largest finite 448).  The release ships
 * BF16 and FP8 weights ([EXPL] "The news"; [MAP] "inference quantization");
 * the pages name no 8-bit format, E4M3 is the one implemented.  FP8 is taken
 * by hc_pre_mix, hc_post_mix, hc_post_pre_mix, hc_weights and hc_weights_save
 * (H and W in FP8, fp32 accumulation) and hc_block_tanh; the gradient calls
 * (the *_backward entry points) return HC_ERR_DTYPE for it. */
typedef enum hc_dtype { HC_F32 = 0, HC_BF16 = 1, HC_FP8 = 2 } hc_dtype;

#define HC_MAX_STREAMS 4
#define HC_MAX_HIDDEN 16384
#define HC_MAX_SINKHORN_ITERS 10000
#define HC_RECORD_LEN(n) (2 * (n) + (n) * (n))

/* Pre (read-mix + RMSNorm): u = gamma * x / sqrt(mean_k x_k^2 + eps) with
 * x = sum_i alpha_i H_i.  [GLOSS] definition (mixing before the block);
 * [EXPL] "Jargon", Pre-norm (the block input is normalised); RMSNorm per
 * [GLOSS] "Related concepts".
 *   H      [T][n][d] dt          w  records (only alpha is read)
 *   gamma  [d] fp32              eps > 0
 *   u      [T][d] dt, output (may not overlap H, w or gamma)
 * The reduction over d is done in an order that depends only on d, so alpha =
 * e_0 gives u bitwise equal to the n = 1 call on stream 0. */
hc_status hc_pre_mix(const void* H, const float* w, int64_t w_stride,
                     const float* gamma, float eps, void* u,
                     int64_t T, int32_t n, int32_t d, hc_dtype dt, void* stream);

/* Post (stream-mix + write-back): H_out_i = sum_j A[i][j] H_j + beta_i F.
 * [GLOSS] definition (mixing after the block); [EXPL] "Jargon", Residual
 * connection (the block output is added to what came in).
 *   H      [T][n][d] dt          F  [T][d] dt
 *   w      records (beta and A are read)
 *   H_out  [T][n][d] dt, output; H_out == H is allowed (in place: every
 *          element is read before the same thread writes it), any other
 *          overlap is HC_ERR_ALIAS. */
hc_status hc_post_mix(const void* H, const void* F, const float* w, int64_t w_stride,
                      void* H_out, int64_t T, int32_t n, int32_t d, hc_dtype dt,
                      void* stream);

/* Per-token weights computed from the streams.  The pages publish no rule for
 * per-token weights ([EXPL], the paragraph on what the model card leaves
 * out); the reading implemented: r_i = 1/sqrt(mean_k H_ik^2 + eps),
 * hbar = (1/n) sum_i r_i H_i, z_c = sum_k hbar_k W[c][k] (c < K), then
 *   sinkhorn_iters == 0:  w = w_static + scale * tanh(z)
 *   sinkhorn_iters  > 0:  l = w_static + scale * z, w = the hc_sinkhorn
 *                         transform of l with that many iterations.
 * The projection runs on the matrix cores (MFMA), fp32 accumulation; FP8
 * operands are widened exactly to bf16 first.
 *   H        [T][n][d] dt        W  [K][d] dt (row c = output c; the layout
 *                                   of a linear layer's weight)
 *   w_static [K] fp32            w_out [T][K] fp32, output (stride K)
 *   0 <= sinkhorn_iters <= HC_MAX_SINKHORN_ITERS, eps > 0. */
hc_status hc_weights(const void* H, const void* W, const float* w_static, float scale,
                     float eps, int32_t sinkhorn_iters, float* w_out,
                     int64_t T, int32_t n, int32_t d, hc_dtype dt, void* stream);

/* Bytes of the state hc_weights_save keeps for hc_weights_backward (0 for
 * T <= 0 or n out of range): the per-stream projections P_i = W H_i
 * ([T][n][K] fp32) and norms r_i ([T][n] fp32, starting at float offset
 * T*n*K rounded up to a multiple of 4). */
int64_t hc_weights_saved_bytes(int64_t T, int32_t n);

/* hc_weights for a training forward ([GLOSS] definition: the weight
 * producers are learned, so their backward needs the forward's state): the
 * same records in w_out (bitwise the same as hc_weights), and in `saved`
 * (saved_bytes >= hc_weights_saved_bytes, 16-byte aligned, no overlap with
 * anything) the projections and norms that hc_weights_backward would
 * otherwise recompute with a second read of H.  Arguments and errors
 * otherwise as hc_weights; a short `saved` is HC_ERR_ARG. */
hc_status hc_weights_save(const void* H, const void* W, const float* w_static, float scale,
                          float eps, int32_t sinkhorn_iters, float* w_out, float* saved,
                          int64_t saved_bytes, int64_t T, int32_t n, int32_t d, hc_dtype dt,
                          void* stream);

/* The write-back of one layer fused with the per-token weights of the next
 * ([GLOSS] definition: mixing weights around every block; [EXPL] "What four
 * streams cost per token": the cost is the n-fold state moved across each
 * boundary, and a separate weights pass would read that state once more).
 * Equivalent to
 *   hc_post_mix(H, F, w, w_stride, H_out)                    then
 *   hc_weights(H_out, W, w_static, scale, eps, sinkhorn_iters, w_out)
 * (or hc_weights_save with `saved`), with H_out taken from registers instead
 * of being read back: H_out is bitwise hc_post_mix's; w_out agrees with
 * hc_weights on H_out to fp32 rounding (the projection's sums are taken in
 * another order).  In a layer loop the records w_out feed the next layer's
 * hc_pre_mix and hc_post_mix; only the first layer needs hc_weights.
 *   H, F, w, w_stride, H_out   as hc_post_mix (H_out == H allowed)
 *   W, w_static, scale, eps,
 *   sinkhorn_iters, w_out      as hc_weights (W of the layer the records are
 *                              for); w_out may not overlap anything
 *   saved, saved_bytes         NULL/0, or the state hc_weights_save keeps
 *                              (saved_bytes >= hc_weights_saved_bytes(T, n),
 *                              16-byte aligned, no overlap): short is HC_ERR_ARG
 * bf16 and FP8 storage only (HC_ERR_DTYPE otherwise).  W is held in
 * registers for the whole call, which bounds the width: d <= 4096, else
 * HC_ERR_SHAPE (use hc_post_mix and hc_weights beyond it). */
hc_status hc_post_mix_weights(const void* H, const void* F, const float* w, int64_t w_stride,
                              const void* W, const float* w_static, float scale, float eps,
                              int32_t sinkhorn_iters, void* H_out, float* w_out, float* saved,
                              int64_t saved_bytes, int64_t T, int32_t n, int32_t d, hc_dtype dt,
                              void* stream);

/* mHC step: make the stream mix doubly stochastic with Sinkhorn iterations
 * ([GLOSS] definition; [ATLAS] "Architecture concepts", mHC).  Per token:
 * alpha = sigmoid(l_alpha), beta = sigmoid(l_beta), A = exp(l_A) then `iters`
 * times {divide every row by its sum; divide every column by its sum}.  With
 * iters >= 1 the largest logit of A is subtracted before exp (equal after the
 * first row division in exact arithmetic).  After the last iteration columns
 * sum to 1 to fp32 rounding; rows approach 1 as iters grows.
 *   logits [T][K] fp32, w_out [T][K] fp32 output (may not overlap logits),
 *   0 <= iters <= HC_MAX_SINKHORN_ITERS. */
hc_status hc_sinkhorn(const float* logits, float* w_out, int32_t iters, int64_t T,
                      int32_t n, void* stream);

/* Cross-layer fusion: the write-back of one layer and the read-mix + RMSNorm
 * of the next in one pass over the streams.  Equivalent to hc_post_mix(H, F,
 * w, w_stride, H_out) followed by hc_pre_mix(H_out, w_next, w_next_stride,
 * gamma_next, eps, u_next) with H_out rounded to dt in between, but H_out is
 * read back from registers instead of HBM.  H_out == H is allowed; u_next may
 * not overlap anything else. */
hc_status hc_post_pre_mix(const void* H, const void* F, const float* w, int64_t w_stride,
                          const float* w_next, int64_t w_next_stride,
                          const float* gamma_next, float eps, void* H_out, void* u_next,
                          int64_t T, int32_t n, int32_t d, hc_dtype dt, void* stream);

/* The whole layer boundary with per-token weights in one pass: the
 * write-back of one layer, the next layer's per-token weights from its
 * result, and the next layer's read-mix + RMSNorm with those weights
 * ([GLOSS] definition: learned mixing before and after every block; [EXPL]
 * "What four streams cost per token": every layer boundary hands the n-fold
 * state across, and this moves it once: H and F in, H' and u out).
 * Equivalent to
 *   hc_post_mix_weights(H, F, w, w_stride, W, w_static, scale, eps,
 *                       sinkhorn_iters, H_out, w_out, saved, saved_bytes)
 *   hc_pre_mix(H_out, w_out, K, gamma_next, pre_eps, u_next)
 * with H_out bitwise hc_post_mix's and w_out as hc_post_mix_weights gives
 * it.  u_next uses the alpha stored in w_out and H_out as stored (rounded);
 * it agrees with that hc_pre_mix call to the rounding of the RMSNorm sum
 * (added in another order), i.e. to one unit in the last place of dt.
 *   arguments as hc_post_mix_weights, plus
 *   gamma_next    [d] fp32, 16-byte aligned: the next read-mix's RMSNorm gain
 *   pre_eps       its RMSNorm epsilon (> 0, finite)
 *   u_next        [T][d] in dt, 16-byte aligned, overlapping nothing
 * Errors as hc_post_mix_weights; gamma_next or u_next NULL (T > 0) is
 * HC_ERR_NULL; a bad pre_eps is HC_ERR_ARG. */
hc_status hc_post_weights_pre_mix(const void* H, const void* F, const float* w, int64_t w_stride,
                                  const void* W, const float* w_static, float scale, float eps,
                                  int32_t sinkhorn_iters, const float* gamma_next, float pre_eps,
                                  void* H_out, float* w_out, void* u_next, float* saved,
                                  int64_t saved_bytes, int64_t T, int32_t n, int32_t d,
                                  hc_dtype dt, void* stream);

/* Bytes of device workspace the backward calls need for T tokens of width d
 * with n streams (0 for T <= 0).  The caller owns it; it holds partial sums
 * (per workgroup, or per token and wave for per-token records) and every
 * call writes what it reads. */
int64_t hc_backward_workspace(int64_t T, int32_t n, int32_t d);

/* Gradients of hc_post_mix (the map is linear in H and F):
 *   dH_j = sum_i A[i][j] dH_out_i        dF = sum_i beta_i dH_out_i
 *   dA[i][j] = sum_k dH_out_ik H_jk      dbeta_i = sum_k dH_out_ik F_k
 * [GLOSS] definition: the mixing is learned, so its weights take gradients.
 *   dH_out, H [T][n][d] dt; F [T][d] dt; w records as in hc_post_mix
 *   dH [T][n][d] dt, dF [T][d] dt: outputs (no overlap with anything).
 *      dH may be NULL: the H gradient is then not written, and
 *      hc_pre_mix_backward, given the same dH_out and records, adds it to its
 *      own dH (one write of dH and one read of it saved per layer).
 *   dw fp32, the shape of the weights: one record [dalpha | dbeta | dA]
 *      (dalpha = 0: post does not read alpha) when w_stride == 0, summed over
 *      the tokens in a fixed order; else [T][K], one record per token.
 *   workspace: >= hc_backward_workspace(T, n, d) bytes, 16-byte aligned
 *      (used when w_stride == 0; may be NULL otherwise). */
hc_status hc_post_mix_backward(const void* dH_out, const void* H, const void* F, const float* w,
                               int64_t w_stride, void* dH, void* dF, float* dw,
                               void* workspace, int64_t workspace_bytes, int64_t T,
                               int32_t n, int32_t d, hc_dtype dt, void* stream);

/* hc_post_mix_backward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same gradients, bitwise, with no workspace argument.  A
 * shared record's partial sums go to the library's own scratch array, one
 * per GPU, 1 MiB, held until the process ends (at n <= 4 every T fits; a
 * larger need is HC_ERR_ARG).  Calls on one GPU share that array, and each
 * call overwrites what the last left there: calls that overlap on one GPU
 * (concurrent streams, several host threads) race and must be serialised by
 * the caller.  Per-token records use no scratch.  Arguments, layouts and
 * errors otherwise as hc_post_mix_backward. */
hc_status hc_post_mix_backward_noalloc(const void* dH_out, const void* H, const void* F,
                                       const float* w, int64_t w_stride, void* dH, void* dF,
                                       float* dw, int64_t T, int32_t n, int32_t d, hc_dtype dt,
                                       void* stream);


/* Gradients of hc_pre_mix (RMSNorm and read-mix written out):
 *   dy = gamma * du, dx = r * (dy - x * r^2 * mean_k(dy_k x_k)),
 *   dH_i = alpha_i dx (+ dH_in_i, or + sum_j A[j][i] dH_out_j),
 *   dalpha_i = sum_k dx_k H_ik,
 *   dgamma_k = sum_t du_tk x_tk r_t,
 * with x and r = 1/sqrt(mean x^2 + eps) recomputed from H.
 *   du [T][d] dt; H [T][n][d] dt; w, gamma, eps as in hc_pre_mix
 *   dH_in [T][n][d] dt or NULL: added to dH (a layer's H feeds both pre and
 *     post, so this is where the two gradients meet); dH_in == dH allowed
 *   dH_out [T][n][d] dt or NULL: the gradient at hc_post_mix's output, when
 *     hc_post_mix_backward was called with dH = NULL; the write-back's H
 *     gradient sum_j A[j][i] dH_out_j (A from the same records w) is then
 *     formed here and added to dH before its one rounding.  At most one of
 *     dH_in and dH_out (both: HC_ERR_ARG).
 *   dH [T][n][d] dt, or NULL: then only dw and dgamma are computed (bitwise
 *     the same as with dH), and dH_in and dH_out must be NULL (HC_ERR_ARG):
 *     for weights produced from H, whose gradient needs dalpha before the
 *     layer's dH is formed.  With dH NULL, dgamma may be NULL too (dalpha
 *     alone: hc_post_pre_mix_backward forms dgamma at the same boundary);
 *     dgamma NULL with dH given is HC_ERR_NULL
 *   dw fp32, the shape of the weights: [dalpha | 0 | 0] summed over tokens
 *     when w_stride == 0, else [T][K] per token
 *   dgamma [d] fp32, summed over tokens in a fixed order (deterministic)
 *   workspace: >= hc_backward_workspace(T, n, d) bytes, 16-byte aligned.
 * Outputs may not overlap inputs, each other or the workspace (except
 * dH == dH_in); a short workspace is HC_ERR_ARG. */
hc_status hc_pre_mix_backward(const void* du, const void* H, const float* w, int64_t w_stride,
                              const float* gamma, float eps, const void* dH_in, const void* dH_out,
                              void* dH, float* dw, float* dgamma, void* workspace,
                              int64_t workspace_bytes, int64_t T, int32_t n, int32_t d, hc_dtype dt,
                              void* stream);

/* Gradients of hc_post_pre_mix (the write-back of one layer and the read-mix
 * + RMSNorm of the next) in one pass over the streams: the backward of one
 * layer boundary.  [GLOSS] definition (the mixing before and after every
 * block is learned, so its weights take gradients); [EXPL] "What four
 * streams cost per token" (the n-fold state crosses every boundary, and here
 * it crosses once: H, F, dH_out and du_next in, dH and dF out).
 * With H' = hc_post_mix(H, F, w) recomputed bitwise as the forward stored it
 * (H' is not an argument) and x, r, dx the read-mix's (hc_pre_mix_backward,
 * with alpha from w_next and gamma_next):
 *   G_i = dH_out_i + alpha_i dx      the whole gradient at H' (fp32, not stored)
 *   dH_j = sum_i A[i][j] G_i         dF = sum_i beta_i G_i
 *   dw      = [0 | dbeta | dA],      dbeta_i = G_i . F,  dA[i][j] = G_i . H_j
 *   dw_next = [dalpha | 0 | 0],      dalpha_i = dx . H'_i
 *   dgamma_next = sum_t du_next x r
 * i.e. hc_post_mix_backward(G, H, F, w) and hc_pre_mix_backward(du_next, H',
 * w_next) with G formed in registers.  dH_out is the gradient at H' from
 * everything after the call except the read-mix: in a stack of layers, the
 * dH that the next boundary's call (or the last write-back's
 * hc_post_mix_backward) returned.
 *   dH_out [T][n][d] dt; du_next [T][d] dt; H [T][n][d] dt; F [T][d] dt
 *   w, w_stride, w_next, w_next_stride as in hc_post_pre_mix, both shared
 *     (stride 0) or both per token (stride K); unequal strides: HC_ERR_ARG
 *   gamma_next [d] fp32, eps > 0: the read-mix's RMSNorm
 *   dH [T][n][d] dt (dH == dH_out allowed), dF [T][d] dt
 *   dw, dw_next fp32 in the shape of w and w_next, dgamma_next [d] fp32,
 *     summed over tokens in a fixed order (deterministic)
 *   workspace >= hc_backward_workspace(T, n, d) bytes, 16-byte aligned.
 * Alignment as the other gradient calls; any other overlap of an output with
 * an input, another output or the workspace is HC_ERR_ALIAS; fp32 and bf16
 * only (HC_ERR_DTYPE for HC_FP8). */
hc_status hc_post_pre_mix_backward(const void* dH_out, const void* du_next, const void* H,
                                   const void* F, const float* w, int64_t w_stride,
                                   const float* w_next, int64_t w_next_stride,
                                   const float* gamma_next, float eps, void* dH, void* dF, float* dw,
                                   float* dw_next, float* dgamma_next, void* workspace,
                                   int64_t workspace_bytes, int64_t T, int32_t n, int32_t d,
                                   hc_dtype dt, void* stream);

/* hc_post_pre_mix_backward at a boundary whose next layer's records are
 * produced from H' by the weight producer (hc_post_mix_weights,
 * hc_post_weights_pre_mix; [GLOSS] definition: the weight producers are
 * learned, so their gradient reaches the streams they read).  The producer's
 * share of the gradient at H' is added inside the pass instead of arriving in
 * dH_out:
 *   G_i = dH_out_i + alpha_i dx + a_i dhbar + b_i H'_i
 * with dhbar and (a_i | b_i) from hc_weights_backward_terms for the records
 * w_next and H' (H' recomputed here bitwise as the forward stored it).  Per
 * token this reads one fp32 row (dhbar) where the producer's own dH pass
 * would read and write n rows of dH.
 *   dhbar [T][d] fp32, 16-byte aligned; coef [T][2n] fp32 = (a_1..a_n |
 *     b_1..b_n) per token: inputs, which no output may overlap
 *   w and w_next per token (stride K): shared records are HC_ERR_ARG
 *   every other argument, output and error as hc_post_pre_mix_backward;
 *   dhbar or coef NULL is HC_ERR_NULL. */
hc_status hc_post_pre_mix_backward_terms(const void* dH_out, const void* du_next, const void* H,
                                         const void* F, const float* w, int64_t w_stride,
                                         const float* w_next, int64_t w_next_stride,
                                         const float* gamma_next, float eps, const float* dhbar,
                                         const float* coef, void* dH, void* dF, float* dw,
                                         float* dw_next, float* dgamma_next, void* workspace,
                                         int64_t workspace_bytes, int64_t T, int32_t n, int32_t d,
                                         hc_dtype dt, void* stream);

/* Bytes of device workspace hc_weights_backward needs (0 for T <= 0 or
 * arguments out of range).  It holds the per-stream projections, per-token
 * coefficients, Sinkhorn intermediates (16 floats per token per iteration)
 * and partial sums; every call rewrites it. */
int64_t hc_weights_backward_workspace(int64_t T, int32_t n, int32_t d, int32_t sinkhorn_iters);

/* Gradients of hc_weights ([GLOSS] definition: the weight producers are
 * learned too).  With z = W hbar as in hc_weights and dw = dL/dw_out:
 *   sinkhorn_iters == 0:  dz = scale (1 - tanh(z)^2) dw,   dw_static = sum_t dw
 *   sinkhorn_iters  > 0:  dl = the mHC backward of dw at l = w_static + scale z,
 *                         dz = scale dl,                    dw_static = sum_t dl
 *   dW = sum_t dz hbar^T   (fp32, [K][d], summed in a fixed order)
 *   dH_i = dH_in_i + (r_i dhbar - r_i^3 (H_i . dhbar) H_i / d) / n,  dhbar = W^T dz
 *   H [T][n][d] dt, W [K][d] dt, w_static [K], scale, eps, sinkhorn_iters as in
 *     hc_weights; dw [T][K] fp32 (records of stride K); dw2 [T][K] fp32 or NULL,
 *     added to dw (the records feed both pre and post, whose backward calls
 *     each return a per-token gradient record)
 *   saved: the state hc_weights_save kept for these H, W and eps, or NULL
 *     (then the projections and norms are recomputed from H: one more read
 *     of H); 16-byte aligned, an input
 *   dH_in [T][n][d] dt or NULL; dH [T][n][d] dt (dH == dH_in allowed)
 *   dW [K][d] fp32, dw_static [K] fp32 outputs
 *   workspace >= hc_weights_backward_workspace(T, n, d, sinkhorn_iters), 16-byte
 *     aligned.  fp32 and bf16 storage only (HC_ERR_DTYPE for HC_FP8). */
hc_status hc_weights_backward(const void* H, const void* W, const float* w_static, float scale,
                              float eps, int32_t sinkhorn_iters, const float* dw, const float* dw2,
                              const float* saved, const void* dH_in,
                              void* dH, float* dW, float* dw_static, void* workspace,
                              int64_t workspace_bytes, int64_t T, int32_t n, int32_t d, hc_dtype dt,
                              void* stream);

/* hc_weights_backward without dH: the gradient reaching H is returned as
 * its two factors, for a later pass that holds H_i to form
 *   dH_i = a_i dhbar + b_i H_i
 * itself (hc_post_pre_mix_backward_terms) instead of this call reading and
 * writing n rows of dH per token ([GLOSS] definition, as hc_weights_backward;
 * [EXPL] "What four streams cost per token": the n-fold state is what each
 * pass moves).
 *   dhbar [T][d] fp32 out = W^T dz per token, 16-byte aligned
 *   coef [T][2n] fp32 out = (a_1..a_n | b_1..b_n), a_i = r_i / n,
 *     b_i = -r_i^3 (H_i . dhbar) / (n d)
 *   dW, dw_static and every input, the workspace and the errors as
 *     hc_weights_backward (dhbar, coef take dH's place: NULL is HC_ERR_NULL,
 *     overlap with anything is HC_ERR_ALIAS).  fp32 and bf16 storage only. */
hc_status hc_weights_backward_terms(const void* H, const void* W, const float* w_static,
                                    float scale, float eps, int32_t sinkhorn_iters, const float* dw,
                                    const float* dw2, const float* saved, float* dhbar, float* coef,
                                    float* dW, float* dw_static, void* workspace,
                                    int64_t workspace_bytes, int64_t T, int32_t n, int32_t d,
                                    hc_dtype dt, void* stream);

/* Bytes of device workspace hc_sinkhorn_backward needs: 64 per token per
 * iteration (0 for iters == 0). */
int64_t hc_sinkhorn_backward_workspace(int64_t T, int32_t iters);

/* Gradient of hc_sinkhorn: dlogits [T][K] from dw = dL/dw [T][K] (both fp32,
 * stride K), plus dw2 [T][K] when not NULL (a layer's records feed its
 * read-mix and its write-back, whose gradients arrive from two calls: e.g.
 * the dw_next of one hc_post_pre_mix_backward and the dw of the next).  Each
 * token's forward is re-run keeping the matrix entering every iteration in
 * the workspace; the row and column steps are undone in reverse, then exp and
 * the sigmoids.  dlogits may not overlap the inputs or the workspace. */
hc_status hc_sinkhorn_backward(const float* logits, const float* dw, const float* dw2,
                               float* dlogits, int32_t iters, void* workspace,
                               int64_t workspace_bytes, int64_t T, int32_t n, void* stream);

/* out[c] = sum over t of rec[t * K + c], c < K, summed in a fixed order:
 * turns per-token gradient records into the gradient of one shared record.
 *   rec [T][K] fp32, out [K] fp32 (no overlap), 1 <= K <= 1024.
 * At T == 0 the sum is empty: zeros are written to `out` if it is not NULL,
 * and `rec` is not read (it may be NULL). */
hc_status hc_sum_records(const float* rec, int64_t T, int32_t K, float* out, void* stream);

/* Stand-in block used by the benchmarks and tests, not part of the method:
 * F = tanh(u) elementwise ([EXPL] "Jargon", Residual connection: the block
 * computes f(x)).  count % 16 == 0 (fp8), count % 8 == 0 (bf16) or
 * count % 4 == 0 (fp32). */
hc_status hc_block_tanh(const void* u, void* F, int64_t count, hc_dtype dt, void* stream);

/* Static string naming a status code; never NULL. */
const char* hc_status_str(hc_status s);

/* Version of this ABI (incremented on any signature change). */
int32_t hc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HC_H */
