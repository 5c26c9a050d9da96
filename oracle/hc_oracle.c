/*
 * hc_oracle.c -- plain CPU oracle for the identity Hyper-Connections residual
 * path (read-mix + RMSNorm before the block, stream-mix + write-back after it,
 * per-token weights, Sinkhorn).
 *
 * TEST INFRASTRUCTURE ONLY. This file is compiled with gcc into
 * oracle/liboracle.so and is loaded only by the test suite, the smoke check and
 * the benchmark's CPU-baseline leg. The GPU library shares no code, header,
 * table or helper with it, and neither side includes or links the other.
 *
 * Style: every value is computed in IEEE double precision with scalar loops,
 * one token at a time, in the order the definitions below are written.  Inputs
 * arrive in their storage type (fp32, bf16 bit patterns held in uint16_t, or
 * FP8 E4M3 codes held in uint8_t) and are widened exactly; outputs are written unrounded as doubles.  A
 * separate routine rounds doubles to a storage type (round to nearest, ties to
 * even, subnormals kept) so that callers can model what a bf16/fp32 store
 * does.  The only parallelism is an OpenMP loop over tokens, which are
 * independent of one another; it does not change any arithmetic.
 *
 * Sources (web pages; cited by title and section):
 *   [EXPL]  learnaivisually.com, "Tencent open-sources Hy4 Preview at 770B --
 *           Identity Hyper-Connections -- What does it mean?"
 *   [GLOSS] hfviewer.com glossary entry "Hyper-connections (mHC)"
 *   [BLOG]  mindstudio.ai, "Hunyuan HY4: How Identity Hyper Connections and
 *           Gated DSA Work"
 *   [ATLAS] llm-atlas model card "Tencent Hy4-preview (770B-A49B)"
 *
 * What the pages fix: n parallel residual streams that a block reads from and
 * writes to separately ([EXPL] "Jargon", Hyper-Connections); learned matrices
 * mix the streams before and after the block ([GLOSS] definition); the mHC
 * variant makes the mixing doubly stochastic with a few Sinkhorn iterations
 * ([GLOSS] definition, [ATLAS] "Architecture concepts"); pre-norm normalises the
 * block's input ([EXPL] "Jargon", Pre-norm); RMSNorm is the related block
 * ([GLOSS] "Related concepts").  The explainer states that no mixing rule was
 * published ([EXPL], the "warning label" paragraph), so the concrete formulas
 * below are the plainest readings consistent with those statements:
 *
 *   weight record per token, K = 2n + n^2 doubles:
 *       [ alpha_0 .. alpha_{n-1} | beta_0 .. beta_{n-1} | A row-major ]
 *       A[i][j] (at 2n + i*n + j) weighs input stream j into output stream i.
 *   pre   x = sum_i alpha_i H_i ;  u_k = gamma_k x_k / sqrt(mean_k x_k^2 + eps)
 *   post  H'_i = sum_j A[i][j] H_j + beta_i F
 *   dyn   r_i = 1/sqrt(mean_k H_ik^2 + eps) ; hbar = (1/n) sum_i r_i H_i ;
 *         z_c = sum_k hbar_k W[c][k] ;  w = w_static + scale * tanh(z)
 *   mHC   alpha = sigmoid(l_alpha), beta = sigmoid(l_beta),
 *         A = Sinkhorn_iters(exp(l_A)), one iteration = normalise every row to
 *         sum 1, then every column to sum 1.
 *   gradients (the same formulas differentiated by the chain rule; the
 *         learned weights take gradients, [GLOSS] definition): of post, of
 *         pre (RMSNorm and read-mix), of the per-token weights (projection,
 *         per-stream RMSNorm, tanh or the mHC transform) and of the mHC
 *         transform alone.
 *
 * What pins each function (tests/test_oracle_*.py; none compares the oracle
 * with itself): identity weights on copies give x + f(x) and n = 1 reduces to
 * the plain residual (bitwise); torch's rms_norm and autograd in float64;
 * exact-rational and 60-digit brute force on tiny inputs; closed forms
 * (one-hot, constant, scaled copies, rank-1 Sinkhorn logits, the n = 2
 * Sinkhorn limit, W = 0); invariants (conservation under column-stochastic A,
 * Sinkhorn cross-ratios, scale invariance of RMSNorm); central finite
 * differences of the forward for every gradient; and planted mistakes in
 * copies of this file that the pins must catch.  The per-token weight rule,
 * its tanh combination and the sigmoid alpha/beta of mHC are readings the
 * pages do not state: the pins fix this file's arithmetic for those readings,
 * not the readings themselves.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage types of the inputs.  ORC_F64 holds values that were never
 * rounded to a storage format: it lets a caller run the pure fp64 chain (no
 * store rounding anywhere) that the per-layer drift is reported against. */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2, ORC_F64 = 3 };

/* FP8 E4M3 ("fn", the OCP 8-bit float): sign, 4 exponent bits with bias 7, 3
 * mantissa bits; no infinities; S.1111.111 is NaN; the largest finite value
 * is 448 and the smallest subnormal 2^-9.  Value of one code. */
static double orc_fp8_value(uint8_t b)
{
    const int e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);        /* subnormal: m * 2^-9 */
    else v = ldexp((double)(8 + m), e - 10);          /* (1 + m/8) * 2^(e-7) */
    return (b & 0x80) ? -v : v;
}

/* ---------------------------------------------------------------- storage */

/* Widen one stored element to double.  bf16 is the upper half of an fp32 bit
 * pattern, so the widening is exact. */
static double orc_load(const void* p, int64_t idx, int dt)
{
    if (dt == ORC_F32) return (double)((const float*)p)[idx];
    if (dt == ORC_F64) return ((const double*)p)[idx];
    if (dt == ORC_FP8) return orc_fp8_value(((const uint8_t*)p)[idx]);
    uint32_t bits = (uint32_t)((const uint16_t*)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, keeping subnormals.
 * bf16 carries 8 significant bits and the fp32 exponent range: normal values
 * are m * 2^(e-8) with integer 128 <= m < 256 and e-1 >= -126; below that the
 * spacing is fixed at 2^-133.  Returns the 16-bit pattern. */
uint16_t orc_round_bf16(double v)
{
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    double r;
    if (isinf(a)) {
        r = INFINITY;
    } else if (a == 0.0) {
        r = 0.0;
    } else {
        int e;
        (void)frexp(a, &e);                     /* a = f * 2^e, 0.5 <= f < 1 */
        int q = (e - 1 >= -126) ? e - 8 : -133; /* spacing exponent          */
        double m = rint(ldexp(a, -q));          /* default mode: ties-to-even */
        r = ldexp(m, q);
        /* largest finite bf16 is (2 - 2^-7) * 2^127; anything that rounds
         * past it is infinite */
        if (r > ldexp(255.0, 120)) r = INFINITY;
    }
    float f = (float)r;                         /* exact: r is a bf16 value */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    uint16_t out = (uint16_t)(bits >> 16);
    if (neg) out |= 0x8000u;
    return out;
}

/* Round a double to FP8 E4M3, nearest with ties to even, saturating: magnitudes
 * beyond the largest finite value (448, infinities included) store as +-448;
 * NaN stores as NaN.  4 significant bits for normal values (e-1 >= -6),
 * spacing 2^-9 below.  Returns the code. */
uint8_t orc_round_fp8(double v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs(v);
    if (a > 448.0) a = 448.0;
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);                          /* a = f * 2^e, 0.5 <= f < 1 */
    const int q = (e - 1 >= -6) ? e - 4 : -9;    /* spacing exponent */
    const double r = ldexp(rint(ldexp(a, -q)), q);
    if (r == 0.0) return sign;
    int er;
    (void)frexp(r, &er);
    uint8_t code;
    if (er - 1 >= -6) {                          /* normal: r = (8 + m) 2^(E-10) */
        const int E = er - 1 + 7;
        const int m = (int)ldexp(r, -(E - 10)) - 8;
        code = (uint8_t)((E << 3) | m);
    } else {                                     /* subnormal: r = m 2^-9 */
        code = (uint8_t)(int)ldexp(r, 9);
    }
    return (uint8_t)(sign | code);
}

void orc_round_fp8_array(const double* in, uint8_t* out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = orc_round_fp8(in[i]);
}

void orc_round_bf16_array(const double* in, uint16_t* out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = orc_round_bf16(in[i]);
}

/* IEEE double -> float conversion rounds to nearest, ties to even. */
void orc_round_f32_array(const double* in, float* out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = (float)in[i];
}

void orc_widen_array(const void* in, int dt, double* out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = orc_load(in, i, dt);
}

/* ---------------------------------------------------------------- threads */

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* --------------------------------------------------------------- the path */

/* Pre: read-mix, then RMSNorm of the block input.
 * [GLOSS] definition: learned mixing of the streams before the block runs.
 * [EXPL] "Jargon", Pre-norm: the block's input is what gets normalised; the
 * normalisation is RMSNorm ([GLOSS] "Related concepts"): divide by the root of
 * the mean square over the hidden width, plus eps inside the root, then scale
 * by the per-channel gain gamma.
 *   H      [T][n][d] storage dt
 *   w      weight records, token t at w + t*w_stride (w_stride 0 = shared)
 *   gamma  [d]
 *   u      [T][d] output, unrounded                                         */
void orc_pre_mix(const void* H, int dt, const double* w, int64_t w_stride,
                 const double* gamma, double eps, double* u,
                 int64_t T, int n, int d)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* alpha = w + t * w_stride;
        const int64_t row0 = t * (int64_t)n * d;
        double* ut = u + t * (int64_t)d;
        /* x_k = sum over streams i (ascending) of alpha_i * H_ik.  The sum
         * starts from the first product so that signed zeros are kept. */
        for (int k = 0; k < d; ++k) {
            double x = alpha[0] * orc_load(H, row0 + k, dt);
            for (int i = 1; i < n; ++i)
                x += alpha[i] * orc_load(H, row0 + (int64_t)i * d + k, dt);
            ut[k] = x;
        }
        double ss = 0.0;
        for (int k = 0; k < d; ++k) ss += ut[k] * ut[k];
        double ms = ss / d;
        double denom = sqrt(ms + eps);
        for (int k = 0; k < d; ++k) ut[k] = gamma[k] * ut[k] / denom;
    }
}

/* Post: stream-mix and write-back.
 * [GLOSS] definition: learned mixing of the streams after the block runs;
 * [EXPL] "Jargon", Hyper-Connections: the block writes into the streams
 * separately; "Jargon", Residual connection: the block output is added to what
 * came in.  H'_i = sum_j A[i][j] H_j + beta_i F.
 *   H [T][n][d], F [T][d] storage dt;  Hout [T][n][d] output, unrounded     */
void orc_post_mix(const void* H, const void* F, int dt, const double* w,
                  int64_t w_stride, double* Hout, int64_t T, int n, int d)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* rec = w + t * w_stride;
        const double* beta = rec + n;
        const double* A = rec + 2 * n;
        const int64_t row0 = t * (int64_t)n * d;
        for (int i = 0; i < n; ++i) {
            for (int k = 0; k < d; ++k) {
                double y = A[i * n + 0] * orc_load(H, row0 + k, dt);
                for (int j = 1; j < n; ++j)
                    y += A[i * n + j] * orc_load(H, row0 + (int64_t)j * d + k, dt);
                y += beta[i] * orc_load(F, t * (int64_t)d + k, dt);
                Hout[row0 + (int64_t)i * d + k] = y;
            }
        }
    }
}

/* Logistic sigmoid, 1 / (1 + e^-x). */
static double orc_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* The mHC transform of one logit record l (K = 2n + n^2) into a weight record.
 * [GLOSS] definition: the mixing is constrained to be doubly stochastic with a
 * few Sinkhorn iterations.  M = exp(l_A); each iteration divides every row by
 * its sum and then every column by its sum (Sinkhorn-Knopp).  The read and
 * write weights are squashed to (0, 1) with the logistic function. */
static void orc_mhc_record(const double* l, double* out, int n, int iters)
{
    for (int i = 0; i < n; ++i) out[i] = orc_sigmoid(l[i]);
    for (int i = 0; i < n; ++i) out[n + i] = orc_sigmoid(l[n + i]);
    double* M = out + 2 * n;
    for (int e = 0; e < n * n; ++e) M[e] = exp(l[2 * n + e]);
    for (int it = 0; it < iters; ++it) {
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int j = 0; j < n; ++j) s += M[i * n + j];
            for (int j = 0; j < n; ++j) M[i * n + j] /= s;
        }
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int i = 0; i < n; ++i) s += M[i * n + j];
            for (int i = 0; i < n; ++i) M[i * n + j] /= s;
        }
    }
}

/* Sinkhorn step on given per-token logits: logits [T][K] -> w [T][K]. */
void orc_sinkhorn(const double* logits, double* w, int iters, int64_t T, int n)
{
    const int K = 2 * n + n * n;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        orc_mhc_record(logits + t * K, w + t * K, n, iters);
}

/* Per-token (dynamic) weights from the streams themselves.
 * The pages give no formula for per-token weights (the explainer: no mixing
 * rule published).  Reading taken: normalise every stream with a gain-free
 * RMSNorm, average the n normalised streams, project the d-vector with W
 * (K rows of d), then either
 *   iters == 0:  w = w_static + scale * tanh(z)
 *   iters  > 0:  l = w_static + scale * z, then the mHC transform above.
 *   H [T][n][d] and W [K][d] in storage dt; w_static [K]; w [T][K] output.  */
void orc_weights(const void* H, const void* W, int dt, const double* w_static,
                 double scale, double eps, int iters, double* w,
                 int64_t T, int n, int d)
{
    const int K = 2 * n + n * n;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const int64_t row0 = t * (int64_t)n * d;
        double r[4];
        for (int i = 0; i < n; ++i) {
            double ss = 0.0;
            for (int k = 0; k < d; ++k) {
                double h = orc_load(H, row0 + (int64_t)i * d + k, dt);
                ss += h * h;
            }
            r[i] = 1.0 / sqrt(ss / d + eps);
        }
        double* hbar = (double*)malloc((size_t)d * sizeof(double));
        for (int k = 0; k < d; ++k) {
            double s = 0.0;
            for (int i = 0; i < n; ++i)
                s += r[i] * orc_load(H, row0 + (int64_t)i * d + k, dt);
            hbar[k] = s / n;
        }
        double z[24];
        for (int c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k)
                acc += hbar[k] * orc_load(W, (int64_t)c * d + k, dt);
            z[c] = acc;
        }
        free(hbar);
        double* out = w + t * K;
        if (iters == 0) {
            for (int c = 0; c < K; ++c) out[c] = w_static[c] + scale * tanh(z[c]);
        } else {
            double l[24];
            for (int c = 0; c < K; ++c) l[c] = w_static[c] + scale * z[c];
            orc_mhc_record(l, out, n, iters);
        }
    }
}

/* Stand-in block used by the single-layer and deep-chain workloads: F = tanh(u)
 * elementwise ([EXPL] "Jargon", Residual connection: the block computes f(x)
 * and its output is added back).  u storage dt, F unrounded. */
void orc_block_tanh(const void* u, int dt, double* F, int64_t count)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e) F[e] = tanh(orc_load(u, e, dt));
}

/* ------------------------------------------------------------ backward */

/* Gradients of the post step H'_i = sum_j A[i][j] H_j + beta_i F, given dHo =
 * dL/dH' (chain rule on a linear map):
 *   dH_j = sum_i A[i][j] dHo_i        dF = sum_i beta_i dHo_i
 *   dA[i][j] = sum_k dHo_ik H_jk      dbeta_i = sum_k dHo_ik F_k
 * dw receives one gradient record per token in the weight-record layout
 * [dalpha | dbeta | dA]; dalpha is 0 (post does not read alpha).
 *   dHo, H [T][n][d], F [T][d] storage dt; dH [T][n][d], dF [T][d], dw [T][K]. */
void orc_post_mix_backward(const void* dHo, const void* H, const void* F, int dt,
                           const double* w, int64_t w_stride, double* dH, double* dF,
                           double* dw, int64_t T, int n, int d)
{
    const int K = 2 * n + n * n;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* rec = w + t * w_stride;
        const double* beta = rec + n;
        const double* A = rec + 2 * n;
        const int64_t row0 = t * (int64_t)n * d;
        double* g = dw + t * K;
        for (int c = 0; c < K; ++c) g[c] = 0.0;
        for (int k = 0; k < d; ++k) {
            const double f = orc_load(F, t * (int64_t)d + k, dt);
            double df = 0.0;
            for (int i = 0; i < n; ++i) {
                const double go = orc_load(dHo, row0 + (int64_t)i * d + k, dt);
                df += beta[i] * go;
                g[n + i] += go * f;
                for (int j = 0; j < n; ++j)
                    g[2 * n + i * n + j] += go * orc_load(H, row0 + (int64_t)j * d + k, dt);
            }
            dF[t * (int64_t)d + k] = df;
            for (int j = 0; j < n; ++j) {
                double s = 0.0;
                for (int i = 0; i < n; ++i)
                    s += A[i * n + j] * orc_load(dHo, row0 + (int64_t)i * d + k, dt);
                dH[row0 + (int64_t)j * d + k] = s;
            }
        }
    }
}

/* Gradients of the pre step u = gamma * x * r, r = 1/sqrt(mean_k x_k^2 + eps),
 * x = sum_i alpha_i H_i, given du = dL/du:
 *   dy = gamma * du;  dx = r * (dy - x * r^2 * (sum_k dy_k x_k) / d)
 *   dH_i = alpha_i dx;  dalpha_i = sum_k dx_k H_ik;  dgamma_k = sum_t du_k x_k r
 * (the derivative of the root-mean-square normalisation written out).
 * dH_in (may be NULL) is added to dH: a layer's H feeds both pre and post.
 *   du [T][d], H [T][n][d] storage dt; dH [T][n][d], dw [T][K] (only dalpha
 *   nonzero), dgamma [d] (summed over tokens). */
void orc_pre_mix_backward(const void* du, const void* H, int dt, const double* w,
                          int64_t w_stride, const double* gamma, double eps,
                          const double* dH_in, double* dH, double* dw, double* dgamma,
                          int64_t T, int n, int d)
{
    const int K = 2 * n + n * n;
    for (int k = 0; k < d; ++k) dgamma[k] = 0.0;
    for (int64_t t = 0; t < T; ++t) {   /* serial: dgamma sums over tokens in order */
        const double* alpha = w + t * w_stride;
        const int64_t row0 = t * (int64_t)n * d;
        double* x = (double*)malloc((size_t)d * sizeof(double));
        double* dx = (double*)malloc((size_t)d * sizeof(double));
        double ss = 0.0, sdx = 0.0;
        for (int k = 0; k < d; ++k) {
            double v = alpha[0] * orc_load(H, row0 + k, dt);
            for (int i = 1; i < n; ++i) v += alpha[i] * orc_load(H, row0 + (int64_t)i * d + k, dt);
            x[k] = v;
            ss += v * v;
        }
        const double r = 1.0 / sqrt(ss / d + eps);
        for (int k = 0; k < d; ++k) {
            const double g = orc_load(du, t * (int64_t)d + k, dt);
            sdx += gamma[k] * g * x[k];
            dgamma[k] += g * x[k] * r;
        }
        for (int k = 0; k < d; ++k) {
            const double dy = gamma[k] * orc_load(du, t * (int64_t)d + k, dt);
            dx[k] = r * (dy - x[k] * r * r * sdx / d);
        }
        double* g = dw + t * K;
        for (int c = 0; c < K; ++c) g[c] = 0.0;
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int k = 0; k < d; ++k) {
                const int64_t e = row0 + (int64_t)i * d + k;
                s += dx[k] * orc_load(H, e, dt);
                dH[e] = alpha[i] * dx[k] + (dH_in ? dH_in[e] : 0.0);
            }
            g[i] = s;
        }
        free(x);
        free(dx);
    }
}

/* ---------------------------------------------------------------------
 * Gradients of the per-token weights (the chain rule through the mHC
 * transform, tanh, the projection and the gain-free per-stream RMSNorm of
 * orc_weights above).  The glossary's definition: the mixing is learned, so
 * its producers take gradients too.
 * ------------------------------------------------------------------- */

/* Gradient of the mHC transform of one record, l [K] -> out [K], given
 * dout = dL/dout; writes dl = dL/dl.  The forward is re-run keeping every
 * intermediate matrix; each iteration is undone in reverse:
 *   column step C = R / colsum(R):  dR_ij = (dC_ij - sum_i' dC_i'j C_i'j) / colsum_j
 *   row step    R = M / rowsum(M):  dM_ij = (dR_ij - sum_j' dR_ij' R_ij') / rowsum_i
 * and exp, sigmoid by their derivatives. */
static void orc_mhc_record_backward(const double* l, const double* dout, double* dl, int n,
                                    int iters)
{
    for (int i = 0; i < 2 * n; ++i) {
        const double s = orc_sigmoid(l[i]);
        dl[i] = dout[i] * s * (1.0 - s);
    }
    const int nn = n * n;
    /* Ms[it] = matrix entering iteration it (Ms[0] = exp(l_A)), Rs[it] = after
     * its row step; rs, cs = the row and column sums used */
    double* Ms = (double*)malloc((size_t)(iters + 1) * nn * sizeof(double));
    double* Rs = (double*)malloc((size_t)(iters > 0 ? iters : 1) * nn * sizeof(double));
    double* rs = (double*)malloc((size_t)(iters > 0 ? iters : 1) * n * sizeof(double));
    double* cs = (double*)malloc((size_t)(iters > 0 ? iters : 1) * n * sizeof(double));
    for (int e = 0; e < nn; ++e) Ms[e] = exp(l[2 * n + e]);
    for (int it = 0; it < iters; ++it) {
        const double* M = Ms + (size_t)it * nn;
        double* R = Rs + (size_t)it * nn;
        double* C = Ms + (size_t)(it + 1) * nn;
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int j = 0; j < n; ++j) s += M[i * n + j];
            rs[it * n + i] = s;
            for (int j = 0; j < n; ++j) R[i * n + j] = M[i * n + j] / s;
        }
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int i = 0; i < n; ++i) s += R[i * n + j];
            cs[it * n + j] = s;
            for (int i = 0; i < n; ++i) C[i * n + j] = R[i * n + j] / s;
        }
    }
    double g[16], gr[16];
    for (int e = 0; e < nn; ++e) g[e] = dout[2 * n + e];
    for (int it = iters - 1; it >= 0; --it) {
        const double* R = Rs + (size_t)it * nn;
        const double* C = Ms + (size_t)(it + 1) * nn;
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int i = 0; i < n; ++i) s += g[i * n + j] * C[i * n + j];
            for (int i = 0; i < n; ++i) gr[i * n + j] = (g[i * n + j] - s) / cs[it * n + j];
        }
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int j = 0; j < n; ++j) s += gr[i * n + j] * R[i * n + j];
            for (int j = 0; j < n; ++j) g[i * n + j] = (gr[i * n + j] - s) / rs[it * n + i];
        }
    }
    for (int e = 0; e < nn; ++e) dl[2 * n + e] = g[e] * Ms[e];
    free(Ms);
    free(Rs);
    free(rs);
    free(cs);
}

/* dlogits [T][K] from dw [T][K] through the Sinkhorn step on logits [T][K]. */
void orc_sinkhorn_backward(const double* logits, const double* dw, double* dlogits, int iters,
                           int64_t T, int n)
{
    const int K = 2 * n + n * n;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        orc_mhc_record_backward(logits + t * K, dw + t * K, dlogits + t * K, n, iters);
}

/* Gradients of orc_weights given dw [T][K] = dL/dw:
 *   dz = scale * (1 - tanh(z)^2) * dw                      (iters == 0)
 *   dz = scale * dl,  dl = the mHC backward of dw at l    (iters  > 0)
 *   dW[c][k] = sum_t dz_c hbar_k,   dw_static = sum_t (dw or dl),
 *   dhbar = sum_c dz_c W[c],  s_i = H_i . dhbar,
 *   dH_i = (r_i dhbar - r_i^3 s_i H_i / d) / n.
 * dH [T][n][d], dW [K][d], dws [K] are written (not accumulated).  Tokens are
 * taken in order, so the sums over tokens are reproducible. */
void orc_weights_backward(const void* H, const void* W, int dt, const double* w_static,
                          double scale, double eps, int iters, const double* dw, double* dH,
                          double* dW, double* dws, int64_t T, int n, int d)
{
    const int K = 2 * n + n * n;
    for (int64_t e = 0; e < (int64_t)K * d; ++e) dW[e] = 0.0;
    for (int c = 0; c < K; ++c) dws[c] = 0.0;
    double* hbar = (double*)malloc((size_t)d * sizeof(double));
    double* dhbar = (double*)malloc((size_t)d * sizeof(double));
    for (int64_t t = 0; t < T; ++t) {
        const int64_t row0 = t * (int64_t)n * d;
        double r[4];
        for (int i = 0; i < n; ++i) {
            double ss = 0.0;
            for (int k = 0; k < d; ++k) {
                const double h = orc_load(H, row0 + (int64_t)i * d + k, dt);
                ss += h * h;
            }
            r[i] = 1.0 / sqrt(ss / d + eps);
        }
        for (int k = 0; k < d; ++k) {
            double s = 0.0;
            for (int i = 0; i < n; ++i) s += r[i] * orc_load(H, row0 + (int64_t)i * d + k, dt);
            hbar[k] = s / n;
        }
        double z[24], dz[24], dl[24];
        for (int c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += hbar[k] * orc_load(W, (int64_t)c * d + k, dt);
            z[c] = acc;
        }
        const double* g = dw + t * K;
        if (iters == 0) {
            for (int c = 0; c < K; ++c) {
                const double th = tanh(z[c]);
                dl[c] = g[c];
                dz[c] = g[c] * scale * (1.0 - th * th);
            }
        } else {
            double l[24];
            for (int c = 0; c < K; ++c) l[c] = w_static[c] + scale * z[c];
            orc_mhc_record_backward(l, g, dl, n, iters);
            for (int c = 0; c < K; ++c) dz[c] = scale * dl[c];
        }
        for (int c = 0; c < K; ++c) {
            dws[c] += dl[c];
            for (int k = 0; k < d; ++k) dW[(int64_t)c * d + k] += dz[c] * hbar[k];
        }
        for (int k = 0; k < d; ++k) {
            double s = 0.0;
            for (int c = 0; c < K; ++c) s += dz[c] * orc_load(W, (int64_t)c * d + k, dt);
            dhbar[k] = s;
        }
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int k = 0; k < d; ++k) s += orc_load(H, row0 + (int64_t)i * d + k, dt) * dhbar[k];
            for (int k = 0; k < d; ++k) {
                const int64_t e = row0 + (int64_t)i * d + k;
                dH[e] = (r[i] * dhbar[k] - r[i] * r[i] * r[i] * s * orc_load(H, e, dt) / d) / n;
            }
        }
    }
    free(hbar);
    free(dhbar);
}
