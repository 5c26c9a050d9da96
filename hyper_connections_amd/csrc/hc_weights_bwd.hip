// hc_weights_bwd.hip -- gradients of the per-token weight producer: the mHC
// (Sinkhorn) transform, tanh, the projection W and the gain-free per-stream
// RMSNorm that feeds it.
//
// Sources: hfviewer.com glossary "Hyper-connections (mHC)", definition (the
// mixing weights are learned and the mHC variant normalises them with a few
// Sinkhorn iterations), so every producer of the weights takes gradients.
// The forward being differentiated (the reading implemented by hc_weights):
//   r_i = 1/sqrt(mean_k H_ik^2 + eps), hbar = (1/n) sum_i r_i H_i,
//   z = W hbar, w = w_static + scale tanh(z)      or      w = mhc(w_static + scale z).
// Chain rule, per token:
//   dz = scale (1 - tanh(z)^2) dw                  or      dz = scale dl, dl = mhc'(dw)
//   dW += dz hbar^T,   dhbar = W^T dz,   s_i = H_i . dhbar = P_i . dz  (P_i = W H_i)
//   dH_i = a_i dhbar + b_i H_i,  a_i = r_i / n,  b_i = -r_i^3 s_i / (n d)
//   dw_static = sum over tokens of dw (tanh) or dl (mHC).
// Passes: (1) P_i and r_i per token: kept by the training forward
// (hc_weights_save), or the forward projection again (hc_weights.hip, raw
// mode); (2) one thread per token turns them and dw
// into dz, a_i, b_i and per-workgroup partial sums of dw_static; (3) one
// streaming pass over H computes dH and partial sums of dW on the matrix
// cores; (4) fixed-order sums of the partials.  Everything is deterministic.
#include <type_traits>

#include "hc_device.h"
#include "hc_launch.h"

namespace hc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int64_t kMaxGrid = 1 << 20;
constexpr int kSlot = 16;      // floats per token per iteration in the Sinkhorn scratch

// ------------------------------------------------------ mHC transform backward

// Gradient of the mHC record transform for one token, one thread:
// l [K] logits, g [K] = dL/dw in, dl [K] = dL/dl out.  The forward is re-run
// (with the largest A logit subtracted, as the forward kernels do; the row
// normalisation removes it exactly) and the matrix entering every iteration
// is kept in `scr` (iteration it at scr + it * stride, kSlot floats); the
// iterations are then undone in reverse:
//   column step C = R / colsum:  dR_ij = (dC_ij - sum_i' dC_i'j C_i'j) / colsum_j
//   row step    R = M / rowsum:  dM_ij = (dR_ij - sum_j' dR_ij' R_ij') / rowsum_i
// The derivatives of sigmoid and tanh, written without the cancellation of
// s (1 - s) and 1 - tanh^2 where the function saturates (there 1 - s and
// 1 - tanh^2 are tiny differences of numbers near 1; in fp32 they lose most
// of their digits past |x| ~ 5): with e = exp(-|x|),
//   sigmoid'(x) = e / (1 + e)^2,   tanh'(x) = 4 e^2 / (1 + e^2)^2.
__device__ __forceinline__ float dsigmoid(float x) {
    const float e = expf(-fabsf(x));
    const float q = 1.0f + e;
    return e / (q * q);
}
__device__ __forceinline__ float dtanh(float x) {
    const float e = expf(-2.0f * fabsf(x));
    const float q = 1.0f + e;
    return 4.0f * e / (q * q);
}

template <int N>
__device__ void mhc_record_bwd(const float* l, const float* g, float* dl, int iters, float* scr,
                               int64_t stride) {
    constexpr int NN = N * N;
    for (int i = 0; i < 2 * N; ++i) dl[i] = g[i] * dsigmoid(l[i]);
    float M[NN], M0[NN];
    float m = 0.0f;
    if (iters > 0) {
        m = l[2 * N];
#pragma unroll
        for (int e = 1; e < NN; ++e) m = fmaxf(m, l[2 * N + e]);
    }
#pragma unroll
    for (int e = 0; e < NN; ++e) M0[e] = M[e] = expf(l[2 * N + e] - m);
    for (int it = 0; it < iters; ++it) {
        float* dst = scr + it * stride;
#pragma unroll
        for (int e = 0; e < NN; ++e) dst[e] = M[e];
        // one correctly rounded reciprocal per sum, then products (a division
        // per entry cost about ten instructions each, the bulk of this loop)
#pragma unroll
        for (int i = 0; i < N; ++i) {
            float s = M[i * N];
#pragma unroll
            for (int j = 1; j < N; ++j) s += M[i * N + j];
            const float inv = 1.0f / s;
#pragma unroll
            for (int j = 0; j < N; ++j) M[i * N + j] *= inv;
        }
#pragma unroll
        for (int j = 0; j < N; ++j) {
            float s = M[j];
#pragma unroll
            for (int i = 1; i < N; ++i) s += M[i * N + j];
            const float inv = 1.0f / s;
#pragma unroll
            for (int i = 0; i < N; ++i) M[i * N + j] *= inv;
        }
    }
    float G[NN];
#pragma unroll
    for (int e = 0; e < NN; ++e) G[e] = g[2 * N + e];
    for (int it = iters - 1; it >= 0; --it) {
        const float* src = scr + it * stride;
        float R[NN], rs[N], cs[N];
#pragma unroll
        for (int e = 0; e < NN; ++e) R[e] = src[e];
        // the reciprocals of the row sums and column sums (rs, cs hold 1/sum)
#pragma unroll
        for (int i = 0; i < N; ++i) {
            float s = R[i * N];
#pragma unroll
            for (int j = 1; j < N; ++j) s += R[i * N + j];
            rs[i] = 1.0f / s;
#pragma unroll
            for (int j = 0; j < N; ++j) R[i * N + j] *= rs[i];
        }
#pragma unroll
        for (int j = 0; j < N; ++j) {
            float s = R[j];
#pragma unroll
            for (int i = 1; i < N; ++i) s += R[i * N + j];
            cs[j] = 1.0f / s;
        }
        // column step: C_ij = R_ij / cs_j
#pragma unroll
        for (int j = 0; j < N; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < N; ++i) s = fmaf(G[i * N + j], R[i * N + j] * cs[j], s);
#pragma unroll
            for (int i = 0; i < N; ++i) G[i * N + j] = (G[i * N + j] - s) * cs[j];
        }
        // row step: R_ij = M_ij / rs_i
#pragma unroll
        for (int i = 0; i < N; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < N; ++j) s = fmaf(G[i * N + j], R[i * N + j], s);
#pragma unroll
            for (int j = 0; j < N; ++j) G[i * N + j] = (G[i * N + j] - s) * rs[i];
        }
    }
#pragma unroll
    for (int e = 0; e < NN; ++e) dl[2 * N + e] = G[e] * M0[e];
}

// hc_sinkhorn_backward: the same gradient with four lanes per token.  Lane r
// of a quad holds row r of the 4 x 4 matrix (rows r >= N hold zeros and
// stay zero) and alpha_r, beta_r.  Row sums are the lane's own; column sums
// and the column step's dot products are added over the quad by two DPP
// exchanges (lanes l ^ 1, then l ^ 2), which every lane of the quad adds in
// an order that gives the same bits.  Four times the lanes of the
// one-thread form, so 32768 tokens fill 2048 waves instead of 512; the
// scratch layout is the same (row r of the matrix entering an iteration at
// floats 4r .. 4r + 3 of the token's slot).
__device__ __forceinline__ float quad_swap1(float x) {      // quad_perm [1, 0, 3, 2]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_swap2(float x) {      // quad_perm [2, 3, 0, 1]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_add(float x) {
    x += quad_swap1(x);
    return x + quad_swap2(x);
}
__device__ __forceinline__ float quad_max(float x) {
    x = fmaxf(x, quad_swap1(x));
    return fmaxf(x, quad_swap2(x));
}

// IMAX > 0: at most IMAX iterations, whose matrices stay in registers (a
// row of 4 floats per lane and iteration) instead of the scratch; the
// iteration loops are unrolled with their index known, and the scratch is
// not touched.  IMAX = 0: any count, through the scratch.
template <int N, int IMAX>
__global__ __launch_bounds__(256) void sinkhorn_bwd_quad_kernel(const float* __restrict__ logits,
                                                                const float* __restrict__ dw,
                                                                const float* __restrict__ dw2,
                                                                float* __restrict__ dlogits,
                                                                int iters, float* __restrict__ scr,
                                                                int64_t T) {
    constexpr int K = 2 * N + N * N;
    const int r = threadIdx.x & 3;
    const bool row = r < N;
    const int64_t step = ((int64_t)gridDim.x * blockDim.x) >> 2;
    // a quad's four lanes share t, so they run (and exchange) together
    for (int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 2; t < T; t += step) {
        const float* lt = logits + t * K;
        const float* gt = dw + t * K;
        const float* g2 = dw2 ? dw2 + t * K : nullptr;
        float* ot = dlogits + t * K;
        if (row) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = h * N + r;
                const float g = g2 ? gt[c] + g2[c] : gt[c];
                ot[c] = g * dsigmoid(lt[c]);
            }
        }
        float l[N], G[N], M[N], M0[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int c = 2 * N + r * N + j;
            l[j] = row ? lt[c] : -INFINITY;
            G[j] = row ? (g2 ? gt[c] + g2[c] : gt[c]) : 0.0f;
        }
        float m = 0.0f;
        if (iters > 0) {
            float mx = l[0];
#pragma unroll
            for (int j = 1; j < N; ++j) mx = fmaxf(mx, l[j]);
            m = quad_max(mx);
        }
#pragma unroll
        for (int j = 0; j < N; ++j) M0[j] = M[j] = row ? expf(l[j] - m) : 0.0f;
        const int64_t stride = T * kSlot;
        float* slot = scr + t * kSlot + 4 * r;
        float keep[IMAX > 0 ? IMAX : 1][N];
        auto forward = [&](int it) __attribute__((always_inline)) {
            if constexpr (IMAX > 0) {
#pragma unroll
                for (int j = 0; j < N; ++j) keep[IMAX > 0 ? it : 0][j] = M[j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) slot[it * stride + j] = j < N ? M[j] : 0.0f;
            }
            if (row) {
                float s = M[0];
#pragma unroll
                for (int j = 1; j < N; ++j) s += M[j];
                const float inv = 1.0f / s;
#pragma unroll
                for (int j = 0; j < N; ++j) M[j] *= inv;
            }
#pragma unroll
            for (int j = 0; j < N; ++j) M[j] *= 1.0f / quad_add(M[j]);
        };
        auto backward = [&](int it) __attribute__((always_inline)) {
            float R[N];
#pragma unroll
            for (int j = 0; j < N; ++j) R[j] = IMAX > 0 ? keep[IMAX > 0 ? it : 0][j] : slot[it * stride + j];
            float rs = 0.0f;
            if (row) {
                float s = R[0];
#pragma unroll
                for (int j = 1; j < N; ++j) s += R[j];
                rs = 1.0f / s;
#pragma unroll
                for (int j = 0; j < N; ++j) R[j] *= rs;
            }
            // column step: C_ij = R_ij / cs_j
#pragma unroll
            for (int j = 0; j < N; ++j) {
                const float ci = 1.0f / quad_add(R[j]);
                const float s = quad_add(G[j] * (R[j] * ci));
                G[j] = row ? (G[j] - s) * ci : 0.0f;
            }
            // row step: R_ij = M_ij / rs_i
            if (row) {
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < N; ++j) s = fmaf(G[j], R[j], s);
#pragma unroll
                for (int j = 0; j < N; ++j) G[j] = (G[j] - s) * rs;
            }
        };
        if constexpr (IMAX > 0) {
#pragma unroll
            for (int it = 0; it < IMAX; ++it)
                if (it < iters) forward(it);
#pragma unroll
            for (int it = IMAX - 1; it >= 0; --it)
                if (it < iters) backward(it);
        } else {
            for (int it = 0; it < iters; ++it) forward(it);
            for (int it = iters - 1; it >= 0; --it) backward(it);
        }
        if (row) {
#pragma unroll
            for (int j = 0; j < N; ++j) ot[2 * N + r * N + j] = G[j] * M0[j];
        }
    }
}

// ----------------------------------------------------- per-token coefficients

// From P [T][N][K], r [T][N] (the forward projection pass) and dw [T][K]
// (plus dw2 when given: the records' gradient from a second consumer):
// dz [T][K], ab [T][2][N] = (a_i, b_i), and per workgroup the sum over its
// tokens of dl (the gradient at the logits / records that w_static
// receives): dl_part [workgroup][K].  One thread per token, one wave per
// workgroup.
template <int N>
__global__ __launch_bounds__(256) void wgrad_coef_kernel(
    const float* __restrict__ P, const float* __restrict__ r, const float* __restrict__ dw,
    const float* __restrict__ dw2, const float* __restrict__ w_static, float scale, int iters,
    float* __restrict__ scr,
    float* __restrict__ dz, float* __restrict__ dl_part, float* __restrict__ ab, int64_t T, int d) {
    constexpr int K = 2 * N + N * N;
    float dls[K];
#pragma unroll
    for (int c = 0; c < K; ++c) dls[c] = 0.0f;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T;
         t += (int64_t)gridDim.x * blockDim.x) {
        const float* p = P + t * N * K;
        float ri[N];
#pragma unroll
        for (int i = 0; i < N; ++i) ri[i] = r[t * N + i];
        float z[K], g[K], gl[K], gz[K];
#pragma unroll
        for (int c = 0; c < K; ++c) {
            // z as the forward kernel forms it: sum_i r_i P_ic in stream order, / n
            float v = ri[0] * p[c];
#pragma unroll
            for (int i = 1; i < N; ++i) v = fmaf(ri[i], p[i * K + c], v);
            z[c] = v / (float)N;
            g[c] = dw2 ? dw[t * K + c] + dw2[t * K + c] : dw[t * K + c];
        }
        if (iters == 0) {
#pragma unroll
            for (int c = 0; c < K; ++c) {
                gl[c] = g[c];
                gz[c] = g[c] * scale * dtanh(z[c]);
            }
        } else {
            float l[K];
#pragma unroll
            for (int c = 0; c < K; ++c) l[c] = fmaf(scale, z[c], w_static[c]);
            mhc_record_bwd<N>(l, g, gl, iters, scr + t * kSlot, T * kSlot);
#pragma unroll
            for (int c = 0; c < K; ++c) gz[c] = scale * gl[c];
        }
#pragma unroll
        for (int c = 0; c < K; ++c) {
            dz[t * K + c] = gz[c];
            dls[c] += gl[c];
        }
#pragma unroll
        for (int i = 0; i < N; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < K; ++c) s = fmaf(p[i * K + c], gz[c], s);
            ab[t * 2 * N + i] = ri[i] / (float)N;
            ab[t * 2 * N + N + i] = -(ri[i] * ri[i] * ri[i]) * s / ((float)N * (float)d);
        }
    }
    // this wave's share of dw_static (the workgroup is one wave)
#pragma unroll
    for (int c = 0; c < K; ++c) {
        const float v = wave_sum(dls[c]);
        if (threadIdx.x == 0) dl_part[(int64_t)blockIdx.x * K + c] = v;
    }
}

// The tanh-mode coefficients with four lanes per token: lane q of a quad
// takes outputs c = q, q + 4, ... (dz_c, its share of dl and of
// s_i = sum_c P_ic dz_c, the quad adding the shares), so a 256-thread
// workgroup covers the 64 tokens that one wave covers in wgrad_coef_kernel
// and the same dl_part rows come out; the loads of a token's P row are
// spread over four lanes.  dz is bitwise wgrad_coef_kernel's; s_i, and so
// b_i, are added in another order.  The workgroup's dl sums go through LDS
// in token order.
template <int N>
__global__ __launch_bounds__(256) void wgrad_coef4_kernel(
    const float* __restrict__ P, const float* __restrict__ r, const float* __restrict__ dw,
    const float* __restrict__ dw2, float scale, float* __restrict__ dz,
    float* __restrict__ dl_part, float* __restrict__ ab, int64_t T, int d) {
    constexpr int K = 2 * N + N * N;
    constexpr int J = (K + 3) / 4;                  // outputs per lane
    __shared__ float dlw[J][4][64];
    const int q = threadIdx.x & 3, tk = threadIdx.x >> 2;
    float dls[J];
#pragma unroll
    for (int j = 0; j < J; ++j) dls[j] = 0.0f;
    for (int64_t b = blockIdx.x; b * 64 < T; b += gridDim.x) {
        const int64_t t = b * 64 + tk;
        const bool ok = t < T;
        const int64_t tc = ok ? t : T - 1;
        const float* p = P + tc * N * K;
        float ri[N];
#pragma unroll
        for (int i = 0; i < N; ++i) ri[i] = r[tc * N + i];
        float si[N];
#pragma unroll
        for (int i = 0; i < N; ++i) si[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int c = q + 4 * j;
            const int cc = c < K ? c : K - 1;
            // z as the forward kernel forms it: sum_i r_i P_ic in stream order, / n
            float v = ri[0] * p[cc];
#pragma unroll
            for (int i = 1; i < N; ++i) v = fmaf(ri[i], p[i * K + cc], v);
            const float z = v / (float)N;
            const float g = dw2 ? dw[tc * K + cc] + dw2[tc * K + cc] : dw[tc * K + cc];
            const float gz = g * scale * dtanh(z);
            const bool live = ok && c < K;
            if (live) dz[t * K + c] = gz;
            dls[j] += live ? g : 0.0f;
#pragma unroll
            for (int i = 0; i < N; ++i) si[i] = fmaf(p[i * K + cc], live ? gz : 0.0f, si[i]);
        }
#pragma unroll
        for (int i = 0; i < N; ++i) si[i] = quad_sum(si[i]);
        if (ok && q < N) {
            float sq = si[0];
#pragma unroll
            for (int i = 1; i < N; ++i) sq = q == i ? si[i] : sq;
            const float rq = ri[q];
            ab[t * 2 * N + q] = rq / (float)N;
            ab[t * 2 * N + N + q] = -(rq * rq * rq) * sq / ((float)N * (float)d);
        }
    }
    // the workgroup's dl: each output's 64 token lanes added in token order
#pragma unroll
    for (int j = 0; j < J; ++j) dlw[j][q][tk] = dls[j];
    __syncthreads();
    if (threadIdx.x < K) {
        const int c = threadIdx.x, j = c / 4, qq = c % 4;
        float v = dlw[j][qq][0];
        for (int k = 1; k < 64; ++k) v += dlw[j][qq][k];
        dl_part[(int64_t)blockIdx.x * K + c] = v;
    }
}

// ---------------------------------------------------- streaming dH and dW pass

// The four waves' partial dW (A x B tiles of f32x4, the same layout in every
// wave: they share the workgroup's columns) added into wave 0's registers in
// wave order, ((w0 + w1) + w2) + w3, through `lds` (3 * A * B * 256 floats),
// so each workgroup writes one partial instead of four.
template <int A, int B>
__device__ __forceinline__ void sum_wave_partials(f32x4 (&acc)[A][B], float* lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave > 0) {
#pragma unroll
        for (int a = 0; a < A; ++a)
#pragma unroll
            for (int b = 0; b < B; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) lds[((((wave - 1) * A + a) * B + b) * 4 + j) * 64 + lane] = acc[a][b][j];
    }
    __syncthreads();
    if (wave == 0) {
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int a = 0; a < A; ++a)
#pragma unroll
                for (int b = 0; b < B; ++b)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[a][b][j] += lds[(((w * A + a) * B + b) * 4 + j) * 64 + lane];
    }
}

// fp32 storage (bf16 takes wgrad_mfma_kernel below).  One workgroup owns a
// slice of CB = 16 V columns (16 lanes x one 16-byte vector) and a range of
// tokens.  Each wave takes 4 tokens per step: lane l
// works on token l / 16 of the step and columns (slice + l % 16) * V .. + V-1,
// so every load is 16 lanes x 16 contiguous bytes of one row.  Per element:
//   hbar = (1/n) sum_i r_i H_i,  dhbar = sum_c dz_c W[c] (W slice in LDS),
//   dH_i = dH_in_i + a_i dhbar + b_i H_i.
// dW: the 4 tokens of a step are the contraction of v_mfma_f32_16x16x4f32:
// A[m = c][k = token] = dz (c = l % 16 + 16 q), B[k = token][n] = the lane's
// hbar element e, so "virtual tile" e has output column (slice + n) V + e --
// the lane's own columns, no shuffles.  Each wave keeps its partial dW
// (2 x V tiles); at the end the workgroup's four are added (wave order) and
// written to part[split][K][d].
//
// TERMS: dH is not formed; the lane's dhbar values are written to dhbar
// [T][d] (fp32) instead, for a later pass that holds H_i to add
// a_i dhbar + b_i H_i itself (dH_in and dH unused).
template <int N, typename S, bool TERMS = false>
__global__ __launch_bounds__(256) void wgrad_stream_kernel(
    const uint8_t* __restrict__ H, const uint8_t* __restrict__ W, const float* __restrict__ dz,
    const float* __restrict__ ab, const float* __restrict__ r, const uint8_t* dH_in,
    uint8_t* dH, float* __restrict__ part, int64_t T, int d, int64_t tok_per_split,
    float* __restrict__ dhbar) {
    constexpr int V = Store<S>::kElems, SB = Store<S>::kBytes;
    constexpr int K = 2 * N + N * N;
    constexpr int CB = 16 * V;                       // columns per workgroup
    __shared__ __attribute__((aligned(16))) uint8_t wl[K * CB * SB];
    __shared__ float wsum[3 * 2 * V * 256];          // sum_wave_partials

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, cl = lane & 15;
    const int nvec = d / V;
    const int cv = blockIdx.x * 16 + cl;             // this lane's vector column
    const bool col_ok = cv < nvec;
    const int64_t row_bytes = (int64_t)d * SB;

    // the W slice: K rows x CB columns
    for (int p = threadIdx.x; p < K * 16; p += 256) {
        const int c = p / 16, v = blockIdx.x * 16 + p % 16;
        *reinterpret_cast<uint4*>(wl + (c * 16 + p % 16) * 16) =
            v < nvec ? ld16(W + ((int64_t)c * d + (int64_t)v * V) * SB) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();

    f32x4 acc[2][V];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[q][e] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t t_begin = (int64_t)blockIdx.y * tok_per_split;
    const int64_t t_end = t_begin + tok_per_split < T ? t_begin + tok_per_split : T;
    for (int64_t t0 = t_begin + 4 * wave; t0 < t_end; t0 += 16) {
        const int64_t t = t0 + g;
        const bool ok = t < t_end;
        const bool live = ok && col_ok;
        const int64_t r0 = (ok ? t : t_begin) * N * row_bytes + (int64_t)cv * 16;
        uint4 rh[N], rin[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            rh[i] = live ? ld16_stream(H + r0 + i * row_bytes) : make_uint4(0, 0, 0, 0);
            rin[i] = (!TERMS && live && dH_in) ? ld16_stream(dH_in + r0 + i * row_bytes)
                                               : make_uint4(0, 0, 0, 0);
        }
        const int64_t tt = ok ? t : t_begin;
        float gz[K];
#pragma unroll
        for (int c = 0; c < K; ++c) gz[c] = ok ? dz[tt * K + c] : 0.0f;
        float ri[N], ai[N], bi[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            ri[i] = ok ? r[tt * N + i] : 0.0f;
            ai[i] = ok ? ab[tt * 2 * N + i] : 0.0f;
            bi[i] = ok ? ab[tt * 2 * N + N + i] : 0.0f;
        }
        // dhbar for the lane's V columns
        float dhb[V];
#pragma unroll
        for (int e = 0; e < V; ++e) dhb[e] = 0.0f;
#pragma unroll
        for (int c = 0; c < K; ++c) {
            float wv[V];
            unpack<S>(*reinterpret_cast<const uint4*>(wl + (c * 16 + cl) * 16), wv);
#pragma unroll
            for (int e = 0; e < V; ++e) dhb[e] = fmaf(gz[c], wv[e], dhb[e]);
        }
        float hb[V];
#pragma unroll
        for (int e = 0; e < V; ++e) hb[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            float h[V], o[V];
            unpack<S>(rh[i], h);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                hb[e] = fmaf(ri[i], h[e], hb[e]);
                o[e] = fmaf(ai[i], dhb[e], bi[i] * h[e]);
            }
            if constexpr (!TERMS) {
                if (dH_in) {
                    float p[V];
                    unpack<S>(rin[i], p);
#pragma unroll
                    for (int e = 0; e < V; ++e) o[e] += p[e];
                }
                if (live) st16_stream(dH + r0 + i * row_bytes, pack<S>(o));
            }
        }
        if constexpr (TERMS) {
            if (live) {
#pragma unroll
                for (int q = 0; q < V / 4; ++q)
                    st16_stream(dhbar + t * d + (int64_t)cv * V + 4 * q,
                                make_uint4(__float_as_uint(dhb[4 * q]), __float_as_uint(dhb[4 * q + 1]),
                                           __float_as_uint(dhb[4 * q + 2]), __float_as_uint(dhb[4 * q + 3])));
            }
        }
#pragma unroll
        for (int e = 0; e < V; ++e) hb[e] = hb[e] / (float)N;
        // dW partial on the matrix cores
        float a0 = 0.0f, a1 = 0.0f;
        if (ok) {
            a0 = cl < K ? dz[tt * K + cl] : 0.0f;
            a1 = cl + 16 < K ? dz[tt * K + 16 + cl] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float bv = col_ok ? hb[e] : 0.0f;
            acc[0][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, bv, acc[0][e], 0, 0, 0);
            acc[1][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bv, acc[1][e], 0, 0, 0);
        }
    }
    // the workgroup's partial: C[m = 4 g + j][n = cl] of tile (q, e) is
    // dW[c = 16 q + 4 g + j][column cv * V + e]
    sum_wave_partials(acc, wsum);
    float* out = part + (int64_t)blockIdx.y * K * (int64_t)d;
    if (wave == 0 && col_ok) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 16 * q + 4 * g + j;
                if (c < K) {
#pragma unroll
                    for (int e = 0; e < V; ++e) out[(int64_t)c * d + (int64_t)cv * V + e] = acc[q][e][j];
                }
            }
    }
}

// bf16 storage: both contractions on the matrix cores, with dz (and hbar)
// split into a bf16 pair hi + lo (hi = dz rounded to bf16, lo = the rest
// rounded again), so a product keeps about 16 mantissa bits (the lo x lo term
// is below fp32 resolution of the sum and dropped; W is exact in bf16).
// A wave takes 16 tokens per step; lane l = 16 g + cl works on tokens
// g + 4 j (j = 0..3) of the step, columns 8 (slice + cl) .. + 7, so one load
// instruction covers 4 neighbouring tokens x 256 contiguous bytes.
//   dhbar: v_mfma_f32_16x16x32_bf16 with A[m][k = c] = dz of token
//     sigma(m) = m / 4 + 4 (m % 4) and B[k = c][n = cl] = W[c][8 (slice + n) + q]
//     for tile q = 0..7, so element j of tile q in lane l is
//     dhbar[token g + 4 j][column 8 (slice + cl) + q]: the lane's own tokens
//     and columns.
//   dW: v_mfma_f32_16x16x16_bf16 with A[m = c][k] = dz and
//     B[k][n = cl] = hbar[token][8 (slice + n) + q], k = 4 g + j standing for
//     token g + 4 j, which the lane holds.
// Per element: hbar = sum_i a_i H_i (a_i = r_i / n), dH_i = dH_in_i + a_i dhbar + b_i H_i.
// The 16-token steps are dealt round robin to the waves of the grid's rows,
// so the tokens in flight across the chip stay close together; the loads of
// a lane's next token are in flight while one is computed.  Loads are
// unconditional from valid addresses (tokens past T read the step's first
// token and are zeroed after the fact): no branches in the loop.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

struct Split2 { uint32_t hi, lo; };
// (x0, x1) -> hi and lo bf16 pairs, element 0 in the low half.
__device__ __forceinline__ Split2 split_bf16x2(float x0, float x1) {
    const uint32_t h = pack_bf16x2(x0, x1);
    return {h, pack_bf16x2(x0 - lo_bf16(h), x1 - hi_bf16(h))};
}

// TERMS (IN false): no dH; the lane's dhbar values (8 columns of each of
// its 4 tokens) go to dhbar [T][d] fp32 instead, for the pass that adds
// a_i dhbar + b_i H_i where it holds H_i.
template <int N, bool IN, bool TERMS = false>
__global__ __launch_bounds__(256) void wgrad_mfma_kernel(
    const uint8_t* __restrict__ H, const uint8_t* __restrict__ W, const float* __restrict__ dz,
    const float* __restrict__ ab, const float* __restrict__ r, const uint8_t* dH_in,
    uint8_t* dH, float* __restrict__ part, int64_t T, int d, int64_t tok_per_split,
    float* __restrict__ dhbar) {
    static_assert(!(IN && TERMS), "the terms take no incoming dH");
    // the fp32 kernel's signature: this one takes hbar's weights from ab (a_i =
    // r_i / n) and deals its steps round robin, so r and the split size go unused
    (void)r;
    (void)tok_per_split;
    constexpr int K = 2 * N + N * N;                 // <= 24
    constexpr int MT = (K + 15) / 16;                // 16-row tiles of dW
    // B operands of the dhbar product: wl[(q * 16 + cl) * 32 + c] = W[c][8 (slice + cl) + q],
    // zero for c >= K and for columns past d
    __shared__ __attribute__((aligned(16))) uint16_t wl[8 * 16 * 32];
    __shared__ float wsum[3 * MT * 8 * 256];         // sum_wave_partials

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, cl = lane & 15;
    const int nvec = d / 8;
    const int cv = blockIdx.x * 16 + cl;
    const bool col_ok = cv < nvec;
    const int64_t row_bytes = (int64_t)d * 2;
    const int64_t col_off = (int64_t)(col_ok ? cv : 0) * 16;

    for (int p = threadIdx.x; p < 32 * 16; p += 256) {
        const int c = p / 16, l = p % 16, v = blockIdx.x * 16 + l;
        const uint4 x = (c < K && v < nvec) ? ld16(W + ((int64_t)c * d + (int64_t)v * 8) * 2)
                                            : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            wl[(q * 16 + l) * 32 + c] = (uint16_t)(word(x, q / 2) >> (16 * (q & 1)));
    }
    __syncthreads();

    f32x4 acc[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[m][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t nsteps = (T + 15) / 16, sstride = (int64_t)gridDim.y * 4;
    for (int64_t st = (int64_t)blockIdx.y * 4 + wave; st < nsteps; st += sstride) {
        const int64_t t0 = st * 16;
        struct Tok { uint32_t h[N][4], din[N][4]; float a[N], b[N]; };
        auto fetch = [&](int j, Tok& L) {
            const int64_t t = t0 + g + 4 * j;
            const int64_t r0 = (t < T ? t : t0) * N * row_bytes + col_off;
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(H + r0 + i * row_bytes));
                L.h[i][0] = v.x; L.h[i][1] = v.y; L.h[i][2] = v.z; L.h[i][3] = v.w;
                if constexpr (IN) {
                    const u32x4 u =
                        __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dH_in + r0 + i * row_bytes));
                    L.din[i][0] = u.x; L.din[i][1] = u.y; L.din[i][2] = u.z; L.din[i][3] = u.w;
                }
            }
            const float* abt = ab + (t < T ? t : t0) * 2 * N;
#pragma unroll
            for (int i = 0; i < N; ++i) {
                L.a[i] = abt[i];
                L.b[i] = abt[N + i];
            }
        };
        Tok L0, L1;
        fetch(0, L0);
        // dhbar for the 16 tokens of the step
        f32x4 dhb[8];
        {
            const int64_t t = t0 + (cl >> 2) + 4 * (cl & 3);
            const bool ok = t < T;
            const int64_t tt = ok ? t : t0;
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = 8 * g + i;
                const float v = dz[tt * K + (c < K ? c : K - 1)];
                x[i] = (ok && c < K) ? v : 0.0f;
            }
            uint32_t ah[4], al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const Split2 s = split_bf16x2(x[2 * i], x[2 * i + 1]);
                ah[i] = s.hi;
                al[i] = s.lo;
            }
            const bf16x8_t Ah = __builtin_bit_cast(bf16x8_t, make_uint4(ah[0], ah[1], ah[2], ah[3]));
            const bf16x8_t Al = __builtin_bit_cast(bf16x8_t, make_uint4(al[0], al[1], al[2], al[3]));
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const bf16x8_t B =
                    __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(wl + (q * 16 + cl) * 32 + 8 * g));
                dhb[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, B, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                dhb[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, B, dhb[q], 0, 0, 0);
            }
        }
        // the lane's 4 tokens: dH, and hbar for the dW product
        float hb[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Tok& L = (j & 1) ? L1 : L0;
            if (j < 3) fetch(j + 1, (j & 1) ? L0 : L1);
            __builtin_amdgcn_sched_barrier(0);
            const int64_t t = t0 + g + 4 * j;
            const bool ok = t < T;
            const int64_t r0 = (ok ? t : t0) * N * row_bytes + col_off;
#pragma unroll
            for (int q = 0; q < 8; ++q) hb[j][q] = 0.0f;
#pragma unroll
            for (int i = 0; i < N; ++i) {
                uint32_t ow[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float h0 = lo_bf16(L.h[i][k]), h1 = hi_bf16(L.h[i][k]);
                    float o0 = 0.0f, o1 = 0.0f;
                    if constexpr (IN) {
                        o0 = lo_bf16(L.din[i][k]);
                        o1 = hi_bf16(L.din[i][k]);
                    }
                    hb[j][2 * k] = fmaf(L.a[i], h0, hb[j][2 * k]);
                    hb[j][2 * k + 1] = fmaf(L.a[i], h1, hb[j][2 * k + 1]);
                    if constexpr (!TERMS) {
                        o0 = fmaf(L.b[i], h0, fmaf(L.a[i], dhb[2 * k][j], o0));
                        o1 = fmaf(L.b[i], h1, fmaf(L.a[i], dhb[2 * k + 1][j], o1));
                        ow[k] = pack_bf16x2(o0, o1);
                    }
                }
                if constexpr (!TERMS)
                    if (ok && col_ok) st16_stream(dH + r0 + i * row_bytes, make_uint4(ow[0], ow[1], ow[2], ow[3]));
            }
            if constexpr (TERMS) {
                // the lane's 32 bytes go out as two 16-byte halves, each
                // store instruction covering every other 16 bytes of the
                // row's 512; as ordinary (cached) stores the halves meet in
                // L2 and each line is written to HBM whole
                if (ok && col_ok) {
                    float* o = dhbar + t * d + (int64_t)cv * 8;
                    st16(o, make_uint4(__float_as_uint(dhb[0][j]), __float_as_uint(dhb[1][j]),
                                       __float_as_uint(dhb[2][j]), __float_as_uint(dhb[3][j])));
                    st16(o + 4, make_uint4(__float_as_uint(dhb[4][j]), __float_as_uint(dhb[5][j]),
                                           __float_as_uint(dhb[6][j]), __float_as_uint(dhb[7][j])));
                }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) hb[j][q] = ok ? hb[j][q] : 0.0f;
            __builtin_amdgcn_sched_barrier(0);
        }
        // dW += dz^T hbar over the 16 tokens
        i16x4_t Ah[MT], Al[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int c = 16 * m + cl;
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t t = t0 + g + 4 * j;
                const float v = dz[(t < T ? t : t0) * K + (c < K ? c : K - 1)];
                x[j] = (t < T && c < K) ? v : 0.0f;
            }
            const Split2 s0 = split_bf16x2(x[0], x[1]), s1 = split_bf16x2(x[2], x[3]);
            Ah[m] = __builtin_bit_cast(i16x4_t, make_uint2(s0.hi, s1.hi));
            Al[m] = __builtin_bit_cast(i16x4_t, make_uint2(s0.lo, s1.lo));
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const Split2 s0 = split_bf16x2(hb[0][q], hb[1][q]), s1 = split_bf16x2(hb[2][q], hb[3][q]);
            const i16x4_t Bh = __builtin_bit_cast(i16x4_t, make_uint2(s0.hi, s1.hi));
            const i16x4_t Bl = __builtin_bit_cast(i16x4_t, make_uint2(s0.lo, s1.lo));
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Ah[m], Bh, acc[m][q], 0, 0, 0);
                acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Ah[m], Bl, acc[m][q], 0, 0, 0);
                acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Al[m], Bh, acc[m][q], 0, 0, 0);
            }
        }
    }
    // the workgroup's partial: element j of tile (m, q) is dW[c = 16 m + 4 g + j][8 cv + q]
    sum_wave_partials(acc, wsum);
    float* out = part + (int64_t)blockIdx.y * K * (int64_t)d;
    if (wave == 0 && col_ok) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 16 * m + 4 * g + j;
                if (c < K) {
                    float* o = out + (int64_t)c * d + (int64_t)cv * 8;
                    *reinterpret_cast<float4*>(o) =
                        make_float4(acc[m][0][j], acc[m][1][j], acc[m][2][j], acc[m][3][j]);
                    *reinterpret_cast<float4*>(o + 4) =
                        make_float4(acc[m][4][j], acc[m][5][j], acc[m][6][j], acc[m][7][j]);
                }
            }
    }
}

inline int64_t coef_blocks(int64_t T) {
    const int64_t b = (T + 63) / 64;
    return b < kMaxGrid ? b : kMaxGrid;
}

template <int N>
hipError_t coef_go(const float* P, const float* r, const float* dw, const float* dw2, const float* ws,
                   float scale, int iters, float* scr, float* dz, float* dl_part, float* ab, int64_t T,
                   int d, hipStream_t s) {
    // 64 tokens per workgroup either way (the dl_part rows): one lane per
    // token for the mHC transform, four for tanh
    if (iters == 0)
        return launch(wgrad_coef4_kernel<N>, dim3((unsigned)coef_blocks(T)), dim3(256), 0, s, P, r,
                      dw, dw2, scale, dz, dl_part, ab, T, d);
    return launch(wgrad_coef_kernel<N>, dim3((unsigned)coef_blocks(T)), dim3(64), 0, s, P, r, dw, dw2,
                  ws, scale, iters, scr, dz, dl_part, ab, T, d);
}

template <int N, typename S>
hipError_t stream_go(const void* H, const void* W, const float* dz, const float* ab, const float* r,
                     const void* dH_in, void* dH, float* part, int64_t T, int d, int splits,
                     int64_t tps, float* dhbar, hipStream_t s) {
    const int nvec = d / Store<S>::kElems;
    const dim3 grid((unsigned)((nvec + 15) / 16), (unsigned)splits);
    void (*kernel)(const uint8_t*, const uint8_t*, const float*, const float*, const float*,
                   const uint8_t*, uint8_t*, float*, int64_t, int, int64_t, float*) =
        !std::is_same<S, bf16_t>::value ? (dhbar ? wgrad_stream_kernel<N, S, true> : wgrad_stream_kernel<N, S>)
        : dhbar                          ? wgrad_mfma_kernel<N, false, true>
        : dH_in                          ? wgrad_mfma_kernel<N, true>
                                         : wgrad_mfma_kernel<N, false>;
    return launch(kernel, grid, dim3(256), 0, s, static_cast<const uint8_t*>(H),
                  static_cast<const uint8_t*>(W), dz, ab, r, static_cast<const uint8_t*>(dH_in),
                  static_cast<uint8_t*>(dH), part, T, d, tps, dhbar);
}

template <typename S>
hipError_t stream_by_n(int n, const void* H, const void* W, const float* dz, const float* ab,
                       const float* r, const void* dH_in, void* dH, float* part, int64_t T, int d,
                       int splits, int64_t tps, float* dhbar, hipStream_t s) {
    switch (n) {
        case 1: return stream_go<1, S>(H, W, dz, ab, r, dH_in, dH, part, T, d, splits, tps, dhbar, s);
        case 2: return stream_go<2, S>(H, W, dz, ab, r, dH_in, dH, part, T, d, splits, tps, dhbar, s);
        case 3: return stream_go<3, S>(H, W, dz, ab, r, dH_in, dH, part, T, d, splits, tps, dhbar, s);
        case 4: return stream_go<4, S>(H, W, dz, ab, r, dH_in, dH, part, T, d, splits, tps, dhbar, s);
    }
    return hipErrorInvalidValue;
}

// Tokens per dW split: enough workgroups (columns x splits) to fill the chip,
// at least 64 tokens each; at most 64 splits.
inline int64_t splits_of(int64_t T) {
    int64_t s = (T + 511) / 512;
    if (s > 64) s = 64;
    return s < 1 ? 1 : s;
}

// Workspace layout (floats): P [T][n][K] | r [T][n] | dz [T][K] |
// dw_static partials [coefficient workgroups][K] | ab [T][2n] | Sinkhorn
// scratch [iters][T][16] | dW partials [splits][K][d] | the two sums'
// level scratch.  Every region starts 16-byte aligned.
struct WgSpace {
    int64_t P, r, dz, dl, ab, scr, part, tmp, tmp2, total;
};
inline int64_t up4(int64_t x) { return (x + 3) / 4 * 4; }
inline WgSpace wg_space(int64_t T, int n, int d, int iters) {
    const int64_t K = 2 * n + int64_t(n) * n;
    WgSpace w;
    w.P = 0;
    w.r = w.P + up4(T * n * K);
    w.dz = w.r + up4(T * n);
    w.dl = w.dz + up4(T * K);
    w.ab = w.dl + up4(coef_blocks(T) * K);
    w.scr = w.ab + up4(T * 2 * n);
    w.part = w.scr + up4(int64_t(iters) * T * kSlot);
    const int64_t rows = splits_of(T);
    w.tmp = w.part + up4(rows * K * d);
    w.tmp2 = w.tmp + up4(sum_rows_tmp_floats(rows, K * d));
    w.total = w.tmp2 + up4(sum_rows_tmp_floats(coef_blocks(T), K));
    return w;
}

}  // namespace

int64_t saved_r_offset(int64_t T, int n) {
    const int64_t K = 2 * n + int64_t(n) * n;
    return up4(T * n * K);
}
int64_t saved_floats(int64_t T, int n) { return saved_r_offset(T, n) + up4(T * n); }

int64_t weights_backward_workspace_bytes(int64_t T, int n, int d, int iters) {
    if (T <= 0 || n <= 0 || d <= 0 || iters < 0) return 0;
    return wg_space(T, n, d, iters).total * 4;
}

int64_t sinkhorn_backward_workspace_bytes(int64_t T, int iters) {
    if (T <= 0 || iters <= 0) return 0;
    return int64_t(iters) * T * kSlot * 4;
}

hipError_t launch_sinkhorn_backward(const float* logits, const float* dw, const float* dw2,
                                    float* dlogits, int iters, void* work, int64_t T, int n,
                                    hipStream_t s) {
    // four lanes per token, 64 tokens per 256-thread workgroup
    const int64_t blocks = (4 * T + 255) / 256;
    const dim3 grid((unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid));
    float* scr = static_cast<float*>(work);
    // up to kKeep iterations keep their matrices in registers
    constexpr int kKeep = 20;
    const bool reg = iters <= kKeep;
#define HC_SKB(NN)                                                                              \
    return reg ? launch(sinkhorn_bwd_quad_kernel<NN, kKeep>, grid, dim3(256), 0, s, logits, dw, \
                        dw2, dlogits, iters, scr, T)                                            \
               : launch(sinkhorn_bwd_quad_kernel<NN, 0>, grid, dim3(256), 0, s, logits, dw, dw2, \
                        dlogits, iters, scr, T);
    switch (n) {
        case 1: HC_SKB(1)
        case 2: HC_SKB(2)
        case 3: HC_SKB(3)
        case 4: HC_SKB(4)
    }
#undef HC_SKB
    return hipErrorInvalidValue;
}

hipError_t launch_weights_backward(const void* H, const void* W, const float* w_static, float scale,
                                   float eps, int iters, const float* dw, const float* dw2,
                                   const float* saved, const void* dH_in,
                                   void* dH, float* dW, float* dws, void* work, int64_t T, int n,
                                   int d, int dt, hipStream_t s, float* dhbar, float* coef) {
    const WgSpace sp = wg_space(T, n, d, iters);
    float* ws = static_cast<float*>(work);
    const int K = 2 * n + n * n;
    // the coefficients (a_i | b_i): the caller's buffer when the terms are
    // returned, else the workspace
    float* const ab = dhbar ? coef : ws + sp.ab;
    // (1) per-stream projections and row norms: kept by the forward, or
    // computed again
    const float* Pp = saved ? saved : ws + sp.P;
    const float* rp = saved ? saved + saved_r_offset(T, n) : ws + sp.r;
    hipError_t e = hipSuccess;
    if (!saved) {
        e = launch_weights_raw(H, W, eps, ws + sp.P, ws + sp.r, T, n, d, dt, s);
        if (e != hipSuccess) return e;
    }
    // (2) per-token coefficients
    switch (n) {
        case 1: e = coef_go<1>(Pp, rp, dw, dw2, w_static, scale, iters, ws + sp.scr, ws + sp.dz, ws + sp.dl, ab, T, d, s); break;
        case 2: e = coef_go<2>(Pp, rp, dw, dw2, w_static, scale, iters, ws + sp.scr, ws + sp.dz, ws + sp.dl, ab, T, d, s); break;
        case 3: e = coef_go<3>(Pp, rp, dw, dw2, w_static, scale, iters, ws + sp.scr, ws + sp.dz, ws + sp.dl, ab, T, d, s); break;
        case 4: e = coef_go<4>(Pp, rp, dw, dw2, w_static, scale, iters, ws + sp.scr, ws + sp.dz, ws + sp.dl, ab, T, d, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    // (3) dH and the dW partials
    const int64_t splits = splits_of(T);
    const int64_t tps = (T + splits - 1) / splits;
    e = dt == 0 ? stream_by_n<f32_t>(n, H, W, ws + sp.dz, ab, rp, dH_in, dH, ws + sp.part,
                                     T, d, (int)splits, tps, dhbar, s)
                : stream_by_n<bf16_t>(n, H, W, ws + sp.dz, ab, rp, dH_in, dH,
                                      ws + sp.part, T, d, (int)splits, tps, dhbar, s);
    if (e != hipSuccess) return e;
    // (4) fixed-order sums: dW over the partials, dw_static over the
    // coefficient workgroups' partials, in shared launches
    const SumJob jobs[2] = {{ws + sp.part, splits, K * d, ws + sp.tmp, dW, nullptr, 0},
                           {ws + sp.dl, coef_blocks(T), K, ws + sp.tmp2, dws, nullptr, 0}};
    return launch_sum_rows(jobs, 2, s);
}

}  // namespace hc
