// hc_backward.hip -- gradients of the Hyper-Connections residual path: the
// write-back (post) and the read-mix + RMSNorm (pre), and the deterministic
// sums that turn per-block partial gradients into gradients of shared
// parameters.
//
// Sources: hfviewer.com glossary "Hyper-connections (mHC)", definition (the
// mixing before and after the block is learned, so its weights need
// gradients, and the page credits the parallel streams with more paths for
// gradients than a single residual offers);
// learnaivisually.com "Tencent open-sources Hy4 Preview at 770B -- Identity
// Hyper-Connections", section "Jargon", Residual connection (gradients take
// the short path back through the residual).
//
// Post:  H'_i = sum_j A[i][j] H_j + beta_i F is linear, so
//   dH_j = sum_i A[i][j] dH'_i,  dF = sum_i beta_i dH'_i,
//   dA[i][j] = sum_k dH'_ik H_jk,  dbeta_i = sum_k dH'_ik F_k.
// Pre:   u = gamma * x * r, r = (mean x^2 + eps)^(-1/2), x = sum_i alpha_i H_i:
//   dy = gamma * du,  dx = r * (dy - x * r^2 * mean(dy * x)),
//   dH_i = alpha_i dx,  dalpha_i = sum_k dx_k H_ik,  dgamma = sum_t du x r.
// A layer's H feeds both, so its gradient is the sum of the two dH above.
// Either post writes its share and pre adds into it, or (folded) post skips
// it and pre forms sum_j A[j][i] dH'_j itself, which moves n rows per token
// fewer and rounds once.
// In a stack of layers the write-back of one layer and the read-mix of the
// next meet at the same H' (the forward's fused boundary), and
// post_pre_bwd_kernel takes both gradients there in one pass: it recomputes
// H' from the write-back's inputs, adds the read-mix's share to the
// gradient arriving at H', and applies the write-back's gradient to the sum
// without storing it.
//
// Weight gradients take the shape of the weights: one record per token for
// per-token weights (post: a workgroup reduction per token; pre: per-wave
// sums in the workspace, added in wave order by token_records_kernel), one
// record in total for shared weights.  Shared-record gradients and dgamma are
// summed over the tokens of a block in registers, written once per block to
// the caller's workspace, and summed over blocks by sum_rows_kernel in a
// fixed order (64 rows per level), so every result is deterministic.
//
// The kernels stream rows like the forward ones (one 16-byte vector per
// thread per stream, all loads of a token issued first).
#include <mutex>

#include "hc_device.h"
#include "hc_launch.h"

namespace hc {

namespace {

constexpr int64_t kMaxGridB = 1 << 20;
constexpr int kSumRows = 64;            // rows summed per block in sum_rows_kernel

// Sum M values over the block at once; every thread gets all M sums.  `red`
// holds 16 * M floats.
template <int M>
__device__ __forceinline__ void block_sum_vec(float (&v)[M], float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        v[m] = wave_sum(v[m]);
        if (lane == 0) red[wave * M + m] = v[m];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float s = red[m];
        for (int w = 1; w < nw; ++w) s += red[w * M + m];
        v[m] = s;
    }
    __syncthreads();
}

// One DPP lane exchange inside a row of 16 lanes (row_ror:8, row_half_mirror
// and quad_perm patterns: every lane has a source).
template <int CTRL>
__device__ __forceinline__ float dpp_swap(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// A reduce-scatter step: pairs (in[2k], in[2k+1]) (a missing in[2k+1] is 0)
// become out[k], the half of the pair that `upper` selects plus the partner
// lane's copy of that same half (the partner's `upper` is the opposite).
template <int L, int CTRL>
__device__ __forceinline__ void halve(const float* in, float* out, bool upper) {
#pragma unroll
    for (int k = 0; k < (L + 1) / 2; ++k) {
        const float lo = in[2 * k], hi = 2 * k + 1 < L ? in[2 * k + 1] : 0.0f;
        out[k] = (upper ? hi : lo) + dpp_swap<CTRL>(upper ? lo : hi);
    }
}

// Sum M <= 24 values over the block for threads 0..M-1 only: thread m returns
// sum m (the others 0).  Inside a wave the values are reduce-scattered: three
// exchanges inside each 16-lane row, with lanes l ^ 8, l ^ 7 and l ^ 2, each
// halve what a lane carries (24 -> 12 -> 6 -> 3), and then lanes l ^ 1 and
// the four rows (v_permlane16_swap, v_permlane32_swap) are added whole.  Lane
// l then holds the wave's sums of values 8k + g (k = 0, 1, 2), g = 4 b1 +
// 2 b2 + b3 from l's bits; lanes 0, 2, .., 14 cover every g.  The waves'
// sums meet in LDS (24 floats per wave in `red`) and are added in wave order.
// About 80 instructions for 20 values, against 7 or 8 per value for one
// reduction per value.
// wave_sums_to is the part inside one wave: the wave's sum of value m goes to
// out[m] (m < M), stored by the lane that holds it.
template <int M>
__device__ __forceinline__ void wave_sums_to(const float (&v)[M], float* out) {
    static_assert(M <= 24, "wave_sums_to takes at most 24 values");
    const int lane = threadIdx.x & 63;
    const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
    constexpr int LA = (M + 1) / 2, LB = (LA + 1) / 2, LC = (LB + 1) / 2;
    float a[LA], b[LB], c[LC];
    halve<M, 0x128>(v, a, b3);        // row_ror:8, partner l ^ 8
    halve<LA, 0x141>(a, b, b2);       // row_half_mirror, partner l ^ 7
    halve<LB, 0x4E>(b, c, b1);        // quad_perm [2, 3, 0, 1], partner l ^ 2
#pragma unroll
    for (int k = 0; k < LC; ++k) {
        float x = c[k] + dpp_swap<0xB1>(c[k]);    // quad_perm [1, 0, 3, 2]: l ^ 1
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        c[k] = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    }
    if (lane < 16 && !(lane & 1)) {
        const int g = (b1 ? 4 : 0) + (b2 ? 2 : 0) + (b3 ? 1 : 0);
#pragma unroll
        for (int k = 0; k < LC; ++k)
            if (8 * k + g < M) out[8 * k + g] = c[k];
    }
}

template <int M>
__device__ __forceinline__ float block_sum_to(const float (&v)[M], float* red) {
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    wave_sums_to<M>(v, red + wave * 24);
    __syncthreads();
    float s = 0.0f;
    if ((int)threadIdx.x < M) {
        s = red[threadIdx.x];
        for (int w = 1; w < nw; ++w) s += red[w * 24 + threadIdx.x];
    }
    __syncthreads();
    return s;
}

// acc + the dot product of two storage words: fp32 one product; bf16 both
// halves at once with v_dot2_f32_bf16 (bf16 products are exact in fp32), so
// the words need no unpacking.
template <typename S> __device__ __forceinline__ float dot_word(uint32_t a, uint32_t b, float acc);
template <> __device__ __forceinline__ float dot_word<f32_t>(uint32_t a, uint32_t b, float acc) {
    return fmaf(__uint_as_float(a), __uint_as_float(b), acc);
}
template <> __device__ __forceinline__ float dot_word<bf16_t>(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                           acc, false);
}

// Tokens per block for shared-record gradients: enough blocks to fill the
// chip several times over, at least 8 tokens each (pre: its per-block
// partials include a d-wide dgamma row).
inline int64_t group_of(int64_t T) {
    const int64_t g = T / 2048;
    return g < 8 ? 8 : g;
}
// Post's partials are only n + n^2 floats per block, so it takes fewer
// tokens per block: about 4096 blocks, at least 2 tokens each (measured at
// T = 8192, n = 4, d = 4096 bf16: 2 tokens per block 167 us, 4 171 us, and
// 1 token per block 170 us with its longer sum).
inline int64_t post_group_of(int64_t T) {
    const int64_t g = T / 4096;
    return g < 2 ? 2 : g;
}

// ------------------------------------------------------------ post backward

// PER_TOKEN: dw is [T][K], one block reduction per token.  Otherwise the
// block's tokens are summed in registers and one partial record per block
// goes to part[blk][M] (M = n + n^2: dbeta then dA).  HG false: dH is not
// written; the pre gradient forms A^T dH' itself (pre_bwd_kernel's dHo),
// which saves writing dH here and reading it back there.
template <int N, typename S, int VPT, bool PER_TOKEN, bool HG>
__global__ __launch_bounds__(1024) void post_bwd_kernel(
    const uint8_t* __restrict__ dHo, const uint8_t* __restrict__ H, const uint8_t* __restrict__ F,
    const float* __restrict__ w, int64_t w_stride, uint8_t* __restrict__ dH,
    uint8_t* __restrict__ dF, float* __restrict__ dw, float* __restrict__ part, int64_t T, int d,
    int group) {
    constexpr int V = Store<S>::kElems, E = Word<S>::kElems;
    constexpr int K = 2 * N + N * N;
    constexpr int M = N + N * N;            // dbeta, dA
    __shared__ float red[16 * 24];          // block_sum_to: 24 floats per wave
    const int B = blockDim.x;
    const int nvec = d / V;
    const int64_t row_bytes = (int64_t)d * Store<S>::kBytes;

    // Block blk takes tokens blk, blk + nb, blk + 2 nb, ... (at most `group`
    // of them), so the tokens in flight at any moment lie close together in
    // memory (consecutive tokens per block spread them over the whole
    // tensor; the pre gradient ran 8% slower that way).
    const int64_t nb = (T + group - 1) / group;
    for (int64_t blk = blockIdx.x; blk < nb; blk += gridDim.x) {
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = 0.0f;
        uint4 rg[N][VPT], rh[N][VPT], rf[VPT];
        // Every path assigns the vectors (zeros where there is no token or
        // column), so the last token's values are dead once used and their
        // registers free for the next phase; otherwise they stay live
        // around the loop.
        auto clear = [&](int j) {
#pragma unroll
            for (int i = 0; i < N; ++i) rg[i][j] = rh[i][j] = make_uint4(0, 0, 0, 0);
            rf[j] = make_uint4(0, 0, 0, 0);
        };
        auto fetch = [&](int64_t t) {
            const int64_t r0 = t * N * row_bytes;
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int v = threadIdx.x + j * B;
                if (v < nvec) {
#pragma unroll
                    for (int i = 0; i < N; ++i) {
                        rg[i][j] = ld16_stream(dHo + r0 + i * row_bytes + v * 16);
                        rh[i][j] = ld16_stream(H + r0 + i * row_bytes + v * 16);
                    }
                    rf[j] = ld16_stream(F + t * row_bytes + v * 16);
                } else {
                    clear(j);
                }
            }
        };
        // Per-token records with one vector per thread: a token's loads are
        // issued before the previous token's block-wide sums.  (Measured at
        // n = 4 when it was introduced: fewer registers than loading at the
        // top of the loop, one more wave per SIMD, and 16% faster; with more
        // vectors per thread it needs more registers, so it is not used there.)
        constexpr bool kAhead = PER_TOKEN && VPT == 1;
        if constexpr (kAhead) {
            if (blk < T) fetch(blk);
        }
        for (int64_t t = blk; t < T; t += nb) {
            if constexpr (!kAhead) fetch(t);
            const float* rec = w + t * w_stride;
            float beta[N], A[N][N];
#pragma unroll
            for (int i = 0; i < N; ++i) beta[i] = rec[N + i];
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int j = 0; j < N; ++j) A[i][j] = rec[2 * N + i * N + j];

            const int64_t r0 = t * N * row_bytes;
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int v = threadIdx.x + j * B;
                if (v < nvec) {
                    // partials of dbeta_i = dH'_i . F and dA[i][jj] = dH'_i . H_jj
                    // first, from the storage words; after them only the dH'
                    // vectors stay live
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
#pragma unroll
                        for (int i = 0; i < N; ++i) {
                            const uint32_t gw = word(rg[i][j], q);
#pragma unroll
                            for (int jj = 0; jj < N; ++jj)
                                acc[N + i * N + jj] = dot_word<S>(gw, word(rh[jj][j], q), acc[N + i * N + jj]);
                            acc[i] = dot_word<S>(gw, word(rf[j], q), acc[i]);
                        }
                    }
                    // (kept apart by the scheduler: interleaving the two phases
                    // keeps every input and output live at once)
                    __builtin_amdgcn_sched_barrier(0);
                    // dH_jj = sum_i A[i][jj] dH'_i (HG only) and dF = sum_i
                    // beta_i dH'_i, one output row at a time from the dH'
                    // vectors unpacked once (the raw words die here)
                    float g[N][4][E];
#pragma unroll
                    for (int i = 0; i < N; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q) unpack_word<S>(word(rg[i][j], q), g[i][q]);
#pragma unroll
                    for (int jj = HG ? 0 : N; jj <= N; ++jj) {
                        uint32_t oh[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            float o[E];
#pragma unroll
                            for (int e = 0; e < E; ++e) {
                                float sum = (jj < N ? A[0][jj] : beta[0]) * g[0][q][e];
#pragma unroll
                                for (int i = 1; i < N; ++i)
                                    sum = fmaf(jj < N ? A[i][jj] : beta[i], g[i][q][e], sum);
                                o[e] = sum;
                            }
                            oh[q] = pack_word<S>(o);
                        }
                        uint8_t* dst = jj < N ? dH + r0 + jj * row_bytes : dF + t * row_bytes;
                        st16_stream(dst + v * 16, make_uint4(oh[0], oh[1], oh[2], oh[3]));
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            if constexpr (PER_TOKEN) {
                if constexpr (kAhead) {
                    if (t + nb < T) {
                        fetch(t + nb);
                    } else {
#pragma unroll
                        for (int j = 0; j < VPT; ++j) clear(j);
                    }
                }
                const float sum = block_sum_to<M>(acc, red);
                // thread m < M holds sum m; the record is [dalpha = 0 (post does
                // not read alpha) | dbeta | dA]
                if ((int)threadIdx.x < N) dw[t * K + threadIdx.x] = 0.0f;
                if ((int)threadIdx.x < M) dw[t * K + N + threadIdx.x] = sum;
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m] = 0.0f;
            }
        }
        if constexpr (!PER_TOKEN) {
            const float sum = block_sum_to<M>(acc, red);
            if ((int)threadIdx.x < M) part[blk * M + threadIdx.x] = sum;
        }
    }
}

// ------------------------------------------------------------- pre backward

// A block walks up to `group` tokens (see post_bwd_kernel).  The dgamma partial of each
// thread's columns stays in registers and goes to dg_part[blk][d] once;
// dalpha goes per token and wave to da_part[t][wave][N] (PER_TOKEN; dw is
// then filled by token_records_kernel) or is summed over the block's tokens
// into da_part[blk][N].  dH gets dH_in added (when given), or with FOLD the
// write-back's H gradient sum_i A[i][j] dH'_i, formed here from dHo (the
// gradient at the write-back's output) and the same record.
// HG false: dH is not written (dH == NULL); the records and dgamma come out
// bitwise as with it (per-token weights produced from H need dalpha before
// the layer's dH can be formed).
template <int N, typename S, int VPT, bool PER_TOKEN, bool FOLD, bool HG = true>
__global__ __launch_bounds__(1024) void pre_bwd_kernel(
    const uint8_t* __restrict__ du, const uint8_t* __restrict__ H, const float* __restrict__ w,
    int64_t w_stride, const float* __restrict__ gamma, float eps, const uint8_t* dH_in,
    const uint8_t* dHo, uint8_t* dH, float* __restrict__ dw, float* __restrict__ dg_part,
    float* __restrict__ da_part, int64_t T, int d, int group) {
    constexpr int V = Store<S>::kElems, E = Word<S>::kElems;
    __shared__ float red[16 * (N > 2 ? N : 2)];   // block_sum_vec<2> and <N>
    const int B = blockDim.x;
    const int nvec = d / V;
    const int64_t row_bytes = (int64_t)d * Store<S>::kBytes;

    // Block blk takes tokens blk, blk + nb, blk + 2 nb, ... (at most `group`
    // of them), so the tokens in flight at any moment lie close together in
    // memory (consecutive tokens per block spread them over the whole
    // tensor; the pre gradient ran 8% slower that way).
    const int64_t nb = (T + group - 1) / group;
    for (int64_t blk = blockIdx.x; blk < nb; blk += gridDim.x) {
        float dgp[VPT][V];
#pragma unroll
        for (int j = 0; j < VPT; ++j)
#pragma unroll
            for (int e = 0; e < V; ++e) dgp[j][e] = 0.0f;
        float dab[N];
#pragma unroll
        for (int i = 0; i < N; ++i) dab[i] = 0.0f;

        for (int64_t t = blk; t < T; t += nb) {
            const float* a = w + t * w_stride;
            float alpha[N], A[N][N];
#pragma unroll
            for (int i = 0; i < N; ++i) alpha[i] = a[i];
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int k = 0; k < N; ++k) A[i][k] = FOLD ? a[2 * N + i * N + k] : 0.0f;
            const int64_t r0 = t * N * row_bytes;
            // every load of the token first, dH_in or dH' included (they do
            // not depend on the reduction)
            const uint8_t* add = FOLD ? dHo : dH_in;
            uint4 rh[N][VPT], ru[VPT], rin[N][VPT];
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int v = threadIdx.x + j * B;
                const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < N; ++i)
                    rh[i][j] = v < nvec ? ld16_stream(H + r0 + i * row_bytes + v * 16) : z;
                ru[j] = v < nvec ? ld16_stream(du + t * row_bytes + v * 16) : z;
#pragma unroll
                for (int i = 0; i < N; ++i)
                    rin[i][j] = (add && v < nvec) ? ld16_stream(add + r0 + i * row_bytes + v * 16) : z;
            }
            // x = sum_i alpha_i H_i, dword by dword (recomputed the same way
            // after the reduction instead of being kept)
            auto mix_word = [&](int j, int q, float (&x)[E]) {
                float h[E];
                unpack_word<S>(word(rh[0][j], q), h);
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = alpha[0] * h[e];
#pragma unroll
                for (int i = 1; i < N; ++i) {
                    unpack_word<S>(word(rh[i][j], q), h);
#pragma unroll
                    for (int e = 0; e < E; ++e) x[e] = fmaf(alpha[i], h[e], x[e]);
                }
            };
            // mean square of x and mean(gamma * du * x)
            float s2[2] = {0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int v = threadIdx.x + j * B;
                if (v < nvec) {
                    float g[V];
#pragma unroll
                    for (int q = 0; q < V / 4; ++q) unpack<f32_t>(ld16(gamma + v * V + 4 * q), &g[4 * q]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float x[E], ug[E];
                        mix_word(j, q, x);
                        unpack_word<S>(word(ru[j], q), ug);
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            s2[0] = fmaf(x[e], x[e], s2[0]);
                            s2[1] = fmaf(g[q * E + e] * ug[e], x[e], s2[1]);
                        }
                    }
                }
            }
            // both sums in one reduction: the mean square of x does not
            // depend on r, and mean(dy * x) is needed only after r is known
            block_sum_vec<2>(s2, red);
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
#pragma unroll
                for (int i = 0; i < N; ++i) opaque(rh[i][j]);
                opaque(ru[j]);
            }
            const float r = 1.0f / sqrtf(s2[0] / (float)d + eps);
            const float c2 = r * r * s2[1] / (float)d;
            float da[N];
#pragma unroll
            for (int i = 0; i < N; ++i) da[i] = 0.0f;
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int v = threadIdx.x + j * B;
                if (v < nvec) {
                    float g[V], dx[V];
#pragma unroll
                    for (int q = 0; q < V / 4; ++q) unpack<f32_t>(ld16(gamma + v * V + 4 * q), &g[4 * q]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float x[E], ug[E];
                        mix_word(j, q, x);
                        unpack_word<S>(word(ru[j], q), ug);
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            dx[q * E + e] = r * (g[q * E + e] * ug[e] - x[e] * c2);
                            dgp[j][q * E + e] = fmaf(ug[e], x[e] * r, dgp[j][q * E + e]);
                        }
                    }
                    // one output row at a time
#pragma unroll
                    for (int i = 0; i < N; ++i) {
                        uint32_t oh[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            float h[E], o[E];
                            unpack_word<S>(word(rh[i][j], q), h);
#pragma unroll
                            for (int e = 0; e < E; ++e) {
                                da[i] = fmaf(dx[q * E + e], h[e], da[i]);
                                o[e] = alpha[i] * dx[q * E + e];
                            }
                            if constexpr (!HG) continue;
                            if (!FOLD && dH_in) {
                                float p[E];
                                unpack_word<S>(word(rin[i][j], q), p);
#pragma unroll
                                for (int e = 0; e < E; ++e) o[e] += p[e];
                            } else if constexpr (FOLD) {
                                // + sum_k A[k][i] dH'_k, formed as the write-back's
                                // gradient forms it, then one rounding
                                float g[N][E];
#pragma unroll
                                for (int k = 0; k < N; ++k) unpack_word<S>(word(rin[k][j], q), g[k]);
#pragma unroll
                                for (int e = 0; e < E; ++e) {
                                    float sum = A[0][i] * g[0][e];
#pragma unroll
                                    for (int k = 1; k < N; ++k) sum = fmaf(A[k][i], g[k][e], sum);
                                    o[e] = fmaf(alpha[i], dx[q * E + e], sum);
                                }
                            }
                            oh[q] = pack_word<S>(o);
                        }
                        if constexpr (HG)
                            st16_stream(dH + r0 + i * row_bytes + v * 16, make_uint4(oh[0], oh[1], oh[2], oh[3]));
                    }
                }
            }
            if constexpr (PER_TOKEN) {
                // per-wave sums, no workgroup barrier: token_records_kernel
                // adds the waves' partials in wave order, the order a
                // workgroup reduction would take
                const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = B >> 6;
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    const float v = wave_sum(da[i]);
                    if (lane == 0) da_part[(t * nw + wave) * N + i] = v;
                }
            } else {
#pragma unroll
                for (int i = 0; i < N; ++i) dab[i] += da[i];
            }
        }
        // the block's partials: dgamma of its columns (unless not asked for),
        // dalpha (shared record)
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec && dg_part) {
#pragma unroll
                for (int q = 0; q < V / 4; ++q)
                    st16(dg_part + blk * (int64_t)d + v * V + 4 * q,
                         make_uint4(__float_as_uint(dgp[j][4 * q]), __float_as_uint(dgp[j][4 * q + 1]),
                                    __float_as_uint(dgp[j][4 * q + 2]), __float_as_uint(dgp[j][4 * q + 3])));
            }
        }
        if constexpr (!PER_TOKEN) {
            block_sum_vec<N>(dab, red);
            if (threadIdx.x < N) {
                float val = 0.0f;
#pragma unroll
                for (int i = 0; i < N; ++i)
                    if ((int)threadIdx.x == i) val = dab[i];
                da_part[blk * N + threadIdx.x] = val;
            }
        }
    }
}

// ------------------------------------------------ layer boundary backward

// The gradient of hc_post_pre_mix (one layer's write-back and the next
// layer's read-mix + RMSNorm) in one pass.  Per token, with beta and A from
// w and alpha from wn:
//   H' = A H + beta F, recomputed in the forward's order and rounded as it
//     is stored, so bitwise the H' that the forward wrote (not read back);
//   x = sum_i alpha_i H'_i, r and dx as in pre_bwd_kernel;
//   G_i = dHo_i + alpha_i dx, the whole gradient at H' (the next layer's
//     write-back sends dHo), in fp32 registers only;
//   dH_j = sum_i A[i][j] G_i and dF = sum_i beta_i G_i, the rows written;
//   dalpha_i = dx . H'_i, dbeta_i = G_i . F, dA[i][j] = G_i . H_j and
//   dgamma = sum_t du x r.
// Rows per token: H, F, dHo and du in, dH and dF out (3n + 3), against
// 5n + 3 for post_bwd_kernel without dH followed by pre_bwd_kernel with the
// fold, which also read the stored H' and read dHo twice.
//
// Record partials come in record order [dalpha | dbeta | dA] (K values).
// PER_TOKEN: per token and wave, rpart[t][wave][K], added in wave order by
// boundary_records_kernel (no block reduction per token).  Otherwise summed
// over the block's tokens in registers: dalpha to rpart[blk][n], the rest to
// rpart[nb * n + blk * M] (nb blocks, M = n + n^2).
//
// WT (with per-token records produced from H' by the weight producer): the
// producer's share of the gradient at H' is added to G as well,
//   G_i += a_i dhbar + b_i H'_i,
// from dhb [T][d] fp32 (dhbar = W^T dz) and coef [T][2n] = (a_i | b_i), which
// the weight producer's gradient pass wrote instead of a dH row per stream
// (hc_weights_bwd.hip); H'_i is the recomputed H' already in hand.
template <int N, typename S, int VPT, bool PER_TOKEN, bool WT = false>
__global__ __launch_bounds__(1024) void post_pre_bwd_kernel(
    const uint8_t* __restrict__ dHo, const uint8_t* __restrict__ du, const uint8_t* __restrict__ H,
    const uint8_t* __restrict__ F, const float* __restrict__ w, const float* __restrict__ wn,
    int64_t w_stride, const float* __restrict__ gamma, float eps, uint8_t* __restrict__ dH,
    uint8_t* __restrict__ dF, float* __restrict__ dg_part, float* __restrict__ rpart, int64_t T,
    int d, int group, const float* __restrict__ dhb, const float* __restrict__ coef) {
    constexpr int V = Store<S>::kElems, E = Word<S>::kElems;
    constexpr int DV = V / 4;               // 16-byte vectors of dhbar per stream vector
    constexpr int K = 2 * N + N * N;
    constexpr int M = N + N * N;
    __shared__ float red[16 * 24];          // block_sum_vec<2> and block_sum_to<K>
    // With one vector per thread the rounded H' waits for the second phase in
    // dynamic LDS, [wave][stream][word][lane] (16 n bytes per thread; each
    // thread reads back only what it wrote, so no barrier; a wave's accesses
    // are consecutive words, and the offsets are constants): at n = 4 that
    // keeps the kernel within 128 VGPRs.  With more vectors per thread it
    // stays in registers.
    constexpr bool kLds = VPT == 1;
    extern __shared__ uint32_t hol[];
    uint32_t* const hl = hol + (threadIdx.x >> 6) * (N * 4 * 64) + (threadIdx.x & 63);
    const int B = blockDim.x;
    // WT with one vector per thread: dhbar waits for the second phase in the
    // same way, after the whole block's H' ([wave][element][lane], V words
    // per thread)
    uint32_t* const dl = hol + (B >> 6) * (N * 4 * 64) + (threadIdx.x >> 6) * (V * 64) + (threadIdx.x & 63);
    const int nvec = d / V;
    const int64_t row_bytes = (int64_t)d * Store<S>::kBytes;
    const int wave = threadIdx.x >> 6, nw = B >> 6;

    // tokens blk, blk + nb, ... as in the other gradient kernels
    const int64_t nb = (T + group - 1) / group;
    for (int64_t blk = blockIdx.x; blk < nb; blk += gridDim.x) {
        float dgp[VPT][V];
#pragma unroll
        for (int j = 0; j < VPT; ++j)
#pragma unroll
            for (int e = 0; e < V; ++e) dgp[j][e] = 0.0f;
        float acc[K];
#pragma unroll
        for (int m = 0; m < K; ++m) acc[m] = 0.0f;

        for (int64_t t = blk; t < T; t += nb) {
            const float* rec = w + t * w_stride;
            const float* recn = wn + t * w_stride;
            float alpha[N], beta[N], A[N][N];
#pragma unroll
            for (int i = 0; i < N; ++i) {
                alpha[i] = recn[i];
                beta[i] = rec[N + i];
            }
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int k = 0; k < N; ++k) A[i][k] = rec[2 * N + i * N + k];
            float ca[N], cb[N];
            if constexpr (WT) {
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    ca[i] = coef[t * 2 * N + i];
                    cb[i] = coef[t * 2 * N + N + i];
                }
            }
            const int64_t r0 = t * N * row_bytes;
            // every load of the token first
            uint4 rh[N][VPT], rg[N][VPT], rf[VPT], ru[VPT], rd[VPT][WT ? DV : 1];
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int v = threadIdx.x + j * B;
                const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < N; ++i)
                    rh[i][j] = v < nvec ? ld16_stream(H + r0 + i * row_bytes + v * 16) : z;
                rf[j] = v < nvec ? ld16_stream(F + t * row_bytes + v * 16) : z;
#pragma unroll
                for (int i = 0; i < N; ++i)
                    rg[i][j] = v < nvec ? ld16_stream(dHo + r0 + i * row_bytes + v * 16) : z;
                ru[j] = v < nvec ? ld16_stream(du + t * row_bytes + v * 16) : z;
                if constexpr (WT) {
#pragma unroll
                    for (int q = 0; q < DV; ++q)
                        rd[j][q] = v < nvec ? ld16_stream(reinterpret_cast<const uint8_t*>(dhb + t * d + v * V) + 16 * q) : z;
                }
            }
            // H' as the forward stores it, and the RMSNorm gradient's two sums
            uint4 ro[N][VPT];
            float s2[2] = {0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int v = threadIdx.x + j * B;
                uint32_t o[N][4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float h[N][E], f[E];
#pragma unroll
                    for (int i = 0; i < N; ++i) unpack_word<S>(word(rh[i][j], q), h[i]);
                    unpack_word<S>(word(rf[j], q), f);
#pragma unroll
                    for (int i = 0; i < N; ++i) {
                        float y[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            float sum = A[i][0] * h[0][e];
#pragma unroll
                            for (int k = 1; k < N; ++k) sum = fmaf(A[i][k], h[k][e], sum);
                            y[e] = fmaf(beta[i], f[e], sum);
                        }
                        o[i][q] = pack_word<S>(y);
                    }
                }
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    if constexpr (kLds) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) hl[(i * 4 + q) * 64] = o[i][q];
                    } else {
                        ro[i][j] = make_uint4(o[i][0], o[i][1], o[i][2], o[i][3]);
                    }
                }
                if constexpr (WT && kLds) {
#pragma unroll
                    for (int el = 0; el < V; ++el) dl[el * 64] = word(rd[j][el / 4], el % 4);
                }
                if (v < nvec) {
                    float g[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if ((q * E) % 4 == 0) unpack<f32_t>(ld16(gamma + v * V + q * E), g);
                        float x[E], yr[E], ug[E];
                        unpack_word<S>(o[0][q], yr);
#pragma unroll
                        for (int e = 0; e < E; ++e) x[e] = alpha[0] * yr[e];
#pragma unroll
                        for (int i = 1; i < N; ++i) {
                            unpack_word<S>(o[i][q], yr);
#pragma unroll
                            for (int e = 0; e < E; ++e) x[e] = fmaf(alpha[i], yr[e], x[e]);
                        }
                        unpack_word<S>(word(ru[j], q), ug);
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            s2[0] = fmaf(x[e], x[e], s2[0]);
                            s2[1] = fmaf(g[(q * E) % 4 + e] * ug[e], x[e], s2[1]);
                        }
                    }
                }
            }
            block_sum_vec<2>(s2, red);
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    opaque(rh[i][j]);
                    opaque(rg[i][j]);
                    if constexpr (!kLds) opaque(ro[i][j]);
                }
                opaque(rf[j]);
                opaque(ru[j]);
                if constexpr (WT && !kLds) {
#pragma unroll
                    for (int q = 0; q < DV; ++q) opaque(rd[j][q]);
                }
            }
            const float r = 1.0f / sqrtf(s2[0] / (float)d + eps);
            const float c2 = r * r * s2[1] / (float)d;
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int v = threadIdx.x + j * B;
                if (v < nvec) {
                    float g[4];
                    uint32_t oh[N][4], of[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if ((q * E) % 4 == 0) unpack<f32_t>(ld16(gamma + v * V + q * E), g);
                        float h[N][E], ho[N][E], gr[N][E], f[E], ug[E];
#pragma unroll
                        for (int i = 0; i < N; ++i) {
                            unpack_word<S>(word(rh[i][j], q), h[i]);
                            unpack_word<S>(kLds ? hl[(i * 4 + q) * 64] : word(ro[i][j], q), ho[i]);
                            unpack_word<S>(word(rg[i][j], q), gr[i]);
                        }
                        unpack_word<S>(word(rf[j], q), f);
                        unpack_word<S>(word(ru[j], q), ug);
                        float o[N][E], ofe[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            float x = alpha[0] * ho[0][e];
#pragma unroll
                            for (int i = 1; i < N; ++i) x = fmaf(alpha[i], ho[i][e], x);
                            const float dx = r * (g[(q * E) % 4 + e] * ug[e] - x * c2);
                            dgp[j][q * E + e] = fmaf(ug[e], x * r, dgp[j][q * E + e]);
                            float G[N];
#pragma unroll
                            for (int i = 0; i < N; ++i) {
                                acc[i] = fmaf(dx, ho[i][e], acc[i]);
                                G[i] = fmaf(alpha[i], dx, gr[i][e]);
                                if constexpr (WT) {
                                    const int el = q * E + e;          // element of the vector
                                    const float hd = __uint_as_float(
                                        kLds ? dl[el * 64] : word(rd[j][(el / 4) % DV], el % 4));
                                    G[i] = fmaf(cb[i], ho[i][e], fmaf(ca[i], hd, G[i]));
                                }
                                acc[N + i] = fmaf(G[i], f[e], acc[N + i]);
#pragma unroll
                                for (int k = 0; k < N; ++k)
                                    acc[2 * N + i * N + k] = fmaf(G[i], h[k][e], acc[2 * N + i * N + k]);
                            }
#pragma unroll
                            for (int k = 0; k < N; ++k) {
                                float sum = A[0][k] * G[0];
#pragma unroll
                                for (int i = 1; i < N; ++i) sum = fmaf(A[i][k], G[i], sum);
                                o[k][e] = sum;
                            }
                            float sum = beta[0] * G[0];
#pragma unroll
                            for (int i = 1; i < N; ++i) sum = fmaf(beta[i], G[i], sum);
                            ofe[e] = sum;
                        }
#pragma unroll
                        for (int k = 0; k < N; ++k) oh[k][q] = pack_word<S>(o[k]);
                        of[q] = pack_word<S>(ofe);
                    }
#pragma unroll
                    for (int k = 0; k < N; ++k)
                        st16_stream(dH + r0 + k * row_bytes + v * 16,
                                    make_uint4(oh[k][0], oh[k][1], oh[k][2], oh[k][3]));
                    st16_stream(dF + t * row_bytes + v * 16, make_uint4(of[0], of[1], of[2], of[3]));
                }
            }
            if constexpr (PER_TOKEN) {
                wave_sums_to<K>(acc, rpart + (t * nw + wave) * K);
#pragma unroll
                for (int m = 0; m < K; ++m) acc[m] = 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
#pragma unroll
                for (int q = 0; q < V / 4; ++q)
                    st16(dg_part + blk * (int64_t)d + v * V + 4 * q,
                         make_uint4(__float_as_uint(dgp[j][4 * q]), __float_as_uint(dgp[j][4 * q + 1]),
                                    __float_as_uint(dgp[j][4 * q + 2]), __float_as_uint(dgp[j][4 * q + 3])));
            }
        }
        if constexpr (!PER_TOKEN) {
            const float sum = block_sum_to<K>(acc, red);
            const int m = threadIdx.x;
            if (m < N) rpart[blk * N + m] = sum;
            else if (m < K) rpart[nb * N + blk * M + (m - N)] = sum;
        }
    }
}

// One level of a column sum: out[s][c] = sum of in[r][c] over the rows r of
// segment s (kSumRows rows each), in row order; a thread per column.  The
// final level of a sum may also clear `zero` (nzero floats: record entries
// that the gradient leaves at 0).
struct SumLevel {
    const float* in;
    int64_t rows;
    int cols;
    float* out;
    float* zero;
    int nzero;
};

// Up to three independent sums per launch (blockIdx.z picks one), so that the
// short sums of a backward call share launches.
__global__ __launch_bounds__(256) void sum_rows_kernel(SumLevel a, SumLevel b, SumLevel c) {
    const SumLevel& j = blockIdx.z == 0 ? a : blockIdx.z == 1 ? b : c;
    if (blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < j.nzero; i += 256) j.zero[i] = 0.0f;
    const int64_t r0 = (int64_t)blockIdx.y * kSumRows;
    if (r0 >= j.rows) return;
    const int64_t r1 = r0 + kSumRows < j.rows ? r0 + kSumRows : j.rows;
    for (int c = blockIdx.x * 256 + threadIdx.x; c < j.cols; c += gridDim.x * 256) {
        float s = 0.0f;
#pragma unroll 8
        for (int64_t r = r0; r < r1; ++r) s += j.in[r * j.cols + c];
        j.out[(int64_t)blockIdx.y * j.cols + c] = s;
    }
}

// out[c] = sum_t rec[t * K + c] for c < K: one 1024-thread block per column,
// a strided per-thread sum in token order, then the block reduction.
__global__ __launch_bounds__(1024) void sum_records_kernel(const float* __restrict__ rec, int64_t T,
                                                           int K, float* __restrict__ out) {
    __shared__ float red[16];
    const int c = blockIdx.x;
    // eight independent partial sums keep eight loads in flight per thread;
    // they are combined in a fixed order
    float p[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = 0.0f;
    int64_t t = threadIdx.x;
    for (; t + 7 * 1024 < T; t += 8 * 1024) {
#pragma unroll
        for (int k = 0; k < 8; ++k) p[k] += rec[(t + k * 1024) * K + c];
    }
#pragma unroll
    for (int k = 0; k < 7; ++k)
        if (t + k * 1024 < T) p[k] += rec[(t + k * 1024) * K + c];
    float s = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    s = block_sum(s, red);
    if (threadIdx.x == 0) out[c] = s;
}

// dw[t][c] = sum over the nw waves of part[t][w][c] (c < n, in wave order),
// 0 for c >= n: pre's per-token records from its per-wave partials.
__global__ __launch_bounds__(256) void token_records_kernel(const float* __restrict__ part, int nw,
                                                            int n, int K, int64_t T,
                                                            float* __restrict__ dw) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < T * K;
         e += (int64_t)gridDim.x * 256) {
        const int64_t t = e / K;
        const int c = (int)(e % K);
        float s = 0.0f;
        if (c < n) {
            const float* p = part + t * nw * n + c;
            s = p[0];
            for (int w = 1; w < nw; ++w) s += p[w * n];
        }
        dw[e] = s;
    }
}

// The layer boundary's per-token records from its per-wave partials
// part[t][wave][K] (added in wave order): dw[t] = [0 | dbeta | dA] for the
// write-back's records, dwn[t] = [dalpha | 0 | 0] for the read-mix's.
__global__ __launch_bounds__(256) void boundary_records_kernel(const float* __restrict__ part,
                                                               int nw, int n, int K, int64_t T,
                                                               float* __restrict__ dw,
                                                               float* __restrict__ dwn) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < T * K;
         e += (int64_t)gridDim.x * 256) {
        const int64_t t = e / K;
        const int c = (int)(e % K);
        const float* p = part + t * nw * K + c;
        float s = p[0];
        for (int w = 1; w < nw; ++w) s += p[w * K];
        dw[e] = c < n ? 0.0f : s;
        dwn[e] = c < n ? s : 0.0f;
    }
}

// ----------------------------------------------------------------- dispatch

inline dim3 grid_of(int64_t blocks) { return dim3((unsigned)(blocks < kMaxGridB ? blocks : kMaxGridB)); }

}  // namespace

// Deterministic column sums, up to three at once: every level folds kSumRows
// rows into one (rows -> ceil(rows / 64) rows in tmp -> ... -> out), so the
// order depends only on the shapes.  Each job's tmp holds
// sum_rows_tmp_floats(rows, cols) floats; the jobs' levels share launches.
hipError_t launch_sum_rows(const SumJob* jobs, int njobs, hipStream_t s) {
    constexpr int kJobs = 3;
    if (njobs < 1 || njobs > kJobs) return hipErrorInvalidValue;
    SumJob j[kJobs];
    bool done[kJobs];
    for (int k = 0; k < kJobs; ++k) {
        j[k] = jobs[k < njobs ? k : 0];
        done[k] = k >= njobs;
    }
    while (!(done[0] && done[1] && done[2])) {
        SumLevel lv[kJobs];
        int idx[kJobs], nz = 0;
        unsigned gx = 1, gy = 1;
        for (int k = 0; k < kJobs; ++k) {
            if (done[k]) continue;
            const int64_t segs = (j[k].rows + kSumRows - 1) / kSumRows;
            const bool last = segs <= 1;
            lv[nz] = {j[k].in, j[k].rows, j[k].cols, last ? j[k].out : j[k].tmp,
                      last ? j[k].zero : nullptr, last ? j[k].nzero : 0};
            idx[nz++] = k;
            const unsigned x = (unsigned)((j[k].cols + 255) / 256), y = (unsigned)(segs > 1 ? segs : 1);
            gx = x > gx ? x : gx;
            gy = y > gy ? y : gy;
        }
        hipError_t e = launch(sum_rows_kernel, dim3(gx, gy, (unsigned)nz), dim3(256), 0, s, lv[0],
                              nz > 1 ? lv[1] : lv[0], nz > 2 ? lv[2] : lv[0]);
        if (e != hipSuccess) return e;
        for (int q = 0; q < nz; ++q) {
            SumJob& x = j[idx[q]];
            const int64_t segs = (x.rows + kSumRows - 1) / kSumRows;
            if (segs <= 1) {
                done[idx[q]] = true;
            } else {
                x.in = x.tmp;
                x.rows = segs;
                x.tmp += segs * x.cols;
            }
        }
    }
    return hipSuccess;
}

namespace {

// Per-token records: post's gradient runs fastest with at most 16 waves per
// CU, two 512-thread workgroups, held there by an LDS request (160 KiB per
// CU) that the kernel does not use.  Measured at 16384 tokens, n = 4, d =
// 4096 bf16: two workgroups per CU 240.0 us, three (the register limit)
// 248.7, one 267.0, four 262.6; shared records showed no difference.
inline size_t post_token_lds(int block) {
    const int per_cu = 16 / (block / 64);
    return per_cu >= 2 ? (size_t)(160 * 1024) / (per_cu + 1) + 1024 : 0;
}

template <int N, typename S, int VPT, bool HG>
hipError_t post_bwd_go2(RowCfg c, const void* dHo, const void* H, const void* F, const float* w,
                        int64_t ws, void* dH, void* dF, float* dw, float* part, int64_t T, int d,
                        int group, hipStream_t s) {
    const dim3 grid = grid_of((T + group - 1) / group);
    if (ws != 0)
        return launch(post_bwd_kernel<N, S, VPT, true, HG>, grid, dim3(c.block),
                      post_token_lds(c.block), s,
                      static_cast<const uint8_t*>(dHo), static_cast<const uint8_t*>(H),
                      static_cast<const uint8_t*>(F), w, ws, static_cast<uint8_t*>(dH),
                      static_cast<uint8_t*>(dF), dw, part, T, d, group);
    return launch(post_bwd_kernel<N, S, VPT, false, HG>, grid, dim3(c.block), 0, s,
                  static_cast<const uint8_t*>(dHo), static_cast<const uint8_t*>(H),
                  static_cast<const uint8_t*>(F), w, ws, static_cast<uint8_t*>(dH),
                  static_cast<uint8_t*>(dF), dw, part, T, d, group);
}

template <int N, typename S, int VPT>
hipError_t post_bwd_go(RowCfg c, const void* dHo, const void* H, const void* F, const float* w,
                       int64_t ws, void* dH, void* dF, float* dw, float* part, int64_t T, int d,
                       int group, hipStream_t s) {
    return dH ? post_bwd_go2<N, S, VPT, true>(c, dHo, H, F, w, ws, dH, dF, dw, part, T, d, group, s)
              : post_bwd_go2<N, S, VPT, false>(c, dHo, H, F, w, ws, dH, dF, dw, part, T, d, group, s);
}

template <int N, typename S, int VPT, bool FOLD, bool HG = true>
hipError_t pre_bwd_go2(RowCfg c, const void* du, const void* H, const float* w, int64_t ws,
                       const float* gamma, float eps, const void* dH_in, const void* dHo, void* dH,
                       float* dw, float* dg_part, float* da_part, int64_t T, int d, int group,
                       hipStream_t s) {
    const dim3 grid = grid_of((T + group - 1) / group);
    if (ws != 0)
        return launch(pre_bwd_kernel<N, S, VPT, true, FOLD, HG>, grid, dim3(c.block), 0, s,
                      static_cast<const uint8_t*>(du), static_cast<const uint8_t*>(H), w, ws, gamma,
                      eps, static_cast<const uint8_t*>(dH_in), static_cast<const uint8_t*>(dHo),
                      static_cast<uint8_t*>(dH), dw, dg_part, da_part, T, d, group);
    return launch(pre_bwd_kernel<N, S, VPT, false, FOLD, HG>, grid, dim3(c.block), 0, s,
                  static_cast<const uint8_t*>(du), static_cast<const uint8_t*>(H), w, ws, gamma,
                  eps, static_cast<const uint8_t*>(dH_in), static_cast<const uint8_t*>(dHo),
                  static_cast<uint8_t*>(dH), dw, dg_part, da_part, T, d, group);
}

template <int N, typename S, int VPT>
hipError_t pre_bwd_go(RowCfg c, const void* du, const void* H, const float* w, int64_t ws,
                      const float* gamma, float eps, const void* dH_in, const void* dHo, void* dH,
                      float* dw, float* dg_part, float* da_part, int64_t T, int d, int group,
                      hipStream_t s) {
    if (!dH)   // records and dgamma only (no addend: the API checks)
        return pre_bwd_go2<N, S, VPT, false, false>(c, du, H, w, ws, gamma, eps, nullptr, nullptr,
                                                    nullptr, dw, dg_part, da_part, T, d, group, s);
    return dHo ? pre_bwd_go2<N, S, VPT, true>(c, du, H, w, ws, gamma, eps, dH_in, dHo, dH, dw, dg_part,
                                               da_part, T, d, group, s)
               : pre_bwd_go2<N, S, VPT, false>(c, du, H, w, ws, gamma, eps, dH_in, dHo, dH, dw, dg_part,
                                                da_part, T, d, group, s);
}

#define HC_BWD_VPT(FN, ...)                                  \
    switch (c.vpt) {                                         \
        case 1: return FN<N, S, 1>(c, __VA_ARGS__);          \
        case 2: return FN<N, S, 2>(c, __VA_ARGS__);          \
        case 3: return FN<N, S, 3>(c, __VA_ARGS__);          \
        case 4: return FN<N, S, 4>(c, __VA_ARGS__);          \
    }                                                        \
    return hipErrorInvalidConfiguration;

template <int N, typename S>
hipError_t post_bwd_vpt(RowCfg c, const void* dHo, const void* H, const void* F, const float* w,
                        int64_t ws, void* dH, void* dF, float* dw, float* part, int64_t T, int d,
                        int group, hipStream_t s) {
    HC_BWD_VPT(post_bwd_go, dHo, H, F, w, ws, dH, dF, dw, part, T, d, group, s)
}

template <int N, typename S>
hipError_t pre_bwd_vpt(RowCfg c, const void* du, const void* H, const float* w, int64_t ws,
                       const float* gamma, float eps, const void* dH_in, const void* dHo, void* dH,
                       float* dw, float* dg_part, float* da_part, int64_t T, int d, int group,
                       hipStream_t s) {
    HC_BWD_VPT(pre_bwd_go, du, H, w, ws, gamma, eps, dH_in, dHo, dH, dw, dg_part, da_part, T, d, group,
               s)
}
template <int N, typename S, int VPT>
hipError_t post_pre_bwd_go(RowCfg c, const void* dHo, const void* du, const void* H, const void* F,
                           const float* w, const float* wn, int64_t ws, const float* gamma,
                           float eps, void* dH, void* dF, float* dg_part, float* rpart, int64_t T,
                           int d, int group, const float* dhb, const float* coef, hipStream_t s) {
    const dim3 grid = grid_of((T + group - 1) / group);
    // the weight producer's terms come only with per-token records
    auto* k = dhb ? post_pre_bwd_kernel<N, S, VPT, true, true>
              : ws != 0 ? post_pre_bwd_kernel<N, S, VPT, true> : post_pre_bwd_kernel<N, S, VPT, false>;
    // the parked H', and with the producer's terms dhbar (V floats per thread)
    const size_t lds = VPT == 1 ? ((size_t)N * 16 + (dhb ? Store<S>::kElems * 4 : 0)) * c.block : 0;
    return launch(k, grid, dim3(c.block), lds, s, static_cast<const uint8_t*>(dHo),
                  static_cast<const uint8_t*>(du), static_cast<const uint8_t*>(H),
                  static_cast<const uint8_t*>(F), w, wn, ws, gamma, eps, static_cast<uint8_t*>(dH),
                  static_cast<uint8_t*>(dF), dg_part, rpart, T, d, group, dhb, coef);
}

template <int N, typename S>
hipError_t post_pre_bwd_vpt(RowCfg c, const void* dHo, const void* du, const void* H, const void* F,
                            const float* w, const float* wn, int64_t ws, const float* gamma,
                            float eps, void* dH, void* dF, float* dg_part, float* rpart, int64_t T,
                            int d, int group, const float* dhb, const float* coef, hipStream_t s) {
    HC_BWD_VPT(post_pre_bwd_go, dHo, du, H, F, w, wn, ws, gamma, eps, dH, dF, dg_part, rpart, T, d,
               group, dhb, coef, s)
}
#undef HC_BWD_VPT

template <typename S, typename... A>
hipError_t post_bwd_n(int n, A... a) {
    switch (n) {
        case 1: return post_bwd_vpt<1, S>(a...);
        case 2: return post_bwd_vpt<2, S>(a...);
        case 3: return post_bwd_vpt<3, S>(a...);
        case 4: return post_bwd_vpt<4, S>(a...);
    }
    return hipErrorInvalidValue;
}

template <typename S, typename... A>
hipError_t post_pre_bwd_n(int n, A... a) {
    switch (n) {
        case 1: return post_pre_bwd_vpt<1, S>(a...);
        case 2: return post_pre_bwd_vpt<2, S>(a...);
        case 3: return post_pre_bwd_vpt<3, S>(a...);
        case 4: return post_pre_bwd_vpt<4, S>(a...);
    }
    return hipErrorInvalidValue;
}

template <typename S, typename... A>
hipError_t pre_bwd_n(int n, A... a) {
    switch (n) {
        case 1: return pre_bwd_vpt<1, S>(a...);
        case 2: return pre_bwd_vpt<2, S>(a...);
        case 3: return pre_bwd_vpt<3, S>(a...);
        case 4: return pre_bwd_vpt<4, S>(a...);
    }
    return hipErrorInvalidValue;
}

// Workspace layout for T tokens of width d with n streams (floats), shared
// by every gradient call here:
//   [rows][d]   dgamma partials         (rows = blocks = ceil(T / group))
//   [rr][K]     record partials         (post: M = n + n^2 per row; pre: n;
//               the layer boundary: n and M, K = 2n + n^2 in all)
//   tmp         the levels of the dgamma sum (sum_rows_tmp_floats(rows, d))
//   tmp2        the levels of the record sums (sum_rows_tmp_floats(rr, K):
//               the floats it needs grow linearly with the columns)
//   wp          per-token, per-wave partials (T x 16 waves x K at most)
struct BwdSpace {
    int64_t rows, prows, dg, rec, tmp, tmp2, wp, total;   // offsets and total, in floats
};
inline BwdSpace bwd_space(int64_t T, int n, int d) {
    BwdSpace b;
    const int64_t g = group_of(T);
    b.rows = (T + g - 1) / g;
    const int64_t K = 2 * n + int64_t(n) * n;
    b.dg = 0;
    b.rec = b.rows * d;
    const int64_t pg = post_group_of(T);
    b.prows = (T + pg - 1) / pg;                          // post's partial records
    const int64_t rr = b.prows > b.rows ? b.prows : b.rows;
    b.tmp = b.rec + rr * K;                               // the dgamma sum's levels
    b.tmp2 = b.tmp + sum_rows_tmp_floats(b.rows, d);      // the record sums' levels
    b.wp = b.tmp2 + sum_rows_tmp_floats(rr, K);           // per-token, per-wave partials
    b.total = b.wp + T * 16 * K;
    return b;
}

}  // namespace

int64_t backward_workspace_bytes(int64_t T, int n, int d) {
    if (T <= 0 || d <= 0 || n <= 0) return 0;
    return bwd_space(T, n, d).total * 4;
}

namespace {

// Post's gradient with its scratch given as two regions: the per-block
// partial records (`part`, prows x M floats) and the levels of their sum
// (`tmp`); both unused with per-token records.
hipError_t post_backward_with(const void* dHo, const void* H, const void* F, const float* w,
                              int64_t w_stride, void* dH, void* dF, float* dw, float* part,
                              float* tmp, int64_t T, int n, int d, int dt, hipStream_t s) {
    const int group = w_stride != 0 ? 1 : (int)post_group_of(T);
    if (w_stride != 0) part = nullptr;
    hipError_t e =
        dt == 0 ? post_bwd_n<f32_t>(n, row_config(d / Store<f32_t>::kElems), dHo, H, F, w, w_stride,
                                    dH, dF, dw, part, T, d, group, s)
                : post_bwd_n<bf16_t>(n, row_config(d / Store<bf16_t>::kElems), dHo, H, F, w, w_stride,
                                     dH, dF, dw, part, T, d, group, s);
    if (e != hipSuccess || w_stride != 0) return e;
    // shared record: dw = [0 (dalpha) | sum of the block partials]
    const int M = n + n * n;
    const int64_t prows = (T + post_group_of(T) - 1) / post_group_of(T);
    const SumJob job = {part, prows, M, tmp, dw + n, dw, n};
    return launch_sum_rows(&job, 1, s);
}

// The allocation-free variant's scratch: one array per GPU for the life of
// the process, shared by every call on that GPU (calls that overlap on one
// GPU race for it).  Host code never passes the array's name to a kernel
// (in host code it is a host-side stand-in, not a device address); it
// passes the device address that hipGetSymbolAddress returns for the
// current device, looked up once per device.
constexpr int64_t kScratchBytes = int64_t(1) << 20;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

hipError_t scratch_on_current_device(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *out = static_cast<float*>(g_scratch_ptr[dev]);
    return hipSuccess;
}

}  // namespace

hipError_t launch_post_mix_backward(const void* dHo, const void* H, const void* F, const float* w,
                                    int64_t w_stride, void* dH, void* dF, float* dw, void* work,
                                    int64_t T, int n, int d, int dt, hipStream_t s) {
    const BwdSpace sp = bwd_space(T, n, d);
    float* ws = static_cast<float*>(work);
    return post_backward_with(dHo, H, F, w, w_stride, dH, dF, dw, ws ? ws + sp.rec : nullptr,
                              ws ? ws + sp.tmp2 : nullptr, T, n, d, dt, s);
}

int64_t post_backward_scratch_bytes(int64_t T, int n) {
    if (T <= 0 || n <= 0) return 0;
    const int64_t M = n + int64_t(n) * n;
    const int64_t prows = (T + post_group_of(T) - 1) / post_group_of(T);
    return (prows * M + sum_rows_tmp_floats(prows, M)) * 4;
}

int64_t post_backward_scratch_max_bytes() { return kScratchBytes; }

hipError_t launch_post_mix_backward_noalloc(const void* dHo, const void* H, const void* F,
                                            const float* w, int64_t w_stride, void* dH, void* dF,
                                            float* dw, int64_t T, int n, int d, int dt, hipStream_t s) {
    float* part = nullptr;
    float* tmp = nullptr;
    if (w_stride == 0) {
        float* base = nullptr;
        const hipError_t e = scratch_on_current_device(&base);
        if (e != hipSuccess) return e;
        const int64_t M = n + int64_t(n) * n;
        const int64_t prows = (T + post_group_of(T) - 1) / post_group_of(T);
        part = base;
        tmp = base + prows * M;
    }
    return post_backward_with(dHo, H, F, w, w_stride, dH, dF, dw, part, tmp, T, n, d, dt, s);
}

hipError_t launch_pre_mix_backward(const void* du, const void* H, const float* w, int64_t w_stride,
                                   const float* gamma, float eps, const void* dH_in, const void* dHo,
                                   void* dH, float* dw, float* dgamma, void* work, int64_t T, int n,
                                   int d, int dt, hipStream_t s) {
    const BwdSpace sp = bwd_space(T, n, d);
    float* ws = static_cast<float*>(work);
    // dalpha alone with per-token records (no dH, no dgamma): no per-block
    // row of partials to keep, so one token per workgroup, as the forward
    // read-mix runs
    const bool alone = !dgamma && w_stride != 0;
    const int group = alone ? 1 : (int)group_of(T);
    float* dg_part = dgamma ? ws + sp.dg : nullptr;
    // dalpha: per-workgroup partials (shared record), or per token and wave
    float* da_part = w_stride != 0 ? ws + sp.wp : ws + sp.rec;
    hipError_t e =
        dt == 0 ? pre_bwd_n<f32_t>(n, row_config(d / Store<f32_t>::kElems), du, H, w, w_stride,
                                   gamma, eps, dH_in, dHo, dH, dw, dg_part, da_part, T, d, group, s)
                : pre_bwd_n<bf16_t>(n, row_config(d / Store<bf16_t>::kElems), du, H, w, w_stride,
                                    gamma, eps, dH_in, dHo, dH, dw, dg_part, da_part, T, d, group, s);
    if (e != hipSuccess) return e;
    const int K = 2 * n + n * n;
    if (w_stride != 0) {
        const int nw = row_config(d / (dt == 0 ? Store<f32_t>::kElems : Store<bf16_t>::kElems)).block / 64;
        const int64_t blocks = (T * K + 255) / 256;
        e = launch(token_records_kernel, grid_of(blocks), dim3(256), 0, s,
                   static_cast<const float*>(da_part), nw, n, K, T, dw);
        if (e != hipSuccess) return e;
    }
    // dgamma; with a shared record also dw = [sum of the dalpha partials |
    // 0 (dbeta, dA)], in the same launches
    const SumJob jobs[2] = {{dg_part, sp.rows, d, ws + sp.tmp, dgamma, nullptr, 0},
                            {da_part, sp.rows, n, ws + sp.tmp2, dw, dw + n, K - n}};
    if (!dgamma)
        return w_stride != 0 ? hipSuccess : launch_sum_rows(jobs + 1, 1, s);
    return launch_sum_rows(jobs, w_stride != 0 ? 1 : 2, s);
}

hipError_t launch_post_pre_mix_backward(const void* dHo, const void* du, const void* H, const void* F,
                                        const float* w, const float* wn, int64_t w_stride,
                                        const float* gamma, float eps, void* dH, void* dF, float* dw,
                                        float* dwn, float* dgamma, void* work, int64_t T, int n,
                                        int d, int dt, hipStream_t s, const float* dhb,
                                        const float* coef) {
    const BwdSpace sp = bwd_space(T, n, d);
    float* ws = static_cast<float*>(work);
    const int group = (int)group_of(T);
    float* dg_part = ws + sp.dg;
    // record partials: per token and wave, or per workgroup
    float* rpart = w_stride != 0 ? ws + sp.wp : ws + sp.rec;
    const RowCfg c = row_config(d / (dt == 0 ? Store<f32_t>::kElems : Store<bf16_t>::kElems));
    hipError_t e =
        dt == 0 ? post_pre_bwd_n<f32_t>(n, c, dHo, du, H, F, w, wn, w_stride, gamma, eps, dH, dF,
                                        dg_part, rpart, T, d, group, dhb, coef, s)
                : post_pre_bwd_n<bf16_t>(n, c, dHo, du, H, F, w, wn, w_stride, gamma, eps, dH, dF,
                                         dg_part, rpart, T, d, group, dhb, coef, s);
    if (e != hipSuccess) return e;
    const int K = 2 * n + n * n, M = n + n * n;
    const SumJob dg_job = {dg_part, sp.rows, d, ws + sp.tmp, dgamma, nullptr, 0};
    if (w_stride != 0) {
        const int64_t blocks = (T * K + 255) / 256;
        e = launch(boundary_records_kernel, grid_of(blocks), dim3(256), 0, s,
                   static_cast<const float*>(rpart), c.block / 64, n, K, T, dw, dwn);
        if (e != hipSuccess) return e;
        return launch_sum_rows(&dg_job, 1, s);
    }
    // shared records: dwn = [sum of the dalpha partials | 0], dw = [0 | sums
    // of the dbeta and dA partials], in the dgamma sum's launches
    const SumJob jobs[3] = {dg_job,
                            {rpart, sp.rows, n, ws + sp.tmp2, dwn, dwn + n, K - n},
                            {rpart + sp.rows * n, sp.rows, M,
                             ws + sp.tmp2 + sum_rows_tmp_floats(sp.rows, n), dw + n, dw, n}};
    return launch_sum_rows(jobs, 3, s);
}

int64_t sum_rows_tmp_floats(int64_t rows, int64_t cols) {
    const int64_t segs = (rows + kSumRows - 1) / kSumRows;
    return 2 * (segs + 1) * cols;
}


hipError_t launch_sum_records(const float* rec, int64_t T, int K, float* out, hipStream_t s) {
    return launch(sum_records_kernel, dim3(K), dim3(1024), 0, s, rec, T, K, out);
}

}  // namespace hc
