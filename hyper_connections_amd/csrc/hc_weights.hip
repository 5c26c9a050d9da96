// hc_weights.hip -- per-token mixing weights: the projection of the
// normalised streams on the matrix cores, tanh, and the Sinkhorn (mHC) step.
//
// Sources: hfviewer.com glossary "Hyper-connections (mHC)", definition (the
// mHC variant makes the stream mixing doubly stochastic with a few Sinkhorn
// iterations); llm-atlas "Tencent Hy4-preview (770B-A49B)", "Architecture
// concepts" (constrained mixing between parallel streams).  The pages give no
// rule for computing weights per token; the reading implemented is
//   r_i = 1/sqrt(mean_k H_ik^2 + eps), hbar = (1/n) sum_i r_i H_i,
//   z = W hbar (W is K x d, K = 2n + n^2),
//   w = w_static + scale * tanh(z)            (sinkhorn_iters == 0)
//   w = mhc(w_static + scale * z)             (sinkhorn_iters  > 0)
// where mhc(l) = [sigmoid(l_alpha) | sigmoid(l_beta) | Sinkhorn(exp(l_A))].
//
// Projection as a GEMM.  Because z is linear in the streams,
//   z_c = (1/n) sum_i r_i P_ic,   P_ic = sum_k H_ik W_ck,
// so the kernel multiplies the raw stream rows (H viewed as a (T*n) x d
// matrix) by W^T on MFMA while the same registers feed the per-row sums of
// squares; r_i is applied in the epilogue.  One HBM pass over H.  bf16 uses
// v_mfma_f32_16x16x32_bf16, FP8 (E4M3 H and W) the same after an exact
// widening to bf16, fp32 v_mfma_f32_16x16x4f32.
//
// Tiling (one wave = 16 matrix rows = 16/n tokens; 4 waves per workgroup):
//  - A operand: the wave's 16 rows.  Lane l supplies row l % 16; its lane
//    group g = l / 16 supplies the k-slice the MFMA assigns to that group.
//    The physical k of every slice is our choice as long as the B operand
//    uses the same one: at step t of half chunk h, group g takes 16-byte
//    slice 16h + 4t + g of the chunk.
//  - Loading the A layout directly would make every load instruction touch
//    16 rows x 64 bytes; loads of 4 rows x 256 contiguous bytes run about
//    12% faster on MI355X.  So the rows are loaded that way and each half
//    chunk passes through a per-wave LDS buffer into the A layout.
//  - B operand: W staged through LDS one k-chunk at a time (shared by the
//    four waves; rows >= K and k >= d are zero).
//  - Both LDS buffers pad their rows by 32 bytes.  With 16 bytes the
//    row-strided 16-byte reads of 16 lanes conflicted: measured on MI355X,
//    bank-conflict cycles were 34% of the LDS active cycles (16 bytes on
//    both), 15% (32 on W only), 26% (32 on the transpose only) and 0.9% (32
//    on both).
//  - C: one 16x16 tile per 16 outputs (two tiles for K = 24).
//  - Epilogue through LDS (the wave's transpose buffer): the C tile and the
//    row sums of squares are combined per token, then tanh or the mHC
//    transform, then stored.
#include <type_traits>

#include "hc_device.h"
#include "hc_launch.h"

namespace hc {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;    // waves per weights workgroup
constexpr int kLV = 8;         // 16-byte vectors per lane per k-chunk
constexpr int64_t kMaxGrid = 1 << 20;

// --------------------------------------------------------------- sinkhorn

// Four lanes per token (lane r owns row r); 64 tokens per 256-thread block.
// Records are staged through LDS so that global traffic is coalesced (a
// record is K floats, K = 3, 8, 15 or 24: not a multiple of 16 bytes).
template <int N>
__global__ __launch_bounds__(256) void sinkhorn_kernel(const float* __restrict__ logits,
                                                       float* __restrict__ w_out, int iters,
                                                       int64_t T) {
    constexpr int K = 2 * N + N * N;
    constexpr int TB = 64;      // tokens per block
    __shared__ float rec[TB * K];
    const int tl = threadIdx.x >> 2, r = threadIdx.x & 3;
    for (int64_t t0 = (int64_t)blockIdx.x * TB; t0 < T; t0 += (int64_t)gridDim.x * TB) {
        const int ntok = (int)((T - t0) < TB ? (T - t0) : TB);
        const float* src = logits + t0 * K;
        for (int e = threadIdx.x; e < ntok * K; e += 256) rec[e] = src[e];
        __syncthreads();
        const bool mine = tl < ntok && r < N;
        float a = 0.0f, b = 0.0f, row[N];
        if (mine) {
            a = rec[tl * K + r];
            b = rec[tl * K + N + r];
        }
#pragma unroll
        for (int j = 0; j < N; ++j) row[j] = mine ? rec[tl * K + 2 * N + r * N + j] : 0.0f;
        mhc_quad<N>(r, a, b, row, iters);
        __syncthreads();
        if (mine) {
            rec[tl * K + r] = a;
            rec[tl * K + N + r] = b;
#pragma unroll
            for (int j = 0; j < N; ++j) rec[tl * K + 2 * N + r * N + j] = row[j];
        }
        __syncthreads();
        float* dst = w_out + t0 * K;
        for (int e = threadIdx.x; e < ntok * K; e += 256) dst[e] = rec[e];
        __syncthreads();
    }
}

// ---------------------------------------------------------------- weights

template <typename S> struct Mfma;
template <> struct Mfma<bf16_t> {
    // one 16-byte vector (8 bf16) is one K = 32 step across the 4 lane groups
    static __device__ __forceinline__ f32x4 step(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<f32_t> {
    // one 16-byte vector (4 fp32) is four K = 4 steps
    static __device__ __forceinline__ f32x4 step(uint4 a, uint4 b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
        return c;
    }
};

template <> struct Mfma<fp8_t> {
    // one 16-byte vector (16 fp8 E4M3) is two K = 32 bf16 steps: every FP8
    // value is exactly a bf16 value, so the operands are widened to bf16
    // (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and multiplied on the bf16
    // matrix path, whose fp32 accumulation matches the other dtypes
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
        const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
        const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
        const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
        const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
        return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
    }
    static __device__ __forceinline__ f32x4 step(uint4 a, uint4 b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(a.x, a.y), widen8(b.x, b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(a.z, a.w), widen8(b.z, b.w), c, 0, 0, 0);
        return c;
    }
};

constexpr int kWThreads = kWaves * 64;

template <int N, typename S>
struct WeightsGeom {
    static constexpr int K = 2 * N + N * N;           // outputs per token
    static constexpr int NT = (K + 15) / 16;          // 16-wide C tiles
    static constexpr int TPW = 16 / N;                // tokens per wave
    static constexpr int V = Store<S>::kElems;        // elements per vector
    static constexpr int KC = 4 * kLV * V;            // k per chunk
    static constexpr int RS = KC * Store<S>::kBytes + 32;  // LDS row pitch (bytes)
    static constexpr int WBYTES = NT * 16 * RS;       // one W chunk in LDS
    static constexpr int PIECES = KC * Store<S>::kBytes / 16;  // 16-byte pieces per W row
    static constexpr int CPITCH = NT * 16 + 1;        // epilogue C row pitch (floats)
    static constexpr int EPI = 16 * CPITCH + 16 + TPW * K;  // floats per wave
    static constexpr int KH = KC * Store<S>::kBytes / 2;     // bytes per row per half chunk
    static constexpr int TP = KH + 32;                // transpose row pitch (bytes)
    static constexpr int TBYTES = 16 * TP;            // transpose buffer per wave
    static_assert(EPI * 4 <= TBYTES, "the epilogue reuses the transpose buffer");
};

// MODE kRecord: the records into w_out.  kRaw: instead of records, the
// per-stream projections P_i = W H_i ([T][n][K] into p_out) and the row norms
// r_i ([T][n] into r_out), the quantities the gradient pass needs.  kSave:
// both (the records, and P and r kept for the gradient pass).
enum WeightsMode { kRecord = 0, kRaw = 1, kSave = 2 };
template <int N, typename S, int MODE>
__global__ __launch_bounds__(kWThreads) void weights_kernel(
    const uint8_t* __restrict__ H, const uint8_t* __restrict__ W, const float* __restrict__ w_static,
    float scale, float eps, int iters, float* __restrict__ w_out, float* __restrict__ p_out,
    float* __restrict__ r_out, int64_t T, int d) {
    using G = WeightsGeom<N, S>;
    constexpr int V = G::V, KC = G::KC, NT = G::NT, K = G::K, TPW = G::TPW;
    constexpr int SB = Store<S>::kBytes;
    __shared__ __attribute__((aligned(16))) uint8_t wlds[G::WBYTES];
    // per wave: the transpose buffer of the stream rows, then the epilogue
    __shared__ __attribute__((aligned(16))) uint8_t tbuf[kWaves * G::TBYTES];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rho = lane & 15, grp = lane >> 4;
    const int64_t row_bytes = (int64_t)d * SB;
    const int nchunks = (d + KC - 1) / KC;
    const int tok_per_block = kWaves * TPW;
    uint8_t* const tb = tbuf + wave * G::TBYTES;
    constexpr int KH = G::KH, TP = G::TP;

    // zero the padding rows (>= K) of the W tile once; chunks never write them
    for (int p = threadIdx.x; p < (NT * 16 - K) * G::PIECES; p += kWThreads) {
        const int r = K + p / G::PIECES, c = p % G::PIECES;
        *reinterpret_cast<uint4*>(wlds + r * G::RS + c * 16) = make_uint4(0, 0, 0, 0);
    }

    for (int64_t b = blockIdx.x; b * tok_per_block < T; b += gridDim.x) {
        const int64_t tok0 = b * tok_per_block + wave * TPW;    // first token of this wave

        f32x4 acc[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        float ss = 0.0f;

        // Stream loads are row-contiguous: load s of a half chunk gives
        // 16 lanes each of rows 4s .. 4s+3 (lane -> row 4s + lane/16, 16-byte
        // piece lane%16), i.e. 256 contiguous bytes per row.  The MFMA A
        // operand wants lane -> row lane%16, so each half chunk is passed
        // through the wave's LDS buffer (rows padded so that the
        // row-strided reads are conflict-free).
        const int lrow = lane >> 4, lpiece = lane & 15;
        for (int c = 0; c < nchunks; ++c) {
            const int k0 = c * KC;
            // fp32 inputs: the chunk's own sums, added to the running ones at
            // its end.  Its MFMA adds 4 products per step (against 32 for
            // bf16 and FP8), so one running sum over a 16384-wide row would
            // take 4096 roundings; the two-level order keeps the error near
            // that of a 128-wide row.  (For bf16 and FP8 the single sum is
            // within the records' tolerance, and the extra registers cost
            // FP8 a wave per SIMD.)
            constexpr bool kTwoLevel = std::is_same<S, f32_t>::value;
            f32x4 cacc[NT];
            float css = 0.0f;
            if constexpr (kTwoLevel) {
#pragma unroll
                for (int q = 0; q < NT; ++q) cacc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            f32x4* const sum = kTwoLevel ? cacc : acc;
            float& sq = kTwoLevel ? css : ss;
            // W chunk pieces first (L2 hits), so that storing them to LDS waits
            // only for these loads and not for the stream loads behind them
            constexpr int WP = (K * G::PIECES + kWThreads - 1) / kWThreads;
            uint4 wv[WP];
#pragma unroll
            for (int i = 0; i < WP; ++i) {
                const int p = threadIdx.x + i * kWThreads;
                const int r = p / G::PIECES, pc = p % G::PIECES;
                const int k = k0 + pc * (16 / SB);
                wv[i] = (p < K * G::PIECES && k < d) ? ld16(W + ((int64_t)r * d + k) * SB)
                                                     : make_uint4(0, 0, 0, 0);
            }
            // this wave's stream rows for the chunk (zero past d, past T and
            // on the padding rows of n = 3)
            uint4 a[kLV];
#pragma unroll
            for (int s = 0; s < kLV; ++s) {
                const int h = s / 4, r = 4 * (s % 4) + lrow;
                const int kb = h * KH + lpiece * 16;                 // byte in the chunk
                const bool ok = r < TPW * N && tok0 + r / N < T && k0 + kb / SB < d;
                a[s] = ok ? ld16_stream(H + (tok0 * N + r) * row_bytes + (int64_t)k0 * SB + kb)
                          : make_uint4(0, 0, 0, 0);
            }
            __syncthreads();   // previous chunk's readers are done
#pragma unroll
            for (int i = 0; i < WP; ++i) {
                const int p = threadIdx.x + i * kWThreads;
                if (p < K * G::PIECES) {
                    const int r = p / G::PIECES, pc = p % G::PIECES;
                    *reinterpret_cast<uint4*>(wlds + r * G::RS + pc * 16) = wv[i];
                }
            }
            __syncthreads();
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // rows of this half chunk into the wave's buffer; LDS
                // operations of one wave complete in order, so the reads
                // below see these writes
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    *reinterpret_cast<uint4*>(tb + (4 * s + lrow) * TP + lpiece * 16) = a[4 * h + s];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int sl = 4 * t + grp;                      // 16-byte slice of the half
                    const uint4 av = *reinterpret_cast<const uint4*>(tb + rho * TP + sl * 16);
                    float f[V];
                    unpack<S>(av, f);
#pragma unroll
                    for (int e = 0; e < V; ++e) sq = fmaf(f[e], f[e], sq);
                    const int kb = h * KH + sl * 16;                 // byte offset in the chunk
#pragma unroll
                    for (int q = 0; q < NT; ++q) {
                        const uint4 bv = *reinterpret_cast<const uint4*>(wlds + (q * 16 + rho) * G::RS + kb);
                        sum[q] = Mfma<S>::step(av, bv, sum[q]);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            if constexpr (kTwoLevel) {
#pragma unroll
                for (int q = 0; q < NT; ++q) acc[q] += cacc[q];
                ss += css;
            }
        }

        // row sums of squares: the 4 lane groups of a row hold partials
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);

        float* E = reinterpret_cast<float*>(tb);
        float* Cs = E;                          // [16][CPITCH]
        float* rs = E + 16 * G::CPITCH;         // [16]
        float* ls = rs + 16;                    // [TPW][K]
#pragma unroll
        for (int q = 0; q < NT; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) Cs[(4 * grp + r) * G::CPITCH + q * 16 + rho] = acc[q][r];
        if (grp == 0) rs[rho] = 1.0f / sqrtf(ss / (float)d + eps);
        __syncthreads();

        if constexpr (MODE != kRecord) {
            for (int o = lane; o < TPW * N * K; o += 64) {
                const int row = o / K, col = o % K;
                if (tok0 + row / N < T) p_out[(tok0 * N + row) * K + col] = Cs[row * G::CPITCH + col];
            }
            if (lane < TPW * N && tok0 + lane / N < T) r_out[tok0 * N + lane] = rs[lane];
        }
        if constexpr (MODE == kRaw) {
            __syncthreads();
            continue;
        }
        for (int o = lane; o < TPW * K; o += 64) {
            const int tl = o / K, col = o % K;
            float z = rs[tl * N] * Cs[(tl * N) * G::CPITCH + col];
#pragma unroll
            for (int i = 1; i < N; ++i) z = fmaf(rs[tl * N + i], Cs[(tl * N + i) * G::CPITCH + col], z);
            z = z / (float)N;
            if (iters == 0) {
                if (tok0 + tl < T) w_out[(tok0 + tl) * K + col] = w_static[col] + scale * tanhf(z);
            } else {
                ls[tl * K + col] = fmaf(scale, z, w_static[col]);
            }
        }
        if (iters > 0) {
            __syncthreads();
            // four lanes per token, lane r owns row r (TPW * 4 <= 64)
            const int tl = lane >> 2, r = lane & 3;
            const bool mine = tl < TPW && tok0 + tl < T && r < N;
            float a = 0.0f, bb = 0.0f, row[N];
            if (mine) {
                a = ls[tl * K + r];
                bb = ls[tl * K + N + r];
            }
#pragma unroll
            for (int j = 0; j < N; ++j) row[j] = mine ? ls[tl * K + 2 * N + r * N + j] : 0.0f;
            mhc_quad<N>(r, a, bb, row, iters);
            if (mine) {
                float* o = w_out + (tok0 + tl) * K;
                o[r] = a;
                o[N + r] = bb;
#pragma unroll
                for (int j = 0; j < N; ++j) o[2 * N + r * N + j] = row[j];
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_sinkhorn(const float* logits, float* w_out, int iters, int64_t T, int n,
                           hipStream_t s) {
    const int64_t blocks = (T + 63) / 64;
    const dim3 grid((unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid));
    switch (n) {
        case 1: return launch(sinkhorn_kernel<1>, grid, dim3(256), 0, s, logits, w_out, iters, T);
        case 2: return launch(sinkhorn_kernel<2>, grid, dim3(256), 0, s, logits, w_out, iters, T);
        case 3: return launch(sinkhorn_kernel<3>, grid, dim3(256), 0, s, logits, w_out, iters, T);
        case 4: return launch(sinkhorn_kernel<4>, grid, dim3(256), 0, s, logits, w_out, iters, T);
    }
    return hipErrorInvalidValue;
}

namespace {
template <int N, typename S>
hipError_t weights_go(const void* H, const void* W, const float* w_static, float scale, float eps,
                      int iters, float* w_out, float* p_out, float* r_out, int64_t T, int d,
                      hipStream_t s) {
    const int64_t per_block = kWaves * WeightsGeom<N, S>::TPW;
    const int64_t blocks = (T + per_block - 1) / per_block;
    const dim3 grid((unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid));
    void (*kernel)(const uint8_t*, const uint8_t*, const float*, float, float, int, float*, float*,
                   float*, int64_t, int) = !p_out ? weights_kernel<N, S, kRecord>
                                           : w_out ? weights_kernel<N, S, kSave>
                                                   : weights_kernel<N, S, kRaw>;
    return launch(kernel, grid, dim3(kWThreads), 0, s, static_cast<const uint8_t*>(H),
                  static_cast<const uint8_t*>(W), w_static, scale, eps, iters, w_out, p_out, r_out, T,
                  d);
}
template <typename S>
hipError_t weights_by_n(int n, const void* H, const void* W, const float* w_static, float scale,
                        float eps, int iters, float* w_out, float* p_out, float* r_out, int64_t T,
                        int d, hipStream_t s) {
    switch (n) {
        case 1: return weights_go<1, S>(H, W, w_static, scale, eps, iters, w_out, p_out, r_out, T, d, s);
        case 2: return weights_go<2, S>(H, W, w_static, scale, eps, iters, w_out, p_out, r_out, T, d, s);
        case 3: return weights_go<3, S>(H, W, w_static, scale, eps, iters, w_out, p_out, r_out, T, d, s);
        case 4: return weights_go<4, S>(H, W, w_static, scale, eps, iters, w_out, p_out, r_out, T, d, s);
    }
    return hipErrorInvalidValue;
}
hipError_t weights_by_dt(int dt, int n, const void* H, const void* W, const float* w_static,
                         float scale, float eps, int iters, float* w_out, float* p_out, float* r_out,
                         int64_t T, int d, hipStream_t s) {
    if (dt == 0) return weights_by_n<f32_t>(n, H, W, w_static, scale, eps, iters, w_out, p_out, r_out, T, d, s);
    if (dt == 2) return weights_by_n<fp8_t>(n, H, W, w_static, scale, eps, iters, w_out, p_out, r_out, T, d, s);
    return weights_by_n<bf16_t>(n, H, W, w_static, scale, eps, iters, w_out, p_out, r_out, T, d, s);
}
}  // namespace

hipError_t launch_weights(const void* H, const void* W, const float* w_static, float scale,
                          float eps, int iters, float* w_out, int64_t T, int n, int d, int dt,
                          hipStream_t s) {
    return weights_by_dt(dt, n, H, W, w_static, scale, eps, iters, w_out, nullptr, nullptr, T, d, s);
}

hipError_t launch_weights_raw(const void* H, const void* W, float eps, float* P, float* r, int64_t T,
                              int n, int d, int dt, hipStream_t s) {
    return weights_by_dt(dt, n, H, W, nullptr, 0.0f, eps, 0, nullptr, P, r, T, d, s);
}

hipError_t launch_weights_save(const void* H, const void* W, const float* w_static, float scale,
                               float eps, int iters, float* w_out, float* P, float* r, int64_t T,
                               int n, int d, int dt, hipStream_t s) {
    return weights_by_dt(dt, n, H, W, w_static, scale, eps, iters, w_out, P, r, T, d, s);
}

}  // namespace hc
