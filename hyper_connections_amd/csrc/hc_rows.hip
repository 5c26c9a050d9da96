// hc_rows.hip -- the streaming kernels of the Hyper-Connections residual path:
// read-mix + RMSNorm (pre), stream-mix + write-back (post), the two fused
// across a layer boundary (post+pre), and the stand-in tanh block.
//
// Sources: hfviewer.com glossary "Hyper-connections (mHC)", definition
// (learned mixing of the parallel streams before and after each block);
// learnaivisually.com "Tencent open-sources Hy4 Preview at 770B -- Identity
// Hyper-Connections", section "Jargon" (residual connection x + f(x),
// pre-norm, identity initialization) and section "What four streams cost per
// token" (the n-fold state handed across every layer boundary is what these
// kernels move).
//
// Design (HBM-bound, 1.9 flop/byte at n = 4 bf16, 3.8 at fp8):
//  - One workgroup per token row; a thread owns VPT 16-byte vectors of the
//    row at positions tid, tid + B, ... (B = blockDim) and the same positions
//    of every stream, so each wave instruction touches 1 KiB of contiguous
//    memory and every HBM byte is read or written exactly once.
//  - All loads of a row are issued before any arithmetic (n*VPT + VPT
//    outstanding 16-byte loads per thread) to keep enough bytes in flight.
//  - The token's weights are wave-uniform and live in scalar registers.
//  - The RMSNorm reduction: per-thread sum in (vector, element) order, wave
//    butterfly, then per-wave partials added in wave order.  The order
//    depends only on d, never on n or the weights.
//  - Results are rounded once, to nearest even, when stored.
#include "hc_device.h"
#include "hc_launch.h"

namespace hc {

namespace {

constexpr int64_t kMaxGrid = 1 << 20;

// ------------------------------------------------------------------- pre

template <int N, typename S, int VPT>
__global__ __launch_bounds__(1024) void pre_mix_kernel(
    const uint8_t* __restrict__ H, const float* __restrict__ w, int64_t w_stride,
    const float* __restrict__ gamma, float eps, uint8_t* __restrict__ u, int64_t T, int d) {
    constexpr int V = Store<S>::kElems, E = Word<S>::kElems;
    __shared__ float red[16];
    const int B = blockDim.x;
    const int nvec = d / V;
    const int64_t row_bytes = (int64_t)d * Store<S>::kBytes;

    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const float* a = w + t * w_stride;
        float alpha[N];
#pragma unroll
        for (int i = 0; i < N; ++i) alpha[i] = a[i];

        const uint8_t* Ht = H + t * N * row_bytes;
        uint4 raw[N][VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
#pragma unroll
                for (int i = 0; i < N; ++i) raw[i][j] = ld16_stream(Ht + i * row_bytes + v * 16);
            }
        }

        float x[VPT][V];
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float h[E];
                    float* xq = &x[j][q * E];
                    unpack_word<S>(word(raw[0][j], q), h);
#pragma unroll
                    for (int e = 0; e < E; ++e) xq[e] = alpha[0] * h[e];
#pragma unroll
                    for (int i = 1; i < N; ++i) {
                        unpack_word<S>(word(raw[i][j], q), h);
#pragma unroll
                        for (int e = 0; e < E; ++e) xq[e] = fmaf(alpha[i], h[e], xq[e]);
                    }
                }
#pragma unroll
                for (int e = 0; e < V; ++e) ss = fmaf(x[j][e], x[j][e], ss);
            }
        }

        float g[VPT][V];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
#pragma unroll
                for (int q = 0; q < V / 4; ++q) {
                    uint4 gv = ld16(gamma + v * V + 4 * q);
                    unpack<f32_t>(gv, &g[j][4 * q]);
                }
            }
        }

        ss = block_sum(ss, red);
        const float r = 1.0f / sqrtf(ss / (float)d + eps);

        uint8_t* ut = u + t * row_bytes;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) o[e] = g[j][e] * (x[j][e] * r);
                st16_stream(ut + v * 16, pack<S>(o));
            }
        }
    }
}

// ------------------------------------------------------------------ post

// H and H_out may be the same buffer: a thread reads every stream at its
// positions before it writes them, and no other thread touches them.
template <int N, typename S, int VPT>
__global__ __launch_bounds__(1024) void post_mix_kernel(
    const uint8_t* H, const uint8_t* __restrict__ F, const float* __restrict__ w,
    int64_t w_stride, uint8_t* H_out, int64_t T, int d) {
    constexpr int V = Store<S>::kElems, E = Word<S>::kElems;
    const int B = blockDim.x;
    const int nvec = d / V;
    const int64_t row_bytes = (int64_t)d * Store<S>::kBytes;

    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const float* rec = w + t * w_stride;
        float beta[N], A[N][N];
#pragma unroll
        for (int i = 0; i < N; ++i) beta[i] = rec[N + i];
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int j = 0; j < N; ++j) A[i][j] = rec[2 * N + i * N + j];

        const uint8_t* Ht = H + t * N * row_bytes;
        const uint8_t* Ft = F + t * row_bytes;
        uint4 rh[N][VPT], rf[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
#pragma unroll
                for (int i = 0; i < N; ++i) rh[i][j] = ld16_stream(Ht + i * row_bytes + v * 16);
                rf[j] = ld16_stream(Ft + v * 16);
            }
        }

        uint8_t* Ot = H_out + t * N * row_bytes;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
                uint32_t o[N][4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {          // dword by dword
                    float h[N][E], f[E];
#pragma unroll
                    for (int i = 0; i < N; ++i) unpack_word<S>(word(rh[i][j], q), h[i]);
                    unpack_word<S>(word(rf[j], q), f);
#pragma unroll
                    for (int i = 0; i < N; ++i) {
                        float y[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            float acc = A[i][0] * h[0][e];
#pragma unroll
                            for (int k = 1; k < N; ++k) acc = fmaf(A[i][k], h[k][e], acc);
                            y[e] = fmaf(beta[i], f[e], acc);
                        }
                        o[i][q] = pack_word<S>(y);
                    }
                }
#pragma unroll
                for (int i = 0; i < N; ++i)
                    st16_stream(Ot + i * row_bytes + v * 16, make_uint4(o[i][0], o[i][1], o[i][2], o[i][3]));
            }
        }
    }
}

// ------------------------------------------------------------- post + pre

// Write-back of layer l fused with the read-mix + RMSNorm of layer l+1.  The
// next layer's input is formed from the rounded H_out values exactly as
// pre_mix_kernel would form it after reading them back, so the fused result
// is bitwise that of the two separate calls.
template <int N, typename S, int VPT>
__global__ __launch_bounds__(1024) void post_pre_mix_kernel(
    const uint8_t* H, const uint8_t* __restrict__ F, const float* __restrict__ w,
    int64_t w_stride, const float* __restrict__ w_next, int64_t w_next_stride,
    const float* __restrict__ gamma, float eps, uint8_t* H_out, uint8_t* __restrict__ u_next,
    int64_t T, int d) {
    constexpr int V = Store<S>::kElems, E = Word<S>::kElems;
    __shared__ float red[16];
    const int B = blockDim.x;
    const int nvec = d / V;
    const int64_t row_bytes = (int64_t)d * Store<S>::kBytes;

    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const float* rec = w + t * w_stride;
        const float* rec_next = w_next + t * w_next_stride;
        float beta[N], A[N][N], alpha[N];
#pragma unroll
        for (int i = 0; i < N; ++i) beta[i] = rec[N + i];
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int j = 0; j < N; ++j) A[i][j] = rec[2 * N + i * N + j];
#pragma unroll
        for (int i = 0; i < N; ++i) alpha[i] = rec_next[i];

        const uint8_t* Ht = H + t * N * row_bytes;
        const uint8_t* Ft = F + t * row_bytes;
        uint4 rh[N][VPT], rf[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
#pragma unroll
                for (int i = 0; i < N; ++i) rh[i][j] = ld16_stream(Ht + i * row_bytes + v * 16);
                rf[j] = ld16_stream(Ft + v * 16);
            }
        }

        uint8_t* Ot = H_out + t * N * row_bytes;
        float x[VPT][V];
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
                uint32_t o[N][4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {          // dword by dword
                    float h[N][E], f[E];
                    float* xq = &x[j][q * E];
#pragma unroll
                    for (int i = 0; i < N; ++i) unpack_word<S>(word(rh[i][j], q), h[i]);
                    unpack_word<S>(word(rf[j], q), f);
#pragma unroll
                    for (int i = 0; i < N; ++i) {
                        float y[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            float acc = A[i][0] * h[0][e];
#pragma unroll
                            for (int k = 1; k < N; ++k) acc = fmaf(A[i][k], h[k][e], acc);
                            y[e] = fmaf(beta[i], f[e], acc);
                        }
                        o[i][q] = pack_word<S>(y);
                        float yr[E];
                        unpack_word<S>(o[i][q], yr);   // the stored (rounded) values
                        if (i == 0) {
#pragma unroll
                            for (int e = 0; e < E; ++e) xq[e] = alpha[0] * yr[e];
                        } else {
#pragma unroll
                            for (int e = 0; e < E; ++e) xq[e] = fmaf(alpha[i], yr[e], xq[e]);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < N; ++i)
                    st16_stream(Ot + i * row_bytes + v * 16, make_uint4(o[i][0], o[i][1], o[i][2], o[i][3]));
#pragma unroll
                for (int e = 0; e < V; ++e) ss = fmaf(x[j][e], x[j][e], ss);
            }
        }

        float g[VPT][V];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
#pragma unroll
                for (int q = 0; q < V / 4; ++q) {
                    uint4 gv = ld16(gamma + v * V + 4 * q);
                    unpack<f32_t>(gv, &g[j][4 * q]);
                }
            }
        }

        ss = block_sum(ss, red);
        const float r = 1.0f / sqrtf(ss / (float)d + eps);

        uint8_t* ut = u_next + t * row_bytes;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = threadIdx.x + j * B;
            if (v < nvec) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) o[e] = g[j][e] * (x[j][e] * r);
                st16_stream(ut + v * 16, pack<S>(o));
            }
        }
    }
}

// ------------------------------------------------------------ tanh block

// tanh from the hardware base-2 exponential and reciprocal (each about one
// ulp): tanh|x| = (1 - t) / (1 + t) with t = 2^(-2|x| log2 e), sign restored.
// The error is a few fp32 ulps of the result, and about 1e-7 absolute near 0
// where 1 - t cancels; the stored F is rounded to its storage type anyway.
// tanh(+-inf) = +-1 and NaN stays NaN.  About a third of the instructions of
// the library tanhf, which made the kernel bound by its arithmetic.
__device__ __forceinline__ float tanh_fast(float x) {
    const float t = __builtin_amdgcn_exp2f(-2.88539008177792681f * fabsf(x));   // 2 log2(e)
    return copysignf((1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t), x);
}

template <typename S>
__global__ __launch_bounds__(256) void block_tanh_kernel(const uint8_t* __restrict__ u,
                                                         uint8_t* __restrict__ F, int64_t nvec) {
    constexpr int V = Store<S>::kElems;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
         v += (int64_t)gridDim.x * blockDim.x) {
        float x[V];
        unpack<S>(ld16_stream(u + v * 16), x);
#pragma unroll
        for (int e = 0; e < V; ++e) x[e] = tanh_fast(x[e]);
        st16_stream(F + v * 16, pack<S>(x));
    }
}

// --------------------------------------------------------------- dispatch

inline dim3 row_grid(int64_t T) { return dim3((unsigned)(T < kMaxGrid ? T : kMaxGrid)); }

struct PreL {
    template <int N, typename S, int VPT, typename... A>
    static hipError_t go(RowCfg c, int64_t T, hipStream_t s, A... a) {
        return launch(pre_mix_kernel<N, S, VPT>, row_grid(T), dim3(c.block), 0, s, a...);
    }
};
struct PostL {
    template <int N, typename S, int VPT, typename... A>
    static hipError_t go(RowCfg c, int64_t T, hipStream_t s, A... a) {
        return launch(post_mix_kernel<N, S, VPT>, row_grid(T), dim3(c.block), 0, s, a...);
    }
};
struct PostPreL {
    template <int N, typename S, int VPT, typename... A>
    static hipError_t go(RowCfg c, int64_t T, hipStream_t s, A... a) {
        return launch(post_pre_mix_kernel<N, S, VPT>, row_grid(T), dim3(c.block), 0, s, a...);
    }
};

template <class L, int N, typename S, typename... A>
hipError_t by_cfg(RowCfg c, int64_t T, hipStream_t s, A... a) {
    if constexpr (Store<S>::kElems == 16) {
        // fp8 rows hold at most HC_MAX_HIDDEN / 16 = 1024 vectors: one per thread
        if (c.vpt == 1) return L::template go<N, S, 1>(c, T, s, a...);
        return hipErrorInvalidConfiguration;
    } else {
        switch (c.vpt) {
            case 1: return L::template go<N, S, 1>(c, T, s, a...);
            case 2: return L::template go<N, S, 2>(c, T, s, a...);
            case 3: return L::template go<N, S, 3>(c, T, s, a...);
            case 4: return L::template go<N, S, 4>(c, T, s, a...);
        }
        return hipErrorInvalidConfiguration;
    }
}

template <class L, typename S, typename... A>
hipError_t by_n(int n, RowCfg c, int64_t T, hipStream_t s, A... a) {
    switch (n) {
        case 1: return by_cfg<L, 1, S>(c, T, s, a...);
        case 2: return by_cfg<L, 2, S>(c, T, s, a...);
        case 3: return by_cfg<L, 3, S>(c, T, s, a...);
        case 4: return by_cfg<L, 4, S>(c, T, s, a...);
    }
    return hipErrorInvalidValue;
}

template <class L, typename... A>
hipError_t dispatch_rows(int n, int d, int dt, int64_t T, hipStream_t s, A... a) {
    if (dt == 0) return by_n<L, f32_t>(n, row_config(d / Store<f32_t>::kElems), T, s, a...);
    if (dt == 2) return by_n<L, fp8_t>(n, row_config(d / Store<fp8_t>::kElems), T, s, a...);
    return by_n<L, bf16_t>(n, row_config(d / Store<bf16_t>::kElems), T, s, a...);
}

}  // namespace

hipError_t launch_pre_mix(const void* H, const float* w, int64_t w_stride, const float* gamma,
                          float eps, void* u, int64_t T, int n, int d, int dt, hipStream_t s) {
    return dispatch_rows<PreL>(n, d, dt, T, s, static_cast<const uint8_t*>(H), w, w_stride, gamma,
                               eps, static_cast<uint8_t*>(u), T, d);
}

hipError_t launch_post_mix(const void* H, const void* F, const float* w, int64_t w_stride,
                           void* H_out, int64_t T, int n, int d, int dt, hipStream_t s) {
    return dispatch_rows<PostL>(n, d, dt, T, s, static_cast<const uint8_t*>(H),
                                static_cast<const uint8_t*>(F), w, w_stride,
                                static_cast<uint8_t*>(H_out), T, d);
}

hipError_t launch_post_pre_mix(const void* H, const void* F, const float* w, int64_t w_stride,
                               const float* w_next, int64_t w_next_stride, const float* gamma,
                               float eps, void* H_out, void* u_next, int64_t T, int n, int d,
                               int dt, hipStream_t s) {
    return dispatch_rows<PostPreL>(n, d, dt, T, s, static_cast<const uint8_t*>(H),
                                   static_cast<const uint8_t*>(F), w, w_stride, w_next,
                                   w_next_stride, gamma, eps, static_cast<uint8_t*>(H_out),
                                   static_cast<uint8_t*>(u_next), T, d);
}

hipError_t launch_block_tanh(const void* u, void* F, int64_t count, int dt, hipStream_t s) {
    const int V = dt == 0 ? Store<f32_t>::kElems
                          : (dt == 2 ? Store<fp8_t>::kElems : Store<bf16_t>::kElems);
    const int64_t nvec = count / V;
    const int64_t blocks = (nvec + 255) / 256;
    const dim3 grid((unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid));
    if (dt == 0)
        return launch(block_tanh_kernel<f32_t>, grid, dim3(256), 0, s,
                      static_cast<const uint8_t*>(u), static_cast<uint8_t*>(F), nvec);
    if (dt == 2)
        return launch(block_tanh_kernel<fp8_t>, grid, dim3(256), 0, s,
                      static_cast<const uint8_t*>(u), static_cast<uint8_t*>(F), nvec);
    return launch(block_tanh_kernel<bf16_t>, grid, dim3(256), 0, s,
                  static_cast<const uint8_t*>(u), static_cast<uint8_t*>(F), nvec);
}

}  // namespace hc
