// hc_launch.h -- internal (C++) launchers behind the C ABI.  The ABI layer
// validates every argument before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace hc {

// Launch `kernel` with arguments converted to its exact parameter types and
// return the runtime's verdict on the launch itself.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                  hipStream_t stream, Args&&... args) {
    std::tuple<KArgs...> params(std::forward<Args>(args)...);
    void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    std::apply([&](auto&... p) {
        int i = 0;
        ((argv[i++] = static_cast<void*>(&p)), ...);
    }, params);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem, stream);
}

// Row kernels (one workgroup per token row): block size and 16-byte vectors
// per thread for a row of `nvec` vectors.  As few vectors per thread as a
// 1024-thread block allows (one up to d = 8192 bf16): measured on MI355X, one
// vector per thread in 512-thread blocks streams faster than two in 256.
// Shared by pre, post and the fused post+pre so that their reductions over d
// run in the same order; the order depends on d only.
struct RowCfg { int block; int vpt; };
inline RowCfg row_config(int nvec) {
    const int vpt = (nvec + 1023) / 1024;                    // 1..4 for d <= 16384
    const int block = ((nvec + vpt - 1) / vpt + 63) / 64 * 64;
    return {block, vpt};
}

hipError_t launch_pre_mix(const void* H, const float* w, int64_t w_stride, const float* gamma,
                          float eps, void* u, int64_t T, int n, int d, int dt, hipStream_t s);
hipError_t launch_post_mix(const void* H, const void* F, const float* w, int64_t w_stride,
                           void* H_out, int64_t T, int n, int d, int dt, hipStream_t s);
hipError_t launch_post_pre_mix(const void* H, const void* F, const float* w, int64_t w_stride,
                               const float* w_next, int64_t w_next_stride, const float* gamma,
                               float eps, void* H_out, void* u_next, int64_t T, int n, int d,
                               int dt, hipStream_t s);
hipError_t launch_block_tanh(const void* u, void* F, int64_t count, int dt, hipStream_t s);
hipError_t launch_weights(const void* H, const void* W, const float* w_static, float scale,
                          float eps, int iters, float* w_out, int64_t T, int n, int d, int dt,
                          hipStream_t s);
hipError_t launch_post_mix_backward(const void* dHo, const void* H, const void* F, const float* w,
                                    int64_t w_stride, void* dH, void* dF, float* dw, void* work,
                                    int64_t T, int n, int d, int dt, hipStream_t s);
hipError_t launch_pre_mix_backward(const void* du, const void* H, const float* w, int64_t w_stride,
                                   const float* gamma, float eps, const void* dH_in, const void* dHo,
                                   void* dH, float* dw, float* dgamma, void* work, int64_t T, int n,
                                   int d, int dt, hipStream_t s);
hipError_t launch_post_pre_mix_backward(const void* dHo, const void* du, const void* H, const void* F,
                                        const float* w, const float* wn, int64_t w_stride,
                                        const float* gamma, float eps, void* dH, void* dF, float* dw,
                                        float* dwn, float* dgamma, void* work, int64_t T, int n,
                                        int d, int dt, hipStream_t s, const float* dhb = nullptr,
                                        const float* coef = nullptr);
int64_t backward_workspace_bytes(int64_t T, int n, int d);
// The post gradient with its scratch in the library's own per-GPU array
// (nothing allocated): bytes it needs, and the array's size.
int64_t post_backward_scratch_bytes(int64_t T, int n);
int64_t post_backward_scratch_max_bytes();
hipError_t launch_post_mix_backward_noalloc(const void* dHo, const void* H, const void* F,
                                            const float* w, int64_t w_stride, void* dH, void* dF,
                                            float* dw, int64_t T, int n, int d, int dt, hipStream_t s);
hipError_t launch_sum_records(const float* rec, int64_t T, int K, float* out, hipStream_t s);
hipError_t launch_sinkhorn(const float* logits, float* w_out, int iters, int64_t T, int n,
                           hipStream_t s);
hipError_t launch_weights_raw(const void* H, const void* W, float eps, float* P, float* r, int64_t T,
                              int n, int d, int dt, hipStream_t s);
hipError_t launch_weights_save(const void* H, const void* W, const float* w_static, float scale,
                               float eps, int iters, float* w_out, float* P, float* r, int64_t T,
                               int n, int d, int dt, hipStream_t s);
// Post fused with the next layer's per-token weights (W held in registers)
// and, when u_out is not null, with the next layer's read-mix (gain gamma,
// RMSNorm eps pre_eps): the largest d it takes for storage dtype dt (0: dt
// not taken).
int post_weights_max_hidden(int dt);
hipError_t launch_post_mix_weights(const void* H, const void* F, const float* w, int64_t w_stride,
                                   const void* W, const float* w_static, float scale, float eps,
                                   int iters, const float* gamma, float pre_eps, void* H_out,
                                   float* w_out, void* u_out, float* P, float* rn, int64_t T, int n,
                                   int d, int dt, hipStream_t s);
// The per-stream projections P [T][n][K] and norms r [T][n] the forward keeps
// for the gradient pass: floats, r at saved_r_offset(T, n).
int64_t saved_r_offset(int64_t T, int n);
int64_t saved_floats(int64_t T, int n);
int64_t sum_rows_tmp_floats(int64_t rows, int64_t cols);
// A deterministic column sum: out[c] = sum over r of in[r * cols + c], in a
// fixed order of levels (tmp: sum_rows_tmp_floats(rows, cols) floats); the
// last level also writes nzero zeros at `zero` (may be NULL).
struct SumJob {
    const float* in;
    int64_t rows;
    int cols;
    float* tmp;
    float* out;
    float* zero;
    int nzero;
};
// One to three independent sums; their levels share launches.
hipError_t launch_sum_rows(const SumJob* jobs, int njobs, hipStream_t s);
int64_t weights_backward_workspace_bytes(int64_t T, int n, int d, int iters);
int64_t sinkhorn_backward_workspace_bytes(int64_t T, int iters);
// With dhbar (and coef) given, the stream pass writes dhbar = W^T dz [T][d]
// and the coefficients (a_i | b_i) [T][2n] instead of dH (dH_in, dH unused).
hipError_t launch_weights_backward(const void* H, const void* W, const float* w_static, float scale,
                                   float eps, int iters, const float* dw, const float* dw2,
                                   const float* saved, const void* dH_in,
                                   void* dH, float* dW, float* dws, void* work, int64_t T, int n,
                                   int d, int dt, hipStream_t s, float* dhbar = nullptr,
                                   float* coef = nullptr);
hipError_t launch_sinkhorn_backward(const float* logits, const float* dw, const float* dw2,
                                    float* dlogits, int iters, void* work, int64_t T, int n,
                                    hipStream_t s);

}  // namespace hc
