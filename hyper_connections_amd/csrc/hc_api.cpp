// hc_api.cpp -- the extern "C" boundary of libhc.so (declared in include/hc.h).
//
// Every entry point validates all arguments before it launches anything, so
// a failed check leaves the stream untouched.  Validation uses only pointer
// values and sizes (no HIP calls), which also lets it run on hosts without a
// GPU.  No exception crosses the boundary and nothing is printed.
#include "hc.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "hc_launch.h"

namespace {

constexpr int64_t kMaxBytes = int64_t(1) << 52;   // any single buffer (4 PiB)

struct Span {
    const void* p;
    int64_t bytes;
};

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

bool overlap(Span a, Span b) {
    if (a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
    return x < y + static_cast<uintptr_t>(b.bytes) && y < x + static_cast<uintptr_t>(a.bytes);
}

int elem_bytes(int dt) { return dt == HC_F32 ? 4 : (dt == HC_FP8 ? 1 : 2); }
int vec_elems(int dt) { return 16 / elem_bytes(dt); }

// The streaming calls (pre, post, post+pre, tanh block) take every storage
// dtype; the weight producer and the gradients take fp32 and bf16.
bool dtype_ok(int dt) { return dt == HC_F32 || dt == HC_BF16 || dt == HC_FP8; }
bool dtype_wide(int dt) { return dt == HC_F32 || dt == HC_BF16; }

int record_len(int n) { return 2 * n + n * n; }

// Bytes of T records read through a stride (0 = one shared record).
int64_t record_span(int64_t T, int64_t stride, int K) {
    return (stride == 0 ? int64_t(K) : (T - 1) * stride + K) * 4;
}

// Shape checks shared by the row kernels.  Order of checks: dtype, n, d, T.
hc_status check_nd(int32_t n, int32_t d, int64_t T, int dt) {
    if (!dtype_ok(dt)) return HC_ERR_DTYPE;
    if (n < 1 || n > HC_MAX_STREAMS) return HC_ERR_SHAPE;
    if (d < 1 || d > HC_MAX_HIDDEN || d % vec_elems(dt) != 0) return HC_ERR_SHAPE;
    if (T < 0) return HC_ERR_ARG;
    if (T > kMaxBytes / (int64_t(n) * d * elem_bytes(dt))) return HC_ERR_ARG;
    return HC_OK;
}

hc_status check_stride(int64_t stride, int K, int64_t T) {
    if (stride != 0 && stride < K) return HC_ERR_SHAPE;
    if (stride > 0 && T > kMaxBytes / 4 / stride) return HC_ERR_ARG;
    return HC_OK;
}

bool eps_ok(float eps) { return std::isfinite(eps) && eps > 0.0f; }

hc_status from_hip(hipError_t e) { return e == hipSuccess ? HC_OK : HC_ERR_HIP; }

// The value a C caller passed for an enum parameter.  C lets any int through
// an enum type; in C++ reading an enum object that holds a value outside its
// enumerators' range is undefined, so the argument is read through its bytes.
template <typename E>
int enum_value(const E& e) {
    int v = 0;
    static_assert(sizeof(E) == sizeof(int), "enum parameters are int-sized");
    std::memcpy(&v, &e, sizeof v);
    return v;
}

}  // namespace

extern "C" {

const char* hc_status_str(hc_status status) {
    switch (enum_value(status)) {
        case HC_OK: return "HC_OK: success";
        case HC_ERR_NULL: return "HC_ERR_NULL: a required pointer is NULL";
        case HC_ERR_SHAPE: return "HC_ERR_SHAPE: n, d or a stride is outside the supported set";
        case HC_ERR_DTYPE: return "HC_ERR_DTYPE: storage dtype unknown or not taken by this call";
        case HC_ERR_ALIGN: return "HC_ERR_ALIGN: a pointer is not aligned as required";
        case HC_ERR_ALIAS: return "HC_ERR_ALIAS: an output overlaps an input or another output";
        case HC_ERR_ARG: return "HC_ERR_ARG: T, eps or iters out of range";
        case HC_ERR_HIP: return "HC_ERR_HIP: the HIP runtime reported a launch error";
    }
    return "HC_ERR_UNKNOWN: unknown status code";
}

int32_t hc_abi_version(void) { return 8; }

hc_status hc_pre_mix(const void* H, const float* w, int64_t w_stride, const float* gamma, float eps,
                     void* u, int64_t T, int32_t n, int32_t d, hc_dtype dt_arg, void* stream) {
    const int dt = enum_value(dt_arg);
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    const int K = record_len(n);
    if ((st = check_stride(w_stride, K, T)) != HC_OK) return st;
    if (!eps_ok(eps)) return HC_ERR_ARG;
    if (T == 0) return HC_OK;
    if (!H || !w || !gamma || !u) return HC_ERR_NULL;
    if (misaligned(H, 16) || misaligned(u, 16) || misaligned(gamma, 16) || misaligned(w, 4))
        return HC_ERR_ALIGN;
    const int64_t s = elem_bytes(dt);
    const Span sH{H, T * n * d * s}, sU{u, T * d * s}, sW{w, record_span(T, w_stride, K)},
        sG{gamma, int64_t(d) * 4};
    if (overlap(sU, sH) || overlap(sU, sW) || overlap(sU, sG)) return HC_ERR_ALIAS;
    return from_hip(hc::launch_pre_mix(H, w, w_stride, gamma, eps, u, T, n, d, dt,
                                       static_cast<hipStream_t>(stream)));
}

hc_status hc_post_mix(const void* H, const void* F, const float* w, int64_t w_stride, void* H_out,
                      int64_t T, int32_t n, int32_t d, hc_dtype dt_arg, void* stream) {
    const int dt = enum_value(dt_arg);
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    const int K = record_len(n);
    if ((st = check_stride(w_stride, K, T)) != HC_OK) return st;
    if (T == 0) return HC_OK;
    if (!H || !F || !w || !H_out) return HC_ERR_NULL;
    if (misaligned(H, 16) || misaligned(F, 16) || misaligned(H_out, 16) || misaligned(w, 4))
        return HC_ERR_ALIGN;
    const int64_t s = elem_bytes(dt);
    const Span sH{H, T * n * d * s}, sF{F, T * d * s}, sO{H_out, T * n * d * s},
        sW{w, record_span(T, w_stride, K)};
    if ((H_out != H && overlap(sO, sH)) || overlap(sO, sF) || overlap(sO, sW)) return HC_ERR_ALIAS;
    return from_hip(hc::launch_post_mix(H, F, w, w_stride, H_out, T, n, d, dt,
                                        static_cast<hipStream_t>(stream)));
}

hc_status hc_post_pre_mix(const void* H, const void* F, const float* w, int64_t w_stride,
                          const float* w_next, int64_t w_next_stride, const float* gamma_next,
                          float eps, void* H_out, void* u_next, int64_t T, int32_t n, int32_t d,
                          hc_dtype dt_arg, void* stream) {
    const int dt = enum_value(dt_arg);
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    const int K = record_len(n);
    if ((st = check_stride(w_stride, K, T)) != HC_OK) return st;
    if ((st = check_stride(w_next_stride, K, T)) != HC_OK) return st;
    if (!eps_ok(eps)) return HC_ERR_ARG;
    if (T == 0) return HC_OK;
    if (!H || !F || !w || !w_next || !gamma_next || !H_out || !u_next) return HC_ERR_NULL;
    if (misaligned(H, 16) || misaligned(F, 16) || misaligned(H_out, 16) || misaligned(u_next, 16) ||
        misaligned(gamma_next, 16) || misaligned(w, 4) || misaligned(w_next, 4))
        return HC_ERR_ALIGN;
    const int64_t s = elem_bytes(dt);
    const Span sH{H, T * n * d * s}, sF{F, T * d * s}, sO{H_out, T * n * d * s},
        sU{u_next, T * d * s}, sW{w, record_span(T, w_stride, K)},
        sW2{w_next, record_span(T, w_next_stride, K)}, sG{gamma_next, int64_t(d) * 4};
    if ((H_out != H && overlap(sO, sH)) || overlap(sO, sF) || overlap(sO, sW) || overlap(sO, sW2) ||
        overlap(sO, sG) || overlap(sU, sH) || overlap(sU, sF) || overlap(sU, sW) ||
        overlap(sU, sW2) || overlap(sU, sG) || overlap(sU, sO))
        return HC_ERR_ALIAS;
    return from_hip(hc::launch_post_pre_mix(H, F, w, w_stride, w_next, w_next_stride, gamma_next,
                                            eps, H_out, u_next, T, n, d, dt,
                                            static_cast<hipStream_t>(stream)));
}

hc_status hc_weights(const void* H, const void* W, const float* w_static, float scale, float eps,
                     int32_t sinkhorn_iters, float* w_out, int64_t T, int32_t n, int32_t d,
                     hc_dtype dt_arg, void* stream) {
    const int dt = enum_value(dt_arg);
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    if (!eps_ok(eps) || !std::isfinite(scale)) return HC_ERR_ARG;
    if (sinkhorn_iters < 0 || sinkhorn_iters > HC_MAX_SINKHORN_ITERS) return HC_ERR_ARG;
    if (T == 0) return HC_OK;
    if (!H || !W || !w_static || !w_out) return HC_ERR_NULL;
    if (misaligned(H, 16) || misaligned(W, 16) || misaligned(w_static, 4) || misaligned(w_out, 4))
        return HC_ERR_ALIGN;
    const int K = record_len(n);
    const int64_t s = elem_bytes(dt);
    const Span sH{H, T * n * d * s}, sW{W, int64_t(K) * d * s}, sS{w_static, int64_t(K) * 4},
        sO{w_out, T * K * 4};
    if (overlap(sO, sH) || overlap(sO, sW) || overlap(sO, sS)) return HC_ERR_ALIAS;
    return from_hip(hc::launch_weights(H, W, w_static, scale, eps, sinkhorn_iters, w_out, T, n, d,
                                       dt, static_cast<hipStream_t>(stream)));
}

int64_t hc_weights_saved_bytes(int64_t T, int32_t n) {
    if (T <= 0 || n < 1 || n > HC_MAX_STREAMS) return 0;
    return hc::saved_floats(T, n) * 4;
}

hc_status hc_weights_save(const void* H, const void* W, const float* w_static, float scale,
                          float eps, int32_t sinkhorn_iters, float* w_out, float* saved,
                          int64_t saved_bytes, int64_t T, int32_t n, int32_t d, hc_dtype dt_arg,
                          void* stream) {
    const int dt = enum_value(dt_arg);
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    if (!eps_ok(eps) || !std::isfinite(scale)) return HC_ERR_ARG;
    if (sinkhorn_iters < 0 || sinkhorn_iters > HC_MAX_SINKHORN_ITERS) return HC_ERR_ARG;
    if (T == 0) return HC_OK;
    if (!H || !W || !w_static || !w_out || !saved) return HC_ERR_NULL;
    const int64_t need = hc_weights_saved_bytes(T, n);
    if (saved_bytes < need) return HC_ERR_ARG;
    if (misaligned(H, 16) || misaligned(W, 16) || misaligned(w_static, 4) || misaligned(w_out, 4) ||
        misaligned(saved, 16))
        return HC_ERR_ALIGN;
    const int K = record_len(n);
    const int64_t s = elem_bytes(dt);
    const Span sH{H, T * n * d * s}, sW{W, int64_t(K) * d * s}, sS{w_static, int64_t(K) * 4},
        sO{w_out, T * K * 4}, sv{saved, need};
    for (const Span& o : {sO, sv})
        if (overlap(o, sH) || overlap(o, sW) || overlap(o, sS)) return HC_ERR_ALIAS;
    if (overlap(sO, sv)) return HC_ERR_ALIAS;
    return from_hip(hc::launch_weights_save(H, W, w_static, scale, eps, sinkhorn_iters, w_out, saved,
                                            saved + hc::saved_r_offset(T, n), T, n, d, dt,
                                            static_cast<hipStream_t>(stream)));
}

namespace {

// The write-back fused with the next layer's weights and, when u_next is
// given, its read-mix (gamma_next, pre_eps); checks every argument first.
hc_status post_weights(const void* H, const void* F, const float* w, int64_t w_stride,
                       const void* W, const float* w_static, float scale, float eps,
                       int32_t sinkhorn_iters, const float* gamma_next, float pre_eps, void* H_out,
                       float* w_out, void* u_next, float* saved, int64_t saved_bytes, int64_t T,
                       int32_t n, int32_t d, int dt, void* stream) {
    const bool pre = u_next != nullptr || gamma_next != nullptr;
    if (dt != HC_BF16 && dt != HC_FP8) return HC_ERR_DTYPE;
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    if (d > hc::post_weights_max_hidden(dt)) return HC_ERR_SHAPE;
    const int K = record_len(n);
    if ((st = check_stride(w_stride, K, T)) != HC_OK) return st;
    if (!eps_ok(eps) || !std::isfinite(scale)) return HC_ERR_ARG;
    if (pre && !eps_ok(pre_eps)) return HC_ERR_ARG;
    if (sinkhorn_iters < 0 || sinkhorn_iters > HC_MAX_SINKHORN_ITERS) return HC_ERR_ARG;
    if (T == 0) return HC_OK;
    if (!H || !F || !w || !W || !w_static || !H_out || !w_out) return HC_ERR_NULL;
    if (pre && (!gamma_next || !u_next)) return HC_ERR_NULL;
    const int64_t need = saved ? hc_weights_saved_bytes(T, n) : 0;
    if (saved && saved_bytes < need) return HC_ERR_ARG;
    if (misaligned(H, 16) || misaligned(F, 16) || misaligned(H_out, 16) || misaligned(W, 16) ||
        misaligned(w, 4) || misaligned(w_static, 4) || misaligned(w_out, 4) ||
        misaligned(saved, 16) || misaligned(u_next, 16) || misaligned(gamma_next, 16))
        return HC_ERR_ALIGN;
    const int64_t s = elem_bytes(dt);
    const Span sH{H, T * n * d * s}, sF{F, T * d * s}, sw{w, record_span(T, w_stride, K)},
        sW{W, int64_t(K) * d * s}, sS{w_static, int64_t(K) * 4}, sO{H_out, T * n * d * s},
        sR{w_out, T * K * 4}, sv{saved, need}, sG{gamma_next, pre ? int64_t(d) * 4 : 0},
        sU{u_next, pre ? T * d * s : 0};
    if ((H_out != H && overlap(sO, sH)) || overlap(sO, sF) || overlap(sO, sw) || overlap(sO, sW) ||
        overlap(sO, sS) || overlap(sO, sG))
        return HC_ERR_ALIAS;
    for (const Span& o : {sR, sv, sU})
        if (overlap(o, sH) || overlap(o, sF) || overlap(o, sw) || overlap(o, sW) || overlap(o, sS) ||
            overlap(o, sO) || overlap(o, sG))
            return HC_ERR_ALIAS;
    if (overlap(sR, sv) || overlap(sR, sU) || overlap(sv, sU)) return HC_ERR_ALIAS;
    return from_hip(hc::launch_post_mix_weights(
        H, F, w, w_stride, W, w_static, scale, eps, sinkhorn_iters, gamma_next, pre_eps, H_out,
        w_out, u_next, saved, saved ? saved + hc::saved_r_offset(T, n) : nullptr, T, n, d, dt,
        static_cast<hipStream_t>(stream)));
}

}  // namespace

hc_status hc_post_mix_weights(const void* H, const void* F, const float* w, int64_t w_stride,
                              const void* W, const float* w_static, float scale, float eps,
                              int32_t sinkhorn_iters, void* H_out, float* w_out, float* saved,
                              int64_t saved_bytes, int64_t T, int32_t n, int32_t d, hc_dtype dt_arg,
                              void* stream) {
    return post_weights(H, F, w, w_stride, W, w_static, scale, eps, sinkhorn_iters, nullptr, 0.0f,
                        H_out, w_out, nullptr, saved, saved_bytes, T, n, d, enum_value(dt_arg),
                        stream);
}

hc_status hc_post_weights_pre_mix(const void* H, const void* F, const float* w, int64_t w_stride,
                                  const void* W, const float* w_static, float scale, float eps,
                                  int32_t sinkhorn_iters, const float* gamma_next, float pre_eps,
                                  void* H_out, float* w_out, void* u_next, float* saved,
                                  int64_t saved_bytes, int64_t T, int32_t n, int32_t d,
                                  hc_dtype dt_arg, void* stream) {
    // the read-mix half needs both of its buffers
    if (T > 0 && (!gamma_next || !u_next)) return HC_ERR_NULL;
    return post_weights(H, F, w, w_stride, W, w_static, scale, eps, sinkhorn_iters, gamma_next,
                        pre_eps, H_out, w_out, u_next, saved, saved_bytes, T, n, d,
                        enum_value(dt_arg), stream);
}

hc_status hc_sinkhorn(const float* logits, float* w_out, int32_t iters, int64_t T, int32_t n,
                      void* stream) {
    if (n < 1 || n > HC_MAX_STREAMS) return HC_ERR_SHAPE;
    if (T < 0 || iters < 0 || iters > HC_MAX_SINKHORN_ITERS) return HC_ERR_ARG;
    const int K = record_len(n);
    if (T > kMaxBytes / (4 * K)) return HC_ERR_ARG;
    if (T == 0) return HC_OK;
    if (!logits || !w_out) return HC_ERR_NULL;
    if (misaligned(logits, 4) || misaligned(w_out, 4)) return HC_ERR_ALIGN;
    if (overlap(Span{logits, T * K * 4}, Span{w_out, T * K * 4})) return HC_ERR_ALIAS;
    return from_hip(hc::launch_sinkhorn(logits, w_out, iters, T, n, static_cast<hipStream_t>(stream)));
}

int64_t hc_backward_workspace(int64_t T, int32_t n, int32_t d) {
    if (n < 1 || n > HC_MAX_STREAMS || d < 1 || d > HC_MAX_HIDDEN) return 0;
    return hc::backward_workspace_bytes(T, n, d);
}

hc_status hc_post_mix_backward(const void* dH_out, const void* H, const void* F, const float* w,
                               int64_t w_stride, void* dH, void* dF, float* dw, void* workspace,
                               int64_t workspace_bytes, int64_t T, int32_t n, int32_t d,
                               hc_dtype dt_arg, void* stream) {
    const int dt = enum_value(dt_arg);
    if (!dtype_wide(dt)) return HC_ERR_DTYPE;
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    const int K = record_len(n);
    if ((st = check_stride(w_stride, K, T)) != HC_OK) return st;
    if (T == 0) return HC_OK;
    if (!dH_out || !H || !F || !w || !dF || !dw) return HC_ERR_NULL;     // dH may be NULL
    const bool shared = w_stride == 0;
    if (shared && !workspace) return HC_ERR_NULL;
    if (shared && workspace_bytes < hc_backward_workspace(T, n, d)) return HC_ERR_ARG;
    if (misaligned(dH_out, 16) || misaligned(H, 16) || misaligned(F, 16) || misaligned(dH, 16) ||
        misaligned(dF, 16) || misaligned(w, 4) || misaligned(dw, 4) ||
        (shared && misaligned(workspace, 16)))
        return HC_ERR_ALIGN;
    const int64_t s = elem_bytes(dt);
    const Span sG{dH_out, T * n * d * s}, sH{H, T * n * d * s}, sF{F, T * d * s},
        sW{w, record_span(T, w_stride, K)}, sdH{dH, dH ? T * n * d * s : 0}, sdF{dF, T * d * s},
        sdw{dw, (shared ? 1 : T) * K * 4},
        sws{workspace, shared ? hc_backward_workspace(T, n, d) : 0};
    const Span ins[] = {sG, sH, sF, sW};
    for (const Span& o : {sdH, sdF, sdw, sws})
        for (const Span& i : ins)
            if (overlap(o, i)) return HC_ERR_ALIAS;
    if (overlap(sdH, sdF) || overlap(sdH, sdw) || overlap(sdF, sdw) || overlap(sws, sdH) ||
        overlap(sws, sdF) || overlap(sws, sdw))
        return HC_ERR_ALIAS;
    return from_hip(hc::launch_post_mix_backward(dH_out, H, F, w, w_stride, dH, dF, dw, workspace,
                                                 T, n, d, dt, static_cast<hipStream_t>(stream)));
}

hc_status hc_post_mix_backward_noalloc(const void* dH_out, const void* H, const void* F,
                                       const float* w, int64_t w_stride, void* dH, void* dF,
                                       float* dw, int64_t T, int32_t n, int32_t d, hc_dtype dt_arg,
                                       void* stream) {
    const int dt = enum_value(dt_arg);
    if (!dtype_wide(dt)) return HC_ERR_DTYPE;
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    const int K = record_len(n);
    if ((st = check_stride(w_stride, K, T)) != HC_OK) return st;
    if (T == 0) return HC_OK;
    if (!dH_out || !H || !F || !w || !dF || !dw) return HC_ERR_NULL;     // dH may be NULL
    const bool shared = w_stride == 0;
    if (shared && hc::post_backward_scratch_bytes(T, n) > hc::post_backward_scratch_max_bytes())
        return HC_ERR_ARG;
    if (misaligned(dH_out, 16) || misaligned(H, 16) || misaligned(F, 16) || misaligned(dH, 16) ||
        misaligned(dF, 16) || misaligned(w, 4) || misaligned(dw, 4))
        return HC_ERR_ALIGN;
    const int64_t s = elem_bytes(dt);
    const Span sG{dH_out, T * n * d * s}, sH{H, T * n * d * s}, sF{F, T * d * s},
        sW{w, record_span(T, w_stride, K)}, sdH{dH, dH ? T * n * d * s : 0}, sdF{dF, T * d * s},
        sdw{dw, (shared ? 1 : T) * K * 4};
    const Span ins[] = {sG, sH, sF, sW};
    for (const Span& o : {sdH, sdF, sdw})
        for (const Span& i : ins)
            if (overlap(o, i)) return HC_ERR_ALIAS;
    if (overlap(sdH, sdF) || overlap(sdH, sdw) || overlap(sdF, sdw)) return HC_ERR_ALIAS;
    return from_hip(hc::launch_post_mix_backward_noalloc(dH_out, H, F, w, w_stride, dH, dF, dw, T, n,
                                                         d, dt, static_cast<hipStream_t>(stream)));
}

hc_status hc_pre_mix_backward(const void* du, const void* H, const float* w, int64_t w_stride,
                              const float* gamma, float eps, const void* dH_in, const void* dH_out,
                              void* dH, float* dw, float* dgamma, void* workspace,
                              int64_t workspace_bytes, int64_t T, int32_t n, int32_t d, hc_dtype dt_arg,
                              void* stream) {
    const int dt = enum_value(dt_arg);
    if (!dtype_wide(dt)) return HC_ERR_DTYPE;
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    const int K = record_len(n);
    if ((st = check_stride(w_stride, K, T)) != HC_OK) return st;
    if (!eps_ok(eps)) return HC_ERR_ARG;
    if (dH_in && dH_out) return HC_ERR_ARG;     // at most one addend
    if (!dH && (dH_in || dH_out)) return HC_ERR_ARG;   // an addend needs the dH it adds into
    if (T == 0) return HC_OK;
    if (!du || !H || !w || !gamma || !dw || !workspace) return HC_ERR_NULL;
    if (!dgamma && dH) return HC_ERR_NULL;             // dgamma may be left out only with dH
    if (workspace_bytes < hc_backward_workspace(T, n, d)) return HC_ERR_ARG;
    if (misaligned(du, 16) || misaligned(H, 16) || misaligned(gamma, 16) || misaligned(dH, 16) ||
        misaligned(dH_in, 16) || misaligned(dH_out, 16) || misaligned(workspace, 16) ||
        misaligned(w, 4) || misaligned(dw, 4) || misaligned(dgamma, 4))
        return HC_ERR_ALIGN;
    const int64_t s = elem_bytes(dt);
    const bool shared = w_stride == 0;
    const Span su{du, T * d * s}, sH{H, T * n * d * s}, sW{w, record_span(T, w_stride, K)},
        sg{gamma, int64_t(d) * 4}, sin{dH_in, dH_in ? T * n * d * s : 0},
        sdH{dH, dH ? T * n * d * s : 0},
        sdw{dw, (shared ? 1 : T) * K * 4}, sdg{dgamma, dgamma ? int64_t(d) * 4 : 0},
        sws{workspace, hc_backward_workspace(T, n, d)},
        sout{dH_out, dH_out ? T * n * d * s : 0};
    const Span ins[] = {su, sH, sW, sg, sout};
    for (const Span& o : {sdH, sdw, sdg, sws})
        for (const Span& i : ins)
            if (overlap(o, i)) return HC_ERR_ALIAS;
    if (dH_in && dH_in != dH && overlap(sdH, sin)) return HC_ERR_ALIAS;
    for (const Span& o : {sdw, sdg, sws})
        if (overlap(o, sin)) return HC_ERR_ALIAS;
    if (overlap(sdH, sdw) || overlap(sdH, sdg) || overlap(sdH, sws) || overlap(sdw, sdg) ||
        overlap(sdw, sws) || overlap(sdg, sws))
        return HC_ERR_ALIAS;
    return from_hip(hc::launch_pre_mix_backward(du, H, w, w_stride, gamma, eps, dH_in, dH_out, dH,
                                                dw, dgamma, workspace, T, n, d, dt,
                                                static_cast<hipStream_t>(stream)));
}

namespace {

// hc_post_pre_mix_backward, and with the weight producer's terms (dhbar and
// coef not NULL: per-token records only) hc_post_pre_mix_backward_terms.
hc_status post_pre_backward(const void* dH_out, const void* du_next, const void* H, const void* F,
                            const float* w, int64_t w_stride, const float* w_next,
                            int64_t w_next_stride, const float* gamma_next, float eps, void* dH,
                            void* dF, float* dw, float* dw_next, float* dgamma_next,
                            const float* dhbar, const float* coef, bool terms, void* workspace,
                            int64_t workspace_bytes, int64_t T, int32_t n, int32_t d, int dt,
                            void* stream) {
    if (!dtype_wide(dt)) return HC_ERR_DTYPE;
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    const int K = record_len(n);
    if ((st = check_stride(w_stride, K, T)) != HC_OK) return st;
    if ((st = check_stride(w_next_stride, K, T)) != HC_OK) return st;
    if (w_stride != w_next_stride) return HC_ERR_ARG;   // both shared or both per token
    if (terms && w_stride == 0) return HC_ERR_ARG;     // the producer's records are per token
    if (!eps_ok(eps)) return HC_ERR_ARG;
    if (T == 0) return HC_OK;
    if (!dH_out || !du_next || !H || !F || !w || !w_next || !gamma_next || !dH || !dF || !dw ||
        !dw_next || !dgamma_next || !workspace)
        return HC_ERR_NULL;
    if (terms && (!dhbar || !coef)) return HC_ERR_NULL;
    if (misaligned(dhbar, 16) || misaligned(coef, 4)) return HC_ERR_ALIGN;
    if (workspace_bytes < hc_backward_workspace(T, n, d)) return HC_ERR_ARG;
    if (misaligned(dH_out, 16) || misaligned(du_next, 16) || misaligned(H, 16) ||
        misaligned(F, 16) || misaligned(gamma_next, 16) || misaligned(dH, 16) ||
        misaligned(dF, 16) || misaligned(workspace, 16) || misaligned(w, 4) ||
        misaligned(w_next, 4) || misaligned(dw, 4) || misaligned(dw_next, 4) ||
        misaligned(dgamma_next, 4))
        return HC_ERR_ALIGN;
    const int64_t s = elem_bytes(dt);
    const bool shared = w_stride == 0;
    const Span sO{dH_out, T * n * d * s}, su{du_next, T * d * s}, sH{H, T * n * d * s},
        sF{F, T * d * s}, sW{w, record_span(T, w_stride, K)},
        sW2{w_next, record_span(T, w_next_stride, K)}, sg{gamma_next, int64_t(d) * 4},
        sdH{dH, T * n * d * s}, sdF{dF, T * d * s}, sdw{dw, (shared ? 1 : T) * K * 4},
        sdw2{dw_next, (shared ? 1 : T) * K * 4}, sdg{dgamma_next, int64_t(d) * 4},
        sws{workspace, hc_backward_workspace(T, n, d)},
        sdb{dhbar, terms ? T * d * 4 : 0}, sco{coef, terms ? T * 2 * n * 4 : 0};
    // dH == dH_out is allowed (every element is read before the same thread
    // writes it); any other overlap of an output is an error
    if (dH != dH_out && overlap(sdH, sO)) return HC_ERR_ALIAS;
    for (const Span& i : {su, sH, sF, sW, sW2, sg, sdb, sco})
        if (overlap(sdH, i)) return HC_ERR_ALIAS;
    const Span outs[] = {sdF, sdw, sdw2, sdg, sws};
    for (const Span& o : outs) {
        for (const Span& i : {sO, su, sH, sF, sW, sW2, sg, sdH, sdb, sco})
            if (overlap(o, i)) return HC_ERR_ALIAS;
    }
    for (int a = 0; a < 5; ++a)
        for (int b = a + 1; b < 5; ++b)
            if (overlap(outs[a], outs[b])) return HC_ERR_ALIAS;
    return from_hip(hc::launch_post_pre_mix_backward(dH_out, du_next, H, F, w, w_next, w_stride,
                                                     gamma_next, eps, dH, dF, dw, dw_next,
                                                     dgamma_next, workspace, T, n, d, dt,
                                                     static_cast<hipStream_t>(stream),
                                                     terms ? dhbar : nullptr,
                                                     terms ? coef : nullptr));
}

}  // namespace

hc_status hc_post_pre_mix_backward(const void* dH_out, const void* du_next, const void* H,
                                   const void* F, const float* w, int64_t w_stride,
                                   const float* w_next, int64_t w_next_stride,
                                   const float* gamma_next, float eps, void* dH, void* dF, float* dw,
                                   float* dw_next, float* dgamma_next, void* workspace,
                                   int64_t workspace_bytes, int64_t T, int32_t n, int32_t d,
                                   hc_dtype dt, void* stream) {
    return post_pre_backward(dH_out, du_next, H, F, w, w_stride, w_next, w_next_stride, gamma_next,
                             eps, dH, dF, dw, dw_next, dgamma_next, nullptr, nullptr, false,
                             workspace, workspace_bytes, T, n, d, enum_value(dt), stream);
}

hc_status hc_post_pre_mix_backward_terms(const void* dH_out, const void* du_next, const void* H,
                                         const void* F, const float* w, int64_t w_stride,
                                         const float* w_next, int64_t w_next_stride,
                                         const float* gamma_next, float eps, const float* dhbar,
                                         const float* coef, void* dH, void* dF, float* dw,
                                         float* dw_next, float* dgamma_next, void* workspace,
                                         int64_t workspace_bytes, int64_t T, int32_t n, int32_t d,
                                         hc_dtype dt, void* stream) {
    return post_pre_backward(dH_out, du_next, H, F, w, w_stride, w_next, w_next_stride, gamma_next,
                             eps, dH, dF, dw, dw_next, dgamma_next, dhbar, coef, true, workspace,
                             workspace_bytes, T, n, d, enum_value(dt), stream);
}

int64_t hc_weights_backward_workspace(int64_t T, int32_t n, int32_t d, int32_t sinkhorn_iters) {
    if (n < 1 || n > HC_MAX_STREAMS || d < 1 || d > HC_MAX_HIDDEN) return 0;
    if (sinkhorn_iters < 0 || sinkhorn_iters > HC_MAX_SINKHORN_ITERS) return 0;
    return hc::weights_backward_workspace_bytes(T, n, d, sinkhorn_iters);
}

namespace {

// hc_weights_backward (terms false: dH out), or hc_weights_backward_terms
// (dhbar and coef out; dH_in and dH NULL).
hc_status weights_backward(const void* H, const void* W, const float* w_static, float scale,
                           float eps, int32_t sinkhorn_iters, const float* dw, const float* dw2,
                           const float* saved, const void* dH_in, void* dH, float* dhbar,
                           float* coef, bool terms, float* dW, float* dw_static, void* workspace,
                           int64_t workspace_bytes, int64_t T, int32_t n, int32_t d, int dt,
                           void* stream) {
    if (!dtype_wide(dt)) return HC_ERR_DTYPE;
    hc_status st = check_nd(n, d, T, dt);
    if (st != HC_OK) return st;
    if (!eps_ok(eps) || !std::isfinite(scale)) return HC_ERR_ARG;
    if (sinkhorn_iters < 0 || sinkhorn_iters > HC_MAX_SINKHORN_ITERS) return HC_ERR_ARG;
    if (T == 0) return HC_OK;
    if (!H || !W || !w_static || !dw || !dW || !dw_static || !workspace) return HC_ERR_NULL;
    if (terms ? (!dhbar || !coef) : !dH) return HC_ERR_NULL;
    if (terms && (dH || dH_in)) return HC_ERR_ARG;
    const int64_t need = hc_weights_backward_workspace(T, n, d, sinkhorn_iters);
    if (workspace_bytes < need) return HC_ERR_ARG;
    if (misaligned(H, 16) || misaligned(W, 16) || misaligned(dH, 16) || misaligned(dH_in, 16) ||
        misaligned(workspace, 16) || misaligned(w_static, 4) || misaligned(dw, 4) ||
        misaligned(dW, 4) || misaligned(dw_static, 4) || misaligned(dw2, 4) || misaligned(saved, 16) ||
        misaligned(dhbar, 16) || misaligned(coef, 4))
        return HC_ERR_ALIGN;
    const int K = record_len(n);
    const int64_t s = elem_bytes(dt);
    // the terms' two outputs take dH's place in the checks below: dhbar
    // [T][d] fp32 and coef [T][2n] fp32, which may not overlap each other
    const Span sdb{dhbar, terms ? T * d * 4 : 0}, sco{coef, terms ? T * 2 * n * 4 : 0};
    if (overlap(sdb, sco)) return HC_ERR_ALIAS;
    const Span sH{H, T * n * d * s}, sW{W, int64_t(K) * d * s}, sS{w_static, int64_t(K) * 4},
        sg{dw, T * K * 4}, sg2{dw2, dw2 ? T * K * 4 : 0}, sin{dH_in, dH_in ? T * n * d * s : 0},
        sdH = terms ? Span{dhbar, T * d * 4} : Span{dH, T * n * d * s},
        sdW{dW, int64_t(K) * d * 4}, sds{dw_static, int64_t(K) * 4},
        sws{workspace, need}, ssv{saved, saved ? hc_weights_saved_bytes(T, n) : 0};
    if (terms)
        for (const Span& i : {sH, sW, sS, sg, sg2, ssv, sdW, sds, sws})
            if (overlap(sco, i)) return HC_ERR_ALIAS;
    const Span ins[] = {sH, sW, sS, sg, sg2, ssv};
    for (const Span& o : {sdH, sdW, sds, sws})
        for (const Span& i : ins)
            if (overlap(o, i)) return HC_ERR_ALIAS;
    if (dH_in && dH_in != dH && overlap(sdH, sin)) return HC_ERR_ALIAS;
    for (const Span& o : {sdW, sds, sws})
        if (overlap(o, sin)) return HC_ERR_ALIAS;
    if (overlap(sdH, sdW) || overlap(sdH, sds) || overlap(sdH, sws) || overlap(sdW, sds) ||
        overlap(sdW, sws) || overlap(sds, sws))
        return HC_ERR_ALIAS;
    return from_hip(hc::launch_weights_backward(H, W, w_static, scale, eps, sinkhorn_iters, dw, dw2,
                                                saved, dH_in, dH, dW, dw_static, workspace, T, n, d, dt,
                                                static_cast<hipStream_t>(stream),
                                                terms ? dhbar : nullptr, terms ? coef : nullptr));
}

}  // namespace

hc_status hc_weights_backward(const void* H, const void* W, const float* w_static, float scale,
                              float eps, int32_t sinkhorn_iters, const float* dw, const float* dw2,
                              const float* saved, const void* dH_in,
                              void* dH, float* dW, float* dw_static, void* workspace,
                              int64_t workspace_bytes, int64_t T, int32_t n, int32_t d, hc_dtype dt,
                              void* stream) {
    return weights_backward(H, W, w_static, scale, eps, sinkhorn_iters, dw, dw2, saved, dH_in, dH,
                            nullptr, nullptr, false, dW, dw_static, workspace, workspace_bytes, T, n,
                            d, enum_value(dt), stream);
}

hc_status hc_weights_backward_terms(const void* H, const void* W, const float* w_static,
                                    float scale, float eps, int32_t sinkhorn_iters, const float* dw,
                                    const float* dw2, const float* saved, float* dhbar, float* coef,
                                    float* dW, float* dw_static, void* workspace,
                                    int64_t workspace_bytes, int64_t T, int32_t n, int32_t d,
                                    hc_dtype dt, void* stream) {
    return weights_backward(H, W, w_static, scale, eps, sinkhorn_iters, dw, dw2, saved, nullptr,
                            nullptr, dhbar, coef, true, dW, dw_static, workspace, workspace_bytes, T,
                            n, d, enum_value(dt), stream);
}

int64_t hc_sinkhorn_backward_workspace(int64_t T, int32_t iters) {
    if (iters < 0 || iters > HC_MAX_SINKHORN_ITERS) return 0;
    return hc::sinkhorn_backward_workspace_bytes(T, iters);
}

hc_status hc_sinkhorn_backward(const float* logits, const float* dw, const float* dw2,
                               float* dlogits, int32_t iters, void* workspace,
                               int64_t workspace_bytes, int64_t T, int32_t n, void* stream) {
    if (n < 1 || n > HC_MAX_STREAMS) return HC_ERR_SHAPE;
    if (T < 0 || iters < 0 || iters > HC_MAX_SINKHORN_ITERS) return HC_ERR_ARG;
    const int K = record_len(n);
    if (T > kMaxBytes / (4 * K)) return HC_ERR_ARG;
    if (T == 0) return HC_OK;
    if (!logits || !dw || !dlogits) return HC_ERR_NULL;
    const int64_t need = hc_sinkhorn_backward_workspace(T, iters);
    if (need > 0 && !workspace) return HC_ERR_NULL;
    if (workspace_bytes < need) return HC_ERR_ARG;
    if (misaligned(logits, 4) || misaligned(dw, 4) || misaligned(dw2, 4) ||
        misaligned(dlogits, 4) || (need > 0 && misaligned(workspace, 4)))
        return HC_ERR_ALIGN;
    const Span sl{logits, T * K * 4}, sg{dw, T * K * 4}, sg2{dw2, dw2 ? T * K * 4 : 0},
        so{dlogits, T * K * 4}, sws{workspace, need};
    if (overlap(so, sl) || overlap(so, sg) || overlap(so, sg2) || overlap(sws, sl) ||
        overlap(sws, sg) || overlap(sws, sg2) || overlap(sws, so))
        return HC_ERR_ALIAS;
    return from_hip(hc::launch_sinkhorn_backward(logits, dw, dw2, dlogits, iters, workspace, T, n,
                                                 static_cast<hipStream_t>(stream)));
}

hc_status hc_sum_records(const float* rec, int64_t T, int32_t K, float* out, void* stream) {
    if (K < 1 || K > 1024) return HC_ERR_SHAPE;
    if (T < 0 || T > kMaxBytes / 4 / K) return HC_ERR_ARG;
    if (T == 0) {
        // the sum over no tokens: zeros into `out` when it is given; `rec`
        // is not read (an empty tensor has no storage) and may be NULL
        if (!out) return HC_OK;
        if (misaligned(out, 4)) return HC_ERR_ALIGN;
        return from_hip(hc::launch_sum_records(rec, 0, K, out, static_cast<hipStream_t>(stream)));
    }
    if (!rec || !out) return HC_ERR_NULL;
    if (misaligned(rec, 4) || misaligned(out, 4)) return HC_ERR_ALIGN;
    if (overlap(Span{rec, T * K * 4}, Span{out, int64_t(K) * 4})) return HC_ERR_ALIAS;
    return from_hip(hc::launch_sum_records(rec, T, K, out, static_cast<hipStream_t>(stream)));
}

hc_status hc_block_tanh(const void* u, void* F, int64_t count, hc_dtype dt_arg, void* stream) {
    const int dt = enum_value(dt_arg);
    if (!dtype_ok(dt)) return HC_ERR_DTYPE;
    if (count < 0 || count > kMaxBytes / 4) return HC_ERR_ARG;
    if (count % vec_elems(dt) != 0) return HC_ERR_SHAPE;
    if (count == 0) return HC_OK;
    if (!u || !F) return HC_ERR_NULL;
    if (misaligned(u, 16) || misaligned(F, 16)) return HC_ERR_ALIGN;
    const int64_t bytes = count * elem_bytes(dt);
    if (overlap(Span{u, bytes}, Span{F, bytes})) return HC_ERR_ALIAS;
    return from_hip(hc::launch_block_tanh(u, F, count, dt, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
