// hc_device.h -- device helpers shared by the libhc.so kernels (gfx950).
//
// Storage: 16-byte vectors (4 fp32, 8 bf16 or 16 fp8 values) are the unit of
// every HBM access; values are widened to fp32 in registers and rounded once
// on the way out (nearest, ties to even, via the hardware packers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

// Tag types for the storage formats.  fp8_t is E4M3 (the OCP 8-bit float:
// 4 exponent bits, bias 7, 3 mantissa bits, no infinities, largest 448).
struct f32_t {};
struct bf16_t {};
struct fp8_t {};

template <typename S> struct Store;
template <> struct Store<f32_t> { static constexpr int kElems = 4; static constexpr int kBytes = 4; };
template <> struct Store<bf16_t> { static constexpr int kElems = 8; static constexpr int kBytes = 2; };
template <> struct Store<fp8_t> { static constexpr int kElems = 16; static constexpr int kBytes = 1; };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
    *reinterpret_cast<uint4*>(p) = v;
}
// Streaming variants: data touched once; hint the caches not to keep it.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16_stream(void* p, uint4 v) {
    const u32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> two bf16 in one dword (element 0 in the low half), rounded to
// nearest even by v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 f = {lo, hi};
    bf16x2 b = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// FP8 E4M3: four codes per dword, element 0 in the low byte.  Widening is
// exact (v_cvt_pk_f32_fp8 decodes two codes).  Narrowing rounds to nearest
// even with v_cvt_pk_fp8_f32, which turns anything beyond the largest finite
// code into NaN; values are first saturated to [-448, 448] with the IEEE
// maximum/minimum operations (v_maximum3/v_minimum3), which pass NaN through,
// so NaN stays NaN and only overflow is clipped.
__device__ __forceinline__ void unpack_fp8x4(uint32_t w, float* f) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo.x; f[1] = lo.y; f[2] = hi.x; f[3] = hi.y;
}
__device__ __forceinline__ float sat_fp8(float x) {
    return __builtin_elementwise_minimum(__builtin_elementwise_maximum(x, -448.0f), 448.0f);
}
__device__ __forceinline__ uint32_t pack_fp8x4(const float* f) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_fp8(f[0]), sat_fp8(f[1]), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_fp8(f[2]), sat_fp8(f[3]), w, true);
    return (uint32_t)w;
}

template <typename S> __device__ __forceinline__ void unpack(uint4 v, float* f);
template <> __device__ __forceinline__ void unpack<bf16_t>(uint4 v, float* f) {
    f[0] = lo_bf16(v.x); f[1] = hi_bf16(v.x);
    f[2] = lo_bf16(v.y); f[3] = hi_bf16(v.y);
    f[4] = lo_bf16(v.z); f[5] = hi_bf16(v.z);
    f[6] = lo_bf16(v.w); f[7] = hi_bf16(v.w);
}
template <> __device__ __forceinline__ void unpack<f32_t>(uint4 v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <> __device__ __forceinline__ void unpack<fp8_t>(uint4 v, float* f) {
    unpack_fp8x4(v.x, f); unpack_fp8x4(v.y, f + 4);
    unpack_fp8x4(v.z, f + 8); unpack_fp8x4(v.w, f + 12);
}

template <typename S> __device__ __forceinline__ uint4 pack(const float* f);
template <> __device__ __forceinline__ uint4 pack<bf16_t>(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}
template <> __device__ __forceinline__ uint4 pack<f32_t>(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
}
template <> __device__ __forceinline__ uint4 pack<fp8_t>(const float* f) {
    return make_uint4(pack_fp8x4(f), pack_fp8x4(f + 4), pack_fp8x4(f + 8), pack_fp8x4(f + 12));
}

// Per-dword access: a 16-byte vector is 4 dwords of kWordElems values each
// (1 fp32, 2 bf16, 4 fp8).  Kernels that work dword by dword keep fewer
// values live at once than a whole-vector unpack.
template <typename S> struct Word { static constexpr int kElems = 4 / Store<S>::kBytes; };

__device__ __forceinline__ uint32_t word(const uint4& v, int q) {
    return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
}

template <typename S> __device__ __forceinline__ void unpack_word(uint32_t w, float* f);
template <> __device__ __forceinline__ void unpack_word<f32_t>(uint32_t w, float* f) {
    f[0] = __uint_as_float(w);
}
template <> __device__ __forceinline__ void unpack_word<bf16_t>(uint32_t w, float* f) {
    f[0] = lo_bf16(w); f[1] = hi_bf16(w);
}
template <> __device__ __forceinline__ void unpack_word<fp8_t>(uint32_t w, float* f) {
    unpack_fp8x4(w, f);
}

template <typename S> __device__ __forceinline__ uint32_t pack_word(const float* f);
template <> __device__ __forceinline__ uint32_t pack_word<f32_t>(const float* f) {
    return __float_as_uint(f[0]);
}
template <> __device__ __forceinline__ uint32_t pack_word<bf16_t>(const float* f) {
    return pack_bf16x2(f[0], f[1]);
}
template <> __device__ __forceinline__ uint32_t pack_word<fp8_t>(const float* f) {
    return pack_fp8x4(f);
}

// Makes the compiler treat v as changed here, so values it derived from v
// before (unpacked fp32 copies) are recomputed after this point instead of
// being kept live in registers.  Emits no instruction.
__device__ __forceinline__ void opaque(uint4& v) {
    u32x4 x = {v.x, v.y, v.z, v.w};
    asm volatile("" : "+v"(x));
    v = make_uint4(x.x, x.y, x.z, x.w);
}

// Sum over the 64 lanes of a wave with DPP row shifts and row broadcasts (no
// LDS traffic): prefix sums of 4, 8 and 16 inside each row, then rows 0+1
// and 2+3, then the two halves; the total lands in lane 63 and is broadcast
// from there, so every lane returns the same value in a fixed order.
#define HC_DPP(v, ctrl, rm, bm)                                                         \
    __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), (ctrl), (rm), (bm), false))
__device__ __forceinline__ float wave_sum(float v) {
    v += HC_DPP(v, 0x111, 0xF, 0xF);    // row_shr:1
    v += HC_DPP(v, 0x112, 0xF, 0xF);    // row_shr:2
    v += HC_DPP(v, 0x114, 0xF, 0xE);    // row_shr:4, lanes 4..15 of each row
    v += HC_DPP(v, 0x118, 0xF, 0xC);    // row_shr:8, lanes 8..15 of each row
    v += HC_DPP(v, 0x142, 0xA, 0xF);    // row_bcast:15 into rows 1 and 3
    v += HC_DPP(v, 0x143, 0xC, 0xF);    // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
#undef HC_DPP

// Sum over the block: waves reduce, then every thread adds the per-wave
// partials in wave order.  The order depends only on blockDim.  `red` holds
// at least blockDim/64 floats; the trailing barrier lets the caller reuse it.
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = red[0];
    for (int i = 1; i < nw; ++i) s += red[i];
    __syncthreads();
    return s;
}

// ---------------------------------------------------------- mHC record

// DPP quad permutes: swap neighbours (1,0,3,2) and pairs (2,3,0,1).
__device__ __forceinline__ float quad_swap1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_swap2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// Sum / max over the 4 lanes of a quad; every lane gets the same value (each
// step adds the same two operands on both partners).
__device__ __forceinline__ float quad_sum(float v) {
    v += quad_swap1(v);
    return v + quad_swap2(v);
}
__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, quad_swap1(v));
    return fmaxf(v, quad_swap2(v));
}

// The mHC transform of one token, spread over the 4 lanes of a quad: lane r
// owns alpha_r, beta_r and row r of the n x n mix (lanes r >= N hold zeros
// and take part only in the column sums).  On entry a, b and row[] are the
// logits, on exit the weights:
//   alpha = sigmoid(l_alpha), beta = sigmoid(l_beta),
//   A = exp(l_A) normalised `iters` times, rows then columns.
// With iters >= 1 the largest logit of A is subtracted before exp; the first
// row division removes any common factor, so exact results are unchanged.
// Must be called by all 4 lanes of the quad (no divergence around DPP).
template <int N>
__device__ __forceinline__ void mhc_quad(int r, float& a, float& b, float (&row)[N], int iters) {
    const bool live = r < N;
    a = 1.0f / (1.0f + expf(-a));
    b = 1.0f / (1.0f + expf(-b));
    float m = 0.0f;
    if (iters > 0) {
        m = live ? row[0] : -INFINITY;
#pragma unroll
        for (int j = 1; j < N; ++j) m = live ? fmaxf(m, row[j]) : m;
        m = quad_max(m);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) row[j] = live ? expf(row[j] - m) : 0.0f;
    for (int it = 0; it < iters; ++it) {
        float s = row[0];
#pragma unroll
        for (int j = 1; j < N; ++j) s += row[j];
        const float sd = live ? s : 1.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) row[j] = row[j] / sd;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const float c = quad_sum(row[j]);
            row[j] = row[j] / c;
        }
    }
}

}  // namespace hc
