// hc_device.h -- device helpers shared by the libhc.so kernels (gfx950).
//
// Storage: 16-byte vectors (8 bf16 or 4 fp32 values) are the unit of every
// HBM access; values are widened to fp32 in registers and rounded once on the
// way out (nearest, ties to even, via the hardware bf16 packer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

// Tag types for the two storage formats.
struct f32_t {};
struct bf16_t {};

template <typename S> struct Store;
template <> struct Store<f32_t> { static constexpr int kElems = 4; static constexpr int kBytes = 4; };
template <> struct Store<bf16_t> { static constexpr int kElems = 8; static constexpr int kBytes = 2; };

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

template <typename S> __device__ __forceinline__ uint4 pack(const float* f);
template <> __device__ __forceinline__ uint4 pack<bf16_t>(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}
template <> __device__ __forceinline__ uint4 pack<f32_t>(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
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

}  // namespace hc
