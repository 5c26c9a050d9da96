// hc_post_weights.hip -- the write-back of one layer fused with the per-token
// weights of the next: H' = post(H, F, w) is stored, and the weight record of
// every token is formed from the stored H' while the token is still on chip.
//
// Sources: hfviewer.com glossary "Hyper-connections (mHC)", definition
// (learned mixing of the streams before and after every block; the mHC
// variant's few Sinkhorn iterations); learnaivisually.com "Tencent
// open-sources Hy4 Preview at 770B -- Identity Hyper-Connections", section
// "What four streams cost per token": the cost is the n-fold state moved
// across each layer boundary, so a separate weights pass, which reads that
// state a second time, is the cost to remove.  The per-token weight rule is
// the one hc_weights implements (the pages publish none):
//   r_i = 1/sqrt(mean_k H'_ik^2 + eps),  z_c = (1/n) sum_i r_i (W_c . H'_i),
//   w = w_static + scale * tanh(z)  or  mhc(w_static + scale * z).
//
// Layout ("stream-split"): one workgroup works on one token at a time and
// loops over tokens (persistent).  Four lanes form a quad; lane r of quad Q
// holds stream r at the quad's positions (VPL 16-byte vectors: vector
// Q + v * qn of the row for v < VPL, so that every wave load instruction
// covers 16 consecutive vectors of each stream).  In that layout:
//  - the stream mix H'_r = sum_j A[r][j] H_j + beta_r F takes H_j from quad
//    lane j with a DPP broadcast (quad_perm [j,j,j,j]) that the compiler
//    folds into the multiply-adds, in the same order of operations as
//    hc_post_mix, so H' is bitwise the same;
//  - F is loaded once per quad, a quarter per lane, and broadcast the same
//    way;
//  - the projection is v_mfma_f32_4x4x4_16b_bf16: its 16 independent 4x4
//    blocks are the 16 quads of a wave.  Block rows are the streams (A
//    operand: lane r's own rounded H'_r, 4 positions per k-step), block
//    columns are 4 of the K outputs (B operand: lane c holds W[4g + c] at the
//    same positions), so lane c, register i accumulates the quad's part of
//    P_i[4g + c] = W_{4g+c} . H'_i.  W lives in registers for the whole
//    kernel: each lane holds a quarter of the quad's slice (48 VGPRs at
//    n = 4, d = 4096), loaded once, instead of being re-read per token.
// Per token, the partial P (and the per-stream sums of squares) are added
// over the quads of a row with two DPP rotations, written to LDS, and after
// one workgroup barrier one wave (a different one for each token) adds the
// waves' partials in a fixed order, forms z and the record and stores it.
// The record is not needed by the write-back itself, so nothing waits for
// it; the next token's loads are already in flight.
//
// Limits: W must fit the register budget: d <= 4096 (VPL <= 2 bf16
// vectors, or one FP8 vector, per lane); bf16 and FP8 storage (FP8 values are
// widened exactly to bf16 for the matrix cores, as in hc_weights).
#include <type_traits>

#include "hc_device.h"
#include "hc_launch.h"

namespace hc {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxWaves = 8;    // 512-thread workgroups
#ifndef PFD
#define PFD 1
#endif

// Value of lane J of this lane's quad (DPP quad_perm [J,J,J,J]); written
// with bound_ctrl so that the compiler folds it into the VOP2 instruction
// that consumes it (v_mul_f32_dpp, v_add_f32_dpp).
template <int J>
__device__ __forceinline__ float qb(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), J * 0x55, 0xF, 0xF, true));
}
// x + the same register of the lane 4 (then 8) places round the 16-lane row:
// after both, every lane holds the sum over the 4 quads of its row.
__device__ __forceinline__ float row_quads_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, true));  // row_ror:4
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, true));  // row_ror:8
    return x;
}

// One dword of the write-back: E values (2 bf16 or 4 FP8) of this lane's
// stream, y_e = A[r][0] x0_e + ... + A[r][N-1] x{N-1}_e + beta_r f_e with
// x_j from quad lane j and every f_e from quad lane L.  The first product
// is a v_mul_f32_dpp the compiler emits; the rest are v_fmac_f32 with a
// DPP source, which the compiler does not fold (the accumulator is tied),
// written here with one s_nop 1 for the dword: the two wait states a DPP
// read needs after a VALU write of its source (x and f are computed by the
// instructions just before).  Each value's terms are added in
// hc_post_mix's order: A[r][1], A[r][2], A[r][3], then beta_r f.
#define HC_QP(J) " quad_perm:[" #J "," #J "," #J "," #J "] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define HC_FM(ACC, SRC, MUL, J) "v_fmac_f32_dpp %" #ACC ", %" #SRC ", %" #MUL HC_QP(J)
template <int N, int E, int L> struct MixWord;
template <> struct MixWord<1, 2, 0> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[1], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 6, 0) HC_FM(1, 5, 6, 0)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<1, 2, 1> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[1], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 6, 1) HC_FM(1, 5, 6, 1)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<1, 2, 2> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[1], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 6, 2) HC_FM(1, 5, 6, 2)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<1, 2, 3> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[1], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 6, 3) HC_FM(1, 5, 6, 3)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<2, 2, 0> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[2], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 5, 7, 0) HC_FM(1, 6, 7, 0)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<2, 2, 1> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[2], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 5, 7, 1) HC_FM(1, 6, 7, 1)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<2, 2, 2> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[2], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 5, 7, 2) HC_FM(1, 6, 7, 2)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<2, 2, 3> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[2], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 5, 7, 3) HC_FM(1, 6, 7, 3)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<3, 2, 0> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[3], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 2, 5, 2) HC_FM(1, 3, 5, 2) HC_FM(0, 6, 8, 0) HC_FM(1, 7, 8, 0)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(Ar[2]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<3, 2, 1> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[3], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 2, 5, 2) HC_FM(1, 3, 5, 2) HC_FM(0, 6, 8, 1) HC_FM(1, 7, 8, 1)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(Ar[2]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<3, 2, 2> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[3], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 2, 5, 2) HC_FM(1, 3, 5, 2) HC_FM(0, 6, 8, 2) HC_FM(1, 7, 8, 2)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(Ar[2]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<3, 2, 3> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[3], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 2, 5, 2) HC_FM(1, 3, 5, 2) HC_FM(0, 6, 8, 3) HC_FM(1, 7, 8, 3)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(Ar[2]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<4, 2, 0> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[4], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 2, 5, 2) HC_FM(1, 3, 5, 2) HC_FM(0, 2, 6, 3) HC_FM(1, 3, 6, 3) HC_FM(0, 7, 9, 0) HC_FM(1, 8, 9, 0)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(Ar[2]), "v"(Ar[3]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<4, 2, 1> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[4], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 2, 5, 2) HC_FM(1, 3, 5, 2) HC_FM(0, 2, 6, 3) HC_FM(1, 3, 6, 3) HC_FM(0, 7, 9, 1) HC_FM(1, 8, 9, 1)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(Ar[2]), "v"(Ar[3]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<4, 2, 2> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[4], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 2, 5, 2) HC_FM(1, 3, 5, 2) HC_FM(0, 2, 6, 3) HC_FM(1, 3, 6, 3) HC_FM(0, 7, 9, 2) HC_FM(1, 8, 9, 2)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(Ar[2]), "v"(Ar[3]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<4, 2, 3> {
    static __device__ __forceinline__ void run(float (&y)[2], const float (&x)[2],
                                               const float (&Ar)[4], float br, const float (&f)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 2, 4, 1) HC_FM(1, 3, 4, 1) HC_FM(0, 2, 5, 2) HC_FM(1, 3, 5, 2) HC_FM(0, 2, 6, 3) HC_FM(1, 3, 6, 3) HC_FM(0, 7, 9, 3) HC_FM(1, 8, 9, 3)
            : "+v"(y[0]), "+v"(y[1])
            : "v"(x[0]), "v"(x[1]), "v"(Ar[1]), "v"(Ar[2]), "v"(Ar[3]), "v"(f[0]), "v"(f[1]), "v"(br));
    }
};
template <> struct MixWord<1, 4, 0> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[1], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 8, 12, 0) HC_FM(1, 9, 12, 0) HC_FM(2, 10, 12, 0) HC_FM(3, 11, 12, 0)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<1, 4, 1> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[1], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 8, 12, 1) HC_FM(1, 9, 12, 1) HC_FM(2, 10, 12, 1) HC_FM(3, 11, 12, 1)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<1, 4, 2> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[1], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 8, 12, 2) HC_FM(1, 9, 12, 2) HC_FM(2, 10, 12, 2) HC_FM(3, 11, 12, 2)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<1, 4, 3> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[1], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 8, 12, 3) HC_FM(1, 9, 12, 3) HC_FM(2, 10, 12, 3) HC_FM(3, 11, 12, 3)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<2, 4, 0> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[2], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 9, 13, 0) HC_FM(1, 10, 13, 0) HC_FM(2, 11, 13, 0) HC_FM(3, 12, 13, 0)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<2, 4, 1> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[2], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 9, 13, 1) HC_FM(1, 10, 13, 1) HC_FM(2, 11, 13, 1) HC_FM(3, 12, 13, 1)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<2, 4, 2> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[2], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 9, 13, 2) HC_FM(1, 10, 13, 2) HC_FM(2, 11, 13, 2) HC_FM(3, 12, 13, 2)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<2, 4, 3> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[2], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 9, 13, 3) HC_FM(1, 10, 13, 3) HC_FM(2, 11, 13, 3) HC_FM(3, 12, 13, 3)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<3, 4, 0> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[3], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 4, 9, 2) HC_FM(1, 5, 9, 2) HC_FM(2, 6, 9, 2) HC_FM(3, 7, 9, 2) HC_FM(0, 10, 14, 0) HC_FM(1, 11, 14, 0) HC_FM(2, 12, 14, 0) HC_FM(3, 13, 14, 0)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(Ar[2]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<3, 4, 1> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[3], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 4, 9, 2) HC_FM(1, 5, 9, 2) HC_FM(2, 6, 9, 2) HC_FM(3, 7, 9, 2) HC_FM(0, 10, 14, 1) HC_FM(1, 11, 14, 1) HC_FM(2, 12, 14, 1) HC_FM(3, 13, 14, 1)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(Ar[2]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<3, 4, 2> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[3], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 4, 9, 2) HC_FM(1, 5, 9, 2) HC_FM(2, 6, 9, 2) HC_FM(3, 7, 9, 2) HC_FM(0, 10, 14, 2) HC_FM(1, 11, 14, 2) HC_FM(2, 12, 14, 2) HC_FM(3, 13, 14, 2)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(Ar[2]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<3, 4, 3> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[3], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 4, 9, 2) HC_FM(1, 5, 9, 2) HC_FM(2, 6, 9, 2) HC_FM(3, 7, 9, 2) HC_FM(0, 10, 14, 3) HC_FM(1, 11, 14, 3) HC_FM(2, 12, 14, 3) HC_FM(3, 13, 14, 3)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(Ar[2]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<4, 4, 0> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[4], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 4, 9, 2) HC_FM(1, 5, 9, 2) HC_FM(2, 6, 9, 2) HC_FM(3, 7, 9, 2) HC_FM(0, 4, 10, 3) HC_FM(1, 5, 10, 3) HC_FM(2, 6, 10, 3) HC_FM(3, 7, 10, 3) HC_FM(0, 11, 15, 0) HC_FM(1, 12, 15, 0) HC_FM(2, 13, 15, 0) HC_FM(3, 14, 15, 0)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(Ar[2]), "v"(Ar[3]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<4, 4, 1> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[4], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 4, 9, 2) HC_FM(1, 5, 9, 2) HC_FM(2, 6, 9, 2) HC_FM(3, 7, 9, 2) HC_FM(0, 4, 10, 3) HC_FM(1, 5, 10, 3) HC_FM(2, 6, 10, 3) HC_FM(3, 7, 10, 3) HC_FM(0, 11, 15, 1) HC_FM(1, 12, 15, 1) HC_FM(2, 13, 15, 1) HC_FM(3, 14, 15, 1)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(Ar[2]), "v"(Ar[3]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<4, 4, 2> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[4], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 4, 9, 2) HC_FM(1, 5, 9, 2) HC_FM(2, 6, 9, 2) HC_FM(3, 7, 9, 2) HC_FM(0, 4, 10, 3) HC_FM(1, 5, 10, 3) HC_FM(2, 6, 10, 3) HC_FM(3, 7, 10, 3) HC_FM(0, 11, 15, 2) HC_FM(1, 12, 15, 2) HC_FM(2, 13, 15, 2) HC_FM(3, 14, 15, 2)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(Ar[2]), "v"(Ar[3]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
template <> struct MixWord<4, 4, 3> {
    static __device__ __forceinline__ void run(float (&y)[4], const float (&x)[4],
                                               const float (&Ar)[4], float br, const float (&f)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Ar[0] * qb<0>(x[e]);
        asm("s_nop 1\n\t" HC_FM(0, 4, 8, 1) HC_FM(1, 5, 8, 1) HC_FM(2, 6, 8, 1) HC_FM(3, 7, 8, 1) HC_FM(0, 4, 9, 2) HC_FM(1, 5, 9, 2) HC_FM(2, 6, 9, 2) HC_FM(3, 7, 9, 2) HC_FM(0, 4, 10, 3) HC_FM(1, 5, 10, 3) HC_FM(2, 6, 10, 3) HC_FM(3, 7, 10, 3) HC_FM(0, 11, 15, 3) HC_FM(1, 12, 15, 3) HC_FM(2, 13, 15, 3) HC_FM(3, 14, 15, 3)
            : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
            : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(Ar[1]), "v"(Ar[2]), "v"(Ar[3]), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(br));
    }
};
#undef HC_FM
#undef HC_QP

// bf16x4 (one 4x4x4 MFMA operand) from 4 stored values.
template <typename S> struct Op4;
template <> struct Op4<bf16_t> {
    // a 16-byte vector is two k-steps: dwords (0, 1) and (2, 3)
    static constexpr int kSteps = 2;
    static __device__ __forceinline__ s16x4 get(uint4 v, int s) {
        const u32x2 x = s == 0 ? u32x2{v.x, v.y} : u32x2{v.z, v.w};
        return __builtin_bit_cast(s16x4, x);
    }
};
template <> struct Op4<fp8_t> {
    // a 16-byte vector is four k-steps, one dword each, widened exactly
    static constexpr int kSteps = 4;
    static __device__ __forceinline__ s16x4 get(uint4 v, int s) {
        const uint32_t w = word(v, s);
        const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
        const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
        const u32x2 x = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
        return __builtin_bit_cast(s16x4, x);
    }
};

template <int N, typename S, int VPL>
struct PWGeom {
    static constexpr int K = 2 * N + N * N;       // outputs per token
    static constexpr int G = (K + 3) / 4;         // MFMA column groups
    static constexpr int V = Store<S>::kElems;    // values per 16-byte vector
    static constexpr int SB = Store<S>::kBytes;
    static constexpr int KS = VPL * Op4<S>::kSteps;  // k-steps per group per token
    static constexpr int FB = 4 * VPL;            // bytes of F each quad lane loads
    static constexpr int FE = FB / SB;            // F values per lane
    static constexpr int NV = N * G + 1;          // values per lane to sum: P parts, sum of squares
    static constexpr int NVP = (NV + 3) / 4 * 4;  // a column class's LDS slot, 16-byte multiple
    static constexpr int SLOT = 4 * NVP;          // floats per (wave, row) in LDS
};

// F bytes of one lane: 4, 8 or 16 (one, two or four dwords).
template <int VPL> struct FLoad;
template <> struct FLoad<1> {
    typedef uint32_t T;
    static __device__ __forceinline__ T ld(const uint8_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    static __device__ __forceinline__ uint32_t w(T x, int i) { return x; }
    static __device__ __forceinline__ T make(const uint32_t (&q)[1]) { return q[0]; }
    static __device__ __forceinline__ void st(uint8_t* p, T x) {
        __builtin_nontemporal_store(x, reinterpret_cast<uint32_t*>(p));
    }
};
template <> struct FLoad<2> {
    typedef u32x2 T;
    static __device__ __forceinline__ T ld(const uint8_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    }
    static __device__ __forceinline__ uint32_t w(T x, int i) { return i == 0 ? x.x : x.y; }
    static __device__ __forceinline__ T make(const uint32_t (&q)[2]) { return T{q[0], q[1]}; }
    static __device__ __forceinline__ void st(uint8_t* p, T x) {
        __builtin_nontemporal_store(x, reinterpret_cast<T*>(p));
    }
};
template <> struct FLoad<4> {
    typedef u32x4 T;
    static __device__ __forceinline__ T ld(const uint8_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
    static __device__ __forceinline__ uint32_t w(T x, int i) {
        return i == 0 ? x.x : (i == 1 ? x.y : (i == 2 ? x.z : x.w));
    }
    static __device__ __forceinline__ T make(const uint32_t (&q)[4]) { return T{q[0], q[1], q[2], q[3]}; }
    static __device__ __forceinline__ void st(uint8_t* p, T x) {
        __builtin_nontemporal_store(x, reinterpret_cast<T*>(p));
    }
};

// One token's rows as they arrive: the lane's stream vectors and its share
// of F.
template <int N, typename S, int VPL>
struct Slot {
    uint4 h[VPL];
    typename FLoad<VPL>::T f;
};

// Loads of one token, branch-free: every lane loads from a valid address
// (lanes without data load the token's first vector; tokens past the end
// load the last token) and the values it must not use are zeroed where they
// are consumed.  With loads under branches the compiler cannot count the
// loads in flight and waits for all of them, the prefetch included.
template <int N, typename S, int VPL>
__device__ __forceinline__ void fetch(Slot<N, S, VPL>& sl, const uint8_t* H, const uint8_t* F,
                                      int64_t t, int64_t T, const int64_t (&hoff)[VPL],
                                      int64_t foff, int64_t row_bytes) {
    const int64_t tc = t < T ? t : T - 1;
#pragma unroll
    for (int v = 0; v < VPL; ++v) sl.h[v] = ld16_stream(H + tc * N * row_bytes + hoff[v]);
    sl.f = FLoad<VPL>::ld(F + tc * row_bytes + foff);
}

constexpr int kRing = 32;   // tokens whose records wait in LDS before one store pass

// FULL: every lane holds data (n = 4, the quads cover the row exactly and
// fill the workgroup), so no lane needs a mask.
//
// PRE: the next layer's read-mix as well.  Its input is the stored H' of the
// token, whose alpha is known only once the token's record is formed (after
// the token's barrier, by the wave that forms the record), so the read-mix
// runs two tokens behind the write-back: the rounded H' of every token is
// parked in LDS (each lane its own vectors, three tokens deep), the record
// wave parks alpha beside it, and two steps later every lane reads its share
// of the row of every stream back (lane r of a quad takes the same bytes of
// the row it loads of F), mixes them in hc_pre_mix's order and parks its
// wave's sum of squares; the normalised u is stored a step after that, when
// every wave's sum is visible.  One workgroup barrier per token, as without
// the read-mix; the record ring is halved to leave the LDS for the parked H'.
template <int N, typename S, int VPL, int PF, bool FULL, bool PRE>
__global__ __launch_bounds__(512) void post_weights_kernel(
    const uint8_t* H, const uint8_t* __restrict__ F, const float* __restrict__ w,
    int64_t w_stride, const uint8_t* __restrict__ W, const float* __restrict__ w_static,
    float scale, float eps, int iters, const float* __restrict__ gamma, float pre_eps,
    uint8_t* H_out, float* __restrict__ w_out, uint8_t* __restrict__ u_out,
    float* __restrict__ p_out, float* __restrict__ r_out, int64_t T, int d, int qn) {
    using Gm = PWGeom<N, S, VPL>;
    constexpr int K = Gm::K, G = Gm::G, V = Gm::V, KS = Gm::KS, NV = Gm::NV, NVP = Gm::NVP,
                  FE = Gm::FE, FB = Gm::FB;
    constexpr int E = Word<S>::kElems;
    constexpr int RL = N + N * N;       // [beta | A], the part of a record the write-back reads
    constexpr int SV = N * K + N;       // kept state per token: projections and norms
    constexpr int KP = kMaxWaves * 64 + 1;   // pitch of a parked vector index (16-byte units)
    constexpr int RING = PRE ? kRing / 2 : kRing;
    // per token: the waves' row partials, double-buffered; per wave: the
    // finalising wave's sums and logits; the records (and kept state) of the
    // last 2 RING tokens; the current and next token's [beta | A]; with the
    // read-mix, the parked H' and alpha of three tokens and the waves' sums
    // of squares of two
    __shared__ __attribute__((aligned(16))) float part[2][kMaxWaves][4][Gm::SLOT];
    __shared__ float fin[kMaxWaves][Gm::SLOT + 32];
    __shared__ float oring[2 * RING][K];
    __shared__ float pring[2 * RING][SV];
    __shared__ float recl[2][32];
    __shared__ float wsl[32];
    __shared__ uint4 hkeep[PRE ? 3 * VPL * KP : 1];
    __shared__ float alds[3][4];
    __shared__ float upart[2][kMaxWaves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = FULL ? kMaxWaves : (int)(blockDim.x >> 6);
    const int r = lane & 3, Q = tid >> 2;
    const int nvec = d / V;
    const int64_t row_bytes = (int64_t)d * Gm::SB;
    const int64_t stride = gridDim.x;
    const bool keep = p_out != nullptr;
    // the norms 1/sqrt(sum/d + eps) use the hardware reciprocal square root
    // (v_rsq_f32, about one ulp) on the sum scaled by 1/d: a few
    // instructions where the rounded division and square root took about
    // forty, once per stream for the records and once per token for u
    const float inv_d = 1.0f / (float)d;

    // which of this lane's loads carry data, and from where
    bool hval[VPL];
    int64_t hoff[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int vi = Q + v * qn;
        hval[v] = FULL || (Q < qn && r < N && vi < nvec);
        hoff[v] = hval[v] ? (int64_t)r * row_bytes + (int64_t)vi * 16 : 0;
    }
    // the quad's F bytes: lane r takes bytes [r FB, (r + 1) FB) of its vectors
    const int fvi = Q + ((r * FB) / 16) * qn;
    const bool fval = FULL || (Q < qn && fvi < nvec);
    const int64_t foff = fval ? (int64_t)fvi * 16 + (r * FB) % 16 : 0;

    // this lane's quarter of the quad's W slice: rows 4g + r at the quad's
    // positions, as bf16 MFMA operands (zero past K and past d)
    s16x4 wb[G][KS];
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int c = 4 * g + r, vi = Q + v * qn;
            const uint4 x = (c < K && Q < qn && vi < nvec)
                                ? ld16(W + ((int64_t)c * d + (int64_t)vi * V) * Gm::SB)
                                : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int s = 0; s < Op4<S>::kSteps; ++s) wb[g][v * Op4<S>::kSteps + s] = Op4<S>::get(x, s);
        }
    }
    // the read-mix gain at this lane's share of the row (the F positions)
    float gm[FE];
    if constexpr (PRE) {
        const int64_t g0 = fval ? foff / Gm::SB : 0;
#pragma unroll
        for (int e = 0; e < FE; ++e) gm[e] = gamma[g0 + e];
    }

    // Rows PF tokens ahead.  The record's [beta | A] goes through LDS: every
    // lane loads entry min(lane, RL - 1) of the record PF tokens ahead (one
    // branch-free load), lanes below RL of wave 0 store the next token's into
    // the LDS buffer of that token's parity before the current token's
    // barrier, and every lane reads its own row of A and its beta from there.
    const bool rec_lane = wave == 0 && lane < RL;
    const int rl = lane < RL ? lane : RL - 1;
    // the static part of output lane (loaded once: a load in the loop would
    // wait behind the prefetch)
    const float wst = w_static[lane < K ? lane : K - 1];
    // (every helper below is forced inline: a call would save the live
    // registers to scratch and wait for every load in flight, the prefetch
    // included)
    auto rec_load = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t tc = t < T ? t : T - 1;
        return w[tc * w_stride + N + rl];
    };
    Slot<N, S, VPL> sl[PF + 1];
    float rq[PF + 1];
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        fetch<N, S, VPL>(sl[k], H, F, blockIdx.x + k * stride, T, hoff, foff, row_bytes);
        rq[k] = rec_load(blockIdx.x + k * stride);
    }
    if (rec_lane) recl[0][lane] = rq[0];
    if (tid < K) wsl[tid] = w_static[tid];
    __syncthreads();
    float Arn[N], brn;
    {
        const float* rlds = recl[0];
        brn = r < N ? rlds[r] : 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) Arn[j] = r < N ? rlds[N + r * N + j] : 0.0f;
    }

    // the records (and kept state) of ring block b, in one pass of all lanes
    auto flush = [&](int b, int count) __attribute__((always_inline)) {
        const int base = (b * RING) % (2 * RING);
        for (int e = tid; e < count * K; e += blockDim.x) {
            const int j = e / K, c = e % K;
            const int64_t t = blockIdx.x + (int64_t)(b * RING + j) * stride;
            w_out[t * K + c] = oring[base + j][c];
        }
        if (keep) {
            for (int e = tid; e < count * SV; e += blockDim.x) {
                const int j = e / SV, c = e % SV;
                const int64_t t = blockIdx.x + (int64_t)(b * RING + j) * stride;
                if (c < N * K) p_out[t * N * K + c] = pring[base + j][c];
                else r_out[t * N + (c - N * K)] = pring[base + j][c];
            }
        }
    };

    // The record of local token tf: its totals (the waves' row partials
    // added in a fixed order, all of a lane's loads issued before its adds),
    // norms, projections, z, then tanh or the mHC transform; into the ring
    // (and the kept state).  One wave.  With the read-mix, its alpha is also
    // parked for the read-mix two steps on (so the two agree bitwise).
    auto finish = [&](int tf) __attribute__((always_inline)) {
        float* tt = &fin[wave][0];
        float* lgs = tt + Gm::SLOT;
        for (int j = lane; j < Gm::SLOT; j += 64) {
            float x[kMaxWaves][4];
#pragma unroll
            for (int w2 = 0; w2 < kMaxWaves; ++w2)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) x[w2][rr] = w2 < nw ? part[tf & 1][w2][rr][j] : 0.0f;
            float sum = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < kMaxWaves; ++w2)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sum += x[w2][rr];
            tt[j] = sum;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float* orow = oring[tf % (2 * RING)];
        float* prow = pring[tf % (2 * RING)];
        float* arow = alds[tf % 3];
        float rs[N];
#pragma unroll
        for (int i = 0; i < N; ++i) rs[i] = __builtin_amdgcn_rsqf(fmaf(tt[i * NVP + NV - 1], inv_d, eps));
        if (lane < K) {
            // output c lives in column class c % 4, group c / 4
            const float* pc = tt + (lane & 3) * NVP + (lane >> 2) * N;
            float z = rs[0] * pc[0];
#pragma unroll
            for (int i = 1; i < N; ++i) z = fmaf(rs[i], pc[i], z);
            z = z / (float)N;
            if (keep) {
#pragma unroll
                for (int i = 0; i < N; ++i) prow[i * K + lane] = pc[i];
            }
            if (iters == 0) {
                const float x = wst + scale * tanhf(z);
                orow[lane] = x;
                if (PRE && lane < N) arow[lane] = x;
            } else {
                lgs[lane] = fmaf(scale, z, wst);
            }
        }
        if (keep && lane < N) prow[N * K + lane] = rs[lane];
        if (iters > 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // four lanes, lane r owns row r (the other quads idle)
            const bool mine = lane < 4 && r < N;
            float a = 0.0f, b = 0.0f, row[N];
            if (mine) {
                a = lgs[r];
                b = lgs[N + r];
            }
#pragma unroll
            for (int j = 0; j < N; ++j) row[j] = mine ? lgs[2 * N + r * N + j] : 0.0f;
            mhc_quad<N>(r, a, b, row, iters);
            if (mine) {
                orow[r] = a;
                if constexpr (PRE) arow[r] = a;
                orow[N + r] = b;
#pragma unroll
                for (int j = 0; j < N; ++j) orow[2 * N + r * N + j] = row[j];
            }
        }
    };

    // The tanh-mode record of local token tf, outputs 4g + c of column class
    // c, by one wave (four waves share a token's record).  Two lanes per
    // total: lane q (< 32) adds the partials of slots 0..15, lane q + 32 those
    // of slots 16..31, each in slot order, and the halves are added across
    // the wave halves.  Totals: the N sums of squares, then P_i[4g + c].
    auto finish_c = [&](int tf, int c) __attribute__((always_inline)) {
        constexpr int NT = N + G * N;
        float* tt = &fin[wave][0];
        const int q = lane & 31, half = lane >> 5;
        const int j = q < N ? q * NVP + NV - 1 : c * NVP + (q < NT ? q - N : 0);
        float x[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int sidx = 16 * half + k;
            const float y = part[tf & 1][sidx >> 2][sidx & 3][j];
            x[k] = (FULL || (sidx >> 2) < nw) ? y : 0.0f;
        }
        float v = x[0];
#pragma unroll
        for (int k = 1; k < 16; ++k) v += x[k];
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                         false);
        v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if (lane < NT) tt[lane] = v;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float* orow = oring[tf % (2 * RING)];
        float* prow = pring[tf % (2 * RING)];
        float rs[N];
#pragma unroll
        for (int i = 0; i < N; ++i) rs[i] = __builtin_amdgcn_rsqf(fmaf(tt[i], inv_d, eps));
        const int g = lane, o = 4 * lane + c;
        if (g < G && o < K) {
            const float* pc = tt + N + g * N;
            float z = rs[0] * pc[0];
#pragma unroll
            for (int i = 1; i < N; ++i) z = fmaf(rs[i], pc[i], z);
            z = z / (float)N;
            if (keep) {
#pragma unroll
                for (int i = 0; i < N; ++i) prow[i * K + o] = pc[i];
            }
            const float rec = wsl[o] + scale * tanhf(z);
            orow[o] = rec;
            if (PRE && o < N) alds[tf % 3][o] = rec;
        }
        if (keep && c == 0 && lane < N) prow[N * K + lane] = rs[lane];
    };
    // the record of local token tf: four waves in tanh mode, one in mHC mode
    auto finish_any = [&](int tf) __attribute__((always_inline)) {
        if (iters == 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (c < K && wave == (tf + c) % nw) finish_c(tf, c);
        } else if (wave == tf % nw) {
            finish(tf);
        }
    };

    // The read-mix of local token tf from its parked H': this lane's FE
    // positions of every stream (quad lane j's copy), x = sum_j alpha_j h_j
    // in hc_pre_mix's order, and the wave's sum of x^2 into upart.
    float xk[FE];
    auto pre_mix = [&](int tf, const float (&al)[N]) __attribute__((always_inline)) {
        typedef typename FLoad<VPL>::T FW;
        const int vv = (r * FB) / 16, wo = ((r * FB) % 16) / 4;
        const uint32_t* kp =
            reinterpret_cast<const uint32_t*>(&hkeep[(tf % 3) * VPL * KP + vv * KP + 4 * Q]) + wo;
        float h[N][FE];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const FW x = *reinterpret_cast<const FW*>(kp + 4 * j);
#pragma unroll
            for (int q = 0; q < FE / E; ++q) unpack_word<S>(FLoad<VPL>::w(x, q), h[j] + q * E);
        }
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < FE; ++e) {
            float x = al[0] * h[0][e];
#pragma unroll
            for (int j = 1; j < N; ++j) x = fmaf(al[j], h[j][e], x);
            xk[e] = x;
            ss = fmaf(x, x, ss);
        }
        ss = wave_sum(fval ? ss : 0.0f);
        if (lane == 0) upart[tf & 1][wave] = ss;
    };
    // u of local token tf from xk, once every wave's sum is visible
    auto u_store = [&](int tf) __attribute__((always_inline)) {
        float us[kMaxWaves];
#pragma unroll
        for (int i = 0; i < kMaxWaves; ++i) us[i] = i < nw ? upart[tf & 1][i] : 0.0f;
        float s = us[0];
#pragma unroll
        for (int i = 1; i < kMaxWaves; ++i) s += us[i];
        const float rr = __builtin_amdgcn_rsqf(fmaf(s, inv_d, pre_eps));
        uint32_t q[FB / 4];
#pragma unroll
        for (int k = 0; k < FB / 4; ++k) {
            float o[E];
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = gm[k * E + e] * (xk[k * E + e] * rr);
            q[k] = pack_word<S>(o);
        }
        const int64_t t = blockIdx.x + (int64_t)tf * stride;
        if (fval) FLoad<VPL>::st(u_out + t * row_bytes + foff, FLoad<VPL>::make(q));
    };

    int tl = 0;   // tokens this workgroup has done
    // one token; ST = how many earlier tokens there are, capped at 2 (the
    // read-mix of the token two back needs two)
    auto step = [&](auto kc, auto stc, int64_t t) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        constexpr int ST = decltype(stc)::value;
        const int64_t ta = t + PF * stride;
        fetch<N, S, VPL>(sl[(k + PF) % (PF + 1)], H, F, ta, T, hoff, foff, row_bytes);
        rq[(k + PF) % (PF + 1)] = rec_load(ta);
        Slot<N, S, VPL>& cur = sl[k];

        // the read-mix of the token two back (its alpha parked after the
        // previous barrier), and the u of the one before it
        if constexpr (PRE && ST >= 2) {
            float al[N];
#pragma unroll
            for (int j = 0; j < N; ++j) al[j] = alds[(tl - 2) % 3][j];
            if (tl >= 3) u_store(tl - 3);
            pre_mix(tl - 2, al);
        }

        // this lane's row of A and its beta, read from LDS a token ago
        float Ar[N], br = brn;
#pragma unroll
        for (int j = 0; j < N; ++j) Ar[j] = Arn[j];
        // the quad's F values held by this lane
        float fv[FE];
#pragma unroll
        for (int q = 0; q < FE / E; ++q) {
            const uint32_t fw = FLoad<VPL>::w(cur.f, q);
            unpack_word<S>(fval ? fw : 0u, fv + q * E);
        }

        // write-back, dword by dword, in hc_post_mix's order of operations
        uint4 o[VPL];
        uint8_t* Ot = H_out + t * N * row_bytes;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            uint32_t ow[4];
#pragma unroll
            for (int qw = 0; qw < 4; ++qw) {
                float h[E], y[E];
                const uint32_t hw = word(cur.h[v], qw);
                unpack_word<S>(hval[v] ? hw : 0u, h);
                // positions p0 .. p0 + E - 1 of the quad; their F values are
                // held by quad lane p0 / FE
                const int p0 = v * V + qw * E;
                float fw[E];
#pragma unroll
                for (int e = 0; e < E; ++e) fw[e] = fv[(p0 + e) % FE];
                switch (p0 / FE) {
                    case 0: MixWord<N, E, 0>::run(y, h, Ar, br, fw); break;
                    case 1: MixWord<N, E, 1>::run(y, h, Ar, br, fw); break;
                    case 2: MixWord<N, E, 2>::run(y, h, Ar, br, fw); break;
                    default: MixWord<N, E, 3>::run(y, h, Ar, br, fw); break;
                }
                ow[qw] = pack_word<S>(y);
            }
            o[v] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
            if (FULL || hval[v]) st16_stream(Ot + hoff[v], o[v]);
            if constexpr (PRE) hkeep[(tl % 3) * VPL * KP + v * KP + tid] = o[v];
        }

        // the next layer's weights from the stored values: sums of squares
        // and the quad's part of every projection; each column group is
        // summed over the row's quads and parked in LDS as soon as its
        // k-steps are done
        float* pt = &part[tl & 1][wave][lane >> 4][r * NVP];
        const bool lead = (lane & 12) == 0;     // quad 0 of each row writes
        float ss = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
#pragma unroll
            for (int s = 0; s < Op4<S>::kSteps; ++s) {
                // (the words are copied out of the vector first: hipcc
                // bit-casts a vector element as if it were element 0)
                const u32x2 aw = __builtin_bit_cast(u32x2, Op4<S>::get(o[v], s));
                const uint32_t a0 = aw.x, a1 = aw.y;
                ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a0),
                                                     __builtin_bit_cast(bf16x2, a0), ss, false);
                ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a1),
                                                     __builtin_bit_cast(bf16x2, a1), ss, false);
            }
        }
        ss = row_quads_sum(ss);
        if (lead) pt[NV - 1] = ss;
        // the column groups' accumulators advance together: G independent
        // chains of dependent MFMAs instead of one chain at a time
        f32x4 acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int s = 0; s < Op4<S>::kSteps; ++s) {
                const s16x4 a = Op4<S>::get(o[v], s);
#pragma unroll
                for (int g = 0; g < G; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, wb[g][v * Op4<S>::kSteps + s],
                                                                  acc[g], 0, 0, 0);
            }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float x[4];
#pragma unroll
            for (int i = 0; i < N; ++i) x[i] = row_quads_sum(acc[g][i]);
            if (lead) {
                if constexpr (N == 4) {
                    *reinterpret_cast<float4*>(pt + 4 * g) = make_float4(x[0], x[1], x[2], x[3]);
                } else {
#pragma unroll
                    for (int i = 0; i < N; ++i) pt[g * N + i] = x[i];
                }
            }
        }
        // the next token's [beta | A] for every wave after the barrier
        if (rec_lane) recl[(tl + 1) & 1][lane] = rq[(k + 1) % (PF + 1)];
        __syncthreads();

        // the records in the ring up to the previous token are visible to
        // every lane from here on: store a full block of them
        if (tl % RING == 0 && tl > 0) flush(tl / RING - 1, RING);

        // the next token's row of A and beta, into registers now so that
        // its LDS latency is not on the next token's path
        {
            const float* rlds = recl[(tl + 1) & 1];
            brn = r < N ? rlds[r] : 0.0f;
#pragma unroll
            for (int j = 0; j < N; ++j) Arn[j] = r < N ? rlds[N + r * N + j] : 0.0f;
        }

        // this token's record
        finish_any(tl);
        ++tl;
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    int64_t t0 = blockIdx.x;
    if (t0 + PF * stride < T) {
        // the first round: with the read-mix, its tokens have fewer than two
        // earlier ones
        step(I0{}, I0{}, t0);
        if constexpr (PF >= 1) step(I1{}, I1{}, t0 + stride);
        if constexpr (PF >= 2) step(I2{}, I2{}, t0 + 2 * stride);
        t0 += (PF + 1) * stride;
        // whole rounds of PF + 1 tokens with no test per token, then the rest
        for (; t0 + PF * stride < T; t0 += (PF + 1) * stride) {
            step(I0{}, I2{}, t0);
            if constexpr (PF >= 1) step(I1{}, I2{}, t0 + stride);
            if constexpr (PF >= 2) step(I2{}, I2{}, t0 + 2 * stride);
        }
        if (t0 < T) step(I0{}, I2{}, t0);
        if constexpr (PF >= 1) {
            if (t0 + stride < T) step(I1{}, I2{}, t0 + stride);
        }
        if constexpr (PF >= 2) {
            if (t0 + 2 * stride < T) step(I2{}, I2{}, t0 + 2 * stride);
        }
    } else {
        // fewer than PF + 1 tokens (the grid never exceeds T, so at least one)
        step(I0{}, I0{}, t0);
        if constexpr (PF >= 1) {
            if (t0 + stride < T) step(I1{}, I1{}, t0 + stride);
        }
    }
    if constexpr (PRE) {
        // the read-mix of the last two tokens and the u of the last three,
        // each once what it reads is visible
        float al[N];
        if (tl >= 2) {
#pragma unroll
            for (int j = 0; j < N; ++j) al[j] = alds[(tl - 2) % 3][j];
            if (tl >= 3) u_store(tl - 3);
            pre_mix(tl - 2, al);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < N; ++j) al[j] = alds[(tl - 1) % 3][j];
        if (tl >= 2) u_store(tl - 2);
        pre_mix(tl - 1, al);
        __syncthreads();
        u_store(tl - 1);
    }
    // every record not yet stored, once the last one is visible
    __syncthreads();
    // blocks flushed in the loop: at steps m RING <= tl - 1, m >= 1
    const int done = tl >= 1 ? ((tl - 1) / RING) * RING : 0;
    for (int b = done / RING; b * RING < tl; ++b)
        flush(b, (tl - b * RING) < RING ? tl - b * RING : RING);
}

template <int N, typename S, int VPL, int PF, bool PRE>
hipError_t go(const void* H, const void* F, const float* w, int64_t w_stride, const void* W,
              const float* w_static, float scale, float eps, int iters, const float* gamma,
              float pre_eps, void* H_out, float* w_out, void* u_out, float* P, float* rn, int64_t T,
              int d, hipStream_t s) {
    const int nvec = d / Store<S>::kElems;
    const int qn = (nvec + VPL - 1) / VPL;
    const int block = (4 * qn + 63) / 64 * 64;
    const bool full = N == 4 && qn * VPL == nvec && 4 * qn == block;
    void (*kernel)(const uint8_t*, const uint8_t*, const float*, int64_t, const uint8_t*, const float*,
                   float, float, int, const float*, float, uint8_t*, float*, uint8_t*, float*, float*,
                   int64_t, int, int) = post_weights_kernel<N, S, VPL, PF, false, PRE>;
    if constexpr (N == 4) {
        if (full) kernel = post_weights_kernel<N, S, VPL, PF, true, PRE>;
    }
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel),
                                                         block, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    const int64_t resident = (int64_t)cus * per_cu;
    const dim3 grid((unsigned)(T < resident ? T : resident));
    return launch(kernel, grid, dim3(block), 0, s, static_cast<const uint8_t*>(H),
                  static_cast<const uint8_t*>(F), w, w_stride, static_cast<const uint8_t*>(W), w_static,
                  scale, eps, iters, gamma, pre_eps, static_cast<uint8_t*>(H_out), w_out,
                  static_cast<uint8_t*>(u_out), P, rn, T, d, qn);
}

struct PWArgs {
    const void* H; const void* F; const float* w; int64_t w_stride; const void* W;
    const float* w_static; float scale; float eps; int iters; const float* gamma; float pre_eps;
    void* H_out; float* w_out; void* u_out; float* P; float* rn; int64_t T; int d; hipStream_t s;
};

template <int N, typename S, int VPL>
hipError_t go_pre(const PWArgs& a) {
    if (a.u_out != nullptr)
        return go<N, S, VPL, PFD, true>(a.H, a.F, a.w, a.w_stride, a.W, a.w_static, a.scale, a.eps,
                                        a.iters, a.gamma, a.pre_eps, a.H_out, a.w_out, a.u_out, a.P,
                                        a.rn, a.T, a.d, a.s);
    return go<N, S, VPL, PFD, false>(a.H, a.F, a.w, a.w_stride, a.W, a.w_static, a.scale, a.eps,
                                     a.iters, nullptr, 0.0f, a.H_out, a.w_out, nullptr, a.P, a.rn,
                                     a.T, a.d, a.s);
}

template <typename S, int VPL>
hipError_t by_n(int n, const PWArgs& a) {
    switch (n) {
        case 1: return go_pre<1, S, VPL>(a);
        case 2: return go_pre<2, S, VPL>(a);
        case 3: return go_pre<3, S, VPL>(a);
        case 4: return go_pre<4, S, VPL>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int post_weights_max_hidden(int dt) {
    // W's slice per lane of a 512-thread workgroup: at most four bf16 vectors
    // or two FP8 vectors per lane (96 VGPRs at n = 4)
    return dt == 1 ? 4096 : (dt == 2 ? 4096 : 0);
}

hipError_t launch_post_mix_weights(const void* H, const void* F, const float* w, int64_t w_stride,
                                   const void* W, const float* w_static, float scale, float eps,
                                   int iters, const float* gamma, float pre_eps, void* H_out,
                                   float* w_out, void* u_out, float* P, float* rn, int64_t T, int n,
                                   int d, int dt, hipStream_t s) {
    const PWArgs a = {H, F, w, w_stride, W, w_static, scale, eps, iters, gamma, pre_eps,
                      H_out, w_out, u_out, P, rn, T, d, s};
    // vectors per lane: as few as fill at most 128 quads (512 threads)
    if (dt == 2) {
        const int nvec = d / Store<fp8_t>::kElems;
        if (nvec <= 128) return by_n<fp8_t, 1>(n, a);
        return by_n<fp8_t, 2>(n, a);
    }
    const int nvec = d / Store<bf16_t>::kElems;
    if (nvec <= 128) return by_n<bf16_t, 1>(n, a);
    if (nvec <= 256) return by_n<bf16_t, 2>(n, a);
    return by_n<bf16_t, 4>(n, a);
}

}  // namespace hc
