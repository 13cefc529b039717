// Device helpers shared by the bf16 scan kernels (gfx950): MFMA wrappers, the LDS transpose
// read that builds MFMA operands whose K index is a row index of a row-major LDS tile, a
// wavefront inclusive scan, and the rotation of 8-element row pieces by fp16 (cos, sin) pairs.
#pragma once

#include "m3_common.h"

namespace m3 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read (16-bit elements): within each group of 16 lanes, lane i
// receives element i % 4 of the 4 elements read by lanes i/4 + 4k, k = 0..3.
// With lane i of the group pointing at &M[r0 + i/4][c0 + 4*(i%4)] of a
// row-major bf16 matrix M, lane i receives M[r0 + k][c0 + i] for k = 0..3.
__device__ __forceinline__ bf16x4 ds_read_tr(const bf16 *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}
// 8 K-values (rows r0 .. r0+3 and r1 .. r1+3) of column c0 + (lane % 16) of a
// row-major [rows][ld] bf16 matrix, as an MFMA operand.
__device__ __forceinline__ bf16x8 tr_operand(const bf16 *m, int ld, int r0, int r1, int c0, int l16) {
    const bf16x4 a = ds_read_tr(m + (r0 + l16 / 4) * ld + c0 + 4 * (l16 % 4));
    const bf16x4 b = ds_read_tr(m + (r1 + l16 / 4) * ld + c0 + 4 * (l16 % 4));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// The value, made opaque to the compiler when ON: address math derived from it is then
// recomputed where it is used instead of being hoisted out of the chunk loop (and spilled).
template <bool ON>
__device__ __forceinline__ int opaque(int v) {
    if constexpr (ON) asm volatile("" : "+v"(v));
    return v;
}

// Wait for this wave's outstanding LDS operations (wave-private staging).
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xc07f); }

__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
    (void)lane;
    return wave_scan_dpp(v);   // DPP lane moves (no LDS round trip)
}
// The value of lane l (uniform l) in every lane.
__device__ __forceinline__ float wave_bcast(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Maximum over the 64 lanes of values >= 0, in every lane (a DPP max-scan, then lane 63's value).
__device__ __forceinline__ float wave_max_nonneg(float v) {
    v = fmaxf(v, dpp_move<0x111>(v));
    v = fmaxf(v, dpp_move<0x112>(v));
    v = fmaxf(v, dpp_move<0x114>(v));
    v = fmaxf(v, dpp_move<0x118>(v));
    v = fmaxf(v, dpp_move<0x142, 0xA>(v));
    v = fmaxf(v, dpp_move<0x143, 0xC>(v));
    return wave_bcast(v, 63);
}

// (sin x, cos x) for the fp32 state rotation by a chunk's total angle: x reduced by 2 pi in three
// fused steps (Cody-Waite: 2 pi = C1 + C2 + C3, C1 with 8 significant bits, so k C1 is exact for
// |k| < 2^16), then the hardware sine and cosine of the remainder in [-pi, pi]. Absolute error
// about 4e-7 for |x| up to 1e4, without the branches and the wide-argument path of sincosf (a
// divergent branch that every wave holding one chunk-end lane would execute in full).
__device__ __forceinline__ void sincos_state(float x, float *s, float *c) {
    const float k = rintf(x * 0.15915494309189535f);
    float r = fmaf(-k, 6.28125f, x);
    r = fmaf(-k, 1.9353071693331003e-3f, r);
    r = fmaf(-k, 1.0253131677018246e-11f, r);
    __sincosf(r, s, c);
}
// 2^x for x <= 0 (hardware exp2; results below the fp32 normal range flush to 0)
__device__ __forceinline__ float exp2_neg(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotate the 4 pairs of an 8-element row piece by -Phi: (u, v) -> (c u + s v, -s u + c v),
// with (cos, sin) of the 4 pairs packed as fp16 in cs.
__device__ __forceinline__ void rot_piece_f(const float (&in)[8], const f16x8 cs, float (&o)[8]) {
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const float c = (float)cs[2 * m], sn = (float)cs[2 * m + 1];
        const float u = in[2 * m], v = in[2 * m + 1];
        o[2 * m] = c * u + sn * v;
        o[2 * m + 1] = c * v - sn * u;
    }
}
// The same rotation with (cos, sin) packed as bf16 pairs, on the bf16 dot-product instruction,
// rounded to bf16: each output is one v_dot2_f32_bf16 (two bf16 products summed in fp32) of the
// raw pair, so neither the row nor the table is widened. The first output of a pair takes
// (c, s).(u, v); the second takes the pair swapped (a 16-bit funnel shift) against (c, -s) (the
// instruction's neg_hi modifier on the table operand, which the builtin cannot express). One asm
// block per 8-element piece, ordered for the hazards the compiler cannot see inside it: the
// swaps come first, so every dot product reads registers written at least four instructions
// earlier, and every dot product's result is read at least three instructions after it is
// written (its required wait states) by the block's own multiplies or conversions, so the block
// leaves only VALU-written registers behind. With scale: each result times s before rounding.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 rot_pack_bf(const bf16x8 raw, const bf16x8 cs) {
    const u32x4 x = __builtin_bit_cast(u32x4, raw), c = __builtin_bit_cast(u32x4, cs);
    u32x4 r;
    float t0, t1, t2, t3, t4, t5, t6, t7;
    asm("v_alignbit_b32 %5, %16, %16, 16\n\t"
        "v_alignbit_b32 %7, %17, %17, 16\n\t"
        "v_alignbit_b32 %9, %18, %18, 16\n\t"
        "v_alignbit_b32 %11, %19, %19, 16\n\t"
        "v_dot2_f32_bf16 %4, %12, %16, 0\n\t"
        "v_dot2_f32_bf16 %6, %13, %17, 0\n\t"
        "v_dot2_f32_bf16 %8, %14, %18, 0\n\t"
        "v_dot2_f32_bf16 %10, %15, %19, 0\n\t"
        "v_dot2_f32_bf16 %5, %12, %5, 0 neg_hi:[1,0,0]\n\t"
        "v_dot2_f32_bf16 %7, %13, %7, 0 neg_hi:[1,0,0]\n\t"
        "v_dot2_f32_bf16 %9, %14, %9, 0 neg_hi:[1,0,0]\n\t"
        "v_dot2_f32_bf16 %11, %15, %11, 0 neg_hi:[1,0,0]\n\t"
        "v_cvt_pk_bf16_f32 %0, %4, %5\n\t"
        "v_cvt_pk_bf16_f32 %1, %6, %7\n\t"
        "v_cvt_pk_bf16_f32 %2, %8, %9\n\t"
        "v_cvt_pk_bf16_f32 %3, %10, %11"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]),
          "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
        : "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
    return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ bf16x8 rot_scale_pack_bf(const bf16x8 raw, const bf16x8 cs, float sc) {
    const u32x4 x = __builtin_bit_cast(u32x4, raw), c = __builtin_bit_cast(u32x4, cs);
    u32x4 r;
    float t0, t1, t2, t3, t4, t5, t6, t7;
    asm("v_alignbit_b32 %5, %16, %16, 16\n\t"
        "v_alignbit_b32 %7, %17, %17, 16\n\t"
        "v_alignbit_b32 %9, %18, %18, 16\n\t"
        "v_alignbit_b32 %11, %19, %19, 16\n\t"
        "v_dot2_f32_bf16 %4, %12, %16, 0\n\t"
        "v_dot2_f32_bf16 %6, %13, %17, 0\n\t"
        "v_dot2_f32_bf16 %8, %14, %18, 0\n\t"
        "v_dot2_f32_bf16 %10, %15, %19, 0\n\t"
        "v_dot2_f32_bf16 %5, %12, %5, 0 neg_hi:[1,0,0]\n\t"
        "v_dot2_f32_bf16 %7, %13, %7, 0 neg_hi:[1,0,0]\n\t"
        "v_dot2_f32_bf16 %9, %14, %9, 0 neg_hi:[1,0,0]\n\t"
        "v_dot2_f32_bf16 %11, %15, %11, 0 neg_hi:[1,0,0]\n\t"
        "v_mul_f32 %4, %20, %4\n\t"
        "v_mul_f32 %6, %20, %6\n\t"
        "v_mul_f32 %8, %20, %8\n\t"
        "v_mul_f32 %10, %20, %10\n\t"
        "v_mul_f32 %5, %20, %5\n\t"
        "v_mul_f32 %7, %20, %7\n\t"
        "v_mul_f32 %9, %20, %9\n\t"
        "v_mul_f32 %11, %20, %11\n\t"
        "v_cvt_pk_bf16_f32 %0, %4, %5\n\t"
        "v_cvt_pk_bf16_f32 %1, %6, %7\n\t"
        "v_cvt_pk_bf16_f32 %2, %8, %9\n\t"
        "v_cvt_pk_bf16_f32 %3, %10, %11"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]),
          "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
        : "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(sc));
    return __builtin_bit_cast(bf16x8, r);
}
// A load / store at a wave-uniform base plus a 32-bit per-lane byte offset: the loads take the
// scalar-base addressing form, and a lane holds one 32-bit offset instead of a 64-bit address.
template <class T>
__device__ __forceinline__ T ld_off(const void *base, uint32_t byte_off) {
    return *(const T *)((const char *)base + byte_off);
}
template <class T>
__device__ __forceinline__ void st_off(void *base, uint32_t byte_off, T v) {
    *(T *)((char *)base + byte_off) = v;
}

__device__ __forceinline__ bf16x8 pack8(const float (&o)[8]) {
    return bf16x8{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3], (bf16)o[4], (bf16)o[5], (bf16)o[6], (bf16)o[7]};
}

}  // namespace m3
