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
__device__ __forceinline__ void rot_piece(const bf16x8 raw, const f16x8 cs, float (&o)[8]) {
    float in[8];
#pragma unroll
    for (int e = 0; e < 8; e++) in[e] = (float)raw[e];
    rot_piece_f(in, cs, o);
}
// The same rotation with (cos, sin) packed as bf16 pairs, on the bf16 dot-product unit: each
// output is one v_dot2_f32_bf16 (two bf16 products summed in fp32) of the raw pair, so neither
// the row nor the table is widened first. The first output takes (c, s).(u, v); the second takes
// the pair swapped (a 16-bit funnel shift) against (c, -s) (the instruction's neg_hi modifier on
// the table operand).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void rot_piece_bf(const bf16x8 raw, const bf16x8 cs, float (&o)[8]) {
    const u32x4 x = __builtin_bit_cast(u32x4, raw), c = __builtin_bit_cast(u32x4, cs);
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const unsigned xs = __builtin_amdgcn_alignbit(x[m], x[m], 16);   // (v, u)
        float a, b;
        asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(a) : "v"(c[m]), "v"(x[m]));
        asm("v_dot2_f32_bf16 %0, %1, %2, 0 neg_hi:[1,0,0]" : "=v"(b) : "v"(c[m]), "v"(xs));
        o[2 * m] = a;
        o[2 * m + 1] = b;
    }
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
