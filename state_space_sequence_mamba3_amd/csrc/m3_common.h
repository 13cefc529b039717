// Shared device/host helpers of the HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mamba3.h"

namespace m3 {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

// Token-input element access: fp32 or bf16 (bf16 -> fp32 is exact).
template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16>(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
// gfx950 converts with v_cvt_pk_bf16_f32 (round to nearest even).
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }

// Lane moves by DPP (within the VALU, no LDS round trip). dpp_move<CTRL, ROWS>(v): lane i gets the
// value of the lane CTRL selects, or 0 where that lane does not exist or i's row is not in ROWS.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
// Sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48) by gfx950's row-swap
// instructions, without the LDS crossbar: v_permlane16_swap pairs rows 0-1 and 2-3, then
// v_permlane32_swap the two halves; every lane receives the sum.
__device__ __forceinline__ float sum_across_rows(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8 within each 16-lane row,
// then each row's total carried to the rows after it (row_bcast:15 into rows 1 and 3, row_bcast:31
// into rows 2 and 3).
__device__ __forceinline__ float wave_scan_dpp(float v) {
    v += dpp_move<0x111>(v);
    v += dpp_move<0x112>(v);
    v += dpp_move<0x114>(v);
    v += dpp_move<0x118>(v);
    v += dpp_move<0x142, 0xA>(v);
    v += dpp_move<0x143, 0xC>(v);
    return v;
}
// Inclusive prefix sum within aligned groups of J consecutive lanes (J = 2, 4, 8 or 16; lane j of
// its group, j = lane % J).
template <int J>
__device__ __forceinline__ float group_scan_dpp(float v, int j) {
    static_assert(J == 2 || J == 4 || J == 8 || J == 16, "groups inside a 16-lane row");
    float o;
    o = dpp_move<0x111>(v);
    if (j >= 1) v += o;
    if constexpr (J > 2) {
        o = dpp_move<0x112>(v);
        if (j >= 2) v += o;
    }
    if constexpr (J > 4) {
        o = dpp_move<0x114>(v);
        if (j >= 4) v += o;
    }
    if constexpr (J > 8) {
        o = dpp_move<0x118>(v);
        if (j >= 8) v += o;
    }
    return v;
}

// Launch plumbing shared by the kernels' host-side entry points.
struct ScanPlan {
    const mamba3_scan_args *a;
    int64_t nslab;      // sequences * heads
    int32_t nseq;
};

// The scan launchers accept y == NULL: a state-only scan (final states alone).
mamba3_status launch_scan_f32(const mamba3_scan_args *a, hipStream_t st);
mamba3_status launch_scan_bf16(const mamba3_scan_args *a, hipStream_t st);
bool scan_bf16_supported(int N, int P, int R, int Q);
// The panel kernel of the rank-4 shapes (plain path: no fused prologue / epilogue, no variants).
bool scan_mimo_supported(const mamba3_scan_args *a);
mamba3_status launch_scan_mimo(const mamba3_scan_args *a, hipStream_t st);
// State-only bf16 scan (a->y NULL) that may also write the state entering every chunk into
// ws_state (padded batches only: [S * ceil(seqlen / chunk)][H][P][N] bf16, the MFMA backward's
// chunk states) and each sequence's decay and angle sums into seg_sums (the first K + 1 floats of each
// [S][H][N][P] block: the segment sums of state passing). scan_bf16_states_supported
// covers the scan's shapes and the backward's chunks.
bool scan_bf16_states_supported(int N, int P, int R, int Q);
mamba3_status launch_scan_bf16_states(const mamba3_scan_args *a, bf16 *ws_state, float *seg_sums, hipStream_t st);
size_t scan_f32_lds_bytes(int N, int P, int R, int Q);
mamba3_status launch_decode(const mamba3_decode_args *a, hipStream_t st);
mamba3_status launch_scan_bwd(const mamba3_scan_bwd_args *b, hipStream_t st);
size_t scan_bwd_workspace_bytes(const mamba3_scan_bwd_args *b);
int scan_bwd_chunk(int N, int P, int R);
bool decode_supported(int N, int P, int R, int dtype);
// sums_staged: the segment sums are already in seg_h_in (written by the state-only scan)
mamba3_status launch_state_passing(const mamba3_state_passing_args *a, hipStream_t st, bool sums_staged = false);
size_t state_passing_lds_bytes(int N, int P, int R);
// packed batches: the bound nseq + ceil(seqlen / seg_tokens) on their segment rows (0 for
// seg_tokens < 1), and the kernel writing their segment table (rows + 1 entries)
int64_t segment_rows_packed(int64_t nseq, int64_t seqlen, int64_t seg_tokens);
mamba3_status launch_segment_table(const int32_t *cu, int32_t nseq, int32_t seqlen, int32_t seg_tokens,
                                   int32_t *seg_cu, hipStream_t st);

}  // namespace m3
