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
// State-only bf16 scan (a->y NULL) that may also write, for padded batches only, the state
// entering every chunk into ws_state ([S * ceil(seqlen / chunk)][H][N][P] fp32: the backward's
// chunk states) and each row's decay and angle sums into seg_sums (the first K + 1 floats of
// each [S][H][N][P] block: the segment sums of state passing). scan_bf16_states_supported
// covers the scan's shapes and the backward's chunks.
bool scan_bf16_states_supported(int N, int P, int R, int Q);
mamba3_status launch_scan_bf16_states(const mamba3_scan_args *a, float *ws_state, float *seg_sums, hipStream_t st);
size_t scan_f32_lds_bytes(int N, int P, int R, int Q);
mamba3_status launch_decode(const mamba3_decode_args *a, hipStream_t st);
mamba3_status launch_scan_bwd(const mamba3_scan_bwd_args *b, hipStream_t st);
size_t scan_bwd_workspace_bytes(const mamba3_scan_bwd_args *b);
int scan_bwd_chunk(int N, int P, int R);
bool decode_supported(int N, int P, int R, int dtype);
// sums_staged: the segment sums are already in seg_h_in (written by the state-only scan)
mamba3_status launch_state_passing(const mamba3_state_passing_args *a, hipStream_t st, bool sums_staged = false);
size_t state_passing_lds_bytes(int N, int P, int R);

}  // namespace m3
