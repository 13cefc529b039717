// Decode step: one token for a batch of sequences, fp32 state updated in place.
//
// Per (batch row b, head h), state H in R^{N x P} (fp32, row-major, rows n):
//   H <- alpha R(phi) (H + delta Bprev xprev^T) + gamma B x^T,   y = H^T C + D x
// with alpha = exp(dt A_h), delta = (1 - lam) dt, gamma = lam dt, phi[k] =
// dt theta[k] rotating rows (2k, 2k+1). This is one step of the three-term
// exponential-trapezoidal recurrence of Proposition 4 ("Complex-Valued State
// Space Models") in the physical frame, with the rank-R update of section
// "MIMO Formulation".
//
// The step is HBM-bound (the state is read and written once per step and
// dominates the traffic), so both kernels are streaming kernels with one
// workgroup per (b, h) slab. Head dim 64 uses the column kernel (one lane per
// state column); other head dims use the tile kernel (4 columns x ROWS rows per
// thread). y is reduced over rows in a fixed order (deterministic). Token
// layouts are rank-major (B [R][N], x and y [R][P]).
//
// The EPI instantiations add the block prologue and epilogue (section
// "Architectural Integration"): each staged B, C and Bprev column is scaled to
// unit RMS and gets the head's bias before the update, and y is multiplied by
// SiLU(z) after the D term.
//
// Variants: a per-row decay rate A_t replaces the head's A, and without a lam
// array every row uses the fixed trapezoid weight. Angle rows may be shared by
// groups of heads (head h reads row h / (H / Gth)).
//
// Slot-indexed states (continuous batching): row b updates state slots[b] of a
// pool; a row whose slot is out of range is inactive and its workgroups return
// before touching memory (the slot is uniform across the workgroup).
#include "m3_common.h"

namespace m3 {

struct DecodeParams {
    const void *x, *dt, *lam, *theta, *B, *C, *Bprev, *xprev;
    const float *A, *D;
    float *h;
    void *y;
    int32_t H, G;
    const float *Bb, *Cb;   // prologue biases [H, N], or NULL
    const void *z;          // output gate (token dtype), or NULL
    int32_t norm;           // 1: B, C, Bprev columns scaled to unit RMS
    float eps;
    const void *A_tok;      // per-row decay rate [batch, H] (token dtype), or NULL: A per head
    float lam_fixed;        // trapezoid weight of every row when lam is NULL
    int32_t Gth;            // angle rows per batch row (divides H)
    const int32_t *slots;   // state slot of each batch row, or NULL: row b uses state b
    int32_t nslots;
};

// The state slab of (row b, head hh), or NULL when the row is inactive.
__device__ __forceinline__ float *state_slab(const DecodeParams &pr, int b, int hh, int NP) {
    int64_t row = b;
    if (pr.slots) {
        const int s = pr.slots[b];
        if (s < 0 || s >= pr.nslots) return nullptr;
        row = s;
    }
    return pr.h + (row * pr.H + hh) * NP;
}

// Stand-in for an absent bias row or gate (read-only zeros), so that prologue loads are
// unconditional.
__constant__ float kZeroRow[256];

__device__ __forceinline__ float silu(float v, bool fast) { return v / (1.f + (fast ? __expf(-v) : expf(-v))); }

// Copy `count` elements of T (count * sizeof(T) a multiple of 16) into LDS as
// fp32 with 16-byte loads; piece i goes to thread (t0 + i) mod TPB, so arrays
// staged with different t0 land on different threads.
template <typename T, int TPB>
__device__ __forceinline__ void stage_f32(float *dst, const T *src, int count, int tid, int t0) {
    constexpr int VW = 16 / sizeof(T);
    for (int i = ((tid - t0) % TPB + TPB) % TPB; i < count / VW; i += TPB) {
        if constexpr (sizeof(T) == 2) {
            const bf16x8 v = *(const bf16x8 *)(src + i * VW);
#pragma unroll
            for (int e = 0; e < VW; e++) dst[i * VW + e] = (float)v[e];
        } else {
            *(f32x4 *)(dst + i * VW) = *(const f32x4 *)(src + i * VW);
        }
    }
}

template <typename T, int N, int P, int R, int TPB, bool EPI>
__global__ __launch_bounds__(TPB) void k_decode(DecodeParams pr) {
    constexpr int PG = P / 4;                 // column groups of 4
    constexpr int NRG = TPB / PG;             // row groups
    constexpr int ROWS = N / NRG;             // rows per thread (even)
    constexpr int VW = 16 / sizeof(T);
    static_assert(P % 4 == 0 && TPB % PG == 0 && N % NRG == 0 && ROWS % 2 == 0, "decode tiling");
    static_assert((N * R) % VW == 0 && (P * R) % VW == 0 && (N / 2) % VW == 0, "16-byte staging");
    __shared__ float sB[N * R], sC[N * R], sBp[N * R], sX[P * R], sXp[P * R], sTh[N / 2];
    constexpr int WL = TPB < 64 ? TPB : 64, NWV = (TPB + 63) / 64;   // lanes per wave, waves
    __shared__ float red[NWV][P * R];

    const int tid = threadIdx.x;
    const int pg = tid % PG, rg = tid / PG;
    const int p0 = pg * 4, n0 = rg * ROWS;
    const int bh = blockIdx.x;
    const int H = pr.H, G = pr.G;
    const int b = bh / H, hh = bh % H, g = hh / (H / G);
    float *hs = state_slab(pr, b, hh, N * P);
    if (!hs) return;   // inactive row (uniform across the workgroup)

    // state tile first: the bulk of the traffic, in flight while the token inputs are staged
    f32x4 st[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; r++) st[r] = __builtin_nontemporal_load((const f32x4 *)(hs + (n0 + r) * P + p0));

    const int64_t obc = ((int64_t)b * G + g) * N * R, ox = (int64_t)bh * P * R;
    constexpr int CB = N * R / VW, CX = P * R / VW, CT = N / 2 / VW;
    stage_f32<T, TPB>(sB, (const T *)pr.B + obc, N * R, tid, 0);
    stage_f32<T, TPB>(sC, (const T *)pr.C + obc, N * R, tid, CB);
    stage_f32<T, TPB>(sX, (const T *)pr.x + ox, P * R, tid, 2 * CB);
    stage_f32<T, TPB>(sTh, (const T *)pr.theta + ((int64_t)b * pr.Gth + hh / (H / pr.Gth)) * (N / 2), N / 2, tid,
                      2 * CB + CX);
    if (pr.Bprev) {
        stage_f32<T, TPB>(sBp, (const T *)pr.Bprev + obc, N * R, tid, 2 * CB + CX + CT);
        stage_f32<T, TPB>(sXp, (const T *)pr.xprev + ox, P * R, tid, 3 * CB + CX + CT);
    }
    const float dt = to_f(((const T *)pr.dt)[bh]);
    const float lam = pr.lam ? to_f(((const T *)pr.lam)[bh]) : pr.lam_fixed;
    const float Ah = pr.A_tok ? to_f(((const T *)pr.A_tok)[bh]) : pr.A[hh];
    // fp32 inputs take the precise exp and sincos, bf16 inputs the hardware approximations
    constexpr bool FAST = sizeof(T) == 2;
    const float alpha = FAST ? __expf(dt * Ah) : expf(dt * Ah);
    const float delta = (1.f - lam) * dt, gamma = lam * dt;
    const float Dh = pr.D ? pr.D[hh] : 0.f;
    const bool has_prev = pr.Bprev != nullptr;
    __syncthreads();
    if constexpr (EPI) {   // prologue: one thread per staged column of B, C, Bprev
        static_assert(3 * R <= TPB, "decode prologue");
        const int arr = tid / R, j = tid % R;
        if (tid < 3 * R && (arr < 2 || has_prev)) {
            float *col = (arr == 0 ? sB : arr == 1 ? sC : sBp) + j * N;
            const float *bias = arr == 1 ? pr.Cb : pr.Bb;
            float inv = 1.f;
            if (pr.norm) {
                float ss = 0.f;
                for (int n = 0; n < N; n++) ss += col[n] * col[n];
                inv = 1.f / sqrtf(ss * (1.f / N) + pr.eps);
            }
            for (int n = 0; n < N; n++) col[n] = col[n] * inv + (bias ? bias[hh * N + n] : 0.f);
        }
        __syncthreads();
    }

    float xv[4][R], xpv[4][R];
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
        for (int j = 0; j < R; j++) {
            xv[c][j] = sX[j * P + p0 + c];
            xpv[c][j] = has_prev ? sXp[j * P + p0 + c] : 0.f;
        }

    float yp[4][R];
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
        for (int i = 0; i < R; i++) yp[c][i] = 0.f;

#pragma unroll
    for (int r = 0; r < ROWS; r += 2) {
        const int n = n0 + r;
        float sn, cs;
        if constexpr (FAST) __sincosf(dt * sTh[n / 2], &sn, &cs);
        else sincosf(dt * sTh[n / 2], &sn, &cs);
        float b0[R], b1[R], q0[R], q1[R], bp0[R], bp1[R];
#pragma unroll
        for (int j = 0; j < R; j++) {
            b0[j] = sB[j * N + n];
            b1[j] = sB[j * N + n + 1];
            q0[j] = sC[j * N + n];
            q1[j] = sC[j * N + n + 1];
            bp0[j] = has_prev ? sBp[j * N + n] : 0.f;
            bp1[j] = has_prev ? sBp[j * N + n + 1] : 0.f;
        }
#pragma unroll
        for (int c = 0; c < 4; c++) {
            float v0 = 0.f, v1 = 0.f, w0 = 0.f, w1 = 0.f;
#pragma unroll
            for (int j = 0; j < R; j++) {
                v0 += bp0[j] * xpv[c][j];
                v1 += bp1[j] * xpv[c][j];
                w0 += b0[j] * xv[c][j];
                w1 += b1[j] * xv[c][j];
            }
            const float u0 = st[r][c] + delta * v0;
            const float u1 = st[r + 1][c] + delta * v1;
            const float h0 = alpha * (cs * u0 - sn * u1) + gamma * w0;
            const float h1 = alpha * (sn * u0 + cs * u1) + gamma * w1;
            st[r][c] = h0;
            st[r + 1][c] = h1;
#pragma unroll
            for (int i = 0; i < R; i++) yp[c][i] += q0[i] * h0 + q1[i] * h1;
        }
    }
#pragma unroll
    for (int r = 0; r < ROWS; r++) __builtin_nontemporal_store(st[r], (f32x4 *)(hs + (n0 + r) * P + p0));

    // y = H^T C: sum the row groups' partials, first across the lanes of a wave (the row groups
    // of one wave are PG lanes apart), then across the waves through LDS
#pragma unroll
    for (int off = PG; off < WL; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; c++)
#pragma unroll
            for (int i = 0; i < R; i++) yp[c][i] += __shfl_xor(yp[c][i], off, 64);
    if ((tid & 63) < PG) {
#pragma unroll
        for (int c = 0; c < 4; c++)
#pragma unroll
            for (int i = 0; i < R; i++) red[tid >> 6][i * P + p0 + c] = yp[c][i];
    }
    __syncthreads();
    T *y = (T *)pr.y + (int64_t)bh * P * R;
    for (int e = tid; e < P * R; e += TPB) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < NWV; q++) acc += red[q][e];
        acc += Dh * sX[e];
        if constexpr (EPI)
            if (pr.z) acc *= silu(to_f(((const T *)pr.z)[(int64_t)bh * P * R + e]), FAST);
        y[e] = from_f<T>(acc);
    }
}

// Head dim 64: one lane per state column, so a wave's loads and stores of a state row are one
// coalesced 256-byte access and every y partial is the lane's own column. Wave w updates rows
// [16 w, 16 w + 16). The update is applied term by term (previous-token term, rotation and
// decay, current-token term, readout), each a pass over the lane's 16 rows, so few values are
// live at once and eight waves per SIMD stay resident.
//
// With EPI the prologue is fused into the staging: the 16-byte pieces of one column sit in
// N / VW consecutive lanes of one wave, so each column's sum of squares is a butterfly of wave
// shuffles, and every thread scales its own piece and adds its slice of the bias row.
template <typename T, int N, int R, bool EPI>
__global__ __launch_bounds__(N / 16 * 64) __attribute__((amdgpu_waves_per_eu(8))) void k_decode_col(DecodeParams pr) {
    constexpr int P = 64, ROWS = 16, NW = N / ROWS, TPB = NW * 64;
    static_assert(N % ROWS == 0 && (N * R) % (16 / sizeof(T)) == 0, "decode column tiling");
    static_assert(P * R <= TPB && N <= 256 && P * R * sizeof(T) <= sizeof(kZeroRow), "decode column epilogue");
    __shared__ __attribute__((aligned(16))) float sB[R * N], sC[R * N], sBp[R * N];
    __shared__ __attribute__((aligned(16))) float2 sCS[N / 2];
    __shared__ float red[NW][R * P];

    const int tid = threadIdx.x, p = tid & 63, w = tid >> 6, n0 = w * ROWS;
    const int bh = blockIdx.x;
    const int H = pr.H, G = pr.G;
    const int b = bh / H, hh = bh % H, g = hh / (H / G);
    float *hs = state_slab(pr, b, hh, N * P);
    if (!hs) return;   // inactive row (uniform across the workgroup)

    const int64_t obc = ((int64_t)b * G + g) * N * R, ox = (int64_t)bh * P * R;
    const bool has_prev = pr.Bprev != nullptr;
    const T *xp_src = has_prev ? (const T *)pr.xprev : (const T *)pr.x;   // (no previous token: unused)
    // All token loads are unconditional and issued before the state loads, and each thread
    // waits only for its own: loads complete in order, so the staging below does not wait for
    // the state. Thread t loads 16-byte piece t % PCS of B (t < PCS), C or Bprev.
    constexpr int VW = 16 / sizeof(T), PCS = N * R / VW, CPC = N / VW;   // pieces per array, per column
    static_assert(3 * PCS <= TPB && CPC <= 64 && (CPC & (CPC - 1)) == 0, "decode staging");
    const int arr = tid / PCS, pc = tid % PCS;
    const T *src = (arr == 1) ? (const T *)pr.C : (arr == 2 && has_prev) ? (const T *)pr.Bprev : (const T *)pr.B;
    typedef T vec_t __attribute__((ext_vector_type(VW)));
    const vec_t piece = *(const vec_t *)(src + obc + pc * VW);
    f32x4 bias4[VW / 4];
    T zr{};
    if constexpr (EPI) {
        const float *Bb = pr.Bb ? pr.Bb + hh * N : kZeroRow, *Cb = pr.Cb ? pr.Cb + hh * N : kZeroRow;
        const float *bsrc = ((arr == 1) ? Cb : Bb) + (pc % CPC) * VW;
#pragma unroll
        for (int q = 0; q < VW / 4; q++) bias4[q] = *(const f32x4 *)(bsrc + 4 * q);
        zr = *(pr.z ? (const T *)pr.z + ox + min(tid, P * R - 1) : (const T *)kZeroRow);
    }
    T xr[R], xpr[R];
#pragma unroll
    for (int j = 0; j < R; j++) {
        xr[j] = ((const T *)pr.x)[ox + j * P + p];
        xpr[j] = xp_src[ox + j * P + p];
    }
    const T thr = ((const T *)pr.theta)[((int64_t)b * pr.Gth + hh / (H / pr.Gth)) * (N / 2) + min(tid, N / 2 - 1)];
    const float dt = to_f(((const T *)pr.dt)[bh]);
    const float lam = pr.lam ? to_f(((const T *)pr.lam)[bh]) : pr.lam_fixed;
    const float Ah = pr.A_tok ? to_f(((const T *)pr.A_tok)[bh]) : pr.A[hh];
    const float Dh = pr.D ? pr.D[hh] : 0.f;

    float st[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; r++) st[r] = __builtin_nontemporal_load(hs + (n0 + r) * P + p);

    // fp32 inputs take the precise exp, sincos and root, bf16 inputs the hardware approximations
    constexpr bool FAST = sizeof(T) == 2;
    float pv[VW];
#pragma unroll
    for (int e = 0; e < VW; e++) pv[e] = (float)piece[e];
    if constexpr (EPI) {
        float inv = 1.f;
        if (pr.norm) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < VW; e++) ss += pv[e] * pv[e];
#pragma unroll
            for (int off = 1; off < CPC; off <<= 1) ss += __shfl_xor(ss, off, 64);
            const float ms = ss * (1.f / N) + pr.eps;
            inv = FAST ? rsqrtf(ms) : 1.f / sqrtf(ms);
        }
#pragma unroll
        for (int e = 0; e < VW; e++) pv[e] = pv[e] * inv + bias4[e / 4][e % 4];
    }
    if (arr < 2 || (arr == 2 && has_prev)) {
        float *dst = (arr == 0) ? sB : (arr == 1) ? sC : sBp;
#pragma unroll
        for (int e = 0; e < VW; e++) dst[pc * VW + e] = pv[e];
    }
    float xv[R], xpv[R];
#pragma unroll
    for (int j = 0; j < R; j++) {
        xv[j] = to_f(xr[j]);
        xpv[j] = has_prev ? to_f(xpr[j]) : 0.f;
    }
    if (tid < N / 2) {   // one sincos per state pair, shared through LDS
        const float a = dt * to_f(thr);
        float sn, cs;
        if constexpr (FAST) __sincosf(a, &sn, &cs);
        else sincosf(a, &sn, &cs);
        sCS[tid] = float2{cs, sn};
    }
    const float alpha = FAST ? __expf(dt * Ah) : expf(dt * Ah);
    const float delta = (1.f - lam) * dt, gamma = lam * dt;
    __syncthreads();

    // H + delta Bprev xprev^T
    if (has_prev) {
#pragma unroll
        for (int j = 0; j < R; j++) {
            const float dx = delta * xpv[j];
#pragma unroll
            for (int q = 0; q < ROWS / 4; q++) {
                const f32x4 bq = *(const f32x4 *)(sBp + j * N + n0 + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; e++) st[4 * q + e] += bq[e] * dx;
            }
        }
    }
    // alpha R(phi) (.)
#pragma unroll
    for (int q = 0; q < ROWS / 4; q++) {
        const f32x4 cs2 = *(const f32x4 *)(sCS + (n0 + 4 * q) / 2);   // two pairs
#pragma unroll
        for (int m = 0; m < 2; m++) {
            const float c = alpha * cs2[2 * m], sn = alpha * cs2[2 * m + 1];
            const float u0 = st[4 * q + 2 * m], u1 = st[4 * q + 2 * m + 1];
            st[4 * q + 2 * m] = c * u0 - sn * u1;
            st[4 * q + 2 * m + 1] = sn * u0 + c * u1;
        }
    }
    // + gamma B x^T
#pragma unroll
    for (int j = 0; j < R; j++) {
        const float gx = gamma * xv[j];
#pragma unroll
        for (int q = 0; q < ROWS / 4; q++) {
            const f32x4 bq = *(const f32x4 *)(sB + j * N + n0 + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; e++) st[4 * q + e] += bq[e] * gx;
        }
    }
#pragma unroll
    for (int r = 0; r < ROWS; r++) __builtin_nontemporal_store(st[r], hs + (n0 + r) * P + p);
    // y partial of the lane's column over the wave's rows
    float yp[R];
#pragma unroll
    for (int i = 0; i < R; i++) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < ROWS / 4; q++) {
            const f32x4 cq = *(const f32x4 *)(sC + i * N + n0 + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; e++) acc += cq[e] * st[4 * q + e];
        }
        yp[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < R; i++) red[w][i * P + p] = yp[i];
    __syncthreads();
    T *y = (T *)pr.y + (int64_t)bh * P * R;
    if (tid < P * R) {
        float acc = Dh * to_f(((const T *)pr.x)[ox + tid]);
#pragma unroll
        for (int q = 0; q < NW; q++) acc += red[q][tid];
        if constexpr (EPI)
            if (pr.z) acc *= silu(to_f(zr), FAST);
        y[tid] = from_f<T>(acc);
    }
}

template <typename T, int N, int P, int R, bool EPI>
static void launch_kernel(const DecodeParams &p, int64_t nblk, hipStream_t st) {
    constexpr int TPB = (N * P / 8 >= 256) ? 256 : N * P / 8;
    if constexpr (P == 64)
        hipLaunchKernelGGL((k_decode_col<T, N, R, EPI>), dim3((unsigned)nblk), dim3(N / 16 * 64), 0, st, p);
    else
        hipLaunchKernelGGL((k_decode<T, N, P, R, TPB, EPI>), dim3((unsigned)nblk), dim3(TPB), 0, st, p);
}

template <typename T, int N, int P, int R>
static mamba3_status launch_one(const mamba3_decode_args *a, hipStream_t st) {
    DecodeParams p{a->x, a->dt, a->lam, a->theta, a->B, a->C, a->Bprev, a->xprev, a->A, a->D, a->h, a->y,
                   a->nheads, a->ngroups, a->B_bias, a->C_bias, a->z, a->bc_norm, a->bc_eps, a->A_tok, a->lam_fixed,
                   a->theta_groups ? a->theta_groups : a->nheads, a->slots, a->nslots};
    int64_t nblk = (int64_t)a->batch * a->nheads;
    if (nblk == 0) return MAMBA3_OK;
    if (a->bc_norm || a->B_bias || a->C_bias || a->z)
        launch_kernel<T, N, P, R, true>(p, nblk, st);
    else
        launch_kernel<T, N, P, R, false>(p, nblk, st);
    return hipGetLastError() == hipSuccess ? MAMBA3_OK : MAMBA3_EHIP;
}

#define M3_DECODE_SHAPES(X) \
    X(64, 64, 4) X(128, 64, 4) X(64, 64, 1) X(128, 64, 1) X(16, 16, 1) X(16, 16, 4) X(64, 64, 2) X(32, 32, 2)

bool decode_supported(int N, int P, int R, int dtype) {
    (void)dtype;
#define X(n, p, r) if (N == n && P == p && R == r) return true;
    M3_DECODE_SHAPES(X)
#undef X
    return false;
}

mamba3_status launch_decode(const mamba3_decode_args *a, hipStream_t st) {
    const int N = a->dstate, P = a->headdim, R = a->rank;
#define X(n, p, r)                                                                   \
    if (N == n && P == p && R == r)                                                  \
        return a->dtype == MAMBA3_BF16 ? launch_one<bf16, n, p, r>(a, st)           \
                                       : launch_one<float, n, p, r>(a, st);
    M3_DECODE_SHAPES(X)
#undef X
    return MAMBA3_EUNSUPPORTED;
}

}  // namespace m3
