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
// The step is HBM-bound (the state is read and written once: "the state must
// be read and written at every step"), so the kernel streams the state with
// 16-byte accesses: a workgroup owns one (b, h) slab; thread tid covers 4
// consecutive columns p and ROWS consecutive rows (whole rotation pairs); y is
// reduced over rows through LDS in a fixed order (deterministic).
#include "m3_common.h"

namespace m3 {

struct DecodeParams {
    const void *x, *dt, *lam, *theta, *B, *C, *Bprev, *xprev;
    const float *A, *D;
    float *h;
    void *y;
    int32_t H, G;
};

template <typename T, int N, int P, int R, int TPB>
__global__ __launch_bounds__(TPB) void k_decode(DecodeParams pr) {
    constexpr int PG = P / 4;                 // column groups of 4
    constexpr int NRG = TPB / PG;             // row groups
    constexpr int ROWS = N / NRG;             // rows per thread (even)
    static_assert(P % 4 == 0 && TPB % PG == 0 && N % NRG == 0 && ROWS % 2 == 0, "decode tiling");
    __shared__ float red[NRG][P * R];

    const int tid = threadIdx.x;
    const int pg = tid % PG, rg = tid / PG;
    const int p0 = pg * 4, n0 = rg * ROWS;
    const int bh = blockIdx.x;
    const int H = pr.H, G = pr.G;
    const int b = bh / H, hh = bh % H, g = hh / (H / G);

    const T *x = (const T *)pr.x + (int64_t)bh * P * R;
    const T *xp = pr.xprev ? (const T *)pr.xprev + (int64_t)bh * P * R : nullptr;
    const T *Bv = (const T *)pr.B + ((int64_t)b * G + g) * N * R;
    const T *Cv = (const T *)pr.C + ((int64_t)b * G + g) * N * R;
    const T *Bp = pr.Bprev ? (const T *)pr.Bprev + ((int64_t)b * G + g) * N * R : nullptr;
    const T *th = (const T *)pr.theta + (int64_t)bh * (N / 2);
    float *hs = pr.h + (int64_t)bh * N * P;

    // state tile first: the bulk of the traffic, issued before anything else
    f32x4 st[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; r++) st[r] = *(const f32x4 *)(hs + (n0 + r) * P + p0);

    const float dt = to_f(((const T *)pr.dt)[bh]);
    const float lam = to_f(((const T *)pr.lam)[bh]);
    const float alpha = expf(dt * pr.A[hh]);
    const float delta = (1.f - lam) * dt, gamma = lam * dt;
    const float Dh = pr.D ? pr.D[hh] : 0.f;

    float xv[4][R], xpv[4][R];
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
        for (int j = 0; j < R; j++) {
            xv[c][j] = to_f(x[(p0 + c) * R + j]);
            xpv[c][j] = xp ? to_f(xp[(p0 + c) * R + j]) : 0.f;
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
        sincosf(dt * to_f(th[n / 2]), &sn, &cs);
        float b0[R], b1[R], q0[R], q1[R], bp0[R], bp1[R];
#pragma unroll
        for (int j = 0; j < R; j++) {
            b0[j] = to_f(Bv[n * R + j]);
            b1[j] = to_f(Bv[(n + 1) * R + j]);
            q0[j] = to_f(Cv[n * R + j]);
            q1[j] = to_f(Cv[(n + 1) * R + j]);
            bp0[j] = Bp ? to_f(Bp[n * R + j]) : 0.f;
            bp1[j] = Bp ? to_f(Bp[(n + 1) * R + j]) : 0.f;
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
            float u0 = st[r][c] + delta * v0;
            float u1 = st[r + 1][c] + delta * v1;
            float h0 = alpha * (cs * u0 - sn * u1) + gamma * w0;
            float h1 = alpha * (sn * u0 + cs * u1) + gamma * w1;
            st[r][c] = h0;
            st[r + 1][c] = h1;
#pragma unroll
            for (int i = 0; i < R; i++) yp[c][i] += q0[i] * h0 + q1[i] * h1;
        }
    }
#pragma unroll
    for (int r = 0; r < ROWS; r++) *(f32x4 *)(hs + (n0 + r) * P + p0) = st[r];

#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
        for (int i = 0; i < R; i++) red[rg][(p0 + c) * R + i] = yp[c][i];
    __syncthreads();
    T *y = (T *)pr.y + (int64_t)bh * P * R;
    for (int e = tid; e < P * R; e += TPB) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < NRG; q++) acc += red[q][e];
        acc += Dh * to_f(x[e]);
        y[e] = from_f<T>(acc);
    }
}

template <typename T, int N, int P, int R>
static mamba3_status launch_one(const mamba3_decode_args *a, hipStream_t st) {
    constexpr int TPB = (N * P / 8 >= 256) ? 256 : N * P / 8;
    DecodeParams p{a->x, a->dt, a->lam, a->theta, a->B, a->C, a->Bprev, a->xprev, a->A, a->D, a->h, a->y,
                   a->nheads, a->ngroups};
    int64_t nblk = (int64_t)a->batch * a->nheads;
    if (nblk == 0) return MAMBA3_OK;
    hipLaunchKernelGGL((k_decode<T, N, P, R, TPB>), dim3((unsigned)nblk), dim3(TPB), 0, st, p);
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
