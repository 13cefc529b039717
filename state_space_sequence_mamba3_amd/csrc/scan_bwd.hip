// Backward of the chunked scan: gradients of every input given dL/dy and
// dL/dh_out (VALU, fp32 arithmetic, token inputs fp32 or bf16).
//
// One workgroup owns one (sequence, head) slab. The state entering each chunk
// is first stored in the workspace: by a state-only forward scan (the bf16
// forward kernel without outputs, at this kernel's chunk) for padded bf16
// batches of the shapes it covers, otherwise by a forward walk of this kernel.
// The slab's chunks are then walked in reverse. Per chunk (tokens 0..e, chunk-local log decay S_t,
// cumulative angle Phi_t, B~ = R(-Phi) B, C~ = R(-Phi) C, carried state H'
// entering the chunk, physical frame) the forward is
//   y_t  = e^{S_t} C~_t^T H' + sum_{s<=t} e^{S_t-S_s} w(t,s) (C~_t . B~_s) X_s + D X_t
//   H'_n = R(Phi_e) (e^{S_e} H' + sum_s c_s B~_s X_s^T),  c_s = e^{S_e-S_s} g1_s
//   w(t,s) = gamma_s + delta_{s+1} [s < t],   g1_s = gamma_s + delta_{s+1} [s < e]
// and the next chunk's first token adds delta_0 B_e X_e^T to H'_n (its
// previous-input term, kept as a separate fold). This is the three-term update
// of Proposition 4 ("Complex-Valued State Space Models") in the SSD matrix form
// ("Parallel representation under SSD"). Its gradient, given dY and dH_n
// (= dL/dH'_n), with G^ = R(-Phi_e) dH_n:
//   dH'   = e^{S_e} G^ + sum_t e^{S_t} C~_t dy_t^T
//   dX_s  = sum_t A(t,s) dy_t + c_s G^^T B~_s + D dy_s,   A = M o (C~ B~^T),  M = e^{S_t-S_s} w
//   dC~_t = sum_s M(t,s) dP(t,s) B~_s + e^{S_t} H' dy_t,  dP(t,s) = dy_t . X_s
//   dB~_s = sum_t M(t,s) dP(t,s) C~_t + c_s G^ X_s
//   dS, dw from M, c and the inter term; dPhi from C~, B~ (d/dPhi R(-Phi) v = -J R(-Phi) v)
//   and from R(Phi_e) (dPhi_e = sum_p G^^T J Inner); then reverse prefix sums over the
//   chunk give dPhi -> dphi = dt dtheta and dS -> d(dt A).
// The fold gives d delta_0 = <dH', Bp Xp^T> and the previous token's dB, dX.
// The block prologue (BC norm, biases) and the gate are differentiated as
// applied. Every sum runs in a fixed order (no atomics): per-slab partial sums
// of dA, dD and the bias gradients, (with G < H) per-head dB, dC, dBprev, and
// (with shared angle rows) per-head dtheta go to the workspace and a second
// kernel adds them up.
//
// Variants: a per-token decay rate A_t (its gradient is per token, dt_t dS_t),
// and a fixed trapezoid weight (no lam gradient).
#include <algorithm>
#include <type_traits>

#include "m3_common.h"

namespace m3 {

struct BwdParams {
    const void *x, *dt, *lam, *theta, *B, *C, *Bprev, *xprev, *z, *dy;
    const float *A, *D, *h_in, *dh_out, *Bb, *Cb;
    void *dx, *ddt, *dlam, *dtheta, *dB, *dC, *dBprev, *dxprev, *dz;
    float *dh_in, *dA, *dD, *dB_bias, *dC_bias;
    float *ws_state;          // VALU kernel: [chunks][H][N][P] fp32 state entering each chunk
    bf16 *ws_hs;              // MFMA kernel: [chunks][H][P][N] bf16 state entering each chunk
    float *p_dA, *p_dD;       // [S][H]
    float *p_dBb, *p_dCb;     // [S][H][N]
    float *p_dB, *p_dC;       // [T][H][R][N] per-head partials (G < H), else NULL
    float *p_dBprev;          // [S][H][R][N] per-head partials (G < H), else NULL
    const int32_t *cu;
    int64_t ws_chunks;        // chunk states the workspace holds
    int32_t nseq, seqlen, H, G, P, N, R, Q;
    int32_t norm;
    float eps;
    const void *A_tok;        // per-token decay rate (token dtype, layout of dt), or NULL
    void *dA_tok;             // its gradient
    float lam_fixed;          // trapezoid weight of every token when lam is NULL
    int32_t Gth;              // angle rows per token (divides H): head h reads row h / (H / Gth)
    int32_t fwd_states;       // MFMA kernel: the chunk states are already in ws_hs (no forward walk)
    float *p_dth;             // [T][H][K] per-head dtheta partials (Gth < H), else NULL
};

constexpr int kBwdThreads = 512;

// LDS layout of the backward (offsets in floats)
struct BwdLayout {
    int cs, sn, dphi, dts, lms, gms, dls, S, g1, dS, dgm, ddl, es, cu, at, em, scal_end;
    int invB, invC, rowA, rowB, colS, colG, colD, rows_end;
    int Bt, Ct, dBt, dCt, Xs, dY, Hs, dH, Sc, dPm, Wk, Wk2;
    int Bp, BpRaw, Xp, dBc_in, dXc_in, dBc_out, dXc_out, invBp, bba, cba, misc, total;
};

__host__ __device__ inline BwdLayout bwd_layout(int N, int P, int R, int Q) {
    BwdLayout L;
    const int K = N / 2, QR = Q * R;
    const int NS = N + 1, PS = P + 1, QS = QR + 1;   // padded row strides
    const int WK0 = (QR > K ? QR : K) * PS, WK = WK0 > kBwdThreads ? WK0 : kBwdThreads;   // >= one float per thread
    int o = 0;
    L.cs = o; o += Q * K;
    L.sn = o; o += Q * K;
    L.dphi = o; o += Q * K;
    L.dts = o; o += Q;
    L.lms = o; o += Q;
    L.gms = o; o += Q;
    L.dls = o; o += Q;
    L.S = o; o += Q;
    L.g1 = o; o += Q;
    L.dS = o; o += Q;
    L.dgm = o; o += Q;
    L.ddl = o; o += Q;
    L.es = o; o += Q;
    L.cu = o; o += Q;
    L.at = o; o += Q;
    L.em = o; o += Q * Q;
    L.scal_end = o;
    L.invB = o; o += QR;
    L.invC = o; o += QR;
    L.rowA = o; o += QR;
    L.rowB = o; o += QR;
    L.colS = o; o += QR;
    L.colG = o; o += QR;
    L.colD = o; o += QR;
    L.rows_end = o;
    o = (o + 3) & ~3;
    L.Bt = o; o += QR * NS;
    L.Ct = o; o += QR * NS;
    L.dBt = o; o += QR * NS;
    L.dCt = o; o += QR * NS;
    L.Xs = o; o += QR * PS;
    L.dY = o; o += QR * PS;
    L.Hs = o; o += N * PS;
    L.dH = o; o += N * PS;
    L.Sc = o; o += QR * QS;
    L.dPm = o; o += QR * QS;
    L.Wk = o; o += WK;
    L.Wk2 = o; o += WK;
    L.Bp = o; o += R * N;
    L.BpRaw = o; o += R * N;
    L.Xp = o; o += R * P;
    L.dBc_in = o; o += R * N;
    L.dXc_in = o; o += R * P;
    L.dBc_out = o; o += R * N;
    L.dXc_out = o; o += R * P;
    L.invBp = o; o += R;
    L.bba = o; o += N;
    L.cba = o; o += N;
    L.misc = o; o += 16;
    L.total = o;
    return L;
}

size_t scan_bwd_lds_bytes(int N, int P, int R, int Q) { return (size_t)bwd_layout(N, P, R, Q).total * sizeof(float); }

template <typename T>
__device__ __forceinline__ float ldt(const void *p, int64_t i) {
    return to_f(((const T *)p)[i]);
}
template <typename T>
__device__ __forceinline__ void stt(void *p, int64_t i, float v) {
    ((T *)p)[i] = from_f<T>(v);
}
// Offset of token tok's angle row for head h.
__device__ __forceinline__ int64_t th_row(const BwdParams &p, int64_t tok, int h) {
    return (tok * p.Gth + h / (p.H / p.Gth)) * (int64_t)(p.N / 2);
}
// Head h's share of dtheta at (token tok, pair k): the output itself with one angle row per
// head, else the per-head partial that k_bwd_reduce sums over the heads sharing a row.
template <typename T>
__device__ __forceinline__ void st_dtheta(const BwdParams &p, int64_t tok, int h, int k, float v) {
    const int64_t i = (tok * p.H + h) * (int64_t)(p.N / 2) + k;
    if (p.p_dth) p.p_dth[i] = v;
    else stt<T>(p.dtheta, i, v);
}

// Sum of one value per thread over the workgroup in a fixed order (wave butterflies, then the
// wave sums in order); every thread gets the total. red: one float of LDS per wave. Must be
// reached by every thread.
__device__ float block_sum(float v, float *red) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
    __syncthreads();   // red is free
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); w++) t += red[w];
    return t;
}

template <typename T>
__global__ __launch_bounds__(kBwdThreads) void k_scan_bwd(BwdParams p) {
    extern __shared__ float sm[];
    const int H = p.H, G = p.G, P = p.P, N = p.N, R = p.R, Q = p.Q, K = N / 2, QR = Q * R;
    // LDS row strides padded by one element: column walks across lanes hit distinct banks
    const int NS = N + 1, PS = P + 1, QS = QR + 1;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int s = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / G);
    const BwdLayout L = bwd_layout(N, P, R, Q);
    float *CS = sm + L.cs, *SN = sm + L.sn, *DPHI = sm + L.dphi;
    float *DT = sm + L.dts, *LM = sm + L.lms, *GM = sm + L.gms, *DL = sm + L.dls, *S = sm + L.S, *G1 = sm + L.g1;
    float *DS = sm + L.dS, *DGM = sm + L.dgm, *DDL = sm + L.ddl;
    float *ES = sm + L.es, *CU = sm + L.cu, *EM = sm + L.em;   // e^{S_t}, c_t, e^{S_t - S_u}
    float *AT = sm + L.at;                                       // A_t of each token
    float *INVB = sm + L.invB, *INVC = sm + L.invC, *ROWA = sm + L.rowA, *ROWB = sm + L.rowB;
    float *COLS = sm + L.colS, *COLG = sm + L.colG, *COLD = sm + L.colD;
    float *Bt = sm + L.Bt, *Ct = sm + L.Ct, *dBt = sm + L.dBt, *dCt = sm + L.dCt;
    float *Xs = sm + L.Xs, *dY = sm + L.dY, *Hs = sm + L.Hs, *dH = sm + L.dH;
    float *Sc = sm + L.Sc, *dPm = sm + L.dPm, *Wk = sm + L.Wk, *Wk2 = sm + L.Wk2;
    float *Bp = sm + L.Bp, *BpRaw = sm + L.BpRaw, *Xp = sm + L.Xp, *INVBP = sm + L.invBp;
    float *dBcIn = sm + L.dBc_in, *dXcIn = sm + L.dXc_in, *dBcOut = sm + L.dBc_out, *dXcOut = sm + L.dXc_out;
    float *BBA = sm + L.bba, *CBA = sm + L.cba, *MISC = sm + L.misc;

    // sequence bounds and the index of its first chunk in the state workspace
    int64_t start, len, cbase;
    if (p.cu) {
        const int64_t a = min(max((int64_t)p.cu[s], (int64_t)0), (int64_t)p.seqlen);
        const int64_t b = min(max((int64_t)p.cu[s + 1], a), (int64_t)p.seqlen);
        start = a;
        len = b - a;
        cbase = 0;
        for (int j = 0; j < s; j++) {
            const int64_t a0 = min(max((int64_t)p.cu[j], (int64_t)0), (int64_t)p.seqlen);
            const int64_t b0 = min(max((int64_t)p.cu[j + 1], a0), (int64_t)p.seqlen);
            cbase += (b0 - a0 + Q - 1) / Q;
        }
    } else {
        start = (int64_t)s * p.seqlen;
        len = p.seqlen;
        cbase = (int64_t)s * ((p.seqlen + Q - 1) / Q);
    }
    const int64_t nch = (len + Q - 1) / Q;
    // a sequence table that breaks its contract (decreasing offsets) could ask for more chunk
    // states than the workspace holds: such a slab writes nothing
    if (cbase + nch > p.ws_chunks) return;
    const float Ah = p.A ? p.A[h] : 0.f;
    const float Dh = p.D ? p.D[h] : 0.f;
    const bool pro = p.norm || p.Bb || p.Cb;
    const bool has_prev = p.Bprev != nullptr;
    const int64_t sh = (int64_t)s * H + h;
    const float *Bbh = p.Bb ? p.Bb + (int64_t)h * N : nullptr;
    const float *Cbh = p.Cb ? p.Cb + (int64_t)h * N : nullptr;
    auto wsS = [&](int64_t c) { return p.ws_state + ((cbase + c) * H + h) * (int64_t)N * P; };
    auto tokB = [&](int64_t t) { return ((start + t) * G + g) * (int64_t)R * N; };   // B / C row base of token t
    auto tokX = [&](int64_t t) { return ((start + t) * H + h) * (int64_t)R * P; };   // x / y row base

    // Prologue of `nrows` LDS rows (one thread per row): scale to unit RMS (inv kept in invs) and
    // add the bias row. Rows hold the raw values on entry.
    auto prologue_rows = [&](float *rows, int nrows, int stride, const float *bias, float *invs) {
        for (int r = tid; r < nrows; r += nt) {
            float *v = rows + (int64_t)r * stride;
            float inv = 1.f;
            if (p.norm) {
                float ss = 0.f;
                for (int n = 0; n < N; n++) ss += v[n] * v[n];
                inv = 1.f / sqrtf(ss / (float)N + p.eps);
            }
            invs[r] = inv;
            if (pro)
                for (int n = 0; n < N; n++) v[n] = v[n] * inv + (bias ? bias[n] : 0.f);
        }
    };
    // per-token scalars of the chunk at c0 with nq tokens, the decay prefix and the angle table
    auto load_scalars = [&](int64_t c0, int nq) {
        for (int t = tid; t < Q; t += nt) {
            float dtv = 0.f, lv = 0.f, av = Ah;
            if (t < nq) {
                dtv = ldt<T>(p.dt, (start + c0 + t) * H + h);
                lv = p.lam ? ldt<T>(p.lam, (start + c0 + t) * H + h) : p.lam_fixed;
                if (p.A_tok) av = ldt<T>(p.A_tok, (start + c0 + t) * H + h);
            }
            DT[t] = dtv;
            LM[t] = lv;
            AT[t] = av;
            GM[t] = lv * dtv;
            DL[t] = (1.f - lv) * dtv;
        }
        __syncthreads();
        if (tid == 0) {
            float acc = 0.f;
            for (int t = 0; t < Q; t++) {
                acc += DT[t] * AT[t];
                S[t] = acc;
                G1[t] = GM[t] + ((t + 1 < nq) ? DL[t + 1] : 0.f);
            }
        }
        for (int k = tid; k < K; k += nt) {
            float acc = 0.f;
            for (int t = 0; t < Q; t++) {
                if (t < nq) acc += DT[t] * ldt<T>(p.theta, th_row(p, start + c0 + t, h) + k);
                float sn, cs;
                sincosf(acc, &sn, &cs);
                CS[t * K + k] = cs;
                SN[t * K + k] = sn;
            }
        }
        __syncthreads();
        for (int e = tid; e < Q * Q; e += nt) {
            const int t = e / Q, u = e % Q;
            EM[e] = (u <= t) ? expf(S[t] - S[u]) : 0.f;
        }
        for (int t = tid; t < Q; t += nt) {
            ES[t] = expf(S[t]);
            CU[t] = (t < nq) ? expf(S[nq - 1] - S[t]) * G1[t] : 0.f;
        }
        __syncthreads();
    };
    // the previous token of the chunk at c0 (its B after the prologue, raw B, x): token c0 - 1 of
    // the sequence, or Bprev / xprev at the start; MISC[0] = 1 if it exists
    auto load_prev = [&](int64_t c0) {
        const bool ex = c0 > 0 || has_prev;
        for (int e = tid; e < R * N; e += nt) {
            float v = 0.f;
            if (c0 > 0) v = ldt<T>(p.B, tokB(c0 - 1) + e);
            else if (has_prev) v = ldt<T>(p.Bprev, ((int64_t)s * G + g) * R * N + e);
            Bp[e] = v;
            BpRaw[e] = v;
        }
        for (int e = tid; e < R * P; e += nt) {
            float v = 0.f;
            if (c0 > 0) v = ldt<T>(p.x, tokX(c0 - 1) + e);
            else if (has_prev) v = ldt<T>(p.xprev, ((int64_t)s * H + h) * R * P + e);
            Xp[e] = v;
        }
        if (tid == 0) MISC[0] = ex ? 1.f : 0.f;
        __syncthreads();
        if (ex) prologue_rows(Bp, R, N, Bbh, INVBP);
        __syncthreads();
    };
    // B~ (and C~ when withC) and X of the chunk: raw rows, prologue, rotation by -Phi
    auto load_chunk = [&](int64_t c0, int nq, bool withC) {
        for (int e = tid; e < QR * N; e += nt) {
            const int r = e / N, n = e % N, t = r / R, j = r % R;
            float bv = 0.f, cv = 0.f;
            if (t < nq) {
                const int64_t o = tokB(c0 + t) + j * N + n;
                bv = ldt<T>(p.B, o);
                if (withC) cv = ldt<T>(p.C, o);
            }
            Bt[r * NS + n] = bv;
            if (withC) Ct[r * NS + n] = cv;
        }
        for (int e = tid; e < QR * P; e += nt) {
            const int r = e / P, pp = e % P, t = r / R, j = r % R;
            Xs[r * PS + pp] = (t < nq) ? ldt<T>(p.x, tokX(c0 + t) + j * P + pp) : 0.f;
        }
        __syncthreads();
        prologue_rows(Bt, nq * R, NS, Bbh, INVB);
        if (withC) prologue_rows(Ct, nq * R, NS, Cbh, INVC);
        __syncthreads();
        for (int e = tid; e < nq * K * R; e += nt) {
            const int t = e / (K * R), k = (e / R) % K, j = e % R, r = t * R + j;
            const float cs = CS[t * K + k], sn = SN[t * K + k];
            const float b0 = Bt[r * NS + 2 * k], b1 = Bt[r * NS + 2 * k + 1];
            Bt[r * NS + 2 * k] = cs * b0 + sn * b1;
            Bt[r * NS + 2 * k + 1] = -sn * b0 + cs * b1;
            if (withC) {
                const float q0 = Ct[r * NS + 2 * k], q1 = Ct[r * NS + 2 * k + 1];
                Ct[r * NS + 2 * k] = cs * q0 + sn * q1;
                Ct[r * NS + 2 * k + 1] = -sn * q0 + cs * q1;
            }
        }
        __syncthreads();
    };

    // ------------------------------------------------------------ forward: chunk states
    for (int e = tid; e < N * P; e += nt) Hs[(e / P) * PS + e % P] = p.h_in ? p.h_in[sh * N * P + e] : 0.f;
    __syncthreads();
    for (int64_t c = 0; c < nch; c++) {
        const int64_t c0 = c * Q;
        const int nq = (int)min((int64_t)Q, len - c0);
        load_scalars(c0, nq);
        load_prev(c0);
        const float d0 = DL[0];
        float *ws = wsS(c);
        for (int e = tid; e < N * P; e += nt) {
            const int n = e / P, pp = e % P;
            float acc = 0.f;
            for (int j = 0; j < R; j++) acc += Bp[j * N + n] * Xp[j * P + pp];
            const float v = Hs[n * PS + pp] + d0 * acc;
            Hs[n * PS + pp] = v;
            ws[e] = v;
        }
        load_chunk(c0, nq, false);   // its first barrier also orders the state writes above
        const float eSe = ES[nq - 1];
        for (int e = tid; e < K * P; e += nt) {
            const int k = e / P, pp = e % P;
            float u0 = eSe * Hs[(2 * k) * PS + pp], u1 = eSe * Hs[(2 * k + 1) * PS + pp];
            for (int q = 0; q < nq * R; q++) {
                const int t = q / R;
                const float w = CU[t] * Xs[q * PS + pp];
                u0 += w * Bt[q * NS + 2 * k];
                u1 += w * Bt[q * NS + 2 * k + 1];
            }
            const float cs = CS[(nq - 1) * K + k], sn = SN[(nq - 1) * K + k];
            Hs[(2 * k) * PS + pp] = cs * u0 - sn * u1;
            Hs[(2 * k + 1) * PS + pp] = sn * u0 + cs * u1;
        }
        __syncthreads();
    }

    // ------------------------------------------------------------ reverse
    for (int e = tid; e < N * P; e += nt) dH[(e / P) * PS + e % P] = p.dh_out ? p.dh_out[sh * N * P + e] : 0.f;
    for (int e = tid; e < R * N; e += nt) dBcIn[e] = 0.f;
    for (int e = tid; e < R * P; e += nt) dXcIn[e] = 0.f;
    for (int e = tid; e < N; e += nt) BBA[e] = CBA[e] = 0.f;
    for (int e = tid; e < R * N; e += nt) BpRaw[e] = 0.f;   // (an empty sequence loads no previous token)
    for (int e = tid; e < R; e += nt) INVBP[e] = 1.f;
    float dA_acc = 0.f, dD_acc = 0.f;   // thread partials (fixed order: reduced at the end)
    __syncthreads();
    for (int64_t c = nch - 1; c >= 0; c--) {
        const int64_t c0 = c * Q;
        const int nq = (int)min((int64_t)Q, len - c0), e_ = nq - 1;
        load_scalars(c0, nq);
        load_prev(c0);
        load_chunk(c0, nq, true);
        const float *ws = wsS(c);
        for (int e = tid; e < N * P; e += nt) Hs[(e / P) * PS + e % P] = ws[e];
        for (int e = tid; e < QR * P; e += nt) {
            const int r = e / P, pp = e % P, t = r / R, j = r % R;
            dY[r * PS + pp] = (t < nq) ? ldt<T>(p.dy, tokX(c0 + t) + j * P + pp) : 0.f;
        }
        for (int e = tid; e < QR * NS; e += nt) dBt[e] = dCt[e] = 0.f;
        for (int e = tid; e < Q * K; e += nt) DPHI[e] = 0.f;
        for (int t = tid; t < Q; t += nt) DS[t] = DGM[t] = DDL[t] = 0.f;
        // G^ = R(-Phi_e) dH_n, in place
        for (int e = tid; e < K * P; e += nt) {
            const int k = e / P, pp = e % P;
            const float cs = CS[e_ * K + k], sn = SN[e_ * K + k];
            const float g0 = dH[(2 * k) * PS + pp], g1 = dH[(2 * k + 1) * PS + pp];
            dH[(2 * k) * PS + pp] = cs * g0 + sn * g1;
            dH[(2 * k + 1) * PS + pp] = -sn * g0 + cs * g1;
        }
        // scores C~_r . B~_q over the causal part (zero elsewhere)
        for (int e = tid; e < QR * QR; e += nt) {
            const int r = e / QR, q = e % QR, t = r / R, u = q / R;
            float v = 0.f;
            if (u <= t && t < nq)
                for (int n = 0; n < N; n++) v += Ct[r * NS + n] * Bt[q * NS + n];
            Sc[r * QS + q] = v;
        }
        __syncthreads();
        // outputs before the gate, the gate's gradient, dy0 = dL/d(pre-gate y); Wk = dy0 * inter term
        for (int e = tid; e < QR * P; e += nt) {
            const int r = e / P, pp = e % P, t = r / R, j = r % R;
            float dy0 = 0.f, prod = 0.f;
            if (t < nq) {
                float yin = 0.f;
                for (int n = 0; n < N; n++) yin += Ct[r * NS + n] * Hs[n * PS + pp];
                yin *= ES[t];
                float yintra = 0.f;
                for (int q = 0; q < (t + 1) * R; q++) {
                    const int u = q / R;
                    const float mw = EM[t * Q + u] * ((u < t) ? G1[u] : GM[u]);
                    yintra += mw * Sc[r * QS + q] * Xs[q * PS + pp];
                }
                const float y0 = yin + yintra + Dh * Xs[r * PS + pp];
                const float d = dY[r * PS + pp];
                if (p.z) {
                    const int64_t oz = tokX(c0 + t) + j * P + pp;
                    const float v = ldt<T>(p.z, oz), sg = 1.f / (1.f + expf(-v));
                    dy0 = d * v * sg;
                    if (p.dz) stt<T>(p.dz, oz, d * y0 * (sg + v * sg * (1.f - sg)));
                } else {
                    dy0 = d;
                }
                prod = dy0 * yin;
            }
            dY[r * PS + pp] = dy0;
            Wk[r * PS + pp] = prod;
        }
        __syncthreads();
        // row sums: inter-term share of dS (ROWA), D's gradient; dP over the causal part
        for (int r = tid; r < QR; r += nt) {
            float a = 0.f, d = 0.f;
            for (int pp = 0; pp < P; pp++) {
                a += Wk[r * PS + pp];
                d += dY[r * PS + pp] * Xs[r * PS + pp];
            }
            ROWA[r] = a;
            dD_acc += d;
        }
        for (int e = tid; e < QR * QR; e += nt) {
            const int r = e / QR, q = e % QR, t = r / R, u = q / R;
            float v = 0.f;
            if (u <= t && t < nq)
                for (int pp = 0; pp < P; pp++) v += dY[r * PS + pp] * Xs[q * PS + pp];
            dPm[r * QS + q] = v;
        }
        __syncthreads();
        // d(mask): dMw = Sc * dP. Row sums of dMw * Mw (dS_t), column sums of the same (-dS_s) and of
        // dMw * e^{S_t - S_s} for s <= t (d gamma_s) and s < t (d delta_{s+1})
        for (int r = tid; r < QR; r += nt) {
            const int t = r / R;
            float a = 0.f;
            for (int q = 0; q <= (t + 1) * R - 1 && t < nq; q++) {
                const int u = q / R;
                const float mw = EM[t * Q + u] * ((u < t) ? G1[u] : GM[u]);
                a += Sc[r * QS + q] * dPm[r * QS + q] * mw;
            }
            ROWB[r] = a;
        }
        for (int q = tid; q < QR; q += nt) {
            const int u = q / R;
            float cs_ = 0.f, cg = 0.f, cd = 0.f;
            for (int r = u * R; r < nq * R; r++) {
                const int t = r / R;
                const float E = EM[t * Q + u];
                const float dm = Sc[r * QS + q] * dPm[r * QS + q];
                const float mw = E * ((u < t) ? G1[u] : GM[u]);
                cs_ += dm * mw;
                cg += dm * E;
                if (u < t) cd += dm * E;
            }
            COLS[q] = cs_;
            COLG[q] = cg;
            COLD[q] = cd;
        }
        __syncthreads();
        // dScore = Mw dP (in dPm), A = Mw Sc (in Sc)
        for (int e = tid; e < QR * QR; e += nt) {
            const int r = e / QR, q = e % QR, t = r / R, u = q / R;
            float mw = 0.f;
            if (u <= t && t < nq) mw = EM[t * Q + u] * ((u < t) ? G1[u] : GM[u]);
            dPm[r * QS + q] *= mw;
            Sc[r * QS + q] *= mw;
        }
        __syncthreads();
        // dX, and Wk = (G^^T B~_q)[p] X_q[p] (for dc); dC~; dB~
        for (int e = tid; e < QR * P; e += nt) {
            const int q = e / P, pp = e % P, u = q / R, j = q % R;
            float prod = 0.f;
            if (u < nq) {
                float gb = 0.f;
                for (int n = 0; n < N; n++) gb += dH[n * PS + pp] * Bt[q * NS + n];
                const float cq = CU[u];
                float dx = cq * gb + Dh * dY[q * PS + pp];
                for (int r = u * R; r < nq * R; r++) dx += Sc[r * QS + q] * dY[r * PS + pp];
                if (u == e_) dx += dXcIn[j * P + pp];
                stt<T>(p.dx, tokX(c0 + u) + j * P + pp, dx);
                prod = gb * Xs[q * PS + pp];
            }
            Wk[q * PS + pp] = prod;
        }
        for (int e = tid; e < QR * N; e += nt) {
            const int r = e / N, n = e % N, t = r / R;
            if (t >= nq) continue;
            float a = 0.f;
            for (int q = 0; q < (t + 1) * R; q++) a += dPm[r * QS + q] * Bt[q * NS + n];
            float b = 0.f;
            for (int pp = 0; pp < P; pp++) b += Hs[n * PS + pp] * dY[r * PS + pp];
            dCt[r * NS + n] = a + ES[t] * b;
        }
        for (int e = tid; e < QR * N; e += nt) {
            const int q = e / N, n = e % N, u = q / R;
            if (u >= nq) continue;
            float a = 0.f;
            for (int r = u * R; r < nq * R; r++) a += dPm[r * QS + q] * Ct[r * NS + n];
            float b = 0.f;
            for (int pp = 0; pp < P; pp++) b += dH[n * PS + pp] * Xs[q * PS + pp];
            dBt[q * NS + n] = a + CU[u] * b;
        }
        float gh_acc = 0.f;   // <G^, H'>, this thread's terms
        // dPhi_e: Wk2[k][p] = G^1 Inner0 - G^0 Inner1 with Inner = e^{S_e} H' + sum_q c_q B~_q X_q^T;
        // and <G^, H'> (the state decay's share of dS_e)
        for (int e = tid; e < K * P; e += nt) {
            const int k = e / P, pp = e % P;
            const float eSe = ES[e_];
            float i0 = eSe * Hs[(2 * k) * PS + pp], i1 = eSe * Hs[(2 * k + 1) * PS + pp];
            for (int q = 0; q < nq * R; q++) {
                const int u = q / R;
                const float w = CU[u] * Xs[q * PS + pp];
                i0 += w * Bt[q * NS + 2 * k];
                i1 += w * Bt[q * NS + 2 * k + 1];
            }
            const float g0 = dH[(2 * k) * PS + pp], g1 = dH[(2 * k + 1) * PS + pp];
            Wk2[k * PS + pp] = g1 * i0 - g0 * i1;
            gh_acc += g0 * Hs[(2 * k) * PS + pp] + g1 * Hs[(2 * k + 1) * PS + pp];
        }
        const float gh = block_sum(gh_acc, MISC + 4);   // <G^, H'> (also the barrier of this phase)
        // dc per row q: the sum of Wk's row, kept in the row's first element
        for (int q = tid; q < QR; q += nt) {
            float a = 0.f;
            for (int pp = 0; pp < P; pp++) a += Wk[q * PS + pp];
            Wk[q * PS] = a;   // dc share of row q (first element of the row; read after the barrier)
        }
        for (int k = tid; k < K; k += nt) {
            float a = 0.f;
            for (int pp = 0; pp < P; pp++) a += Wk2[k * PS + pp];
            DPHI[e_ * K + k] += a;
        }
        __syncthreads();
        // dH' = e^{S_e} G^ + sum_r e^{S_t} C~_r dy_r^T (in place: every read of G^ is done)
        for (int e = tid; e < N * P; e += nt) {
            const int n = e / P, pp = e % P;
            float v = ES[e_] * dH[n * PS + pp];
            for (int r = 0; r < nq * R; r++) v += ES[r / R] * Ct[r * NS + n] * dY[r * PS + pp];
            dH[n * PS + pp] = v;
        }
        // dPhi_t from C~ and B~ (thread per (t, k))
        for (int e = tid; e < nq * K; e += nt) {
            const int t = e / K, k = e % K;
            float a = 0.f;
            for (int j = 0; j < R; j++) {
                const int r = t * R + j;
                a += dCt[r * NS + 2 * k] * Ct[r * NS + 2 * k + 1] - dCt[r * NS + 2 * k + 1] * Ct[r * NS + 2 * k];
                a += dBt[r * NS + 2 * k] * Bt[r * NS + 2 * k + 1] - dBt[r * NS + 2 * k + 1] * Bt[r * NS + 2 * k];
            }
            DPHI[t * K + k] += a;
        }
        __syncthreads();
        // per-token scalar gradients: dS (inter rows, mask rows/columns, state), d gamma, d delta
        if (tid == 0) {
            float dSe = ES[e_] * gh;
            for (int u = 0; u < nq; u++) {
                float rowA = 0.f, rowB = 0.f, colS = 0.f, colG = 0.f, colD = 0.f, dc = 0.f;
                for (int j = 0; j < R; j++) {
                    const int q = u * R + j;
                    rowA += ROWA[q];
                    rowB += ROWB[q];
                    colS += COLS[q];
                    colG += COLG[q];
                    colD += COLD[q];
                    dc += Wk[q * PS];
                }
                const float E = EM[e_ * Q + u];
                const float cu = CU[u];
                DS[u] += rowA + rowB - colS - dc * cu;
                dSe += dc * cu;
                DGM[u] += colG + dc * E;
                if (u + 1 < nq) DDL[u + 1] += colD + dc * E;
            }
            DS[e_] += dSe;
        }
        // the fold at the chunk start: d delta_0 = <dH', Bp Xp^T>, carries for the previous token
        float fold_acc = 0.f;   // <dH', Bp Xp^T>, this thread's terms
        if (MISC[0] != 0.f) {
            for (int e = tid; e < R * N; e += nt) {
                const int j = e / N, n = e % N;
                float a = 0.f;
                for (int pp = 0; pp < P; pp++) a += dH[n * PS + pp] * Xp[j * P + pp];
                dBcOut[e] = DL[0] * a;
                fold_acc += Bp[e] * a;
            }
            for (int e = tid; e < R * P; e += nt) {
                const int j = e / P, pp = e % P;
                float a = 0.f;
                for (int n = 0; n < N; n++) a += dH[n * PS + pp] * Bp[j * N + n];
                dXcOut[e] = DL[0] * a;
            }
        } else {
            for (int e = tid; e < R * N; e += nt) dBcOut[e] = 0.f;
            for (int e = tid; e < R * P; e += nt) dXcOut[e] = 0.f;
        }
        const float fold = block_sum(fold_acc, MISC + 4);
        if (tid == 0) DDL[0] += fold;
        __syncthreads();
        // reverse prefix sums over the chunk: dphi (per angle pair) and d(dt A)
        for (int k = tid; k < K; k += nt) {
            float acc = 0.f;
            for (int t = nq - 1; t >= 0; t--) {
                acc += DPHI[t * K + k];
                DPHI[t * K + k] = acc;
            }
        }
        if (tid == 0) {
            float acc = 0.f;
            for (int t = nq - 1; t >= 0; t--) {
                acc += DS[t];
                DS[t] = acc;
            }
        }
        __syncthreads();
        for (int e = tid; e < nq * K; e += nt) {
            const int t = e / K, k = e % K;
            st_dtheta<T>(p, start + c0 + t, h, k, DT[t] * DPHI[e]);
        }
        for (int t = tid; t < nq; t += nt) {
            float ddt = AT[t] * DS[t] + (1.f - LM[t]) * DDL[t] + LM[t] * DGM[t];
            const int64_t tr = th_row(p, start + c0 + t, h);
            for (int k = 0; k < K; k++) ddt += ldt<T>(p.theta, tr + k) * DPHI[t * K + k];
            stt<T>(p.ddt, (start + c0 + t) * H + h, ddt);
            if (p.dlam) stt<T>(p.dlam, (start + c0 + t) * H + h, DT[t] * (DGM[t] - DDL[t]));
            if (p.A_tok) stt<T>(p.dA_tok, (start + c0 + t) * H + h, DT[t] * DS[t]);
            else dA_acc += DT[t] * DS[t];
        }
        // dB, dC: rotate back to the physical frame (+ the carry into the last token), then back
        // through the prologue to the raw columns; bias gradients accumulate per slab
        for (int e = tid; e < nq * K * R; e += nt) {
            const int t = e / (K * R), k = (e / R) % K, j = e % R, r = t * R + j;
            const float cs = CS[t * K + k], sn = SN[t * K + k];
            float d0 = dBt[r * NS + 2 * k], d1 = dBt[r * NS + 2 * k + 1];
            float b0 = cs * d0 - sn * d1, b1 = sn * d0 + cs * d1;
            if (t == e_) {
                b0 += dBcIn[j * N + 2 * k];
                b1 += dBcIn[j * N + 2 * k + 1];
            }
            dBt[r * NS + 2 * k] = b0;
            dBt[r * NS + 2 * k + 1] = b1;
            d0 = dCt[r * NS + 2 * k];
            d1 = dCt[r * NS + 2 * k + 1];
            dCt[r * NS + 2 * k] = cs * d0 - sn * d1;
            dCt[r * NS + 2 * k + 1] = sn * d0 + cs * d1;
        }
        __syncthreads();
        for (int n = tid; n < N; n += nt) {
            float a = 0.f, b = 0.f;
            for (int r = 0; r < nq * R; r++) {
                a += dBt[r * NS + n];
                b += dCt[r * NS + n];
            }
            BBA[n] += a;
            CBA[n] += b;
        }
        for (int r = tid; r < 2 * nq * R; r += nt) {
            const bool isC = r >= nq * R;
            const int rr = isC ? r - nq * R : r, t = rr / R, j = rr % R;
            const float *gout = (isC ? dCt : dBt) + rr * NS;
            const float inv = (isC ? INVC : INVB)[rr];
            const void *src = isC ? p.C : p.B;
            const int64_t o = tokB(c0 + t) + j * N;
            float dot = 0.f;
            if (p.norm)
                for (int n = 0; n < N; n++) dot += gout[n] * ldt<T>(src, o + n);
            const float k3 = p.norm ? dot * inv * inv * inv / (float)N : 0.f;
            float *part = isC ? p.p_dC : p.p_dB;
            for (int n = 0; n < N; n++) {
                const float v = p.norm ? gout[n] * inv - k3 * ldt<T>(src, o + n) : gout[n];
                if (part) part[((start + c0 + t) * H + h) * (int64_t)R * N + j * N + n] = v;
                else stt<T>(isC ? p.dC : p.dB, o + n, v);
            }
        }
        // carries: this chunk's fold feeds the previous chunk's last token
        for (int e = tid; e < R * N; e += nt) dBcIn[e] = dBcOut[e];
        for (int e = tid; e < R * P; e += nt) dXcIn[e] = dXcOut[e];
        __syncthreads();
    }

    // ------------------------------------------------------------ slab results
    if (p.dh_in)
        for (int e = tid; e < N * P; e += nt) p.dh_in[sh * N * P + e] = dH[(e / P) * PS + e % P];
    if (has_prev) {
        // dBprev: the carry of the first chunk's fold (zero for an empty sequence), through the prologue
        for (int j = tid; j < R; j += nt) {
            const float *gout = dBcIn + j * N;
            const float inv = INVBP[j];
            const int64_t o = ((int64_t)s * G + g) * R * N + j * N;
            float dot = 0.f;
            if (p.norm)
                for (int n = 0; n < N; n++) dot += gout[n] * BpRaw[j * N + n];
            const float k3 = p.norm ? dot * inv * inv * inv / (float)N : 0.f;
            for (int n = 0; n < N; n++) {
                const float v = p.norm ? gout[n] * inv - k3 * BpRaw[j * N + n] : gout[n];
                if (p.p_dBprev) p.p_dBprev[sh * (int64_t)R * N + j * N + n] = v;
                else if (p.dBprev) stt<T>(p.dBprev, o + n, v);
            }
        }
        for (int n = tid; n < N; n += nt)
            for (int j = 0; j < R; j++) BBA[n] += dBcIn[j * N + n];
        for (int e = tid; e < R * P; e += nt)
            if (p.dxprev) stt<T>(p.dxprev, sh * R * P + e, dXcIn[e]);
    }
    // per-slab partial sums (thread partials reduced through LDS in thread order)
    __syncthreads();
    Wk[tid] = dA_acc;
    Wk2[tid] = dD_acc;
    __syncthreads();
    if (tid == 0) {
        float a = 0.f, d = 0.f;
        for (int i = 0; i < nt; i++) {
            a += Wk[i];
            d += Wk2[i];
        }
        p.p_dA[sh] = a;
        p.p_dD[sh] = d;
    }
    for (int n = tid; n < N; n += nt) {
        p.p_dBb[sh * N + n] = BBA[n];
        p.p_dCb[sh * N + n] = CBA[n];
    }
}

// ---------------------------------------------------------------- MFMA path (bf16 token inputs)
// The same chunked backward with every chunk contraction on v_mfma_f32_16x16x32_bf16: bf16
// operands staged in LDS, fp32 accumulation. The state entering each chunk (forward pass) and
// the carried gradient dH (reverse pass) live in fp32 accumulator registers; each wave owns
// N x P tiles of both. The chunk states go through the workspace in bf16, column-major per
// chunk ([P][N]: a lane's four consecutive rows are one 8-byte piece): the state's bf16 copy is
// what the contractions read anyway, and only the e^{S_e} H' terms of the rotated state and of
// the chunk's decay gradient see the rounding, each once (the chain itself stays fp32). Per chunk: scores S = C~ B~^T and dP = dY X^T on the causal tiles
// (masked into A = M o S and dS' = M o dP), then dX = A^T dY + c o (B~ G^), dC~ = dS' B~ +
// e^{S} o (dY H'^T), dB~ = dS'^T C~ + c o (X G^^T), dH' = e^{S_e} G^ + C~^T (e^{S} o dY) and the
// rotated state Inner = e^{S_e} H' + B~^T (c o X). Row and column sums that the scalar
// gradients need are formed per tile (DPP row sums, wave shuffles) and added in a fixed order.
// Latency, not bandwidth, sets the time of a chunk, so: each chunk's token inputs (and, in the
// reverse walk, its entering state) are loaded into registers one chunk ahead; the lane index is
// made opaque per chunk so that address math is recomputed rather than spilled; block-wide sums
// go through per-wave partials read after barriers the phases need anyway.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// An empty asm that reads and rewrites v: the compiler's wait for a load into v falls here, and
// later reads of v need none.
template <class V>
__device__ __forceinline__ void held(V &v) {
    if constexpr (sizeof(V) == 16) {
        u32x4 u = __builtin_bit_cast(u32x4, v);
        asm volatile("" : "+v"(u));
        v = __builtin_bit_cast(V, u);
    } else if constexpr (sizeof(V) == 8) {
        u32x2 u = __builtin_bit_cast(u32x2, v);
        asm volatile("" : "+v"(u));
        v = __builtin_bit_cast(V, u);
    } else {
        static_assert(sizeof(V) == 2, "16-bit element");
        unsigned short u = __builtin_bit_cast(unsigned short, v);
        asm volatile("" : "+v"(u));
        v = __builtin_bit_cast(V, u);
    }
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Operands of the 16x16x32 product, lane l: i = l % 16 is the A operand's row / the B operand's
// column, g = l / 16 picks its 8 K-values of the 32-wide K block. Two K orders occur, and the
// two operands of one product always use the same one:
//   natural: K = 8g .. 8g + 7                                  (op_nat)
//   split:   K = 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3         (op_split, op_tr)
// op_nat and op_split read a row of a K-contiguous matrix ([row][K]); op_tr reads column c0 + i
// of a matrix stored with K as its row index ([K][col]) through the LDS transpose read.
__device__ __forceinline__ bf16x8 op_nat(const bf16 *m, int ld, int row, int k0, int g) {
    return *(const bf16x8 *)(m + row * ld + k0 + 8 * g);
}
__device__ __forceinline__ bf16x8 op_split(const bf16 *m, int ld, int row, int k0, int g) {
    const bf16x4 a = *(const bf16x4 *)(m + row * ld + k0 + 4 * g);
    const bf16x4 b = *(const bf16x4 *)(m + row * ld + k0 + 16 + 4 * g);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// LDS transpose read (16-bit elements): within a group of 16 lanes, lane i receives element
// i % 4 of the 4 elements read by lanes i / 4 + 4k, k = 0..3; pointed at &M[r0 + i/4][c0 + 4(i%4)],
// lane i receives M[r0 + k][c0 + i], k = 0..3.
__device__ __forceinline__ bf16x4 ds_tr4(const bf16 *q) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(q));
    return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 op_tr(const bf16 *m, int ld, int k0, int c0, int i, int g) {
    const bf16x4 a = ds_tr4(m + (k0 + 4 * g + i / 4) * ld + c0 + 4 * (i % 4));
    const bf16x4 b = ds_tr4(m + (k0 + 16 + 4 * g + i / 4) * ld + c0 + 4 * (i % 4));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// sum over the 16 lanes of a lane group (i = l % 16), and over the 4 groups (g = l / 16)
// (lane-to-lane moves within a row of 16 lanes: DPP, no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
    v += dppf<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    v += dppf<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    v += dppf<0x141>(v);   // row_half_mirror: the other quad of the 8
    v += dppf<0x140>(v);   // row_mirror: the other 8 lanes of the row
    return v;
}
// (the lane ^ 16 and lane ^ 32 partners through gfx950's row-swap instructions, VALU rather than
// the LDS crossbar: v_permlane16_swap pairs rows 0-1 and 2-3, v_permlane32_swap the two halves;
// each returns the lower and the upper partner, so both lanes of a pair add the same two values)
__device__ __forceinline__ float sum_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// sum over the 64 lanes of a wave (the same pairing order as a xor butterfly 1, 2, ..., 32)
__device__ __forceinline__ float wave_sum(float v) { return sum_groups(sum16(v)); }

template <int N_, int P_, int R_, int Q_, int NW_>
struct BCfg {
    static constexpr int N = N_, P = P_, R = R_, Q = Q_, NW = NW_;
    static constexpr int QR = Q * R, K2 = N / 2, NT = NW * 64;
    // NF: fp32 dC~ / dB~ rows, 16-byte aligned (their pieces are read as vectors; the tile
    // epilogues' 4-byte writes of 16 columns by rows 4 apart still meet no bank conflict)
    static constexpr int NS = N + 8, PS = P + 8, QS = QR + 8, NF = N + 4, SF = QR + 1;
    static constexpr int TQ = QR / 16, TN = N / 16, TP = P / 16, NPT = TN * TP, UPW = NPT / NW;
    static_assert(QR % 32 == 0 && N % 32 == 0 && P % 32 == 0 && NPT % NW == 0, "MFMA backward tiling");
    static_assert((NT & (NT - 1)) == 0, "the thread index is masked to the workgroup size");
    static_assert(R == 1 || R == 2 || R == 4, "rank");
    // LDS layout (bytes; every region 16-byte aligned)
    static constexpr int al(int b) { return (b + 15) / 16 * 16; }
    static constexpr int O_CS = 0, O_SN = O_CS + al(Q * K2 * 4), O_DPHI = O_SN + al(Q * K2 * 4);
    static constexpr int O_SC = O_DPHI + al(Q * K2 * 4);            // 12 float [Q] tables
    static constexpr int O_EM = O_SC + al(12 * Q * 4);              // float [Q][Q]
    static constexpr int O_INV = O_EM + al(Q * Q * 4);              // float [2][QR]
    static constexpr int O_RPM = O_INV + al(2 * QR * 4);            // float [QR][TQ] row partials of dM M
    static constexpr int O_CPM = O_RPM + al(QR * TQ * 4);           // float [3][QR][TQ] column partials
    static constexpr int O_RPI = O_CPM + al(3 * QR * TQ * 4);       // float [QR][TN] dS inter partials
    static constexpr int O_RPC = O_RPI + al(QR * TN * 4);           // float [QR][TP] dc partials
    static constexpr int O_PHE = O_RPC + al(QR * TP * 4);           // float [K2][TP] dPhi_e partials
    static constexpr int O_TH = O_PHE + al(K2 * TP * 4);            // bf16 [Q][K2] theta of the chunk
    static constexpr int O_SMALL = O_TH + al(Q * K2 * 2);           // biases, previous token, carries
    static constexpr int SMALL = 2 * N + 6 * R * N + 4 * R * P + R + 2 * N + 16 + 64;
    static constexpr int O_DCF = O_SMALL + al(SMALL * 4);           // float [QR][NF] dC~ (raw C staging)
    static constexpr int O_DBF = O_DCF + al(QR * NF * 4);           // float [QR][NF] dB~ (raw B staging)
    // float [QR][SF] scores: over the raw C staging when it fits (QR <= N). The staging is dead
    // from the rotation into C~ until dC~ is written, and the scores live from the score tiles to
    // dP, inside that window.
    static constexpr bool SF_ALIAS = QR <= N;
    static constexpr int O_SF = SF_ALIAS ? O_DCF : O_DBF + al(QR * NF * 4);
    static constexpr int O_CT = SF_ALIAS ? O_DBF + al(QR * NF * 4) : O_SF + al(QR * SF * 4);   // bf16 [QR][NS] C~
    static constexpr int O_BT = O_CT + al(QR * NS * 2);             // bf16 [QR][NS] B~
    static constexpr int O_XB = O_BT + al(QR * NS * 2);             // bf16 [QR][PS] X
    static constexpr int O_XC = O_XB + al(QR * PS * 2);             // bf16 [QR][PS] c o X
    static constexpr int O_DY = O_XC + al(QR * PS * 2);             // bf16 [QR][PS] dy0
    static constexpr int O_EDY = O_DY + al(QR * PS * 2);            // bf16 [QR][PS] e^{S} o dy0
    static constexpr int O_HB = O_EDY + al(QR * PS * 2);            // bf16 [N][PS] H'
    static constexpr int O_GB = O_HB + al(N * PS * 2);              // bf16 [N][PS] G^ (then the fold's partials)
    static constexpr int O_AB = O_GB + al(N * PS * 2);              // bf16 [QR][QS] A = M o S
    static constexpr int O_DSB = O_AB + al(QR * QS * 2);            // bf16 [QR][QS] dS' = M o dP
    static constexpr int LDS = O_DSB + al(QR * QS * 2);
    static_assert(LDS <= 160 * 1024, "LDS");
};

template <class CF>
__global__ __launch_bounds__(CF::NT) void k_scan_bwd_mfma(BwdParams p_arg) {
    // The arguments are read through the kernarg segment pointer (p below), which is made opaque
    // at the start of every chunk: each chunk then re-reads the arguments it uses (scalar loads
    // that hit the scalar cache) instead of holding every pointer in SGPRs across the kernel,
    // which spilled them to VGPR lanes and reloaded them all over the chunk body.
    (void)p_arg;
    using KPtr = const __attribute__((address_space(4))) BwdParams *;
    KPtr pk = (KPtr)__builtin_amdgcn_kernarg_segment_ptr();
#define p (*pk)
    constexpr int N = CF::N, P = CF::P, R = CF::R, Q = CF::Q, NW = CF::NW, QR = CF::QR, K = CF::K2, NT = CF::NT;
    constexpr int NS = CF::NS, PS = CF::PS, QS = CF::QS, NF = CF::NF, SF = CF::SF;
    constexpr int TQ = CF::TQ, TN = CF::TN, TP = CF::TP, UPW = CF::UPW;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float *CS = (float *)(smem + CF::O_CS), *SN = (float *)(smem + CF::O_SN), *DPHI = (float *)(smem + CF::O_DPHI);
    float *SC = (float *)(smem + CF::O_SC);
    float *DT = SC, *LM = SC + Q, *GM = SC + 2 * Q, *DL = SC + 3 * Q, *S = SC + 4 * Q, *G1 = SC + 5 * Q;
    float *ES = SC + 6 * Q, *CU = SC + 7 * Q, *DS = SC + 8 * Q, *DGM = SC + 9 * Q, *DDL = SC + 10 * Q;
    float *AT = SC + 11 * Q;   // A_t of each token
    float *EM = (float *)(smem + CF::O_EM);
    float *INVB = (float *)(smem + CF::O_INV), *INVC = INVB + QR;
    float *RPM = (float *)(smem + CF::O_RPM), *CPM = (float *)(smem + CF::O_CPM);
    float *CPG = CPM + QR * TQ, *CPD = CPG + QR * TQ;
    float *RPI = (float *)(smem + CF::O_RPI), *RPC = (float *)(smem + CF::O_RPC), *PHE = (float *)(smem + CF::O_PHE);
    bf16 *TH = (bf16 *)(smem + CF::O_TH);
    float *SMALLp = (float *)(smem + CF::O_SMALL);
    float *BBL = SMALLp, *CBL = BBL + N;   // the head's B and C biases (zero without them)
    float *Bp = CBL + N, *BpRaw = Bp + R * N, *Xp = BpRaw + R * N, *dBcIn = Xp + R * P, *dBcOut = dBcIn + R * N;
    float *dXcIn = dBcOut + R * N, *dXcOut = dXcIn + R * P, *INVBP = dXcOut + R * P, *BBA = INVBP + R;
    float *CBA = BBA + N, *MISC = CBA + N, *RED = MISC + 16, *TMPC = RED + 16;   // RED: 16 floats, TMPC: [Q]
    float *dCf = (float *)(smem + CF::O_DCF), *dBf = (float *)(smem + CF::O_DBF), *Sf = (float *)(smem + CF::O_SF);
    bf16 *Ct = (bf16 *)(smem + CF::O_CT), *Bt = (bf16 *)(smem + CF::O_BT), *Xb = (bf16 *)(smem + CF::O_XB);
    bf16 *XcB = (bf16 *)(smem + CF::O_XC), *dYb = (bf16 *)(smem + CF::O_DY), *EdYb = (bf16 *)(smem + CF::O_EDY);
    bf16 *Hb = (bf16 *)(smem + CF::O_HB), *Gb = (bf16 *)(smem + CF::O_GB), *Ab = (bf16 *)(smem + CF::O_AB);
    bf16 *dSb = (bf16 *)(smem + CF::O_DSB);

    const int H = p.H, G = p.G;
    int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int li = lane & 15, lg = lane >> 4;
    // The lane-derived values are made opaque once per chunk, so that address math is recomputed
    // where it is used instead of being hoisted out of the chunk loops and spilled.
    auto refresh = [&]() {
        asm volatile("" : "+v"(tid));
        asm volatile("" : "+s"(pk));
        tid &= NT - 1;   // (its range, for the address math: full-rate shifts and 24-bit products)
        lane = tid & 63;
        li = lane & 15;
        lg = lane >> 4;
    };
    const int s = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / G);
    const bf16 *gx = (const bf16 *)p.x, *gB = (const bf16 *)p.B, *gC = (const bf16 *)p.C, *gdy = (const bf16 *)p.dy;

    int64_t start, len, cbase;
    if (p.cu) {
        const int64_t a = min(max((int64_t)p.cu[s], (int64_t)0), (int64_t)p.seqlen);
        const int64_t b = min(max((int64_t)p.cu[s + 1], a), (int64_t)p.seqlen);
        start = a;
        len = b - a;
        cbase = 0;
        for (int j = 0; j < s; j++) {
            const int64_t a0 = min(max((int64_t)p.cu[j], (int64_t)0), (int64_t)p.seqlen);
            const int64_t b0 = min(max((int64_t)p.cu[j + 1], a0), (int64_t)p.seqlen);
            cbase += (b0 - a0 + Q - 1) / Q;
        }
    } else {
        start = (int64_t)s * p.seqlen;
        len = p.seqlen;
        cbase = (int64_t)s * ((p.seqlen + Q - 1) / Q);
    }
    const int64_t nch = (len + Q - 1) / Q;
    if (cbase + nch > p.ws_chunks) return;   // a sequence table that breaks its contract
    const float Ah = p.A ? p.A[h] : 0.f;
    const float Dh = p.D ? p.D[h] : 0.f;
    const bool pro = p.norm || p.Bb || p.Cb;
    const bool has_prev = p.Bprev != nullptr;
    const int64_t sh = (int64_t)s * H + h;
    // the biases are read from LDS in every chunk (a global read there would wait for every
    // memory access in flight); the first chunk's barriers order these writes
    for (int e = tid; e < N; e += NT) {
        BBL[e] = p.Bb ? p.Bb[(int64_t)h * N + e] : 0.f;
        CBL[e] = p.Cb ? p.Cb[(int64_t)h * N + e] : 0.f;
    }
    auto wsS = [&](int64_t c) { return p.ws_hs + ((cbase + c) * H + h) * (int64_t)N * P; };
    auto tokB = [&](int64_t t) { return ((start + t) * G + g) * (int64_t)R * N; };
    auto tokX = [&](int64_t t) { return ((start + t) * H + h) * (int64_t)R * P; };
    // this wave's N x P tiles: tile v covers rows n0 .. n0 + 15, columns p0 .. p0 + 15; the lane
    // holds rows n0 + 4 lg + i (i = 0..3) of column p0 + li
    auto tile_n0 = [&](int v) { return ((wave * UPW + v) / TP) * 16; };
    auto tile_p0 = [&](int v) { return ((wave * UPW + v) % TP) * 16; };

    // Prologue of `nrows` LDS rows (raw values on entry): 16 lanes per row, N/16 columns each
    auto prologue_rows = [&](float *rows, int nrows, int stride, const float *bias, float *invs) {   // bias: LDS
        for (int r0 = tid >> 4; r0 < (nrows + NT / 16 - 1) / (NT / 16) * (NT / 16); r0 += NT / 16) {
            const bool ok = r0 < nrows;   // (every lane of a group reaches the shuffles)
            float *v = rows + (int64_t)(ok ? r0 : 0) * stride;
            float inv = 1.f;
            if (p.norm) {
                float ss = 0.f;
                for (int n = li; n < N; n += 16) ss += v[n] * v[n];
                ss = sum16(ss);
                inv = 1.f / sqrtf(ss / (float)N + p.eps);
            }
            if (ok) {
                if (li == 0) invs[r0] = inv;
                if (pro)
                    for (int n = li; n < N; n += 16) v[n] = v[n] * inv + bias[n];
            }
        }
    };
    // A chunk's raw token inputs are loaded into registers one chunk ahead (issued after the
    // current chunk is staged, consumed when the next one is), so their latency overlaps the
    // current chunk's work. Each thread loads the pieces it later stages; a token past the end
    // reads the chunk's last token and is masked when consumed. The pieces: 16 bytes of B (and
    // C), of x (and dy) and of theta; one element of the previous token's B and x; and, in wave 0,
    // one token's dt, lam and A_t.
    constexpr int PF_B = (QR * N / 8 + NT - 1) / NT, PF_X = (QR * P / 8 + NT - 1) / NT;
    constexpr int PF_T = (Q * K / 8 + NT - 1) / NT, PF_V = (R * N + NT - 1) / NT, PF_U = (R * P + NT - 1) / NT;
    bf16x8 pB[PF_B], pC[PF_B], pX[PF_X], pD[PF_X], pT[PF_T];
    bf16 pBp[PF_V], pXp[PF_U], pdt = {}, plm = {}, pat = {};
    bf16x4 pH[UPW];  // reverse walk: the state entering the chunk (rows 4 lg .. 4 lg + 3), from the workspace
    // Addressing: every prefetch load is a wave-uniform base (the chunk's first token; SGPRs) plus
    // a 32-bit per-lane byte offset (a chunk spans at most Q tokens), so the loads take the
    // scalar-base form and a lane holds no 64-bit address; a lane's condition is a clamped index
    // rather than a branch.
    const int hq = h / (H / p.Gth);   // head h's angle row
    const uint32_t tsB = (uint32_t)G * R * N, tsX = (uint32_t)H * R * P, tsT = (uint32_t)p.Gth * K;   // per token
    auto prefetch = [&](int64_t c, bool rev) {
        const int64_t c0 = c * Q;
        const int last = (int)min((int64_t)Q, len - c0) - 1;
        const char *bB = (const char *)(gB + tokB(c0)), *bC = (const char *)(gC + tokB(c0));
        const char *bX = (const char *)(gx + tokX(c0)), *bD = (const char *)(gdy + tokX(c0));
        const char *bT = (const char *)((const bf16 *)p.theta + ((start + c0) * p.Gth + hq) * (int64_t)K);
#pragma unroll
        for (int i = 0; i < PF_B; i++) {
            const int e = min(tid + i * NT, QR * N / 8 - 1);   // (surplus threads repeat the last piece)
            const int r = e / (N / 8), n = (e % (N / 8)) * 8;
            const uint32_t o = ((uint32_t)min(r / R, last) * tsB + (uint32_t)((r % R) * N + n)) * 2u;
            pB[i] = *(const bf16x8 *)(bB + o);
            if (rev) pC[i] = *(const bf16x8 *)(bC + o);
        }
#pragma unroll
        for (int i = 0; i < PF_X; i++) {
            const int e = min(tid + i * NT, QR * P / 8 - 1);
            const int r = e / (P / 8), pp = (e % (P / 8)) * 8;
            const uint32_t o = ((uint32_t)min(r / R, last) * tsX + (uint32_t)((r % R) * P + pp)) * 2u;
            pX[i] = *(const bf16x8 *)(bX + o);
            if (rev) pD[i] = *(const bf16x8 *)(bD + o);
        }
#pragma unroll
        for (int i = 0; i < PF_T; i++) {
            const int e = min(tid + i * NT, Q * K / 8 - 1);
            const uint32_t o = ((uint32_t)min(e / (K / 8), last) * tsT + (uint32_t)((e % (K / 8)) * 8)) * 2u;
            pT[i] = *(const bf16x8 *)(bT + o);
        }
        const bf16 *srcB = c0 > 0 ? gB + tokB(c0 - 1) : has_prev ? (const bf16 *)p.Bprev + ((int64_t)s * G + g) * R * N : nullptr;
        const bf16 *srcX = c0 > 0 ? gx + tokX(c0 - 1) : has_prev ? (const bf16 *)p.xprev + sh * R * P : nullptr;
        if (srcB) {   // (uniform)
#pragma unroll
            for (int i = 0; i < PF_V; i++) pBp[i] = srcB[min(tid + i * NT, R * N - 1)];
#pragma unroll
            for (int i = 0; i < PF_U; i++) pXp[i] = srcX[min(tid + i * NT, R * P - 1)];
        }
        if (wave == 0) {
            const int64_t t0 = (start + c0) * H + h;
            const uint32_t o = (uint32_t)min(lane, last) * (uint32_t)H * 2u;
            pdt = *(const bf16 *)((const char *)((const bf16 *)p.dt + t0) + o);
            if (p.lam) plm = *(const bf16 *)((const char *)((const bf16 *)p.lam + t0) + o);
            if (p.A_tok) pat = *(const bf16 *)((const char *)((const bf16 *)p.A_tok + t0) + o);
        }
    };
    // reverse walk: the state entering chunk c, issued in a phase of its own (the previous chunk's
    // contractions are done by then), so its loads do not queue with the token inputs'
    auto prefetch_state = [&](int64_t c) {
        const char *ws = (const char *)wsS(c);
#pragma unroll
        for (int v = 0; v < UPW; v++)
            pH[v] = *(const bf16x4 *)(ws + (uint32_t)((tile_p0(v) + li) * N + tile_n0(v) + 4 * lg) * 2u);
    };
    // Every prefetched register taken as loaded (the reverse walk). The memory counter is in order
    // and counts stores too, so a first read at the next chunk's start would also wait for every
    // gradient store issued since; taken before the chunk's dtheta, dB and dC stores, the loads
    // have long arrived and nothing is waited for.
    auto settle = [&]() {
#pragma unroll
        for (int i = 0; i < PF_B; i++) {
            held(pB[i]);
            held(pC[i]);
        }
#pragma unroll
        for (int i = 0; i < PF_X; i++) {
            held(pX[i]);
            held(pD[i]);
        }
#pragma unroll
        for (int i = 0; i < PF_T; i++) held(pT[i]);
#pragma unroll
        for (int i = 0; i < PF_V; i++) held(pBp[i]);
#pragma unroll
        for (int i = 0; i < PF_U; i++) held(pXp[i]);
        held(pdt);
        held(plm);
        held(pat);
#pragma unroll
        for (int v = 0; v < UPW; v++) held(pH[v]);
    };
    // em: also the decay table EM (the reverse walk's)
    auto load_scalars = [&](int64_t c0, int nq, bool em) {
        static_assert(Q <= 64, "one wave scans the chunk");
        if (wave == 0) {   // per-token scalars and the log-decay prefix (wave scan)
            const int t = lane;
            float dtv = 0.f, lv = 0.f, av = Ah;
            if (t < nq) {
                dtv = (float)pdt;
                lv = p.lam ? (float)plm : p.lam_fixed;
                if (p.A_tok) av = (float)pat;
            }
            const float acc = wave_scan_dpp(dtv * av);         // DPP lane moves
            const float dln = dpp_move<0x130>((1.f - lv) * dtv);   // wave_shl:1, the next token's
            const float g1 = lv * dtv + ((t + 1 < nq) ? dln : 0.f);
            const float se = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), nq - 1));   // S_e
            if (t < Q) {
                DT[t] = dtv;
                LM[t] = lv;
                AT[t] = av;
                GM[t] = lv * dtv;
                DL[t] = (1.f - lv) * dtv;
                S[t] = acc;
                G1[t] = g1;
                // the exponentials of the log decays here (S <= 0 and S_e - S_t <= 0), from registers
                ES[t] = __expf(acc);
                CU[t] = (t < nq) ? __expf(se - acc) * g1 : 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < PF_T; i++) {   // theta of the chunk (zero past the end), 16-byte pieces
            const int e = tid + i * NT;
            if (e < Q * K / 8) {
                const int t = e / (K / 8), k = (e % (K / 8)) * 8;
                *(bf16x8 *)(TH + t * K + k) = (t < nq) ? pT[i] : bf16x8{};
            }
        }
        __syncthreads();
        {   // cumulative angles: J consecutive lanes per pair, TPG tokens each; a lane's running sum
            // over its tokens, then an exclusive scan of the lane totals across the pair's J lanes
            constexpr int J = NT / K, TPG = Q / J;
            static_assert(NT % K == 0 && Q % J == 0 && (J & (J - 1)) == 0 && J <= 16, "angle split");
            const int k = tid / J, j = tid % J;
            float a[TPG], run = 0.f;
#pragma unroll
            for (int i = 0; i < TPG; i++) {
                const int t = j * TPG + i;
                run += DT[t] * (float)TH[t * K + k];
                a[i] = run;
            }
            const float ex = group_scan_dpp<J>(run, j) - run;
#pragma unroll
            for (int i = 0; i < TPG; i++) {
                const int t = j * TPG + i;
                float sn, cs;
                __sincosf(a[i] + ex, &sn, &cs);   // hardware sin / cos: operands of bf16 products
                CS[t * K + k] = cs;
                SN[t * K + k] = sn;
            }
        }
        // the decay table e^{S_t - S_u} (u <= t, else zero), branch-free
        if (em) {
#pragma unroll
            for (int i = 0; i < (Q * Q + NT - 1) / NT; i++) {
                const int e = tid + i * NT;
                if ((Q * Q) % NT != 0 && e >= Q * Q) break;
                const int t = e / Q, u = e % Q;
                const float x = fminf(S[t] - S[u], 0.f);
                EM[e] = (u <= t) ? __expf(x) : 0.f;
            }
        }
        __syncthreads();
    };
    // the previous token into LDS (no barrier: load_scalars' first one orders it), then its prologue
    auto stage_prev = [&](int64_t c0) {
        const bool ex = c0 > 0 || has_prev;
#pragma unroll
        for (int i = 0; i < PF_V; i++) {
            const int e = tid + i * NT;
            if (e < R * N) {
                const float v = ex ? (float)pBp[i] : 0.f;
                Bp[e] = v;
                BpRaw[e] = v;
            }
        }
#pragma unroll
        for (int i = 0; i < PF_U; i++) {
            const int e = tid + i * NT;
            if (e < R * P) Xp[e] = ex ? (float)pXp[i] : 0.f;
        }
        if (tid == 0) MISC[0] = ex ? 1.f : 0.f;
    };
    auto prologue_prev = [&](int64_t c0) {
        if (pro && (c0 > 0 || has_prev)) {
            prologue_rows(Bp, R, N, BBL, INVBP);
            __syncthreads();
        }
    };
    // B~ (and C~, dy in the reverse pass) and X, c o X of the chunk in bf16. B and C go from the
    // prefetched 16-byte pieces straight to their rotated bf16 rows: a row's pieces sit on the
    // N / 8 consecutive lanes of one DPP row group, which form the row's sum of squares for the
    // prologue; each lane then rotates its 4 pairs by R(-Phi_t) and writes one 16-byte piece.
    static_assert(N / 8 == 8 || N / 8 == 16, "a row's pieces fill half or all of a 16-lane DPP row");
    auto row_sum = [&](float v) {   // over the N / 8 lanes holding one row
        v += dppf<0xB1>(v);
        v += dppf<0x4E>(v);
        v += dppf<0x141>(v);
        if constexpr (N / 8 == 16) v += dppf<0x140>(v);
        return v;
    };
    auto stage_rows = [&](const bf16x8 &raw, int r, int n, int nq_, const float *bias, float *invs, bf16 *dst) {
        const int t = r / R;
        float u[8];
#pragma unroll
        for (int m = 0; m < 8; m++) u[m] = (t < nq_) ? (float)raw[m] : 0.f;
        if (pro) {
            float inv = 1.f;
            if (p.norm) {
                float ss = 0.f;
#pragma unroll
                for (int m = 0; m < 8; m++) ss += u[m] * u[m];
                inv = 1.f / sqrtf(row_sum(ss) / (float)N + p.eps);
            }
            if (n == 0) invs[r] = inv;
            const f32x4 b0 = *(const f32x4 *)(bias + n), b1 = *(const f32x4 *)(bias + n + 4);
#pragma unroll
            for (int m = 0; m < 8; m++) u[m] = (t < nq_) ? u[m] * inv + ((m < 4) ? b0[m] : b1[m - 4]) : 0.f;
        }
        const f32x4 cs = *(const f32x4 *)(CS + t * K + n / 2), sn = *(const f32x4 *)(SN + t * K + n / 2);
        bf16x8 o;
#pragma unroll
        for (int m = 0; m < 4; m++) {
            o[2 * m] = (bf16)(cs[m] * u[2 * m] + sn[m] * u[2 * m + 1]);
            o[2 * m + 1] = (bf16)(-sn[m] * u[2 * m] + cs[m] * u[2 * m + 1]);
        }
        *(bf16x8 *)(dst + r * NS + n) = o;
    };
    float dA_acc = 0.f, dD_acc = 0.f;   // thread partials (fixed order: reduced at the end)
    auto stage_chunk = [&](int64_t c0, int nq, bool rev) {
        (void)c0;
#pragma unroll
        for (int i = 0; i < PF_B; i++) {   // 16-byte pieces; whole rows are active or not
            const int e = tid + i * NT;
            if (e >= QR * N / 8) break;
            const int r = e / (N / 8), n = (e % (N / 8)) * 8;
            stage_rows(pB[i], r, n, nq, BBL, INVB, Bt);
            if (rev) stage_rows(pC[i], r, n, nq, CBL, INVC, Ct);
        }
#pragma unroll
        for (int i = 0; i < PF_X; i++) {
            const int e = tid + i * NT;
            if (e >= QR * P / 8) break;
            const int r = e / (P / 8), pp = (e % (P / 8)) * 8, t = r / R;
            const bf16x8 xv = (t < nq) ? pX[i] : bf16x8{}, dv = (rev && t < nq) ? pD[i] : bf16x8{};
            bf16x8 xc;
#pragma unroll
            for (int m = 0; m < 8; m++) xc[m] = (bf16)(CU[t] * (float)xv[m]);
            *(bf16x8 *)(Xb + r * PS + pp) = xv;
            *(bf16x8 *)(XcB + r * PS + pp) = xc;
            if (rev) {
                *(bf16x8 *)(dYb + r * PS + pp) = dv;
                if (!p.z) {   // e^{S} o dy and D's gradient (with the gate they wait for dy0)
                    bf16x8 ed;
#pragma unroll
                    for (int m = 0; m < 8; m++) {
                        ed[m] = (bf16)(ES[t] * (float)dv[m]);
                        dD_acc += (float)dv[m] * (float)xv[m];
                    }
                    *(bf16x8 *)(EdYb + r * PS + pp) = ed;
                }
            }
        }
        __syncthreads();
    };

    // ------------------------------------------------------------ forward: chunk states
    if (!p.fwd_states) {
    f32x4 hacc[UPW];
#pragma unroll
    for (int v = 0; v < UPW; v++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int n = tile_n0(v) + 4 * lg + i, pp = tile_p0(v) + li;
            hacc[v][i] = p.h_in ? p.h_in[sh * N * P + n * P + pp] : 0.f;
        }
#pragma unroll
    for (int v = 0; v < UPW; v++) held(hacc[v]);
    if (nch > 0) prefetch(0, false);
    for (int64_t c = 0; c < nch; c++) {
        const int64_t c0 = c * Q;
        const int nq = (int)min((int64_t)Q, len - c0), e_ = nq - 1;
        refresh();
        stage_prev(c0);
        load_scalars(c0, nq, false);
        prologue_prev(c0);
        bf16 *ws = wsS(c);
#pragma unroll
        for (int v = 0; v < UPW; v++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int n = tile_n0(v) + 4 * lg + i, pp = tile_p0(v) + li;
                float acc = 0.f;
                for (int j = 0; j < R; j++) acc += Bp[j * N + n] * Xp[j * P + pp];
                hacc[v][i] += DL[0] * acc;
            }
            *(bf16x4 *)(ws + (tile_p0(v) + li) * N + tile_n0(v) + 4 * lg) =
                bf16x4{(bf16)hacc[v][0], (bf16)hacc[v][1], (bf16)hacc[v][2], (bf16)hacc[v][3]};
        }
        stage_chunk(c0, nq, false);
        if (c + 1 < nch) prefetch(c + 1, false);
#pragma unroll
        for (int v = 0; v < UPW; v++) {
            const int n0 = tile_n0(v), p0 = tile_p0(v);
            f32x4 acc = {};
#pragma unroll
            for (int k0 = 0; k0 < QR; k0 += 32)
                acc = mfma16(op_tr(Bt, NS, k0, n0, li, lg), op_tr(XcB, PS, k0, p0, li, lg), acc);
#pragma unroll
            for (int m = 0; m < 2; m++) {   // pairs (rows 4 lg + 2m, + 1)
                const int k = (n0 + 4 * lg) / 2 + m;
                const float cs = CS[e_ * K + k], sn = SN[e_ * K + k];
                const float u0 = ES[e_] * hacc[v][2 * m] + acc[2 * m];
                const float u1 = ES[e_] * hacc[v][2 * m + 1] + acc[2 * m + 1];
                hacc[v][2 * m] = cs * u0 - sn * u1;
                hacc[v][2 * m + 1] = sn * u0 + cs * u1;
            }
        }
        __syncthreads();
    }
    }

    // ------------------------------------------------------------ reverse
    f32x4 dacc[UPW];
#pragma unroll
    for (int v = 0; v < UPW; v++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int n = tile_n0(v) + 4 * lg + i, pp = tile_p0(v) + li;
            dacc[v][i] = p.dh_out ? p.dh_out[sh * N * P + n * P + pp] : 0.f;
        }
#pragma unroll
    for (int v = 0; v < UPW; v++) held(dacc[v]);   // (else every chunk waits for memory at its first read)
    for (int e = tid; e < R * N; e += NT) dBcIn[e] = 0.f;
    for (int e = tid; e < R * P; e += NT) dXcIn[e] = 0.f;
    for (int e = tid; e < N; e += NT) BBA[e] = CBA[e] = 0.f;
    for (int e = tid; e < R * N; e += NT) BpRaw[e] = 0.f;
    for (int e = tid; e < R; e += NT) INVBP[e] = 1.f;
    float bbias[8] = {}, cbias[8] = {};   // this thread's columns of the bias gradients
    __syncthreads();
    if (nch > 0) {
        prefetch(nch - 1, true);
        prefetch_state(nch - 1);
        settle();
    }
    for (int64_t c = nch - 1; c >= 0; c--) {
        const int64_t c0 = c * Q;
        const int nq = (int)min((int64_t)Q, len - c0), e_ = nq - 1;
        refresh();
        stage_prev(c0);
        load_scalars(c0, nq, true);
        prologue_prev(c0);
        // G^ = R(-Phi_e) dH (registers, bf16 copy in Gb); H' entering the chunk from the workspace
        f32x4 gacc[UPW], hcur[UPW];
#pragma unroll
        for (int v = 0; v < UPW; v++) {
            const int n0 = tile_n0(v), p0 = tile_p0(v);
#pragma unroll
            for (int m = 0; m < 2; m++) {
                const int k = (n0 + 4 * lg) / 2 + m;
                const float cs = CS[e_ * K + k], sn = SN[e_ * K + k];
                const float g0 = dacc[v][2 * m], g1 = dacc[v][2 * m + 1];
                gacc[v][2 * m] = cs * g0 + sn * g1;
                gacc[v][2 * m + 1] = -sn * g0 + cs * g1;
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int n = n0 + 4 * lg + i, pp = p0 + li;
                hcur[v][i] = (float)pH[v][i];
                Gb[n * PS + pp] = (bf16)gacc[v][i];
                Hb[n * PS + pp] = (bf16)hcur[v][i];
            }
        }
        stage_chunk(c0, nq, true);
        if (c > 0) prefetch(c - 1, true);
        for (int e = tid; e < Q * K; e += NT) DPHI[e] = 0.f;
        for (int t = tid; t < Q; t += NT) DS[t] = DGM[t] = DDL[t] = 0.f;
        // scores S = C~ B~^T and dP = dY X^T on every QR x QR tile (zero outside the causal part):
        // A = M o S and dS' = M o dP (bf16); d(mask) = S o dP, summed per row and column. Without
        // the gate both run in one pass (the gated dy0 needs all of A first).
        auto mask_tile = [&](int tr, int tc, const f32x4 &sacc, const f32x4 &pacc, bool write_a) {
            // every table read first (indices stay below Q: no conditions), then the selects;
            // the partial sums are stored by every lane holding them (the same value)
            const int q = tc * 16 + li, u = q / R;
            const float g1 = G1[u], gm = GM[u];
            float em[4];
#pragma unroll
            for (int i = 0; i < 4; i++) em[i] = EM[((tr * 16 + 4 * lg + i) / R) * Q + u];
            float cm = 0.f, cg = 0.f, cd = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = tr * 16 + 4 * lg + i, t = r / R;
                const bool ok = u <= t && t < nq;
                const float E = ok ? em[i] : 0.f, w = (u < t) ? g1 : gm;
                if (write_a) Ab[r * QS + q] = (bf16)(E * w * sacc[i]);
                const float dm = sacc[i] * pacc[i];
                dSb[r * QS + q] = (bf16)(E * w * pacc[i]);
                RPM[r * TQ + tc] = sum16(dm * E * w);   // row r's share of this tile
                cm += dm * E * w;
                cg += dm * E;
                cd += (u < t) ? dm * E : 0.f;
            }
            CPM[q * TQ + tr] = sum_groups(cm);
            CPG[q * TQ + tr] = sum_groups(cg);
            CPD[q * TQ + tr] = sum_groups(cd);
        };
        if (!p.z) {
            #pragma unroll
            for (int it_ = 0; it_ < (TQ * TQ + NW - 1) / NW; it_++) {   // a wave's tiles, unrolled
                const int tile = wave + it_ * NW;
                if ((TQ * TQ) % NW != 0 && tile >= TQ * TQ) break;
                const int tr = tile / TQ, tc = tile % TQ;
                f32x4 sacc = {}, pacc = {};
#pragma unroll
                for (int k0 = 0; k0 < N; k0 += 32)
                    sacc = mfma16(op_nat(Ct, NS, tr * 16 + li, k0, lg), op_nat(Bt, NS, tc * 16 + li, k0, lg), sacc);
#pragma unroll
                for (int k0 = 0; k0 < P; k0 += 32)
                    pacc = mfma16(op_nat(dYb, PS, tr * 16 + li, k0, lg), op_nat(Xb, PS, tc * 16 + li, k0, lg), pacc);
                mask_tile(tr, tc, sacc, pacc, true);
            }
            __syncthreads();
        } else {
            // scores first: S (fp32, for the mask's gradient) and A
            #pragma unroll
            for (int it_ = 0; it_ < (TQ * TQ + NW - 1) / NW; it_++) {   // a wave's tiles, unrolled
                const int tile = wave + it_ * NW;
                if ((TQ * TQ) % NW != 0 && tile >= TQ * TQ) break;
                const int tr = tile / TQ, tc = tile % TQ;
                f32x4 acc = {};
#pragma unroll
                for (int k0 = 0; k0 < N; k0 += 32)
                    acc = mfma16(op_nat(Ct, NS, tr * 16 + li, k0, lg), op_nat(Bt, NS, tc * 16 + li, k0, lg), acc);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int r = tr * 16 + 4 * lg + i, q = tc * 16 + li, t = r / R, u = q / R;
                    const bool ok = u <= t && t < nq;
                    const float mw = ok ? EM[t * Q + u] * ((u < t) ? G1[u] : GM[u]) : 0.f;
                    Sf[r * SF + q] = ok ? acc[i] : 0.f;
                    Ab[r * QS + q] = (bf16)(mw * acc[i]);
                }
            }
            __syncthreads();
            // outputs before the gate, y0 = e^{S_t} C~ H' + A X + D X; dy0 = dy SiLU(z), dz
            #pragma unroll
            for (int it_ = 0; it_ < (TQ * TP + NW - 1) / NW; it_++) {   // a wave's tiles, unrolled
                const int tile = wave + it_ * NW;
                if ((TQ * TP) % NW != 0 && tile >= TQ * TP) break;
                const int tr = tile / TP, tp = tile % TP;
                f32x4 yin = {}, yia = {};
#pragma unroll
                for (int k0 = 0; k0 < N; k0 += 32)
                    yin = mfma16(op_split(Ct, NS, tr * 16 + li, k0, lg), op_tr(Hb, PS, k0, tp * 16, li, lg), yin);
#pragma unroll
                for (int k0 = 0; k0 < QR; k0 += 32)
                    yia = mfma16(op_split(Ab, QS, tr * 16 + li, k0, lg), op_tr(Xb, PS, k0, tp * 16, li, lg), yia);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int r = tr * 16 + 4 * lg + i, pp = tp * 16 + li, t = r / R, j = r % R;
                    if (t >= nq) continue;
                    const float y0 = ES[t] * yin[i] + yia[i] + Dh * (float)Xb[r * PS + pp];
                    const float d = (float)dYb[r * PS + pp];
                    const int64_t oz = tokX(c0 + t) + j * P + pp;
                    const float zv = ldt<bf16>(p.z, oz), sg = 1.f / (1.f + expf(-zv));
                    if (p.dz) stt<bf16>(p.dz, oz, d * y0 * (sg + zv * sg * (1.f - sg)));
                    dYb[r * PS + pp] = (bf16)(d * zv * sg);
                }
            }
            __syncthreads();
            // e^{S} o dy0, and D's gradient
            for (int e = tid; e < QR * P; e += NT) {
                const int r = e / P, pp = e % P, t = r / R;
                const float d = (float)dYb[r * PS + pp];
                EdYb[r * PS + pp] = (bf16)(ES[t] * d);
                dD_acc += d * (float)Xb[r * PS + pp];
            }
            __syncthreads();
            // dP with the gated dy0, and the mask's products with the stored scores
            #pragma unroll
            for (int it_ = 0; it_ < (TQ * TQ + NW - 1) / NW; it_++) {   // a wave's tiles, unrolled
                const int tile = wave + it_ * NW;
                if ((TQ * TQ) % NW != 0 && tile >= TQ * TQ) break;
                const int tr = tile / TQ, tc = tile % TQ;
                f32x4 pacc = {}, sacc;
#pragma unroll
                for (int k0 = 0; k0 < P; k0 += 32)
                    pacc = mfma16(op_nat(dYb, PS, tr * 16 + li, k0, lg), op_nat(Xb, PS, tc * 16 + li, k0, lg), pacc);
#pragma unroll
                for (int i = 0; i < 4; i++) sacc[i] = Sf[(tr * 16 + 4 * lg + i) * SF + tc * 16 + li];
                mask_tile(tr, tc, sacc, pacc, false);
            }
            __syncthreads();
        }
        // dX = A^T dy0 + c o (B~ G^) + D dy0 (+ the fold's carry into the last token); dc partials
        #pragma unroll
        for (int it_ = 0; it_ < (TQ * TP + NW - 1) / NW; it_++) {   // a wave's tiles, unrolled
            const int tile = wave + it_ * NW;
            if ((TQ * TP) % NW != 0 && tile >= TQ * TP) break;
            const int tq = tile / TP, tp = tile % TP;
            // transposed products (the dy / G^ operand first): the lane holds row q = 16 tq + li,
            // columns pp .. pp + 3, and stores them as one 8-byte piece
            f32x4 a1 = {}, a2 = {};
#pragma unroll
            for (int k0 = 0; k0 < QR; k0 += 32)
                a1 = mfma16(op_tr(dYb, PS, k0, tp * 16, li, lg), op_tr(Ab, QS, k0, tq * 16, li, lg), a1);
#pragma unroll
            for (int k0 = 0; k0 < N; k0 += 32)
                a2 = mfma16(op_tr(Gb, PS, k0, tp * 16, li, lg), op_split(Bt, NS, tq * 16 + li, k0, lg), a2);
            const int q = tq * 16 + li, pp = tp * 16 + 4 * lg, u = q / R, j = q % R;
            const bf16x4 xv = *(const bf16x4 *)(Xb + q * PS + pp), dv = *(const bf16x4 *)(dYb + q * PS + pp);
            float dc = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i++) dc += a2[i] * (float)xv[i];
            dc = sum_groups(dc);   // row q's share over the tile's 16 columns
            RPC[q * TP + tp] = dc;   // (every lane of the row's group: the same value)
            const float cuu = CU[u];
            const f32x4 cin = *(const f32x4 *)(dXcIn + j * P + pp);
            if (u < nq) {
                const f32x4 carry = (u == e_) ? cin : f32x4{};
                float dx[4];
#pragma unroll
                for (int i = 0; i < 4; i++) dx[i] = a1[i] + cuu * a2[i] + Dh * (float)dv[i] + carry[i];
                *(bf16x4 *)((bf16 *)p.dx + tokX(c0 + u) + j * P + pp) = bf16x4{(bf16)dx[0], (bf16)dx[1], (bf16)dx[2], (bf16)dx[3]};
            }
        }
        // dC~ = dS' B~ + e^{S_t} (dY H'^T); the inter part's share of dS
        #pragma unroll
        for (int it_ = 0; it_ < (TQ * TN + NW - 1) / NW; it_++) {   // a wave's tiles, unrolled
            const int tile = wave + it_ * NW;
            if ((TQ * TN) % NW != 0 && tile >= TQ * TN) break;
            const int tq = tile / TN, tn = tile % TN;
            f32x4 a1 = {}, a2 = {};
#pragma unroll
            for (int k0 = 0; k0 < QR; k0 += 32)
                a1 = mfma16(op_split(dSb, QS, tq * 16 + li, k0, lg), op_tr(Bt, NS, k0, tn * 16, li, lg), a1);
#pragma unroll
            for (int k0 = 0; k0 < P; k0 += 32)
                a2 = mfma16(op_nat(dYb, PS, tq * 16 + li, k0, lg), op_nat(Hb, PS, tn * 16 + li, k0, lg), a2);
            float es[4], cv[4];   // the epilogue's reads first (t < Q: no conditions)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = tq * 16 + 4 * lg + i;
                es[i] = ES[r / R];
                cv[i] = (float)Ct[r * NS + tn * 16 + li];
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = tq * 16 + 4 * lg + i, n = tn * 16 + li, t = r / R;
                const float inter = (t < nq) ? es[i] * a2[i] : 0.f;
                dCf[r * NF + n] = (t < nq) ? a1[i] + inter : 0.f;
                RPI[r * TN + tn] = sum16(cv[i] * inter);   // (every lane of the row: the same value)
            }
        }
        // dB~ = dS'^T C~ + c o (X G^^T)
        #pragma unroll
        for (int it_ = 0; it_ < (TQ * TN + NW - 1) / NW; it_++) {   // a wave's tiles, unrolled
            const int tile = wave + it_ * NW;
            if ((TQ * TN) % NW != 0 && tile >= TQ * TN) break;
            const int tq = tile / TN, tn = tile % TN;
            f32x4 a1 = {}, a2 = {};
#pragma unroll
            for (int k0 = 0; k0 < QR; k0 += 32)
                a1 = mfma16(op_tr(dSb, QS, k0, tq * 16, li, lg), op_tr(Ct, NS, k0, tn * 16, li, lg), a1);
#pragma unroll
            for (int k0 = 0; k0 < P; k0 += 32)
                a2 = mfma16(op_nat(Xb, PS, tq * 16 + li, k0, lg), op_nat(Gb, PS, tn * 16 + li, k0, lg), a2);
            float cu4[4];
#pragma unroll
            for (int i = 0; i < 4; i++) cu4[i] = CU[(tq * 16 + 4 * lg + i) / R];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int q = tq * 16 + 4 * lg + i, n = tn * 16 + li, u = q / R;
                dBf[q * NF + n] = (u < nq) ? a1[i] + cu4[i] * a2[i] : 0.f;
            }
        }
        // dH' = e^{S_e} G^ + C~^T (e^{S} o dY), and the rotated state Inner = e^{S_e} H' + B~^T (c o X)
        // for dPhi_e = sum_p G^^T J Inner; <G^, H'> for dS_e
        float gh_acc = 0.f;
#pragma unroll
        for (int v = 0; v < UPW; v++) {
            const int n0 = tile_n0(v), p0 = tile_p0(v);
            f32x4 a1 = {}, a2 = {};
#pragma unroll
            for (int k0 = 0; k0 < QR; k0 += 32) {
                a1 = mfma16(op_tr(Ct, NS, k0, n0, li, lg), op_tr(EdYb, PS, k0, p0, li, lg), a1);
                a2 = mfma16(op_tr(Bt, NS, k0, n0, li, lg), op_tr(XcB, PS, k0, p0, li, lg), a2);
            }
#pragma unroll
            for (int m = 0; m < 2; m++) {
                const float in0 = ES[e_] * hcur[v][2 * m] + a2[2 * m], in1 = ES[e_] * hcur[v][2 * m + 1] + a2[2 * m + 1];
                const float ph = sum16(gacc[v][2 * m + 1] * in0 - gacc[v][2 * m] * in1);
                PHE[((n0 + 4 * lg) / 2 + m) * TP + p0 / 16] = ph;   // (every lane of the row: the same value)
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                gh_acc += gacc[v][i] * hcur[v][i];
                dacc[v][i] = ES[e_] * gacc[v][i] + a1[i];
            }
        }
        // <G^, H'>: per-wave sums in RED[0, NW), added in wave order by the scalar thread below
        static_assert(NW <= 8, "per-wave partials");
        {
            const float w = wave_sum(gh_acc);
            if (lane == 0) RED[wave] = w;
        }
        __syncthreads();   // (also orders every write above before the reads below)
        if (c > 0) prefetch_state(c - 1);
        // The fold's products with dH' (in registers): dH' Xp^T and dH'^T Bp, as per-tile partial
        // sums in LDS (Gb is free: G^ is no longer read), added up below in a fixed order.
        // A wave's tiles share one row block and cover UPW consecutive column blocks, so dH' Xp^T
        // is summed over them in registers first: TP / UPW partials per row.
        constexpr int FBP = TP / UPW;
        static_assert(TP % UPW == 0, "a wave's tiles share a row block");
        float *FB = (float *)Gb, *FX = FB + R * N * FBP;   // [R][N][FBP], [R][P][TN]
        static_assert(R * N * FBP + R * P * TN <= N * PS / 2, "fold partials fit over G^");
        const bool fold_on = MISC[0] != 0.f;
        if (fold_on) {
            const int n0 = tile_n0(0), pb = tile_p0(0) / 16 / UPW;
#pragma unroll
            for (int j = 0; j < R; j++) {
                float rb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < UPW; v++) {
                    const int pp = tile_p0(v) + li;
                    const float xv = Xp[j * P + pp];
                    float bx = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        rb[i] += dacc[v][i] * xv;
                        bx += dacc[v][i] * Bp[j * N + n0 + 4 * lg + i];
                    }
                    bx = sum_groups(bx);                           // over the tile's 16 rows
                    if (lg == 0) FX[(j * P + pp) * TN + n0 / 16] = bx;
                }
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float r = sum16(rb[i]);                  // over the wave's columns
                    if (li == 0) FB[(j * N + n0 + 4 * lg + i) * FBP + pb] = r;
                }
            }
        }
        // dPhi_e, and dPhi_t from C~ and B~ (thread per (t, k))
        for (int k = tid; k < K; k += NT) {
            float a = 0.f;
            for (int tp = 0; tp < TP; tp++) a += PHE[k * TP + tp];
            DPHI[e_ * K + k] += a;
        }
        __syncthreads();
        for (int e = tid; e < nq * K; e += NT) {
            const int t = e / K, k = e % K;
            float a = 0.f;
            for (int j = 0; j < R; j++) {
                const int r = t * R + j;
                const float2 dc = *(const float2 *)(dCf + r * NF + 2 * k), db = *(const float2 *)(dBf + r * NF + 2 * k);
                const bf16x2 cc = *(const bf16x2 *)(Ct + r * NS + 2 * k), bb = *(const bf16x2 *)(Bt + r * NS + 2 * k);
                a += dc.x * (float)cc[1] - dc.y * (float)cc[0];
                a += db.x * (float)bb[1] - db.y * (float)bb[0];
            }
            DPHI[t * K + k] += a;
        }
        // per-token scalar gradients from the row / column partials (fixed order), one token per
        // thread; the state coefficient's share of dS_e is summed after the barrier below
        for (int u = tid; u < nq; u += NT) {
            float rowA = 0.f, rowB = 0.f, colS = 0.f, colG = 0.f, colD = 0.f, dc = 0.f;
            for (int j = 0; j < R; j++) {
                const int q = u * R + j;
                for (int x = 0; x < TN; x++) rowA += RPI[q * TN + x];
                for (int x = 0; x < TQ; x++) {
                    rowB += RPM[q * TQ + x];
                    colS += CPM[q * TQ + x];
                    colG += CPG[q * TQ + x];
                    colD += CPD[q * TQ + x];
                }
                for (int x = 0; x < TP; x++) dc += RPC[q * TP + x];
            }
            const float E = EM[e_ * Q + u];
            const float cu = CU[u];
            DS[u] += rowA + rowB - colS - dc * cu;
            TMPC[u] = dc * cu;
            DGM[u] += colG + dc * E;
            if (u + 1 < nq) DDL[u + 1] += colD + dc * E;
        }
        // the fold at the chunk start: d delta_0 = <dH', Bp Xp^T>, carries for the previous token
        float fold_acc = 0.f;
        if (fold_on) {   // one output per thread, from the partials
            for (int e = tid; e < R * N; e += NT) {
                float a = 0.f;
                for (int q = 0; q < FBP; q++) a += FB[e * FBP + q];
                dBcOut[e] = DL[0] * a;
                fold_acc += Bp[e] * a;
            }
            for (int e = tid; e < R * P; e += NT) {
                float a = 0.f;
                for (int q = 0; q < TN; q++) a += FX[e * TN + q];
                dXcOut[e] = DL[0] * a;
            }
        } else {
            for (int e = tid; e < R * N; e += NT) dBcOut[e] = 0.f;
            for (int e = tid; e < R * P; e += NT) dXcOut[e] = 0.f;
        }
        {
            const float w = wave_sum(fold_acc);
            if (lane == 0) RED[8 + wave] = w;
        }
        __syncthreads();
        // reverse prefix sums over the chunk's tokens (past the end every term is zero). dPhi: J
        // consecutive lanes per pair, lane j holding TPG tokens counted from the chunk's end; its
        // own suffix sums, then the totals of the lanes holding later tokens (a DPP prefix sum over
        // the J lanes) added to them.
        {
            constexpr int J = NT / K, TPG = Q / J;
            const int k = tid / J, j = tid % J;
            float v[TPG];
#pragma unroll
            for (int i = 0; i < TPG; i++) v[i] = DPHI[((J - 1 - j) * TPG + i) * K + k];
#pragma unroll
            for (int i = TPG - 2; i >= 0; i--) v[i] += v[i + 1];
            const float later = group_scan_dpp<J>(v[0], j) - v[0];
#pragma unroll
            for (int i = 0; i < TPG; i++) DPHI[((J - 1 - j) * TPG + i) * K + k] = v[i] + later;
        }
        if (wave == NW - 1) {   // the last wave: the fold's d delta_0, the state's share of dS_e,
            // then dS's reverse prefix (lane i holds token Q - 1 - i, so a prefix sum over the
            // lanes is the suffix sum over the tokens)
            float gh = 0.f, fold = 0.f;
            for (int w = 0; w < NW; w++) {
                gh += RED[w];
                fold += RED[8 + w];
            }
            if (lane == 0) DDL[0] += fold;
            const float dSe = ES[e_] * gh + wave_sum((lane < nq) ? TMPC[lane] : 0.f);
            const int t = Q - 1 - lane;
            float v = (t >= 0) ? DS[t] + ((t == e_) ? dSe : 0.f) : 0.f;
            v = wave_scan_dpp(v);
            if (t >= 0) DS[t] = v;
        }
        __syncthreads();
        settle();
        {   // dtheta = dt dPhi, 8 pairs of a token per thread (one 16-byte store), and ddt: the
            // token's K / 8 consecutive lanes add up its sum_k theta_k dPhi_k (DPP, within a row)
            constexpr int KG = K / 8;
            static_assert(KG == 4 || KG == 8, "a token's pairs on 4 or 8 lanes");
            for (int e0 = tid; e0 < (Q * KG + NT - 1) / NT * NT; e0 += NT) {
                const int t = e0 / KG, k0 = (e0 % KG) * 8;
                const bool ok = t < nq;   // the same on every lane of the token
                const int tt = ok ? t : 0;
                const f32x4 d0 = *(const f32x4 *)(DPHI + tt * K + k0), d1 = *(const f32x4 *)(DPHI + tt * K + k0 + 4);
                const bf16x8 th = *(const bf16x8 *)(TH + tt * K + k0);
                float a = 0.f;
#pragma unroll
                for (int m = 0; m < 8; m++) a += (float)th[m] * ((m < 4) ? d0[m] : d1[m - 4]);
                a += dppf<0xB1>(a);
                a += dppf<0x4E>(a);
                if constexpr (KG == 8) a += dppf<0x141>(a);
                if (ok) {
                    const float dtv = DT[t];
                    const int64_t tok = start + c0 + t;
                    float o[8];
#pragma unroll
                    for (int m = 0; m < 8; m++) o[m] = dtv * ((m < 4) ? d0[m] : d1[m - 4]);
                    if (p.p_dth) {   // head h's share of a shared angle row
                        float *dst = p.p_dth + (tok * H + h) * (int64_t)K + k0;
                        *(f32x4 *)dst = f32x4{o[0], o[1], o[2], o[3]};
                        *(f32x4 *)(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
                    } else {
                        *(bf16x8 *)((bf16 *)p.dtheta + (tok * H + h) * (int64_t)K + k0) =
                            bf16x8{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3], (bf16)o[4], (bf16)o[5], (bf16)o[6], (bf16)o[7]};
                    }
                    if (k0 == 0) {
                        const float ddt = AT[t] * DS[t] + (1.f - LM[t]) * DDL[t] + LM[t] * DGM[t] + a;
                        stt<bf16>(p.ddt, tok * H + h, ddt);
                        if (p.dlam) stt<bf16>(p.dlam, tok * H + h, DT[t] * (DGM[t] - DDL[t]));
                        if (p.A_tok) stt<bf16>(p.dA_tok, tok * H + h, DT[t] * DS[t]);
                        else dA_acc += DT[t] * DS[t];
                    }
                }
            }
        }
        // dB, dC of the chunk: back to the physical frame (+ the carry into the last token), through
        // the prologue, stored. Thread e holds row r = e / (N / 8), columns n .. n + 7 of both: the
        // rotation of its 4 pairs, the row's dot product over its N / 8 lanes (norm), one store each.
        // The bias gradients accumulate per thread (its columns are the same in every chunk) and
        // are summed over the threads at the end of the slab.
        static_assert(PF_B == 1, "one 16-byte piece of B and of C per thread");
        // (instantiated with and without the norm, so that without it no instruction reads the
        // raw rows' registers, which would wait for every memory access in flight)
        auto tail = [&](auto NORMC) {
        constexpr bool NORM = decltype(NORMC)::value;
        if (tid < QR * N / 8) {   // whole rows are active or not
            const int r = tid / (N / 8), n = (tid % (N / 8)) * 8, t = r / R, j = r % R;
            const bool live = t < nq;   // the same for every lane of the row
            bf16x8 raw[2] = {bf16x8{}, bf16x8{}};
            if (NORM && live) {
                const int64_t o = tokB(c0 + t) + j * N + n;
                raw[0] = *(const bf16x8 *)(gB + o);
                raw[1] = *(const bf16x8 *)(gC + o);
            }
            const f32x4 cs = *(const f32x4 *)(CS + t * K + n / 2), sn = *(const f32x4 *)(SN + t * K + n / 2);
#pragma unroll
            for (int isC = 0; isC < 2; isC++) {
                const float *gsrc = (isC ? dCf : dBf) + r * NF + n;
                const f32x4 g0 = *(const f32x4 *)gsrc, g1 = *(const f32x4 *)(gsrc + 4);
                float v[8];
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    const float d0 = (m < 2) ? g0[2 * m] : g1[2 * m - 4], d1 = (m < 2) ? g0[2 * m + 1] : g1[2 * m - 3];
                    v[2 * m] = cs[m] * d0 - sn[m] * d1;
                    v[2 * m + 1] = sn[m] * d0 + cs[m] * d1;
                }
                if (!isC && t == e_) {   // the carry; the rows of the last token then pass it on
#pragma unroll
                    for (int m = 0; m < 8; m++) {
                        v[m] += dBcIn[j * N + n + m];
                        dBcIn[j * N + n + m] = dBcOut[j * N + n + m];
                    }
                }
                float dot = 0.f;
                if constexpr (NORM) {
#pragma unroll
                    for (int m = 0; m < 8; m++) dot += v[m] * (float)raw[isC][m];
                    dot = row_sum(dot);
                }
                if (!live) continue;
#pragma unroll
                for (int m = 0; m < 8; m++) {
                    if (isC) cbias[m] += v[m];
                    else bbias[m] += v[m];
                }
                float o[8];
                if constexpr (NORM) {
                    const float inv = (isC ? INVC : INVB)[r];
                    const float k3 = dot * inv * inv * inv / (float)N;
#pragma unroll
                    for (int m = 0; m < 8; m++) o[m] = v[m] * inv - k3 * (float)raw[isC][m];
                } else {
#pragma unroll
                    for (int m = 0; m < 8; m++) o[m] = v[m];
                }
                float *part = isC ? p.p_dC : p.p_dB;
                if (part) {
                    float *dst = part + ((start + c0 + t) * H + h) * (int64_t)R * N + j * N + n;
                    *(f32x4 *)dst = f32x4{o[0], o[1], o[2], o[3]};
                    *(f32x4 *)(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
                } else {
                    *(bf16x8 *)((bf16 *)(isC ? p.dC : p.dB) + tokB(c0 + t) + j * N + n) =
                        bf16x8{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3], (bf16)o[4], (bf16)o[5], (bf16)o[6], (bf16)o[7]};
                }
            }
        }
        };
        if (p.norm) tail(std::true_type{});
        else tail(std::false_type{});
        for (int e = tid; e < R * P; e += NT) dXcIn[e] = dXcOut[e];
        __syncthreads();
    }

    // ------------------------------------------------------------ slab results
    if (p.dh_in) {
#pragma unroll
        for (int v = 0; v < UPW; v++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                p.dh_in[sh * N * P + (tile_n0(v) + 4 * lg + i) * P + tile_p0(v) + li] = dacc[v][i];
    }
    if (has_prev) {
        for (int j = tid; j < R; j += NT) {
            const float *gout = dBcIn + j * N;
            const float inv = INVBP[j];
            const int64_t o = ((int64_t)s * G + g) * R * N + j * N;
            float dot = 0.f;
            if (p.norm)
                for (int n = 0; n < N; n++) dot += gout[n] * BpRaw[j * N + n];
            const float k3 = p.norm ? dot * inv * inv * inv / (float)N : 0.f;
            for (int n = 0; n < N; n++) {
                const float v = p.norm ? gout[n] * inv - k3 * BpRaw[j * N + n] : gout[n];
                if (p.p_dBprev) p.p_dBprev[sh * (int64_t)R * N + j * N + n] = v;
                else if (p.dBprev) stt<bf16>(p.dBprev, o + n, v);
            }
        }
        for (int n = tid; n < N; n += NT)
            for (int j = 0; j < R; j++) BBA[n] += dBcIn[j * N + n];
        for (int e = tid; e < R * P; e += NT)
            if (p.dxprev) stt<bf16>(p.dxprev, sh * R * P + e, dXcIn[e]);
    }
    if (p.Bb || p.Cb) {   // the per-thread bias partials, summed over the threads in thread order
        float *scr = dBf;  // [QR * N / 8][8] (dB~'s staging is free after the last chunk)
        for (int isC = 0; isC < 2; isC++) {
            if (tid < QR * N / 8)
#pragma unroll
                for (int m = 0; m < 8; m++) scr[tid * 8 + m] = isC ? cbias[m] : bbias[m];
            __syncthreads();
            for (int n = tid; n < N; n += NT) {
                float a = 0.f;
                for (int q = n / 8; q < QR * N / 8; q += N / 8) a += scr[q * 8 + n % 8];
                (isC ? CBA : BBA)[n] += a;
            }
            __syncthreads();
        }
    }
    const float dA_sum = block_sum(dA_acc, RED);
    const float dD_sum = block_sum(dD_acc, RED);
    if (tid == 0) {
        p.p_dA[sh] = dA_sum;
        p.p_dD[sh] = dD_sum;
    }
    for (int n = tid; n < N; n += NT) {
        p.p_dBb[sh * N + n] = BBA[n];
        p.p_dCb[sh * N + n] = CBA[n];
    }
#undef p
}

// (N, P, R) -> chunk length and waves of the MFMA backward
#define M3_BWD_MFMA_SHAPES(X) \
    X(128, 64, 1, 32, 8)      \
    X(64, 64, 1, 32, 8)       \
    X(64, 64, 4, 16, 8)       \
    X(128, 64, 2, 16, 8)      \
    X(128, 64, 4, 8, 8)       \
    X(64, 64, 2, 32, 8)

int scan_bwd_mfma_chunk(int N, int P, int R) {
#define X(n, pp, r, q, w) if (N == n && P == pp && R == r) return q;
    M3_BWD_MFMA_SHAPES(X)
#undef X
    return 0;
}

template <class CF>
static mamba3_status launch_bwd_mfma_cfg(const BwdParams &p, int64_t nblk, hipStream_t st) {
    if (hipFuncSetAttribute((const void *)k_scan_bwd_mfma<CF>, hipFuncAttributeMaxDynamicSharedMemorySize, CF::LDS) !=
        hipSuccess)
        return MAMBA3_EHIP;
    if (nblk > 0) hipLaunchKernelGGL(k_scan_bwd_mfma<CF>, dim3((unsigned)nblk), dim3(CF::NT), CF::LDS, st, p);
    return MAMBA3_OK;
}

static mamba3_status launch_bwd_mfma(const BwdParams &p, int64_t nblk, hipStream_t st) {
#define X(n, pp, r, q, w) \
    if (p.N == n && p.P == pp && p.R == r) return launch_bwd_mfma_cfg<BCfg<n, pp, r, q, w>>(p, nblk, st);
    M3_BWD_MFMA_SHAPES(X)
#undef X
    return MAMBA3_EUNSUPPORTED;
}

// Fixed-order sums of the per-slab partials: dA, dD, the bias gradients over
// sequences; with G < H, dB, dC, dBprev over the heads of each group; with
// Gth < H, dtheta over the heads sharing an angle row.
template <typename T>
__global__ void k_bwd_reduce(BwdParams p, int64_t T_tok, int32_t S) {
    const int H = p.H, G = p.G, N = p.N, R = p.R;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < H) {
        float a = 0.f, d = 0.f;
        for (int s = 0; s < S; s++) {
            a += p.p_dA[(int64_t)s * H + i];
            d += p.p_dD[(int64_t)s * H + i];
        }
        if (p.dA) p.dA[i] = a;
        if (p.dD) p.dD[i] = d;
    }
    if (i < (int64_t)H * N) {
        const int h = (int)(i / N), n = (int)(i % N);
        float a = 0.f, b = 0.f;
        for (int s = 0; s < S; s++) {
            a += p.p_dBb[((int64_t)s * H + h) * N + n];
            b += p.p_dCb[((int64_t)s * H + h) * N + n];
        }
        if (p.dB_bias) p.dB_bias[i] = a;
        if (p.dC_bias) p.dC_bias[i] = b;
    }
    if (p.p_dB) {
        const int HG = H / G;
        const int64_t RN = (int64_t)R * N;
        if (i < T_tok * G * RN) {
            const int64_t t = i / (G * RN), gg = (i / RN) % G, jn = i % RN;
            float a = 0.f, b = 0.f;
            for (int hh = 0; hh < HG; hh++) {
                const int64_t o = (t * H + gg * HG + hh) * RN + jn;
                a += p.p_dB[o];
                b += p.p_dC[o];
            }
            ((T *)p.dB)[i] = from_f<T>(a);
            ((T *)p.dC)[i] = from_f<T>(b);
        }
        if (p.p_dBprev && i < (int64_t)S * G * RN) {
            const int64_t s = i / (G * RN), gg = (i / RN) % G, jn = i % RN;
            float a = 0.f;
            for (int hh = 0; hh < HG; hh++) a += p.p_dBprev[((s * H) + gg * HG + hh) * RN + jn];
            if (p.dBprev) ((T *)p.dBprev)[i] = from_f<T>(a);
        }
    }
    if (p.p_dth) {
        const int HT = H / p.Gth, K = N / 2;
        if (i < T_tok * p.Gth * K) {
            const int64_t t = i / ((int64_t)p.Gth * K), gq = (i / K) % p.Gth, k = i % K;
            float a = 0.f;
            for (int hh = 0; hh < HT; hh++) a += p.p_dth[(t * H + gq * HT + hh) * K + k];
            ((T *)p.dtheta)[i] = from_f<T>(a);
        }
    }
}

// chunk length of the backward: the largest of 64, 32, ..., 1 whose LDS fits
int scan_bwd_chunk(int N, int P, int R) {
    for (int q = 64; q >= 1; q /= 2)
        if (scan_bwd_lds_bytes(N, P, R, q) <= 160 * 1024) return q;
    return 0;
}

// workspace: states, then the partial sums (each region 256-byte aligned)
struct BwdWs {
    size_t state, pA, pD, pBb, pCb, pB, pC, pBprev, pth, total;
    int64_t chunks;
};
// mfma: the MFMA kernel's chunk states are bf16 (the VALU kernel's fp32)
static BwdWs bwd_ws(const mamba3_scan_bwd_args *b, int Q, bool mfma) {
    const mamba3_scan_args *a = &b->fwd;
    const int64_t S = a->cu_seqlens ? a->nseq : a->batch, T = (int64_t)a->batch * a->seqlen;
    const int64_t H = a->nheads, N = a->dstate, P = a->headdim, R = a->rank;
    const int64_t chunks = a->cu_seqlens ? (T + Q - 1) / Q + S : S * ((a->seqlen + Q - 1) / Q);
    const bool grouped = a->ngroups < a->nheads;
    auto al = [](size_t v) { return (v + 255) / 256 * 256; };
    BwdWs w;
    size_t o = 0;
    w.chunks = chunks;
    w.state = o; o += al((size_t)chunks * H * N * P * (mfma ? 2 : 4));
    w.pA = o; o += al((size_t)S * H * 4);
    w.pD = o; o += al((size_t)S * H * 4);
    w.pBb = o; o += al((size_t)S * H * N * 4);
    w.pCb = o; o += al((size_t)S * H * N * 4);
    w.pB = o; o += grouped ? al((size_t)T * H * R * N * 4) : 0;
    w.pC = o; o += grouped ? al((size_t)T * H * R * N * 4) : 0;
    w.pBprev = o; o += (grouped && a->Bprev) ? al((size_t)S * H * R * N * 4) : 0;
    const bool th_shared = a->theta_groups && a->theta_groups < a->nheads;
    w.pth = o; o += th_shared ? al((size_t)T * H * (N / 2) * 4) : 0;
    w.total = o;
    return w;
}

// chunk length of the path that runs: the MFMA kernel's for bf16 inputs of its shapes, else the
// VALU kernel's
static int bwd_path_chunk(const mamba3_scan_args *a, bool *mfma) {
    const int qm = a->dtype == MAMBA3_BF16 ? scan_bwd_mfma_chunk(a->dstate, a->headdim, a->rank) : 0;
    if (mfma) *mfma = qm > 0;
    return qm > 0 ? qm : scan_bwd_chunk(a->dstate, a->headdim, a->rank);
}

size_t scan_bwd_workspace_bytes(const mamba3_scan_bwd_args *b) {
    bool mfma = false;
    const int Q = bwd_path_chunk(&b->fwd, &mfma);
    return Q ? bwd_ws(b, Q, mfma).total : 0;
}

template <typename T>
static mamba3_status launch_bwd_t(const mamba3_scan_bwd_args *b, hipStream_t st) {
    const mamba3_scan_args *a = &b->fwd;
    bool mfma = false;
    const int Q = bwd_path_chunk(a, &mfma);
    const BwdWs w = bwd_ws(b, Q, mfma);
    char *ws = (char *)b->workspace;
    BwdParams p;
    p.fwd_states = 0;
    p.x = a->x; p.dt = a->dt; p.lam = a->lam; p.theta = a->theta; p.B = a->B; p.C = a->C;
    p.Bprev = a->Bprev; p.xprev = a->xprev; p.z = a->z; p.dy = b->dy;
    p.A = a->A; p.D = a->D; p.h_in = a->h_in; p.dh_out = b->dh_out; p.Bb = a->B_bias; p.Cb = a->C_bias;
    p.dx = b->dx; p.ddt = b->ddt; p.dlam = b->dlam; p.dtheta = b->dtheta; p.dB = b->dB; p.dC = b->dC;
    p.dBprev = b->dBprev; p.dxprev = b->dxprev; p.dz = b->dz; p.dh_in = b->dh_in;
    p.dA = b->dA; p.dD = b->dD; p.dB_bias = b->dB_bias; p.dC_bias = b->dC_bias;
    p.ws_state = (float *)(ws + w.state);
    p.ws_hs = (bf16 *)(ws + w.state);
    p.p_dA = (float *)(ws + w.pA); p.p_dD = (float *)(ws + w.pD);
    p.p_dBb = (float *)(ws + w.pBb); p.p_dCb = (float *)(ws + w.pCb);
    const bool grouped = a->ngroups < a->nheads;
    p.p_dB = grouped ? (float *)(ws + w.pB) : nullptr;
    p.p_dC = grouped ? (float *)(ws + w.pC) : nullptr;
    p.p_dBprev = (grouped && a->Bprev) ? (float *)(ws + w.pBprev) : nullptr;
    p.cu = a->cu_seqlens;
    p.ws_chunks = w.chunks;
    p.nseq = a->cu_seqlens ? a->nseq : a->batch;
    p.seqlen = a->seqlen; p.H = a->nheads; p.G = a->ngroups; p.P = a->headdim; p.N = a->dstate; p.R = a->rank;
    p.Q = Q; p.norm = a->bc_norm; p.eps = a->bc_eps;
    p.A_tok = a->A_tok; p.dA_tok = b->dA_tok; p.lam_fixed = a->lam_fixed;
    p.Gth = a->theta_groups ? a->theta_groups : a->nheads;
    p.p_dth = p.Gth < p.H ? (float *)(ws + w.pth) : nullptr;
    const int64_t S = p.nseq, T_tok = (int64_t)a->batch * a->seqlen;
    const int64_t nblk = S * p.H;
    if constexpr (std::is_same<T, bf16>::value) {
        if (mfma) {
            // padded batches at a chunk the forward kernel covers: the chunk states come from a
            // state-only forward scan, and the backward kernel skips its own forward walk
            p.fwd_states = 0;
            if (!a->cu_seqlens && T_tok > 0 && scan_bf16_states_supported(p.N, p.P, p.R, Q)) {
                mamba3_scan_args f = *a;
                f.y = nullptr;
                f.h_out = nullptr;
                f.z = nullptr;
                f.C_bias = nullptr;
                f.D = nullptr;
                f.chunk = Q;
                f.workspace = nullptr;
                f.workspace_bytes = 0;
                const mamba3_status fs = launch_scan_bf16_states(&f, p.ws_hs, nullptr, st);
                if (fs != MAMBA3_OK) return fs;
                p.fwd_states = 1;
            }
            const mamba3_status ms = launch_bwd_mfma(p, nblk, st);
            if (ms != MAMBA3_OK) return ms;
        }
    }
    if (!mfma) {
        const size_t lds = scan_bwd_lds_bytes(p.N, p.P, p.R, Q);
        if (hipFuncSetAttribute((const void *)k_scan_bwd<T>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
            hipSuccess)
            return MAMBA3_EHIP;
        if (nblk > 0) hipLaunchKernelGGL(k_scan_bwd<T>, dim3((unsigned)nblk), dim3(kBwdThreads), lds, st, p);
    }
    int64_t nred = (int64_t)p.H * p.N;
    if (grouped) nred = std::max(nred, std::max(T_tok * p.G * p.R * p.N, S * p.G * p.R * p.N));
    if (p.p_dth) nred = std::max(nred, T_tok * p.Gth * (p.N / 2));
    if (nred > 0) hipLaunchKernelGGL(k_bwd_reduce<T>, dim3((unsigned)((nred + 255) / 256)), dim3(256), 0, st, p, T_tok, (int32_t)S);
    return hipGetLastError() == hipSuccess ? MAMBA3_OK : MAMBA3_EHIP;
}

mamba3_status launch_scan_bwd(const mamba3_scan_bwd_args *b, hipStream_t st) {
    return b->fwd.dtype == MAMBA3_BF16 ? launch_bwd_t<bf16>(b, st) : launch_bwd_t<float>(b, st);
}

}  // namespace m3
