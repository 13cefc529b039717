// fp32 chunked scan (VALU). One workgroup per (sequence, head) walks the
// sequence chunk by chunk, keeping the fp32 state in LDS.
//
// Chunked form used here (derived from the three-term update of Proposition 4,
// "Complex-Valued State Space Models", and the SSD matrix form of section
// "Parallel representation under SSD"): inside a chunk with first token c0,
// S_t = sum_{c0<=k<=t} dt_k A (log decay), Phi_t[k] = sum_{c0<=j<=t} dt_j theta_j[k]
// (cumulative angle, restarted at every chunk), B~_s = R(-Phi_s) B_s,
// C~_t = R(-Phi_t) C_t. With the carried state H' (physical frame) entering
// the chunk,
//   y_t = e^{S_t} C~_t^T H' + sum_{s<=t} e^{S_t - S_s} w(t,s) (C~_t . B~_s) X_s + D X_t
//   w(t,s) = gamma_s + delta_{s+1} [s < t]
// and the state leaving the chunk (last token e) is
//   H'_next = R(Phi_e) ( e^{S_e} H' + sum_s e^{S_e - S_s} (gamma_s + delta_{s+1}) B~_s X_s^T ),
// where delta_{e+1} is the next chunk's first token's (0 at the sequence end),
// which folds that token's previous-input term into the carried state.
// At the sequence start H' = h_in + delta_0 Bprev xprev^T.
//
// Optional block prologue and epilogue (section "Architectural Integration"):
// each B and C column is scaled to unit RMS and gets its head's bias before
// the rotation, and y is multiplied by SiLU(z) after the D term.
//
// Variants: a per-token decay rate A_t replaces the head's A, and without a
// lam array every token uses the fixed trapezoid weight.
#include "m3_common.h"

namespace m3 {

struct ValuParams {
    const float *x, *dt, *lam, *theta, *B, *C, *Bprev, *xprev;
    const float *A, *D, *h_in;
    float *y, *h_out;
    const int32_t *cu;
    const float *Bb, *Cb, *z;   // prologue biases [H, N] and output gate, or NULL
    const float *A_tok;         // per-token decay rate [T, H], or NULL (A per head)
    int32_t nseq, seqlen, H, G, P, N, R, Q;
    int32_t norm;               // 1: B and C columns scaled to unit RMS
    float eps;
    float lam_fixed;            // trapezoid weight of every token when lam is NULL
    int32_t Gth;                // angle rows per token (divides H): head h reads row h / (H / Gth)
};

// Block prologue on `nrows` LDS rows of N values: scale each row to unit RMS
// (norm) and add the head's bias row (bias may be NULL). One thread per row.
__device__ void bc_prologue_rows(float *rows, int nrows, int N, const float *bias, int norm, float eps, int tid,
                                 int nt) {
    for (int r = tid; r < nrows; r += nt) {
        float *v = rows + (int64_t)r * N;
        float inv = 1.f;
        if (norm) {
            float ss = 0.f;
            for (int n = 0; n < N; n++) ss += v[n] * v[n];
            inv = 1.f / sqrtf(ss / (float)N + eps);
        }
        for (int n = 0; n < N; n++) v[n] = v[n] * inv + (bias ? bias[n] : 0.f);
    }
}

size_t scan_f32_lds_bytes(int N, int P, int R, int Q) {
    size_t QR = (size_t)Q * R, K = N / 2;
    size_t floats = QR * N * 2 + QR * P + QR * QR + (size_t)N * P + (size_t)Q * (8 + K);
    return floats * sizeof(float);
}

__global__ __launch_bounds__(256) void k_scan_f32(ValuParams p) {
    extern __shared__ float smem[];
    const int H = p.H, G = p.G, P = p.P, N = p.N, R = p.R, Q = p.Q, K = N / 2, QR = Q * R;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int s = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / G);

    float *Bt = smem;              // [QR][N]
    float *Ct = Bt + QR * N;       // [QR][N]
    float *Xs = Ct + QR * N;       // [QR][P]
    float *M = Xs + QR * P;        // [QR][QR]
    float *Hs = M + QR * QR;       // [N][P]
    float *S = Hs + N * P;         // [Q] log decay prefix
    float *gm = S + Q;             // [Q] gamma
    float *dl = gm + Q;            // [Q] delta
    float *g1 = dl + Q;            // [Q] gamma_s + delta_{s+1}
    float *dts = g1 + Q;           // [Q] dt
    float *wU = dts + Q;           // [Q] chunk-state weights
    float *misc = wU + Q;          // [Q] (misc[0] = delta of the token after the chunk)
    float *phi = misc + Q;         // [Q][K]
    float *dtA = phi + Q * K;      // [Q] dt_t A_t

    int64_t start, len;
    if (p.cu) {
        int64_t a = min(max((int64_t)p.cu[s], (int64_t)0), (int64_t)p.seqlen);
        int64_t b = min(max((int64_t)p.cu[s + 1], a), (int64_t)p.seqlen);
        start = a;
        len = b - a;
    } else {
        start = (int64_t)s * p.seqlen;
        len = p.seqlen;
    }
    const float Ah = p.A ? p.A[h] : 0.f;
    const float Dh = p.D ? p.D[h] : 0.f;
    const bool pro = p.norm || p.Bb || p.Cb;
    const float *Bbh = p.Bb ? p.Bb + (int64_t)h * N : nullptr;
    const float *Cbh = p.Cb ? p.Cb + (int64_t)h * N : nullptr;
    const int64_t st_off = ((int64_t)s * H + h) * N * P;

    for (int e = tid; e < N * P; e += nt) Hs[e] = p.h_in ? p.h_in[st_off + e] : 0.f;
    __syncthreads();

    for (int64_t c0 = 0; c0 < len; c0 += Q) {
        const int nq = (int)min((int64_t)Q, len - c0);
        // per-token scalars
        for (int t = tid; t < Q; t += nt) {
            float dtv = 0.f, lv = 0.f, av = 0.f;
            if (t < nq) {
                int64_t tg = start + c0 + t;
                dtv = p.dt[tg * H + h];
                lv = p.lam ? p.lam[tg * H + h] : p.lam_fixed;
                av = p.A_tok ? p.A_tok[tg * H + h] : Ah;
            }
            dtA[t] = dtv * av;
            dts[t] = dtv;
            gm[t] = lv * dtv;
            dl[t] = (1.f - lv) * dtv;
        }
        if (tid == 0) {
            float dnext = 0.f;
            if (c0 + nq < len) {
                int64_t tg = start + c0 + nq;
                float dtv = p.dt[tg * H + h], lv = p.lam ? p.lam[tg * H + h] : p.lam_fixed;
                dnext = (1.f - lv) * dtv;
            }
            misc[0] = dnext;
        }
        __syncthreads();
        if (tid == 0) {
            float acc = 0.f;
            for (int t = 0; t < Q; t++) {
                if (t < nq) acc += dtA[t];
                S[t] = acc;
                float dn = (t + 1 < nq) ? dl[t + 1] : (t + 1 == nq ? misc[0] : 0.f);
                g1[t] = gm[t] + dn;
            }
            for (int t = 0; t < Q; t++) wU[t] = (t < nq) ? expf(S[nq - 1] - S[t]) * g1[t] : 0.f;
        }
        for (int k = tid; k < K; k += nt) {
            float acc = 0.f;
            for (int t = 0; t < Q; t++) {
                if (t < nq) acc += dts[t] * p.theta[((start + c0 + t) * p.Gth + h / (H / p.Gth)) * K + k];
                phi[t * K + k] = acc;
            }
        }
        // previous-token fold at the sequence start: H' += delta_0 Bprev xprev^T (Bprev's
        // columns staged in Bt, through the prologue)
        if (c0 == 0 && p.Bprev) {
            const int64_t ob = ((int64_t)s * G + g) * N * R, ox = ((int64_t)s * H + h) * P * R;
            for (int e = tid; e < R * N; e += nt) Bt[e] = p.Bprev[ob + e];
            __syncthreads();
            if (pro) {
                bc_prologue_rows(Bt, R, N, Bbh, p.norm, p.eps, tid, nt);
                __syncthreads();
            }
            const float d0 = dl[0];
            for (int e = tid; e < N * P; e += nt) {
                int n = e / P, pp = e % P;
                float acc = 0.f;
                for (int j = 0; j < R; j++) acc += Bt[j * N + n] * p.xprev[ox + j * P + pp];
                Hs[e] += d0 * acc;
            }
        }
        __syncthreads();
        // B and C columns of the chunk (zero past the sequence end), through the prologue
        for (int e = tid; e < QR * N; e += nt) {
            int r = e / N, n = e % N, t = r / R, j = r % R;
            float bv = 0.f, cv = 0.f;
            if (t < nq) {
                int64_t ob = ((start + c0 + t) * G + g) * N * R + j * N + n;
                bv = p.B[ob];
                cv = p.C[ob];
            }
            Bt[e] = bv;
            Ct[e] = cv;
        }
        if (pro) {
            __syncthreads();
            bc_prologue_rows(Bt, nq * R, N, Bbh, p.norm, p.eps, tid, nt);
            bc_prologue_rows(Ct, nq * R, N, Cbh, p.norm, p.eps, tid, nt);
        }
        __syncthreads();
        // rotated B~, C~ in place
        for (int e = tid; e < nq * K * R; e += nt) {
            int t = e / (K * R), k = (e / R) % K, j = e % R;
            float cs, sn;
            sincosf(phi[t * K + k], &sn, &cs);
            int r = t * R + j;
            const float b0 = Bt[r * N + 2 * k], b1 = Bt[r * N + 2 * k + 1];
            const float q0 = Ct[r * N + 2 * k], q1 = Ct[r * N + 2 * k + 1];
            Bt[r * N + 2 * k] = cs * b0 + sn * b1;
            Bt[r * N + 2 * k + 1] = -sn * b0 + cs * b1;
            Ct[r * N + 2 * k] = cs * q0 + sn * q1;
            Ct[r * N + 2 * k + 1] = -sn * q0 + cs * q1;
        }
        for (int e = tid; e < Q * P * R; e += nt) {
            int t = e / (P * R), pp = (e / R) % P, j = e % R;
            float v = (t < nq) ? p.x[((start + c0 + t) * H + h) * P * R + j * P + pp] : 0.f;
            Xs[(t * R + j) * P + pp] = v;
        }
        __syncthreads();
        // masked score matrix M[(t,i)][(s,j)]
        for (int e = tid; p.y && e < QR * QR; e += nt) {
            int r = e / QR, q = e % QR, tt = r / R, ss = q / R;
            float v = 0.f;
            if (ss <= tt && tt < nq) {
                float gdot = 0.f;
                for (int n = 0; n < N; n++) gdot += Ct[r * N + n] * Bt[q * N + n];
                float w = (ss < tt) ? g1[ss] : gm[ss];
                v = expf(S[tt] - S[ss]) * w * gdot;
            }
            M[e] = v;
        }
        __syncthreads();
        // outputs (none in a state-only scan: y NULL)
        for (int e = tid; p.y && e < QR * P; e += nt) {
            int r = e / P, pp = e % P, tt = r / R, i = r % R;
            if (tt >= nq) continue;
            float inter = 0.f;
            for (int n = 0; n < N; n++) inter += Ct[r * N + n] * Hs[n * P + pp];
            float acc = expf(S[tt]) * inter;
            for (int q = 0; q < (tt + 1) * R; q++) acc += M[r * QR + q] * Xs[q * P + pp];
            acc += Dh * Xs[r * P + pp];
            const int64_t oy = ((start + c0 + tt) * H + h) * P * R + i * P + pp;
            if (p.z) {
                const float v = p.z[oy];
                acc *= v / (1.f + expf(-v));
            }
            p.y[oy] = acc;
        }
        __syncthreads();
        // carried state
        {
            const float eS = expf(S[nq - 1]);
            for (int e = tid; e < K * P; e += nt) {
                int k = e / P, pp = e % P;
                float u0 = eS * Hs[(2 * k) * P + pp], u1 = eS * Hs[(2 * k + 1) * P + pp];
                for (int q = 0; q < nq * R; q++) {
                    float w = wU[q / R] * Xs[q * P + pp];
                    u0 += w * Bt[q * N + 2 * k];
                    u1 += w * Bt[q * N + 2 * k + 1];
                }
                float sn, cs;
                sincosf(phi[(nq - 1) * K + k], &sn, &cs);
                Hs[(2 * k) * P + pp] = cs * u0 - sn * u1;
                Hs[(2 * k + 1) * P + pp] = sn * u0 + cs * u1;
            }
        }
        __syncthreads();
    }
    if (p.h_out)
        for (int e = tid; e < N * P; e += nt) p.h_out[st_off + e] = Hs[e];
}

mamba3_status launch_scan_f32(const mamba3_scan_args *a, hipStream_t st) {
    ValuParams p;
    p.x = (const float *)a->x; p.dt = (const float *)a->dt; p.lam = (const float *)a->lam;
    p.theta = (const float *)a->theta; p.B = (const float *)a->B; p.C = (const float *)a->C;
    p.Bprev = (const float *)a->Bprev; p.xprev = (const float *)a->xprev;
    p.A = a->A; p.D = a->D; p.h_in = a->h_in; p.y = (float *)a->y; p.h_out = a->h_out;
    p.cu = a->cu_seqlens;
    p.nseq = a->cu_seqlens ? a->nseq : a->batch;
    p.seqlen = a->seqlen; p.H = a->nheads; p.G = a->ngroups; p.P = a->headdim; p.N = a->dstate;
    p.R = a->rank; p.Q = a->chunk;
    p.Bb = a->B_bias; p.Cb = a->C_bias; p.z = (const float *)a->z;
    p.norm = a->bc_norm; p.eps = a->bc_eps;
    p.A_tok = (const float *)a->A_tok; p.lam_fixed = a->lam_fixed;
    p.Gth = a->theta_groups ? a->theta_groups : a->nheads;
    size_t lds = scan_f32_lds_bytes(p.N, p.P, p.R, p.Q);
    if (hipFuncSetAttribute((const void *)k_scan_f32, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return MAMBA3_EHIP;
    int64_t nblk = (int64_t)p.nseq * p.H;
    if (nblk == 0) return MAMBA3_OK;
    hipLaunchKernelGGL(k_scan_f32, dim3((unsigned)nblk), dim3(256), lds, st, p);
    return hipGetLastError() == hipSuccess ? MAMBA3_OK : MAMBA3_EHIP;
}

}  // namespace m3
