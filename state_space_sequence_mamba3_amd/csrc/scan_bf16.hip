// bf16 chunked scan on gfx950 MFMA (v_mfma_f32_32x32x16_bf16), fp32 state.
//
// One workgroup owns one (sequence, head) slab and walks it chunk by chunk;
// the fp32 state lives in registers across chunks, so every input byte is read
// from HBM once and every output byte written once. Chunked form (derived from
// the three-term update of Proposition 4, "Complex-Valued State Space Models",
// and the matrix form Y = (L o C B^T) X of "Parallel representation under
// SSD"), with chunk-local log decay S_t and cumulative angles Phi_t restarted
// at each chunk, B~_s = R(-Phi_s) B_s, C~_t = R(-Phi_t) C_t (the RoPE trick of
// Proposition 3 inside a chunk), and H' the carried state:
//   y_t = e^{S_t} C~_t^T H' + sum_{s<=t} e^{S_t-S_s} (gamma_s + delta_{s+1}[s<t]) (C~_t.B~_s) X_s + D X_t
//   H'  <- R(Phi_e) ( e^{S_e} H' + sum_s e^{S_e-S_s} (gamma_s + delta_{s+1}) B~_s X_s^T )
// (delta_{e+1} is the next chunk's first token's, 0 at the sequence end: it
// folds that token's previous-input term into the carried state).
//
// Rank-expanded rows: row (tau, j) = tau*R + j of a chunk, so the chunk is a
// (Q*R) x (Q*R) problem cut into 32-row blocks ("blocks", TOKB = 32/R tokens).
// Work per chunk:
//   * every wave owns "tasks" = (t-block, column group of P) and holds the
//     rotated C~ rows of its t-blocks in registers (MFMA operands) and the
//     output accumulators Y in registers;
//   * the chunk is swept over s-blocks: each s-block's rotated B~, weighted
//     B~^T and X^T are staged through LDS (double buffered, global loads
//     prefetched one block ahead), then each wave computes its lower-triangle
//     score tiles G^T = B~ C~^T (MFMA, K = N), applies the decay/trapezoid mask
//     in registers, converts to bf16 and feeds them straight into the output
//     MFMA (Y += M X) with the K index permuted to match the accumulator lane
//     layout - the score tile never touches LDS;
//   * the state tiles (N x P, fp32, distributed over the waves) accumulate the
//     chunk's rank-R update B~^T X on MFMA and are rotated by Phi_e at the end.
// The state enters the next chunk's inter-chunk term e^{S_t} C~_t^T H' as a
// bf16 copy in LDS.
#include "m3_common.h"

namespace m3 {

namespace {

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Wait for this wave's outstanding LDS operations (wave-private staging).
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xc07f); }

__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

struct BfParams {
    const bf16 *x, *dt, *lam, *theta, *B, *C, *Bprev, *xprev;
    const float *A, *D, *h_in;
    bf16 *y;
    float *h_out;
    const int32_t *cu;
    int32_t seqlen, H, G;
};

template <int N_, int P_, int R_, int Q_, int NW_>
struct Cfg {
    static constexpr int N = N_, P = P_, R = R_, Q = Q_, NW = NW_;
    static constexpr int K = N / 2, QR = Q * R, NB = QR / 32, TOKB = 32 / R;
    static constexpr int NTHR = NW * 64;
    static constexpr int PG = (NB >= NW) ? 1 : NW / NB;   // column groups per t-block
    static constexpr int PT = P / PG, NPT = PT / 32;     // columns / 32-col tiles per task
    static constexpr int NTASK = NB * PG, TPW = NTASK / NW;
    static constexpr int NUT = (N / 32) * (P / 32), UPW = NUT / NW;
    static constexpr int NKK = N / 16;                   // K-steps over N
    static constexpr int NS = N + 8;                     // padded bf16 row stride of [*][N] tiles
    static constexpr int RS = 40;                        // padded bf16 row stride of [*][32] tiles
    static_assert(N % 32 == 0 && P % 32 == 0 && 32 % R == 0 && QR % 32 == 0, "shape");
    static_assert(NTASK % NW == 0 && NUT % NW == 0 && P % PG == 0 && PT % 32 == 0, "work split");
    static_assert(TPW == 1 || TPW % 2 == 0, "task pairing");
    static_assert(K % 8 == 0 && Q % NW == 0 && Q <= 128 && Q < NTHR, "prologue");
    // LDS layout (bytes)
    static constexpr int OFF_PHI = 0;                                  // float [Q][K]
    static constexpr int OFF_S2 = OFF_PHI + Q * K * 4;                 // float [Q] log2 decay prefix
    static constexpr int OFF_A2 = OFF_S2 + Q * 4;                      // float [Q] per-token log2 decay
    static constexpr int OFF_GM = OFF_A2 + Q * 4;                      // float [Q] gamma
    static constexpr int OFF_DL = OFF_GM + Q * 4;                      // float [Q] delta
    static constexpr int OFF_G1 = OFF_DL + Q * 4;                      // float [Q] gamma_s + delta_{s+1}
    static constexpr int OFF_WU = OFF_G1 + Q * 4;                      // float [Q] chunk-state weights
    static constexpr int OFF_TOT = OFF_WU + Q * 4;                     // float [NW][K] angle segment sums
    static constexpr int OFF_MISC = OFF_TOT + NW * K * 4;              // float [4]
    static constexpr int OFF_HB = (OFF_MISC + 16 + 15) / 16 * 16;      // bf16 [P][NS] carried state
    static constexpr int OFF_U = OFF_HB + P * NS * 2;                  // union region
    static constexpr int CST_BYTES = 32 * NS * 2;                      // per-wave C~ staging
    static constexpr int SB_BT = 0, SB_WT = 32 * NS * 2, SB_X = SB_WT + N * RS * 2;
    static constexpr int STAGE = SB_X + P * RS * 2;                    // one s-block stage
    static constexpr int U_BYTES = (NW * CST_BYTES > 2 * STAGE) ? NW * CST_BYTES : 2 * STAGE;
    static constexpr int LDS = OFF_U + U_BYTES;
    static_assert(LDS <= 160 * 1024, "LDS");
    // global loads per s-block (16 bytes each)
    static constexpr int BCH = 32 * N / 8, XCH = 32 * P / 8;
    static constexpr int NLB = (BCH + NTHR - 1) / NTHR, NLX = (XCH + NTHR - 1) / NTHR;
};

template <class CF>
__global__ __launch_bounds__(CF::NTHR) void k_scan_bf16(BfParams pr) {
    constexpr int N = CF::N, P = CF::P, R = CF::R, Q = CF::Q, NW = CF::NW, K = CF::K;
    constexpr int NB = CF::NB, TOKB = CF::TOKB, NTHR = CF::NTHR, PG = CF::PG, PT = CF::PT;
    constexpr int NPT = CF::NPT, TPW = CF::TPW, UPW = CF::UPW, NKK = CF::NKK, NS = CF::NS, RS = CF::RS;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float *phi = (float *)(smem + CF::OFF_PHI);
    float *S2 = (float *)(smem + CF::OFF_S2);
    float *A2 = (float *)(smem + CF::OFF_A2);
    float *GM = (float *)(smem + CF::OFF_GM);
    float *DL = (float *)(smem + CF::OFF_DL);
    float *G1 = (float *)(smem + CF::OFF_G1);
    float *WU = (float *)(smem + CF::OFF_WU);
    float *TOT = (float *)(smem + CF::OFF_TOT);
    float *MISC = (float *)(smem + CF::OFF_MISC);
    bf16 *HB = (bf16 *)(smem + CF::OFF_HB);
    char *UR = smem + CF::OFF_U;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int H = pr.H, G = pr.G;
    const int s = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / G);

    int64_t start, len;
    if (pr.cu) {
        int64_t a = min(max((int64_t)pr.cu[s], (int64_t)0), (int64_t)pr.seqlen);
        int64_t b = min(max((int64_t)pr.cu[s + 1], a), (int64_t)pr.seqlen);
        start = a;
        len = b - a;
    } else {
        start = (int64_t)s * pr.seqlen;
        len = pr.seqlen;
    }
    const float A2h = pr.A[h] * kLog2e;
    const float Dh = pr.D ? pr.D[h] : 0.f;

    // this wave's tasks (t-block, column group) and state tiles
    int task_tb[TPW], task_p0[TPW];
#pragma unroll
    for (int u = 0; u < TPW; u++) {
        int task = (TPW == 1) ? wave : (u / 2) * 2 * NW + ((u % 2 == 0) ? wave : 2 * NW - 1 - wave);
        task_tb[u] = task / PG;
        task_p0[u] = (task % PG) * PT;
    }
    int ut_n0[UPW], ut_p0[UPW];
#pragma unroll
    for (int v = 0; v < UPW; v++) {
        int ut = wave * UPW + v;
        ut_n0[v] = (ut / (P / 32)) * 32;
        ut_p0[v] = (ut % (P / 32)) * 32;
    }

    // ---- initial state: h_in (+ delta_0 Bprev xprev^T) in the MFMA accumulator layout
    f32x16 hreg[UPW];
    {
        const int64_t so = ((int64_t)s * H + h) * N * P;
        float d0 = 0.f;
        if (pr.Bprev && len > 0) {
            float dt0 = to_f(pr.dt[start * H + h]), l0 = to_f(pr.lam[start * H + h]);
            d0 = (1.f - l0) * dt0;
        }
#pragma unroll
        for (int v = 0; v < UPW; v++) {
            const int p = ut_p0[v] + l32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int n = ut_n0[v] + 8 * (r / 4) + 4 * hi + (r % 4);
                float val = pr.h_in ? pr.h_in[so + (int64_t)n * P + p] : 0.f;
                if (pr.Bprev) {
                    const bf16 *bp = pr.Bprev + ((int64_t)s * G + g) * N * R + n * R;
                    const bf16 *xp = pr.xprev + ((int64_t)s * H + h) * P * R + p * R;
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < R; j++) acc += to_f(bp[j]) * to_f(xp[j]);
                    val += d0 * acc;
                }
                hreg[v][r] = val;
            }
            // bf16 copy for the first chunk's inter-chunk term
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int n = ut_n0[v] + 8 * (r / 4) + 4 * hi + (r % 4);
                bf16x2 pk = {(bf16)hreg[v][r], (bf16)hreg[v][r + 1]};
                *(bf16x2 *)(HB + p * NS + n) = pk;
            }
        }
    }
    __syncthreads();

    for (int64_t c0 = 0; c0 < len; c0 += Q) {
        const int nq = (int)min((int64_t)Q, len - c0);
        const int64_t tok0 = start + c0;   // flat token index of chunk row 0

        // ---- prologue 1: per-token scalars and raw angles dt*theta
        if (tid < Q) {
            float dtv = 0.f, lv = 0.f;
            if (tid < nq) {
                dtv = to_f(pr.dt[(tok0 + tid) * H + h]);
                lv = to_f(pr.lam[(tok0 + tid) * H + h]);
            }
            A2[tid] = dtv * A2h;
            GM[tid] = lv * dtv;
            DL[tid] = (1.f - lv) * dtv;
        } else if (tid == Q) {
            float dn = 0.f;
            if (c0 + nq < len) {
                const int64_t tn = tok0 + nq;
                float dtv = to_f(pr.dt[tn * H + h]), lv = to_f(pr.lam[tn * H + h]);
                dn = (1.f - lv) * dtv;
            }
            MISC[0] = dn;
        }
        for (int e = tid; e < Q * K / 8; e += NTHR) {
            const int tau = e / (K / 8), k0 = (e % (K / 8)) * 8;
            float v[8];
            if (tau < nq) {
                const int64_t tg = tok0 + tau;
                const float dtv = to_f(pr.dt[tg * H + h]);
                bf16x8 th = *(const bf16x8 *)(pr.theta + (tg * H + h) * K + k0);
#pragma unroll
                for (int i = 0; i < 8; i++) v[i] = dtv * (float)th[i];
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++) v[i] = 0.f;
            }
            *(f32x4 *)(phi + tau * K + k0) = f32x4{v[0], v[1], v[2], v[3]};
            *(f32x4 *)(phi + tau * K + k0 + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
        __syncthreads();

        // ---- prologue 2: angle prefix within each wave's token segment; log-decay prefix (wave 0)
        constexpr int SEG = Q / NW;
        if (lane < K) {
            float acc = 0.f;
            for (int t = wave * SEG; t < (wave + 1) * SEG; t++) {
                acc += phi[t * K + lane];
                phi[t * K + lane] = acc;
            }
            TOT[wave * K + lane] = acc;
        }
        if (wave == 0) {
            constexpr int PER = (Q + 63) / 64;
            float loc[PER];
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < PER; i++) {
                const int t = lane * PER + i;
                run += (t < Q) ? A2[t] : 0.f;
                loc[i] = run;
            }
            const float incl = wave_incl_scan(run, lane);
            const float excl = incl - run;
#pragma unroll
            for (int i = 0; i < PER; i++) {
                const int t = lane * PER + i;
                if (t < Q) S2[t] = excl + loc[i];
            }
            lds_wait();
            const float S2e = S2[nq - 1];
            const float dn = MISC[0];
#pragma unroll
            for (int i = 0; i < PER; i++) {
                const int t = lane * PER + i;
                if (t < Q) {
                    float next = (t + 1 < nq) ? DL[t + 1] : ((t + 1 == nq) ? dn : 0.f);
                    float g1 = GM[t] + next;
                    G1[t] = g1;
                    WU[t] = (t < nq) ? exp2f(S2e - S2[t]) * g1 : 0.f;
                }
            }
            if (lane == 0) MISC[1] = S2e;
        }
        __syncthreads();
        // carry the segment sums into later segments
        if (lane < K && wave > 0) {
            float carry = 0.f;
            for (int w = 0; w < wave; w++) carry += TOT[w * K + lane];
            for (int t = wave * SEG; t < (wave + 1) * SEG; t++) phi[t * K + lane] += carry;
        }
        __syncthreads();

        // ---- prologue 3: rotated C~ rows of this wave's t-blocks into registers (staged per wave)
        bf16x8 creg[TPW][NKK];
        f32x16 yacc[TPW][NPT];
        {
            bf16 *cst = (bf16 *)(UR + wave * CF::CST_BYTES);
#pragma unroll
            for (int u = 0; u < TPW; u++) {
                const int tb = task_tb[u];
                // raw C of tokens tb*TOKB .. +TOKB: TOKB*N*R bf16 = 32*N, 16-byte pieces over the wave
                for (int c = lane; c < 32 * N / 8; c += 64) {
                    const int flat = c * 8;
                    const int tl = flat / (N * R);               // token within the block
                    const int n0 = (flat % (N * R)) / R;         // first state row of the piece
                    const int tau = tb * TOKB + tl;
                    bf16x8 raw;
                    if (tau < nq) raw = *(const bf16x8 *)(pr.C + ((tok0 + tau) * G + g) * N * R + n0 * R);
                    else raw = bf16x8{};
#pragma unroll
                    for (int q = 0; q < 4 / R; q++) {            // pairs in the piece
                        const int n = n0 + 2 * q;
                        float sn, cs;
                        __sincosf(phi[tau * K + n / 2], &sn, &cs);
#pragma unroll
                        for (int j = 0; j < R; j++) {
                            float c0v = (float)raw[(2 * q) * R + j], c1v = (float)raw[(2 * q + 1) * R + j];
                            bf16x2 pk = {(bf16)(cs * c0v + sn * c1v), (bf16)(-sn * c0v + cs * c1v)};
                            *(bf16x2 *)(cst + (tl * R + j) * NS + n) = pk;
                        }
                    }
                }
                lds_wait();
#pragma unroll
                for (int kk = 0; kk < NKK; kk++) creg[u][kk] = *(const bf16x8 *)(cst + l32 * NS + 16 * kk + 8 * hi);
                lds_wait();
            }
        }

        // ---- inter-chunk term: Y = e^{S_t} C~ H'   (H' bf16 in LDS, [p][n])
#pragma unroll
        for (int u = 0; u < TPW; u++) {
#pragma unroll
            for (int pt = 0; pt < NPT; pt++) {
                f32x16 acc = {};
                const int p = task_p0[u] + pt * 32 + l32;
#pragma unroll
                for (int kk = 0; kk < NKK; kk++) {
                    bf16x8 b = *(const bf16x8 *)(HB + p * NS + 16 * kk + 8 * hi);
                    acc = mfma32(creg[u][kk], b, acc);
                }
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int tau = task_tb[u] * TOKB + (8 * (r / 4) + 4 * hi + (r % 4)) / R;
                    acc[r] *= exp2f(S2[tau]);
                }
                yacc[u][pt] = acc;
            }
        }
        // state decays over the whole chunk before the chunk's update accumulates on it
        {
            const float eS = exp2f(MISC[1]);
#pragma unroll
            for (int v = 0; v < UPW; v++)
#pragma unroll
                for (int r = 0; r < 16; r++) hreg[v][r] *= eS;
        }
        __syncthreads();   // C~ staging and H' reads done: the union region becomes s-block stages

        // ---- s-block sweep
        const int nbv = (nq + TOKB - 1) / TOKB;   // blocks holding valid tokens
        bf16x8 rawB[CF::NLB], rawX[CF::NLX];
        auto load_block = [&](int sb) {
#pragma unroll
            for (int i = 0; i < CF::NLB; i++) {
                const int c = tid + i * NTHR;
                rawB[i] = bf16x8{};
                if (c < CF::BCH) {
                    const int flat = c * 8, tl = flat / (N * R), tau = sb * TOKB + tl;
                    if (tau < nq)
                        rawB[i] = *(const bf16x8 *)(pr.B + ((tok0 + tau) * G + g) * N * R + (flat % (N * R)));
                }
            }
#pragma unroll
            for (int i = 0; i < CF::NLX; i++) {
                const int c = tid + i * NTHR;
                rawX[i] = bf16x8{};
                if (c < CF::XCH) {
                    const int flat = c * 8, tl = flat / (P * R), tau = sb * TOKB + tl;
                    if (tau < nq)
                        rawX[i] = *(const bf16x8 *)(pr.x + ((tok0 + tau) * H + h) * P * R + (flat % (P * R)));
                }
            }
        };
        auto store_block = [&](int sb, int buf) {
            char *stg = UR + buf * CF::STAGE;
            bf16 *bt = (bf16 *)(stg + CF::SB_BT);   // [32 rows][NS]   rotated B~
            bf16 *wt = (bf16 *)(stg + CF::SB_WT);   // [N][RS]         wU * B~, transposed
            bf16 *xt = (bf16 *)(stg + CF::SB_X);    // [P][RS]         X, transposed
#pragma unroll
            for (int i = 0; i < CF::NLB; i++) {
                const int c = tid + i * NTHR;
                if (c < CF::BCH) {
                    const int flat = c * 8, tl = flat / (N * R), n0 = (flat % (N * R)) / R;
                    const int tau = sb * TOKB + tl;
                    const float w = WU[tau];
#pragma unroll
                    for (int q = 0; q < 4 / R; q++) {
                        const int n = n0 + 2 * q;
                        float sn, cs;
                        __sincosf(phi[tau * K + n / 2], &sn, &cs);
                        float r0[R], r1[R];
#pragma unroll
                        for (int j = 0; j < R; j++) {
                            float b0 = (float)rawB[i][(2 * q) * R + j], b1 = (float)rawB[i][(2 * q + 1) * R + j];
                            r0[j] = cs * b0 + sn * b1;
                            r1[j] = -sn * b0 + cs * b1;
                            bf16x2 pk = {(bf16)r0[j], (bf16)r1[j]};
                            *(bf16x2 *)(bt + (tl * R + j) * NS + n) = pk;
                        }
                        if constexpr (R == 4) {
                            bf16x4 w0 = {(bf16)(w * r0[0]), (bf16)(w * r0[1]), (bf16)(w * r0[2]), (bf16)(w * r0[3])};
                            bf16x4 w1 = {(bf16)(w * r1[0]), (bf16)(w * r1[1]), (bf16)(w * r1[2]), (bf16)(w * r1[3])};
                            *(bf16x4 *)(wt + n * RS + tl * 4) = w0;
                            *(bf16x4 *)(wt + (n + 1) * RS + tl * 4) = w1;
                        } else {
#pragma unroll
                            for (int j = 0; j < R; j++) {
                                wt[n * RS + tl * R + j] = (bf16)(w * r0[j]);
                                wt[(n + 1) * RS + tl * R + j] = (bf16)(w * r1[j]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < CF::NLX; i++) {
                const int c = tid + i * NTHR;
                if (c < CF::XCH) {
                    const int flat = c * 8, tl = flat / (P * R), p0 = (flat % (P * R)) / R;
                    if constexpr (R == 4) {
#pragma unroll
                        for (int q = 0; q < 2; q++) {
                            bf16x4 v = {rawX[i][4 * q], rawX[i][4 * q + 1], rawX[i][4 * q + 2], rawX[i][4 * q + 3]};
                            *(bf16x4 *)(xt + (p0 + q) * RS + tl * 4) = v;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; e++) xt[(p0 + e / R) * RS + tl * R + (e % R)] = rawX[i][e];
                    }
                }
            }
        };

        load_block(0);
        store_block(0, 0);
        __syncthreads();
        for (int sb = 0; sb < nbv; sb++) {
            const int buf = sb & 1;
            if (sb + 1 < nbv) load_block(sb + 1);
            const char *stg = UR + buf * CF::STAGE;
            const bf16 *bt = (const bf16 *)(stg + CF::SB_BT);
            const bf16 *wt = (const bf16 *)(stg + CF::SB_WT);
            const bf16 *xt = (const bf16 *)(stg + CF::SB_X);
            // scores and outputs for every owned t-block at or after this s-block
#pragma unroll
            for (int u = 0; u < TPW; u++) {
                const int tb = task_tb[u];
                if (tb < sb) continue;
                f32x16 gt = {};
#pragma unroll
                for (int kk = 0; kk < NKK; kk++) {
                    bf16x8 a = *(const bf16x8 *)(bt + l32 * NS + 16 * kk + 8 * hi);
                    gt = mfma32(a, creg[u][kk], gt);
                }
                // mask: row (s, j), column (t, i) of this lane
                const int tcol = tb * TOKB + l32 / R;
                const float S2t = S2[tcol];
                bf16x8 mop[2];
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int srow = sb * TOKB + (8 * (r / 4) + 4 * hi + (r % 4)) / R;
                    float coef = 0.f;
                    if (srow <= tcol) coef = exp2f(S2t - S2[srow]) * ((srow < tcol) ? G1[srow] : GM[srow]);
                    mop[r / 8][r % 8] = (bf16)(coef * gt[r]);
                }
#pragma unroll
                for (int pt = 0; pt < NPT; pt++) {
                    const int p = task_p0[u] + pt * 32 + l32;
#pragma unroll
                    for (int ks = 0; ks < 2; ks++) {
                        bf16x4 lo = *(const bf16x4 *)(xt + p * RS + 16 * ks + 4 * hi);
                        bf16x4 up = *(const bf16x4 *)(xt + p * RS + 16 * ks + 8 + 4 * hi);
                        bf16x8 b = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
                        yacc[u][pt] = mfma32(mop[ks], b, yacc[u][pt]);
                    }
                    if (tb == sb) {   // skip term D x_t from the staged X of this block
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            bf16x4 xv = *(const bf16x4 *)(xt + p * RS + 8 * q + 4 * hi);
#pragma unroll
                            for (int e = 0; e < 4; e++) yacc[u][pt][4 * q + e] += Dh * (float)xv[e];
                        }
                    }
                }
            }
            // chunk-state update on the owned state tiles: H += (wU B~)^T X
#pragma unroll
            for (int v = 0; v < UPW; v++) {
                const int n = ut_n0[v] + l32, p = ut_p0[v] + l32;
#pragma unroll
                for (int ks = 0; ks < 2; ks++) {
                    bf16x8 a = *(const bf16x8 *)(wt + n * RS + 16 * ks + 8 * hi);
                    bf16x8 b = *(const bf16x8 *)(xt + p * RS + 16 * ks + 8 * hi);
                    hreg[v] = mfma32(a, b, hreg[v]);
                }
            }
            if (sb + 1 < nbv) store_block(sb + 1, buf ^ 1);
            __syncthreads();
        }

        // ---- epilogue: outputs
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int tb = task_tb[u];
#pragma unroll
            for (int pt = 0; pt < NPT; pt++) {
                const int p = task_p0[u] + pt * 32 + l32;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    if constexpr (R == 4) {
                        const int tau = tb * TOKB + 2 * q + hi;
                        if (tau < nq) {
                            bf16x4 o = {(bf16)yacc[u][pt][4 * q], (bf16)yacc[u][pt][4 * q + 1],
                                        (bf16)yacc[u][pt][4 * q + 2], (bf16)yacc[u][pt][4 * q + 3]};
                            *(bf16x4 *)(pr.y + ((tok0 + tau) * H + h) * P * R + p * R) = o;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int row = 8 * q + 4 * hi + e;
                            const int tau = tb * TOKB + row / R, i = row % R;
                            if (tau < nq) pr.y[((tok0 + tau) * H + h) * P * R + p * R + i] = (bf16)yacc[u][pt][4 * q + e];
                        }
                    }
                }
            }
        }
        // ---- epilogue: rotate the state by the chunk's total angle; bf16 copy for the next chunk
        {
            const float *phe = phi + (nq - 1) * K;
#pragma unroll
            for (int v = 0; v < UPW; v++) {
                const int p = ut_p0[v] + l32;
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const int n = ut_n0[v] + 8 * (r / 4) + 4 * hi + (r % 4);
                    float sn, cs;
                    __sincosf(phe[n / 2], &sn, &cs);
                    const float u0 = hreg[v][r], u1 = hreg[v][r + 1];
                    hreg[v][r] = cs * u0 - sn * u1;
                    hreg[v][r + 1] = sn * u0 + cs * u1;
                    bf16x2 pk = {(bf16)hreg[v][r], (bf16)hreg[v][r + 1]};
                    *(bf16x2 *)(HB + p * NS + n) = pk;
                }
            }
        }
        __syncthreads();
    }

    if (pr.h_out) {
        const int64_t so = ((int64_t)s * H + h) * N * P;
#pragma unroll
        for (int v = 0; v < UPW; v++) {
            const int p = ut_p0[v] + l32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int n = ut_n0[v] + 8 * (r / 4) + 4 * hi + (r % 4);
                pr.h_out[so + (int64_t)n * P + p] = hreg[v][r];
            }
        }
    }
}

template <class CF>
mamba3_status launch_cfg(const mamba3_scan_args *a, hipStream_t st) {
    BfParams p;
    p.x = (const bf16 *)a->x; p.dt = (const bf16 *)a->dt; p.lam = (const bf16 *)a->lam;
    p.theta = (const bf16 *)a->theta; p.B = (const bf16 *)a->B; p.C = (const bf16 *)a->C;
    p.Bprev = (const bf16 *)a->Bprev; p.xprev = (const bf16 *)a->xprev;
    p.A = a->A; p.D = a->D; p.h_in = a->h_in; p.y = (bf16 *)a->y; p.h_out = a->h_out;
    p.cu = a->cu_seqlens; p.seqlen = a->seqlen; p.H = a->nheads; p.G = a->ngroups;
    const int64_t nseq = a->cu_seqlens ? a->nseq : a->batch;
    const int64_t nblk = nseq * a->nheads;
    if (nblk == 0) return MAMBA3_OK;
    if (hipFuncSetAttribute((const void *)k_scan_bf16<CF>, hipFuncAttributeMaxDynamicSharedMemorySize, CF::LDS) !=
        hipSuccess)
        return MAMBA3_EHIP;
    hipLaunchKernelGGL(k_scan_bf16<CF>, dim3((unsigned)nblk), dim3(CF::NTHR), CF::LDS, st, p);
    return hipGetLastError() == hipSuccess ? MAMBA3_OK : MAMBA3_EHIP;
}

}  // namespace

// (N, P, R, Q) -> waves per workgroup
#define M3_BF16_SHAPES(X) \
    X(128, 64, 1, 64, 4)  \
    X(64, 64, 4, 64, 4)   \
    X(128, 64, 4, 128, 8) \
    X(64, 64, 1, 64, 4)   \
    X(64, 64, 4, 32, 4)   \
    X(128, 64, 2, 64, 4)  \
    X(128, 64, 4, 64, 8)

bool scan_bf16_supported(int N, int P, int R, int Q) {
#define X(n, p, r, q, w) if (N == n && P == p && R == r && Q == q) return true;
    M3_BF16_SHAPES(X)
#undef X
    return false;
}

mamba3_status launch_scan_bf16(const mamba3_scan_args *a, hipStream_t st) {
    const int N = a->dstate, P = a->headdim, R = a->rank, Q = a->chunk;
#define X(n, p, r, q, w) \
    if (N == n && P == p && R == r && Q == q) return launch_cfg<Cfg<n, p, r, q, w>>(a, st);
    M3_BF16_SHAPES(X)
#undef X
    return MAMBA3_EUNSUPPORTED;
}

}  // namespace m3
