// bf16 chunked scan on gfx950 MFMA, fp32 state.
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
// Rank-expanded rows: row (tau, j) = tau*R + j of a chunk; with the rank-major
// layouts every such row of B, C, x and y is contiguous in memory. A chunk is
// a (Q*R) x (Q*R) problem: outputs are cut into 16-row t-blocks, the sweep over
// inputs into 32-row s-blocks.
//   * Once per chunk the cumulative angles become an fp16 (cos, sin) table in
//     LDS; every rotation of B, C reads it (one sincos per angle and chunk).
//   * Every wave owns t-blocks (balanced pairs along the causal triangle); it
//     loads their C rows straight from memory in MFMA operand layout, rotates
//     them in registers and keeps them, with the output accumulators, in
//     registers for the whole chunk.
//   * Each s-block's rotated B~ rows, X rows and weighted X rows are staged in
//     LDS as plain row copies. Each wave computes its score tiles
//     G^T = B~ C~^T (v_mfma_f32_16x16x32_bf16, K = N), applies the decay and
//     trapezoid mask in registers and feeds the bf16 tile straight back as the
//     A operand of Y += M X, with the K index permuted to the accumulator lane
//     layout; score tiles never touch LDS. Operands that need the token axis
//     as the K index (X for the outputs, B~ and weighted X for the state
//     update) are read with the LDS transpose read ds_read_b64_tr_b16.
//   * The N x P state is split into tiles over the waves; it accumulates the
//     chunk's rank-R update B~^T (w X) on MFMA and is rotated by the chunk's
//     total angle at the end (fp32). A bf16 copy in LDS feeds the next chunk's
//     inter-chunk term e^{S_t} C~^T H'.
//   * Global loads run ahead of use: raw B and X of the sequence's s-blocks
//     stream through two register sets two blocks ahead, and the next chunk's
//     dt, lam, theta and C rows are loaded while the current chunk computes.
//   * Outputs leave through a per-wave LDS transpose as 16-byte row stores.
#include <type_traits>

#include "m3_common.h"

namespace m3 {

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
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

// 2^x for x <= 0 (hardware exp2; results below the fp32 normal range flush to 0)
__device__ __forceinline__ float exp2_neg(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotate the 4 pairs of an 8-element row piece by -Phi: (u, v) -> (c u + s v, -s u + c v),
// with (cos, sin) of the 4 pairs packed as fp16 in cs.
__device__ __forceinline__ void rot_piece(const bf16x8 raw, const f16x8 cs, float (&o)[8]) {
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const float c = (float)cs[2 * m], sn = (float)cs[2 * m + 1];
        const float u = (float)raw[2 * m], v = (float)raw[2 * m + 1];
        o[2 * m] = c * u + sn * v;
        o[2 * m + 1] = c * v - sn * u;
    }
}
__device__ __forceinline__ bf16x8 pack8(const float (&o)[8]) {
    return bf16x8{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3], (bf16)o[4], (bf16)o[5], (bf16)o[6], (bf16)o[7]};
}

struct BfParams {
    const bf16 *x, *dt, *lam, *theta, *B, *C, *Bprev, *xprev;
    const float *A, *D, *h_in;
    bf16 *y;
    float *h_out;
    const int32_t *cu;
    int32_t seqlen, H, G;
};

template <int N_, int P_, int R_, int Q_, int NW_, int UT_>
struct Cfg {
    static constexpr int N = N_, P = P_, R = R_, Q = Q_, NW = NW_, UT = UT_;
    static constexpr int K = N / 2, QR = Q * R;
    static constexpr int NTB = QR / 16, NSB = QR / 32;      // 16-row t-blocks, 32-row s-blocks
    static constexpr int TOKT = 16 / R, TOKS = 32 / R;      // tokens per t-block / s-block
    static constexpr int NTHR = NW * 64, TPW = NTB / NW;
    static constexpr int NKK = N / 32;                      // K-steps over N (16x16x32)
    static constexpr int NPT = P / 16;                      // 16-column tiles of P
    static constexpr int NUT = (N / UT) * (P / UT), UPW = NUT / NW;
    static constexpr int UR_ = (UT == 32) ? 16 : 4;         // state registers per tile
    static constexpr int NS = N + 8, PS = P + 8;            // padded bf16 row strides
    static constexpr bool PFC = TPW <= 2;                   // prefetch the next chunk's C rows
    static_assert(N % 32 == 0 && P % 32 == 0 && (R == 1 || R == 2 || R == 4) && QR % 32 == 0, "shape");
    static_assert(NTB % NW == 0 && (TPW == 1 || TPW % 2 == 0), "t-block split");
    static_assert(NUT % NW == 0 && (UT == 16 || UT == 32), "state tile split");
    static_assert(K % 8 == 0 && Q % NW == 0 && Q <= 128 && Q < NTHR, "prologue");
    static_assert(NSB % 2 == 0, "full chunks alternate the two prefetch register sets");
    // LDS layout (bytes)
    static constexpr int OFF_PHI = 0;                                  // float [Q][K] -> f16x2 (cos, sin)
    static constexpr int OFF_PHC = OFF_PHI + Q * K * 4;                // float2 [K] (cos, sin) of the chunk's total angle
    static constexpr int OFF_S2 = OFF_PHC + K * 8;                     // float [Q] log2 decay prefix
    static constexpr int OFF_A2 = OFF_S2 + Q * 4;                      // float [Q] per-token log2 decay
    static constexpr int OFF_GM = OFF_A2 + Q * 4;                      // float [Q] gamma
    static constexpr int OFF_DL = OFF_GM + Q * 4;                      // float [Q] delta
    static constexpr int OFF_G1 = OFF_DL + Q * 4;                      // float [Q] gamma_s + delta_{s+1}
    static constexpr int OFF_WU = OFF_G1 + Q * 4;                      // float [Q] chunk-state weights
    static constexpr int OFF_F1 = OFF_WU + Q * 4;                      // float [Q] column mask factors, s < t
    static constexpr int OFF_F0 = OFF_F1 + Q * 4;                      // float [Q] column mask factors, s = t
    static constexpr int OFF_TOT = OFF_F0 + Q * 4;                     // float [NW][K] angle segment sums
    static constexpr int OFF_MISC = OFF_TOT + NW * K * 4;              // float [4]
    static constexpr int OFF_HB = (OFF_MISC + 16 + 15) / 16 * 16;      // bf16 [P][NS] carried state
    static constexpr int OFF_U = OFF_HB + P * NS * 2;                  // stage buffers / output staging
    static constexpr int SB_BT = 0, SB_X = 32 * NS * 2, SB_WX = SB_X + 32 * PS * 2;
    static constexpr int STAGE = SB_WX + 32 * PS * 2;                  // one s-block stage
    static constexpr int YST = 16 * PS * 2;                            // per-wave output staging
    static constexpr int U_BYTES = (NW * YST > 2 * STAGE) ? NW * YST : 2 * STAGE;
    static constexpr int LDS = OFF_U + U_BYTES;
    static_assert(LDS <= 160 * 1024, "LDS");
    // global loads (16 bytes each) per s-block, and next-chunk header prefetch
    static constexpr int BCH = 32 * N / 8, XCH = 32 * P / 8;
    static constexpr int NLB = (BCH + NTHR - 1) / NTHR, NLX = (XCH + NTHR - 1) / NTHR;
    static constexpr int NTH = (Q * K / 8 + NTHR - 1) / NTHR;
};

template <class CF>
__global__ __launch_bounds__(CF::NTHR) __attribute__((amdgpu_waves_per_eu(2))) void k_scan_bf16(BfParams pr) {
    constexpr int N = CF::N, P = CF::P, R = CF::R, Q = CF::Q, NW = CF::NW, K = CF::K, UT = CF::UT;
    constexpr int TOKT = CF::TOKT, TOKS = CF::TOKS, NTHR = CF::NTHR, TPW = CF::TPW;
    constexpr int NKK = CF::NKK, NPT = CF::NPT, UPW = CF::UPW, NS = CF::NS, PS = CF::PS, UR_ = CF::UR_;
    using UAcc = std::conditional_t<UT == 32, f32x16, f32x4>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float *phi = (float *)(smem + CF::OFF_PHI);
    const f16x2 *cst = (const f16x2 *)(smem + CF::OFF_PHI);   // after the prologue: (cos, sin) table
    float2 *PHC = (float2 *)(smem + CF::OFF_PHC);
    float *S2 = (float *)(smem + CF::OFF_S2);
    float *A2 = (float *)(smem + CF::OFF_A2);
    float *GM = (float *)(smem + CF::OFF_GM);
    float *DL = (float *)(smem + CF::OFF_DL);
    float *G1 = (float *)(smem + CF::OFF_G1);
    float *WU = (float *)(smem + CF::OFF_WU);
    float *F1 = (float *)(smem + CF::OFF_F1);
    float *F0 = (float *)(smem + CF::OFF_F0);
    float *TOT = (float *)(smem + CF::OFF_TOT);
    float *MISC = (float *)(smem + CF::OFF_MISC);
    bf16 *HB = (bf16 *)(smem + CF::OFF_HB);
    char *UR = smem + CF::OFF_U;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps per-wave branches scalar
    const int l16 = lane & 15, q4 = lane >> 4, l32 = lane & 31, hi = lane >> 5;
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
    // per-(sequence, head) base pointers: add token * stride (+ rank * N or P)
    const bf16 *gB = pr.B + g * (int64_t)R * N;
    const bf16 *gC = pr.C + g * (int64_t)R * N;
    const bf16 *gX = pr.x + h * (int64_t)R * P;
    bf16 *gY = pr.y + h * (int64_t)R * P;
    const bf16 *gTh = pr.theta + h * (int64_t)K;
    const int64_t strBC = (int64_t)G * R * N, strX = (int64_t)H * R * P, strTh = (int64_t)H * K;

    // this wave's t-blocks and state tiles
    // t-block u of this wave in the chunk starting at c0x: balanced pairs along the causal
    // triangle, rotated by the chunk index so the heavy blocks move across the SIMDs
    auto tb_of = [&](int u, int64_t c0x) {
        const int w = (wave + (int)(c0x / Q)) % NW;
        return (TPW == 1) ? w : (u / 2) * 2 * NW + ((u % 2 == 0) ? w : 2 * NW - 1 - w);
    };
    int ut_n0[UPW], ut_p0[UPW];
#pragma unroll
    for (int v = 0; v < UPW; v++) {
        const int ut = wave * UPW + v;
        ut_n0[v] = (ut / (P / UT)) * UT;
        ut_p0[v] = (ut % (P / UT)) * UT;
    }
    // state-tile register r -> row n within the tile; column = ucol
    auto urow = [&](int r) { return (UT == 32) ? 8 * (r / 4) + 4 * hi + (r % 4) : 4 * q4 + r; };
    const int ucol = (UT == 32) ? l32 : l16;

    // ---- initial state: h_in (+ delta_0 Bprev xprev^T) in the accumulator layout
    UAcc hreg[UPW];
    {
        const int64_t so = ((int64_t)s * H + h) * N * P;
        float d0 = 0.f;
        if (pr.Bprev && len > 0) {
            const float dt0 = to_f(pr.dt[start * H + h]), l0 = to_f(pr.lam[start * H + h]);
            d0 = (1.f - l0) * dt0;
        }
#pragma unroll
        for (int v = 0; v < UPW; v++) {
            const int p = ut_p0[v] + ucol;
#pragma unroll
            for (int r = 0; r < UR_; r++) {
                const int n = ut_n0[v] + urow(r);
                float val = pr.h_in ? pr.h_in[so + (int64_t)n * P + p] : 0.f;
                if (pr.Bprev) {
                    const bf16 *bp = pr.Bprev + ((int64_t)s * G + g) * R * N + n;
                    const bf16 *xp = pr.xprev + ((int64_t)s * H + h) * R * P + p;
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < R; j++) acc += to_f(bp[j * N]) * to_f(xp[j * P]);
                    val += d0 * acc;
                }
                hreg[v][r] = val;
            }
#pragma unroll
            for (int r = 0; r < UR_; r += 2) {
                const int n = ut_n0[v] + urow(r);
                *(bf16x2 *)(HB + p * NS + n) = bf16x2{(bf16)hreg[v][r], (bf16)hreg[v][r + 1]};
            }
        }
    }

    // ---- next-chunk header (dt, lam, theta, own C rows) prefetched into registers
    // All prefetch loads are unconditional: a token past the end of the
    // sequence is clamped to the last valid one (or to the sequence start when
    // the whole chunk lies past the end), so the compiler sees a fixed sequence
    // of memory operations. Loaded values stay raw until their use, where
    // tokens past the end are masked; no select or conversion sits next to a
    // load, so nothing waits for a prefetch before its consumer needs it.
    bf16 h_dt = {}, h_lam = {};
    bf16x8 h_th[CF::NTH];
    bf16 h_thdt[CF::NTH];
    bf16x8 h_c[TPW][NKK];
    // C rows of the own t-blocks in operand layout: row 16 tb + l16, columns 32 kk + 8 q4 ..
    auto load_crows = [&](int64_t c0h) {
        const int64_t c0c = c0h < len ? c0h : 0;
        const int64_t t0h = start + c0c, last = len - c0c - 1;
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int row = tb_of(u, c0h) * 16 + l16;
            const int tau = row / R, j = row % R;
            const int64_t tk = t0h + min((int64_t)tau, last);
#pragma unroll
            for (int kk = 0; kk < NKK; kk++) h_c[u][kk] = *(const bf16x8 *)(gC + tk * strBC + j * N + 32 * kk + 8 * q4);
        }
    };
    auto load_header = [&](int64_t c0h) {
        const int64_t c0c = c0h < len ? c0h : 0;
        const int nqh = (int)min((int64_t)Q, len - c0c);
        const int64_t t0h = start + c0c, last = len - c0c - 1;
        {
            const int idx = (tid < Q) ? tid : nqh;                 // thread Q: the token after the chunk
            const int64_t tk = t0h + min((int64_t)idx, last);
            h_dt = pr.dt[tk * H + h];
            h_lam = pr.lam[tk * H + h];
        }
#pragma unroll
        for (int i = 0; i < CF::NTH; i++) {
            const int e = min(tid + i * NTHR, Q * K / 8 - 1);
            const int tau = e / (K / 8), k0 = (e % (K / 8)) * 8;
            const int64_t tk = t0h + min((int64_t)tau, last);
            h_thdt[i] = pr.dt[tk * H + h];
            h_th[i] = *(const bf16x8 *)(gTh + tk * strTh + k0);
        }
        if constexpr (CF::PFC) load_crows(c0h);
    };

    // ---- s-block stream: block j of the sequence lives in register set j % 2
    bf16x8 rb0[CF::NLB], rx0[CF::NLX], rb1[CF::NLB], rx1[CF::NLX];
    auto load_block_into = [&](bf16x8 (&rb)[CF::NLB], bf16x8 (&rx)[CF::NLX], int64_t c0b, int sb) {
        const int64_t c0c = c0b < len ? c0b : 0;                   // past the end: dummy loads, never used
        const int64_t t0b = start + c0c, last = len - c0c - 1;
#pragma unroll
        for (int i = 0; i < CF::NLB; i++) {
            const int c = (tid + i * NTHR) % CF::BCH;
            const int row = c / (N / 8), col = (c % (N / 8)) * 8;
            const int tau = sb * TOKS + row / R;
            const int64_t tk = t0b + min((int64_t)tau, last);
            rb[i] = *(const bf16x8 *)(gB + tk * strBC + (row % R) * N + col);
        }
#pragma unroll
        for (int i = 0; i < CF::NLX; i++) {
            const int c = (tid + i * NTHR) % CF::XCH;
            const int row = c / (P / 8), col = (c % (P / 8)) * 8;
            const int tau = sb * TOKS + row / R;
            const int64_t tk = t0b + min((int64_t)tau, last);
            rx[i] = *(const bf16x8 *)(gX + tk * strX + (row % R) * P + col);
        }
    };
    auto advance = [&](int64_t &c0b, int &sb) {
        if (c0b >= len) return;
        const int nqb = (int)min((int64_t)Q, len - c0b);
        if (sb + 1 < (nqb + TOKS - 1) / TOKS) {
            sb++;
        } else {
            c0b += Q;
            sb = 0;
        }
    };
    int64_t ld_c0 = 0;
    int ld_sb = 0;
    if (len > 0) {
        load_header(0);
        load_block_into(rb0, rx0, ld_c0, ld_sb);
        advance(ld_c0, ld_sb);
        load_block_into(rb1, rx1, ld_c0, ld_sb);
        advance(ld_c0, ld_sb);
    }
    __syncthreads();

    // One chunk. Full chunks (Q tokens) have a compile-time number of s-blocks
    // (NSB, even), so block j of the sequence always sits in register set j % 2
    // and the sweep is fully unrolled; the final partial chunk runs the same
    // steps under a runtime bound.
    auto chunk_body = [&](auto FULLC, int64_t c0) {
        constexpr bool FULL = decltype(FULLC)::value;
        const int nq = FULL ? Q : (int)(len - c0);
        const int64_t tok0 = start + c0;
        int task_tb[TPW];
#pragma unroll
        for (int u = 0; u < TPW; u++) task_tb[u] = tb_of(u, c0);

        // ---- prologue 1: per-token scalars and raw angles dt*theta
        {
            const float dt = to_f(h_dt), lm = to_f(h_lam);
            if (tid < Q) {
                const bool ok = FULL || tid < nq;
                A2[tid] = ok ? dt * A2h : 0.f;
                GM[tid] = ok ? lm * dt : 0.f;
                DL[tid] = ok ? (1.f - lm) * dt : 0.f;
            } else if (tid == Q) {
                MISC[0] = (c0 + nq < len) ? (1.f - lm) * dt : 0.f;   // delta of the token after the chunk
            }
        }
#pragma unroll
        for (int i = 0; i < CF::NTH; i++) {
            const int e = tid + i * NTHR;
            if (e < Q * K / 8) {
                const int tau = e / (K / 8), k0 = (e % (K / 8)) * 8;
                const bool ok = FULL || tau < nq;
                const float dt = to_f(h_thdt[i]);
                float v[8];
#pragma unroll
                for (int q = 0; q < 8; q++) v[q] = ok ? dt * (float)h_th[i][q] : 0.f;
                *(f32x4 *)(phi + tau * K + k0) = f32x4{v[0], v[1], v[2], v[3]};
                *(f32x4 *)(phi + tau * K + k0 + 4) = f32x4{v[4], v[5], v[6], v[7]};
            }
        }
        __syncthreads();

        // ---- prologue 2: angle prefix within each wave's token segment; log-decay prefix (wave 0)
        constexpr int SEG = Q / NW;
        if (lane < K) {
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < SEG; t++) {
                acc += phi[(wave * SEG + t) * K + lane];
                phi[(wave * SEG + t) * K + lane] = acc;
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
                    const float next = (t + 1 < nq) ? DL[t + 1] : ((t + 1 == nq) ? dn : 0.f);
                    const float g1 = GM[t] + next;
                    G1[t] = g1;
                    WU[t] = (t < nq) ? exp2_neg(S2e - S2[t]) * g1 : 0.f;
                    // mask factor relative to the first token of the t's s-block (>= 1)
                    const float f = __builtin_amdgcn_exp2f(S2[(t / TOKS) * TOKS] - S2[t]);
                    F1[t] = f * g1;
                    F0[t] = f * GM[t];
                }
            }
            if (lane == 0) {
                MISC[1] = S2e;
                // the factored mask is used when every factor stays far inside the fp32 range
                MISC[2] = (S2[0] - S2[Q - 1] <= 120.f) ? 1.f : 0.f;
            }
        }
        __syncthreads();
        // ---- prologue 3: carry the segment sums, keep the total angle, turn angles into (cos, sin)
        if (lane < K) {
            float carry = 0.f;
            for (int w = 0; w < wave; w++) carry += TOT[w * K + lane];
#pragma unroll
            for (int t = 0; t < SEG; t++) {
                const int tau = wave * SEG + t;
                const float a = phi[tau * K + lane] + carry;
                if (tau == Q - 1) {                // angles past the end are zero: Phi[Q-1] = Phi[nq-1]
                    float sn, cs;
                    sincosf(a, &sn, &cs);
                    PHC[lane] = float2{cs, sn};
                }
                float sn, cs;
                __sincosf(a, &sn, &cs);
                ((f16x2 *)phi)[tau * K + lane] = f16x2{(_Float16)cs, (_Float16)sn};
            }
        }
        __syncthreads();

        // ---- rotated C~ rows of this wave's t-blocks, from the prefetched (or just loaded) raw rows
        if constexpr (!CF::PFC) load_crows(c0);
        bf16x8 creg[TPW][NKK];
        f32x4 yacc[TPW][NPT];
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int tau = (task_tb[u] * 16 + l16) / R;
#pragma unroll
            for (int kk = 0; kk < NKK; kk++) {
                const f16x8 cs = *(const f16x8 *)(cst + tau * K + 16 * kk + 4 * q4);
                float o[8];
                rot_piece(h_c[u][kk], cs, o);
                creg[u][kk] = (FULL || tau < nq) ? pack8(o) : bf16x8{};
            }
        }

        // ---- inter-chunk term: Y = e^{S_t} C~ H'   (H' bf16 in LDS, [p][n])
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int tb = task_tb[u];
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; i++) sc[i] = exp2_neg(S2[(tb * 16 + 4 * q4 + i) / R]);
#pragma unroll
            for (int pt = 0; pt < NPT; pt++) {
                f32x4 acc = {};
                const int p = pt * 16 + l16;
#pragma unroll
                for (int kk = 0; kk < NKK; kk++)
                    acc = mfma16(creg[u][kk], *(const bf16x8 *)(HB + p * NS + 32 * kk + 8 * q4), acc);
#pragma unroll
                for (int i = 0; i < 4; i++) acc[i] *= sc[i];
                yacc[u][pt] = acc;
            }
        }
        {
            const float eS = exp2_neg(MISC[1]);
#pragma unroll
            for (int v = 0; v < UPW; v++)
#pragma unroll
                for (int r = 0; r < UR_; r++) hreg[v][r] *= eS;
        }
        // the header registers are consumed: prefetch the next chunk's header now
        load_header(c0 + Q);

        // ---- s-block sweep
        // lane coordinates made opaque per chunk: the mask indices derived from them are
        // recomputed in every chunk instead of being hoisted out of the chunk loop (and spilled)
        int l16c = l16, q4c = q4;
        if constexpr (CF::NSB <= 8) asm volatile("" : "+v"(l16c), "+v"(q4c));   // fully unrolled sweeps
        const bool fastmask = __builtin_amdgcn_readfirstlane(__float_as_int(MISC[2])) != 0;
        float S2t[TPW];
#pragma unroll
        for (int u = 0; u < TPW; u++) S2t[u] = S2[(task_tb[u] * 16 + l16) / R];
        const int nbs = FULL ? CF::NSB : (nq + TOKS - 1) / TOKS;   // s-blocks holding valid tokens
        auto store_block = [&](const bf16x8 (&rawB)[CF::NLB], const bf16x8 (&rawX)[CF::NLX], int sb, int buf) {
            char *stg = UR + buf * CF::STAGE;
            bf16 *bt = (bf16 *)(stg + CF::SB_BT);   // [32 rows][NS]  rotated B~
            bf16 *xs = (bf16 *)(stg + CF::SB_X);    // [32 rows][PS]  X
            bf16 *wx = (bf16 *)(stg + CF::SB_WX);   // [32 rows][PS]  wU * X
            // every LDS read of the block first, then the arithmetic and the stores: a read
            // issued after a store would also wait for that store
            f16x8 csb[CF::NLB];
            float wxv[CF::NLX];
#pragma unroll
            for (int i = 0; i < CF::NLB; i++) {
                const int c = min(tid + i * NTHR, CF::BCH - 1);
                csb[i] = *(const f16x8 *)(cst + (sb * TOKS + (c / (N / 8)) / R) * K + (c % (N / 8)) * 4);
            }
#pragma unroll
            for (int i = 0; i < CF::NLX; i++) {
                const int c = min(tid + i * NTHR, CF::XCH - 1);
                wxv[i] = WU[sb * TOKS + (c / (P / 8)) / R];
            }
#pragma unroll
            for (int i = 0; i < CF::NLB; i++) {
                const int c = tid + i * NTHR;
                if (c < CF::BCH) {
                    const int row = c / (N / 8), col = (c % (N / 8)) * 8;
                    const int tau = sb * TOKS + row / R;
                    float o[8];
                    rot_piece(rawB[i], csb[i], o);
                    *(bf16x8 *)(bt + row * NS + col) = (FULL || tau < nq) ? pack8(o) : bf16x8{};
                }
            }
#pragma unroll
            for (int i = 0; i < CF::NLX; i++) {
                const int c = tid + i * NTHR;
                if (c < CF::XCH) {
                    const int row = c / (P / 8), col = (c % (P / 8)) * 8;
                    const int tau = sb * TOKS + row / R;
                    const bool ok = FULL || tau < nq;
                    *(bf16x8 *)(xs + row * PS + col) = ok ? rawX[i] : bf16x8{};
                    float o[8];
#pragma unroll
                    for (int e = 0; e < 8; e++) o[e] = wxv[i] * (float)rawX[i][e];
                    *(bf16x8 *)(wx + row * PS + col) = ok ? pack8(o) : bf16x8{};
                }
            }
        };
        auto compute_block = [&](int sb) {
            const char *stg = UR + (sb & 1) * CF::STAGE;
            const bf16 *bt = (const bf16 *)(stg + CF::SB_BT);
            const bf16 *xs = (const bf16 *)(stg + CF::SB_X);
            const bf16 *wx = (const bf16 *)(stg + CF::SB_WX);
#pragma unroll
            for (int u = 0; u < TPW; u++) {
                const int tb = task_tb[u];
                if (2 * sb > tb) continue;                  // t-block lies before this s-block
                const bool upper = (2 * sb + 1 <= tb);      // second 16-row half of the s-block is causal
                f32x4 g0 = {}, g1 = {};
#pragma unroll
                for (int kk = 0; kk < NKK; kk++) {
                    g0 = mfma16(*(const bf16x8 *)(bt + l16 * NS + 32 * kk + 8 * q4), creg[u][kk], g0);
                    if (upper) g1 = mfma16(*(const bf16x8 *)(bt + (16 + l16) * NS + 32 * kk + 8 * q4), creg[u][kk], g1);
                }
                // decay/trapezoid mask: column (t, i) = lane's t-row, rows (s, j) of the two halves
                const int tt = (tb * 16 + l16c) / R;
                auto sidx = [&](int e) { return (sb * 32 + 16 * (e / 4) + 4 * q4c + (e % 4)) / R; };
                bf16x8 mop;
                if (fastmask) {
                    // e^{S_t - S_s} w_s = 2^{S2_t - S2_ref} * (2^{S2_ref - S2_s} w_s), ref = first token
                    // of the s-block; the second factor is tabulated per chunk
                    const float rf = exp2_neg(S2t[u] - S2[sb * TOKS]);
                    float fc[8];
                    if constexpr (R == 1) {
                        const f32x4 a = *(const f32x4 *)(F1 + sb * 32 + 4 * q4);
                        const f32x4 b = *(const f32x4 *)(F1 + sb * 32 + 16 + 4 * q4);
#pragma unroll
                        for (int e = 0; e < 4; e++) { fc[e] = a[e]; fc[e + 4] = b[e]; }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; e++) fc[e] = F1[sidx(e)];
                    }
                    if (tb >= 2 * sb + 2) {                 // every s of the tile precedes every t
#pragma unroll
                        for (int e = 0; e < 8; e++) mop[e] = (bf16)(rf * fc[e] * ((e < 4) ? g0[e] : g1[e - 4]));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            // masks as 0/1 factors rather than selects of loaded values, which
                            // the compiler would turn into branches around the loads
                            const int ss = sidx(e);
                            const float m1 = (ss < tt) ? 1.f : 0.f, m0 = (ss == tt) ? 1.f : 0.f;
                            float coef = fc[e] * m1 + F0[ss] * m0;
                            if (!(e < 4 || upper)) coef = 0.f;
                            mop[e] = (bf16)(rf * coef * ((e < 4) ? g0[e] : g1[e - 4]));
                        }
                    }
                } else {
                    const float S2tt = S2[tt];
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const int ss = sidx(e);
                        const float m1 = (ss < tt) ? 1.f : 0.f, m0 = (ss == tt) ? 1.f : 0.f;
                        float coef = exp2_neg(fminf(S2tt - S2[ss], 0.f)) * (G1[ss] * m1 + GM[ss] * m0);
                        if (!(e < 4 || upper)) coef = 0.f;
                        mop[e] = (bf16)(coef * ((e < 4) ? g0[e] : g1[e - 4]));
                    }
                }
                const int dblk = tb - 2 * sb;               // 0/1: the t-block's rows are in this s-block
#pragma unroll
                for (int pt = 0; pt < NPT; pt++) {
                    // X rows 4 q4 .. and 16 + 4 q4 .. of column 16 pt + l16 (K permuted like mop)
                    yacc[u][pt] = mfma16(mop, tr_operand(xs, PS, 4 * q4, 16 + 4 * q4, pt * 16, l16), yacc[u][pt]);
                    if (dblk == 0 || dblk == 1) {           // skip term D x_t of the t-block's own rows
                        const bf16x4 xv = ds_read_tr(xs + (16 * dblk + 4 * q4 + l16 / 4) * PS + pt * 16 + 4 * (l16 % 4));
#pragma unroll
                        for (int i = 0; i < 4; i++) yacc[u][pt][i] += Dh * (float)xv[i];
                    }
                }
            }
            // chunk-state update on the owned state tiles: H += B~^T (wU X), K = the s-block's rows
#pragma unroll
            for (int v = 0; v < UPW; v++) {
                if constexpr (UT == 32) {
                    // lane groups: column half c0 = 16 (group % 2), K rows 8 (group / 2) ..
                    const int grp = lane >> 4;
                    const int cn = ut_n0[v] + 16 * (grp & 1), cp = ut_p0[v] + 16 * (grp & 1);
#pragma unroll
                    for (int ks = 0; ks < 2; ks++) {
                        const int r0 = 16 * ks + 8 * (grp >> 1);
                        hreg[v] = mfma32(tr_operand(bt, NS, r0, r0 + 4, cn, l16), tr_operand(wx, PS, r0, r0 + 4, cp, l16),
                                         hreg[v]);
                    }
                } else {
                    hreg[v] = mfma16(tr_operand(bt, NS, 8 * q4, 8 * q4 + 4, ut_n0[v], l16),
                                     tr_operand(wx, PS, 8 * q4, 8 * q4 + 4, ut_p0[v], l16), hreg[v]);
                }
            }
        };

        // block sb of this chunk: set sb % 2 receives block sb + 2 of the stream, then the
        // block is computed and block sb + 1 is staged from the other set
        auto step = [&](auto SETC, int sb) {
            constexpr int ST = decltype(SETC)::value;
            if constexpr (ST == 0) load_block_into(rb0, rx0, ld_c0, ld_sb);
            else load_block_into(rb1, rx1, ld_c0, ld_sb);
            advance(ld_c0, ld_sb);
            compute_block(sb);
            if (sb + 1 < nbs) {
                if constexpr (ST == 0) store_block(rb1, rx1, sb + 1, (sb + 1) & 1);
                else store_block(rb0, rx0, sb + 1, (sb + 1) & 1);
            }
            __syncthreads();
        };
        store_block(rb0, rx0, 0, 0);
        __syncthreads();
        if constexpr (FULL && CF::NSB <= 8) {
#pragma unroll
            for (int sb = 0; sb < CF::NSB; sb += 2) {
                step(std::integral_constant<int, 0>{}, sb);
                step(std::integral_constant<int, 1>{}, sb + 1);
            }
        } else if constexpr (FULL) {
#pragma nounroll
            for (int sb = 0; sb < CF::NSB; sb += 2) {
                step(std::integral_constant<int, 0>{}, sb);
                step(std::integral_constant<int, 1>{}, sb + 1);
            }
        } else {
            for (int sb = 0; sb < nbs; sb += 2) {
                step(std::integral_constant<int, 0>{}, sb);
                if (sb + 1 < nbs) step(std::integral_constant<int, 1>{}, sb + 1);
            }
        }

        // ---- epilogue: outputs through a per-wave LDS transpose, 16-byte row stores
        {
            bf16 *ys = (bf16 *)(UR + wave * CF::YST);   // [16 rows][PS]
#pragma unroll
            for (int u = 0; u < TPW; u++) {
                const int tb = task_tb[u];
#pragma unroll
                for (int pt = 0; pt < NPT; pt++)
#pragma unroll
                    for (int i = 0; i < 4; i++) ys[(4 * q4 + i) * PS + pt * 16 + l16] = (bf16)yacc[u][pt][i];
                lds_wait();
#pragma unroll
                for (int c = lane; c < 16 * P / 8; c += 64) {
                    const int row = c / (P / 8), col = (c % (P / 8)) * 8;
                    const int rr = tb * 16 + row, tau = rr / R;
                    if (FULL || tau < nq) *(bf16x8 *)(gY + (tok0 + tau) * strX + (rr % R) * P + col) =
                        *(const bf16x8 *)(ys + row * PS + col);
                }
                lds_wait();
            }
        }
        // ---- epilogue: rotate the state by the chunk's total angle; bf16 copy for the next chunk
        // (cos, sin) of the pairs of rows urow(4q) .. urow(4q) + 3: two pairs per 16-byte read,
        // all read before the first store
        f32x4 rot4[UPW][UR_ / 4];
#pragma unroll
        for (int v = 0; v < UPW; v++)
#pragma unroll
            for (int q = 0; q < UR_ / 4; q++) rot4[v][q] = *(const f32x4 *)(PHC + (ut_n0[v] + urow(4 * q)) / 2);
#pragma unroll
        for (int v = 0; v < UPW; v++) {
            const int p = ut_p0[v] + ucol;
#pragma unroll
            for (int r = 0; r < UR_; r += 2) {
                const int n = ut_n0[v] + urow(r);
                const float cs = rot4[v][r / 4][r % 4], sn = rot4[v][r / 4][r % 4 + 1];
                const float u0 = hreg[v][r], u1 = hreg[v][r + 1];
                hreg[v][r] = cs * u0 - sn * u1;
                hreg[v][r + 1] = sn * u0 + cs * u1;
                *(bf16x2 *)(HB + p * NS + n) = bf16x2{(bf16)hreg[v][r], (bf16)hreg[v][r + 1]};
            }
        }
        __syncthreads();
    };

    int64_t c0 = 0;
    for (; c0 + Q <= len; c0 += Q) chunk_body(std::true_type{}, c0);
    if (c0 < len) chunk_body(std::false_type{}, c0);

    if (pr.h_out) {
        const int64_t so = ((int64_t)s * H + h) * N * P;
#pragma unroll
        for (int v = 0; v < UPW; v++) {
            const int p = ut_p0[v] + ucol;
#pragma unroll
            for (int r = 0; r < UR_; r++) pr.h_out[so + (int64_t)(ut_n0[v] + urow(r)) * P + p] = hreg[v][r];
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

// (N, P, R, Q) -> waves per workgroup, state tile size
#define M3_BF16_SHAPES(X)      \
    X(128, 64, 1, 64, 4, 32)   \
    X(64, 64, 4, 64, 8, 16)    \
    X(128, 64, 4, 128, 8, 16)  \
    X(64, 64, 1, 64, 4, 32)    \
    X(64, 64, 4, 32, 8, 16)    \
    X(128, 64, 2, 64, 8, 32)   \
    X(128, 64, 4, 64, 8, 32)

bool scan_bf16_supported(int N, int P, int R, int Q) {
#define X(n, p, r, q, w, ut) if (N == n && P == p && R == r && Q == q) return true;
    M3_BF16_SHAPES(X)
#undef X
    return false;
}

mamba3_status launch_scan_bf16(const mamba3_scan_args *a, hipStream_t st) {
    const int N = a->dstate, P = a->headdim, R = a->rank, Q = a->chunk;
#define X(n, p, r, q, w, ut) \
    if (N == n && P == p && R == r && Q == q) return launch_cfg<Cfg<n, p, r, q, w, ut>>(a, st);
    M3_BF16_SHAPES(X)
#undef X
    return MAMBA3_EUNSUPPORTED;
}

}  // namespace m3
