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
//   * Once per chunk the cumulative angles become a (cos, sin) table in LDS;
//     every rotation of B, C reads it (one sincos per angle and chunk). Raw
//     rows are rotated on the bf16 dot-product instruction from bf16 pairs
//     (one v_dot2_f32_bf16 per element, fp32 sums); with the fused prologue
//     the rows are fp32 when rotated, and the table holds fp16 pairs.
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
//     With the fused epilogue the transpose buffers share LDS with the angle
//     table, which is dead from the end of the sweep until the next chunk
//     rebuilds it.
//
// The EPI instantiations fuse the block prologue and epilogue (section
// "Architectural Integration"): every B, C and Bprev column is scaled to unit
// RMS and gets the head's bias (rows kept in LDS) before its rotation, and y
// is multiplied by SiLU(z) after the D term, in fp32 before the single bf16
// rounding. The RMS of a column is a butterfly of wave shuffles over the lanes
// that hold its pieces: the 4 operand lanes of a C row, the N/8 consecutive
// loading lanes of a staged B row. They also carry the variants: a per-token
// decay rate A_t (loaded with dt) and a fixed trapezoid weight.
#include <type_traits>

#include "mfma_ops.h"

namespace m3 {

namespace {

// Prologue of one 8-element piece of a B or C column: scale by inv (the column's inverse RMS,
// or 1) and add the bias slice b (8 fp32 values in LDS).
__device__ __forceinline__ void prologue_piece(const bf16x8 raw, float inv, const float *b, float (&o)[8]) {
    const f32x4 b0 = *(const f32x4 *)b, b1 = *(const f32x4 *)(b + 4);
#pragma unroll
    for (int e = 0; e < 8; e++) o[e] = (float)raw[e] * inv + ((e < 4) ? b0[e] : b1[e - 4]);
}
__device__ __forceinline__ float sumsq8(const bf16x8 v) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) ss += (float)v[e] * (float)v[e];
    return ss;
}

struct BfParams {
    const bf16 *x, *dt, *lam, *theta, *B, *C, *Bprev, *xprev;
    const float *A, *D, *h_in;
    bf16 *y;
    float *h_out;
    const int32_t *cu;
    int32_t seqlen, H, G, nseq;
    const float *Bb, *Cb;   // prologue biases [H, N], or NULL
    const bf16 *z;          // output gate, or NULL
    int32_t norm;           // 1: B, C, Bprev columns scaled to unit RMS
    float eps;
    // variants (EPI instantiations): a per-token decay rate, a fixed trapezoid weight. Atk and
    // lam always point at readable token data (dt stands in for an absent array).
    const bf16 *Atk;
    int32_t atok_on, lam_on;
    float lam_fixed;
    int32_t Gth;            // angle rows per token (divides H): head h reads row h / (H / Gth)
    // state-only scans: the state entering every chunk, [S * chunks][H][P][N] bf16 (the MFMA
    // backward's chunk-state layout: a state column's N rows contiguous), or NULL
    bf16 *ws_state;
    // state-only scans: sum_t dt_t A_t and sum_t dt_t theta_t[k] over each sequence, written to
    // the first K + 1 floats of its [S][H][N][P] block (the segment sums that state passing
    // reads), or NULL
    float *seg_sums;
};

template <int N_, int P_, int R_, int Q_, int NW_, int UT_, int SBR_, bool EPI_, bool YO_ = true>
struct Cfg {
    static constexpr int N = N_, P = P_, R = R_, Q = Q_, NW = NW_, UT = UT_, SBR = SBR_;
    static constexpr bool EPI = EPI_;                        // fused block prologue / epilogue
    // outputs; without them (a state-only scan) a chunk is its chunk-state update alone: no C
    // rows are read, no scores or y are formed
    static constexpr bool YO = YO_;
    static constexpr int K = N / 2, QR = Q * R;
    static constexpr int NTB = QR / 16, NSB = QR / SBR;     // 16-row t-blocks, SBR-row s-blocks
    static constexpr int NSUB = SBR / 32;                    // 32-row score tiles per s-block
    static constexpr int NST = (NSB == 1) ? 1 : 2;           // LDS stages of s-blocks
    static constexpr int TOKT = 16 / R, TOKS = SBR / R;     // tokens per t-block / s-block
    static constexpr int TOKS32 = 32 / R;                   // tokens per 32-row tile
    static constexpr int NTHR = NW * 64, TPW = NTB / NW;
    static constexpr int NKK = N / 32;                      // K-steps over N (16x16x32)
    static constexpr int NPT = P / 16;                      // 16-column tiles of P
    static constexpr int NUT = (N / UT) * (P / UT), UPW = NUT / NW;
    static constexpr int UR_ = (UT == 32) ? 16 : 4;         // state registers per tile
    static constexpr int NS = N + 8, PS = P + 8;            // padded bf16 row strides
    static constexpr bool PFC = TPW <= 2;                   // prefetch the next chunk's C rows
    // angle prefix: wave w owns angles [w KW, (w+1) KW); lane = (angle pair, token group)
    static constexpr int KW = K / NW, KP = KW / 2, TG = 64 / KP, TPL = Q / TG;
    static_assert(K % NW == 0 && KW % 2 == 0 && 64 % KP == 0 && Q % TG == 0, "angle prefix split");
    static_assert(N % 32 == 0 && P % 32 == 0 && (R == 1 || R == 2 || R == 4) && QR % 32 == 0, "shape");
    // t-blocks exist only with outputs (a state-only scan may have fewer 16-row blocks than waves)
    static_assert(!YO || (NTB % NW == 0 && (TPW == 1 || TPW % 2 == 0)), "t-block split");
    static_assert(NUT % NW == 0 && (UT == 16 || UT == 32), "state tile split");
    static_assert(K % 8 == 0 && Q % NW == 0 && Q <= 128 && Q < NTHR, "prologue");
    static_assert(SBR % 32 == 0 && QR % SBR == 0, "s-block size");
    static_assert(NSB == 1 || NSB % 2 == 0, "full chunks alternate the two prefetch register sets");
    static_assert(NTHR % (N / 8) == 0 && N / 8 <= 64, "a staged B row is N/8 consecutive lanes of one wave");
    // LDS layout (bytes)
    static constexpr int YPS = EPI ? P + 4 : PS;                       // output staging row stride (elements)
    static constexpr int YST = 16 * YPS * (EPI ? 4 : 2);               // per-wave output staging (fp32 with EPI)
    // with EPI the output staging shares the angle table's bytes (the table is dead from the end of
    // the sweep to the next chunk's prologue); otherwise it has a region of its own
    static constexpr int REG0 = EPI ? ((Q * K * 4 > NW * YST) ? Q * K * 4 : NW * YST) : Q * K * 4;
    static constexpr int OFF_PHI = 0;                                  // bf16x2 / f16x2 [Q][K] (cos, sin) of Phi
    static constexpr int OFF_PHC = REG0;                               // float2 [K] (cos, sin) of the chunk's total angle
    static constexpr int OFF_S2 = OFF_PHC + K * 8;                     // float [Q] log2 decay prefix
    static constexpr int OFF_A2 = OFF_S2 + Q * 4;                      // float [Q] per-token log2 decay
    static constexpr int OFF_GM = OFF_A2 + Q * 4;                      // float [Q] gamma
    static constexpr int OFF_DL = OFF_GM + Q * 4;                      // float [Q] delta
    static constexpr int OFF_G1 = OFF_DL + Q * 4;                      // float [Q] gamma_s + delta_{s+1}
    static constexpr int OFF_WU = OFF_G1 + Q * 4;                      // float [Q] chunk-state weights
    static constexpr int OFF_F1 = OFF_WU + Q * 4;                      // float [Q] column mask factors, s < t
    static constexpr int OFF_F0 = OFF_F1 + Q * 4;                      // float [Q] column mask factors, s = t
    static constexpr int OFF_DT = OFF_F0 + Q * 4;                      // float [Q] dt (0 past the end)
    static constexpr int OFF_MISC = OFF_DT + Q * 4;                    // float [4]
    static constexpr int OFF_BIA = (OFF_MISC + 16 + 15) / 16 * 16;     // float [2][N] B, C bias rows (EPI)
    static constexpr int OFF_HB = OFF_BIA + (EPI ? 2 * N * 4 : 0);     // bf16 [P][NS] carried state
    static constexpr int OFF_U = OFF_HB + P * NS * 2;                  // stage buffers / output staging
    static constexpr int SB_BT = 0, SB_X = SBR * NS * 2, SB_WX = SB_X + SBR * PS * 2;
    static constexpr int STAGE = SB_WX + SBR * PS * 2;                 // one s-block stage
    static constexpr int OFF_Y = EPI ? 0 : OFF_U + NST * STAGE;        // per-wave output staging
    static constexpr int LDS = EPI ? OFF_U + NST * STAGE : OFF_Y + NW * YST;
    static_assert(LDS <= 160 * 1024, "LDS");
    // global loads (16 bytes each) per s-block, and next-chunk header prefetch
    static constexpr int BCH = SBR * N / 8, XCH = SBR * P / 8;
    static constexpr int NLB = (BCH + NTHR - 1) / NTHR, NLX = (XCH + NTHR - 1) / NTHR;
};

template <class CF>
__global__ __launch_bounds__(CF::NTHR) __attribute__((amdgpu_waves_per_eu(2))) void k_scan_bf16(BfParams pr) {
    constexpr int N = CF::N, P = CF::P, R = CF::R, Q = CF::Q, NW = CF::NW, K = CF::K, UT = CF::UT;
    constexpr int TOKT = CF::TOKT, TOKS = CF::TOKS, TOKS32 = CF::TOKS32, NTHR = CF::NTHR, TPW = CF::TPW;
    constexpr int NKK = CF::NKK, NPT = CF::NPT, UPW = CF::UPW, NS = CF::NS, PS = CF::PS, UR_ = CF::UR_;
    constexpr int TPA = TPW > 0 ? TPW : 1;   // extent of per-t-block arrays (a state-only scan may have none)
    using UAcc = std::conditional_t<UT == 32, f32x16, f32x4>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // (cos, sin) table of the chunk's angles: bf16 pairs for the dot-product rotation of raw rows,
    // fp16 pairs with the fused prologue (whose rows are fp32 when rotated)
    using TabEl = std::conditional_t<CF::EPI, _Float16, bf16>;
    using Tab2 = std::conditional_t<CF::EPI, f16x2, bf16x2>;
    using Tab4 = std::conditional_t<CF::EPI, f16x4, bf16x4>;
    using Tab8 = std::conditional_t<CF::EPI, f16x8, bf16x8>;
    Tab2 *cstw = (Tab2 *)(smem + CF::OFF_PHI);
    const Tab2 *cst = cstw;
    float2 *PHC = (float2 *)(smem + CF::OFF_PHC);
    float *S2 = (float *)(smem + CF::OFF_S2);
    float *A2 = (float *)(smem + CF::OFF_A2);
    float *GM = (float *)(smem + CF::OFF_GM);
    float *DL = (float *)(smem + CF::OFF_DL);
    float *G1 = (float *)(smem + CF::OFF_G1);
    float *WU = (float *)(smem + CF::OFF_WU);
    float *F1 = (float *)(smem + CF::OFF_F1);
    float *F0 = (float *)(smem + CF::OFF_F0);
    float *DT = (float *)(smem + CF::OFF_DT);
    float *MISC = (float *)(smem + CF::OFF_MISC);
    bf16 *HB = (bf16 *)(smem + CF::OFF_HB);
    char *UR = smem + CF::OFF_U;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps per-wave branches scalar
    const int l16 = lane & 15, q4 = lane >> 4, l32 = lane & 31, hi = lane >> 5;
    const int H = pr.H, G = pr.G;
    const int h = blockIdx.x % H, g = h / (H / G);
    // Packed batches of at most 64 sequences run longest first: workgroup rank r = blockIdx / H
    // takes the sequence of rank r by length (ties by index), so the longest sequences start in
    // the first wave of workgroups and the short ones fill in behind them. Every wave ranks the
    // lengths itself (one lane per sequence).
    int s = blockIdx.x / H;
    if (pr.cu && pr.nseq <= 64) {
        const int ns = pr.nseq, i = lane;
        int li = -1;
        if (i < ns) {
            const int a0 = min(max(pr.cu[i], 0), pr.seqlen), a1 = min(max(pr.cu[i + 1], a0), pr.seqlen);
            li = a1 - a0;
        }
        int rank = 0;
        for (int j = 0; j < ns; j++) {
            const int lj = __builtin_amdgcn_readlane(li, j);
            rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        const unsigned long long hit = __ballot(i < ns && rank == s);
        s = __builtin_amdgcn_readfirstlane((int)__ffsll((long long)hit) - 1);
    }

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
    const float A2h = (CF::EPI ? (pr.A ? pr.A[h] : 0.f) : pr.A[h]) * kLog2e;
    // the trapezoid weight of a loaded lam value (the fixed one when there is no lam array)
    auto lamv = [&](bf16 raw) { return (CF::EPI && !pr.lam_on) ? pr.lam_fixed : to_f(raw); };
    // log2 decay rate of a token whose loaded A_t is raw (the head's without per-token A)
    auto a2v = [&](bf16 raw) { return (CF::EPI && pr.atok_on) ? to_f(raw) * kLog2e : A2h; };
    const float Dh = pr.D ? pr.D[h] : 0.f;
    // per-(sequence, head) base pointers: add token * stride (+ rank * N or P)
    const bf16 *gB = pr.B + g * (int64_t)R * N;
    const bf16 *gC = pr.C + g * (int64_t)R * N;
    const bf16 *gX = pr.x + h * (int64_t)R * P;
    bf16 *gY = pr.y + h * (int64_t)R * P;
    const bf16 *gTh = pr.theta + (h / (H / pr.Gth)) * (int64_t)K;
    const int64_t strBC = (int64_t)G * R * N, strX = (int64_t)H * R * P, strTh = (int64_t)pr.Gth * K;
    // prologue bias rows of the head (zeros for an absent bias): [0, N) for B, [N, 2N) for C
    float *BIA = (float *)(smem + CF::OFF_BIA);
    if constexpr (CF::EPI) {
        for (int e = tid; e < 2 * N; e += NTHR) {
            const float *src = (e < N) ? pr.Bb : pr.Cb;
            BIA[e] = src ? src[(int64_t)h * N + e % N] : 0.f;
        }
    }

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
            const float dt0 = to_f(pr.dt[start * H + h]), l0 = lamv(pr.lam[start * H + h]);
            d0 = (1.f - l0) * dt0;
        }
        // prologue of Bprev's columns: inverse RMS per column (every wave computes its own)
        float invp[R];
#pragma unroll
        for (int j = 0; j < R; j++) invp[j] = 1.f;
        if constexpr (CF::EPI) {
            if (pr.Bprev && pr.norm) {
                const bf16 *bp0 = pr.Bprev + ((int64_t)s * G + g) * R * N;
#pragma unroll
                for (int j = 0; j < R; j++) {
                    float ss = 0.f;
                    for (int n = lane; n < N; n += 64) ss += to_f(bp0[j * N + n]) * to_f(bp0[j * N + n]);
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off, 64);
                    invp[j] = rsqrtf(ss * (1.f / N) + pr.eps);
                }
            }
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
                    const float bb = (CF::EPI && pr.Bb) ? pr.Bb[(int64_t)h * N + n] : 0.f;
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < R; j++) acc += (to_f(bp[j * N]) * invp[j] + bb) * to_f(xp[j * P]);
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
    bf16 h_dt = {}, h_lam = {};     // token tid of the chunk (tid < Q)
    bf16 h_A = {};                  // its decay rate A_t (per-token variant)
    bf16 h_dtn = {}, h_lamn = {};   // the token after the chunk (same for every thread)
    bf16x2 h_th2[CF::TPL];          // theta of the lane's angle pair for its TPL tokens
    bf16x8 h_c[TPA][NKK];
    // C rows of the own t-blocks in operand layout: row 16 tb + l16, columns 32 kk + 8 q4 ..
    // tq: the thread index the address math uses (tid, or an opaque copy inside the chunk loop)
    // Addressing: a chunk's loads are a wave-uniform base (the chunk's first token) plus a 32-bit
    // per-lane byte offset (chunk-local token indices stay below Q), clamped to the sequence's last
    // token; lanes hold 32-bit offsets, not 64-bit addresses.
    auto ltok = [&](int64_t c0c, int tau) { return (uint32_t)min(tau, (int)min((int64_t)Q, len - c0c - 1)); };
    auto load_crows = [&](int64_t c0h, int tq) {
        const int64_t c0c = c0h < len ? c0h : 0;
        const bf16 *bC = gC + (start + c0c) * strBC;
        const int l16q = tq & 15, q4q = (tq & 63) >> 4;
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int row = tb_of(u, c0h) * 16 + l16q;
            const uint32_t o = ltok(c0c, row / R) * (uint32_t)strBC + (uint32_t)((row % R) * N + 8 * q4q);
#pragma unroll
            for (int kk = 0; kk < NKK; kk++) h_c[u][kk] = ld_off<bf16x8>(bC, (o + 32 * kk) * 2u);
        }
    };
    auto load_header = [&](int64_t c0h, int tq) {
        const int64_t c0c = c0h < len ? c0h : 0;
        const int nqh = (int)min((int64_t)Q, len - c0c);
        {
            const int64_t b = (start + c0c) * H + h;
            const uint32_t tk = ltok(c0c, min(tq, Q - 1)) * (uint32_t)H * 2u, tn = ltok(c0c, nqh) * (uint32_t)H * 2u;
            h_dt = ld_off<bf16>(pr.dt + b, tk);
            h_lam = ld_off<bf16>(pr.lam + b, tk);
            if constexpr (CF::EPI) h_A = ld_off<bf16>(pr.Atk + b, tk);
            h_dtn = ld_off<bf16>(pr.dt + b, tn);
            h_lamn = ld_off<bf16>(pr.lam + b, tn);
        }
        {
            const int lq = tq & 63;
            const int k = wave * CF::KW + 2 * (lq % CF::KP), g0 = (lq / CF::KP) * CF::TPL;
            const bf16 *bth = gTh + (start + c0c) * strTh;
#pragma unroll
            for (int j = 0; j < CF::TPL; j++)
                h_th2[j] = ld_off<bf16x2>(bth, (ltok(c0c, g0 + j) * (uint32_t)strTh + (uint32_t)k) * 2u);
        }
        if constexpr (CF::PFC && CF::YO) load_crows(c0h, tq);
    };

    // ---- s-block stream: block j of the sequence lives in register set j % 2
    bf16x8 rb0[CF::NLB], rx0[CF::NLX], rb1[CF::NLB], rx1[CF::NLX];
    auto load_block_into = [&](bf16x8 (&rb)[CF::NLB], bf16x8 (&rx)[CF::NLX], int64_t c0b, int sb, int tq) {
        const int64_t c0c = c0b < len ? c0b : 0;                   // past the end: dummy loads, never used
        const bf16 *bB = gB + (start + c0c) * strBC, *bX = gX + (start + c0c) * strX;
#pragma unroll
        for (int i = 0; i < CF::NLB; i++) {
            const int c = (tq + i * NTHR) % CF::BCH;
            const int row = c / (N / 8), col = (c % (N / 8)) * 8;
            const int tau = sb * TOKS + row / R;
            rb[i] = ld_off<bf16x8>(bB, (ltok(c0c, tau) * (uint32_t)strBC + (uint32_t)((row % R) * N + col)) * 2u);
        }
#pragma unroll
        for (int i = 0; i < CF::NLX; i++) {
            const int c = (tq + i * NTHR) % CF::XCH;
            const int row = c / (P / 8), col = (c % (P / 8)) * 8;
            const int tau = sb * TOKS + row / R;
            rx[i] = ld_off<bf16x8>(bX, (ltok(c0c, tau) * (uint32_t)strX + (uint32_t)((row % R) * P + col)) * 2u);
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
        load_header(0, tid);
        load_block_into(rb0, rx0, ld_c0, ld_sb, tid);
        advance(ld_c0, ld_sb);
        if constexpr (CF::NST == 2) {
            load_block_into(rb1, rx1, ld_c0, ld_sb, tid);
            advance(ld_c0, ld_sb);
        }
    }
    __syncthreads();

    // state-only scans: running sums over the chunks of the log2 decay (thread 0) and of the
    // angles of the lane's pair (lanes of the last token group)
    float sum_s2 = 0.f, sum_ph0 = 0.f, sum_ph1 = 0.f;

    // One chunk. Full chunks (Q tokens) have a compile-time number of s-blocks
    // (NSB, even), so block j of the sequence always sits in register set j % 2
    // and the sweep is fully unrolled; the final partial chunk runs the same
    // steps under a runtime bound.
    auto chunk_body = [&](auto FULLC, int64_t c0) {
        constexpr bool FULL = decltype(FULLC)::value;
        const int nq = FULL ? Q : (int)(len - c0);
        // with the fused prologue / epilogue, and at N = 128, R = 4, the registers run short: the
        // lane-derived address math of the prefetch, staging and output code is recomputed in
        // every chunk (for the other plain shapes hoisting it is faster)
        // (the plain kernels also re-mask it to its range, for cheaper address math; in the fused
        // ones that let the compiler hold more derived values, and they spilled)
        const int tq = CF::EPI ? opaque<true>(tid) : (opaque<(CF::N == 128 && CF::R == 4)>(tid) & (NTHR - 1));
        const int64_t tok0 = start + c0;
        if constexpr (!CF::YO) {
            // the state entering the chunk, with the previous-token term of its first token
            // (folded into the previous chunk's last weight, or added from Bprev for chunk 0)
            if (pr.ws_state) {   // registers 4j .. 4j + 3 hold four consecutive rows: one 8-byte piece
                bf16 *wsc = pr.ws_state + ((s * (((int64_t)pr.seqlen + Q - 1) / Q) + c0 / Q) * H + h) * (int64_t)N * P;
#pragma unroll
                for (int v = 0; v < UPW; v++)
#pragma unroll
                    for (int r = 0; r < UR_; r += 4)
                        *(bf16x4 *)(wsc + (ut_p0[v] + ucol) * N + ut_n0[v] + urow(r)) =
                            bf16x4{(bf16)hreg[v][r], (bf16)hreg[v][r + 1], (bf16)hreg[v][r + 2], (bf16)hreg[v][r + 3]};
            }
        }
        int task_tb[TPA];
#pragma unroll
        for (int u = 0; u < TPW; u++) task_tb[u] = tb_of(u, c0);

        // ---- prologue 1: per-token scalars. With Q <= 64 wave 0 holds every token of the chunk
        // and builds the log2-decay prefix and the weight tables in registers.
        if constexpr (Q <= 64) {
            if (wave == 0) {
                const int t = lane;
                const bool ok = (FULL || t < nq) && t < Q;
                const float dt = ok ? to_f(h_dt) : 0.f, lm = ok ? lamv(h_lam) : 0.f;
                const float gm = lm * dt, dl = (1.f - lm) * dt;
                const float s2 = wave_incl_scan(dt * a2v(h_A), lane);
                const float s2e = wave_bcast(s2, nq - 1);
                const float dn = (c0 + nq < len) ? (1.f - lamv(h_lamn)) * to_f(h_dtn) : 0.f;
                const float dl1 = __shfl_down(dl, 1, 64);
                const float g1 = gm + ((t + 1 < nq) ? dl1 : ((t + 1 == nq) ? dn : 0.f));
                // mask factor relative to the first token of t's 32-row tile (>= 1)
                const float f = __builtin_amdgcn_exp2f(__shfl(s2, (t / TOKS32) * TOKS32, 64) - s2);
                const float s2first = wave_bcast(s2, 0), s2last = wave_bcast(s2, Q - 1);
                if (t < Q) {
                    DT[t] = dt;
                    S2[t] = s2;
                    GM[t] = gm;
                    G1[t] = g1;
                    WU[t] = (t < nq) ? exp2_neg(s2e - s2) * g1 : 0.f;
                    F1[t] = f * g1;
                    F0[t] = f * gm;
                }
                if (lane == 0) {
                    MISC[1] = s2e;
                    // the factored mask is used when every factor stays far inside the fp32 range
                    MISC[2] = (s2first - s2last <= 120.f) ? 1.f : 0.f;
                }
            }
        } else {
            if (tid < Q) {
                const bool ok = FULL || tid < nq;
                const float dt = ok ? to_f(h_dt) : 0.f, lm = ok ? lamv(h_lam) : 0.f;
                DT[tid] = dt;
                A2[tid] = dt * a2v(h_A);
                GM[tid] = lm * dt;
                DL[tid] = (1.f - lm) * dt;
            }
            if (tid == 0) MISC[0] = (c0 + nq < len) ? (1.f - lamv(h_lamn)) * to_f(h_dtn) : 0.f;
        }
        __syncthreads();

        // ---- prologue 2: cumulative angles of the wave's angle pairs over the chunk, as a
        // (cos, sin) table; with Q > 64 wave 0 also builds the log2-decay prefix here
        if constexpr (Q > 64) {
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
                        const float f = __builtin_amdgcn_exp2f(S2[(t / TOKS32) * TOKS32] - S2[t]);
                        F1[t] = f * g1;
                        F0[t] = f * GM[t];
                    }
                }
                if (lane == 0) {
                    MISC[1] = S2e;
                    MISC[2] = (S2[0] - S2[Q - 1] <= 120.f) ? 1.f : 0.f;
                }
            }
        }
        {
            constexpr int KP = CF::KP, TPL = CF::TPL;
            const int k = wave * CF::KW + 2 * (lane % KP), g0 = (lane / KP) * TPL;
            float a0[TPL], a1[TPL];
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int j = 0; j < TPL; j++) {
                const float dt = DT[g0 + j];   // 0 past the end: the angle stays put
                r0 += dt * (float)h_th2[j][0];
                r1 += dt * (float)h_th2[j][1];
                a0[j] = r0;
                a1[j] = r1;
            }
            // exclusive prefix of the token groups' sums across the lanes holding the same pair
            float e0 = r0, e1 = r1;
#pragma unroll
            for (int off = KP; off < 64; off <<= 1) {
                const float o0 = __shfl_up(e0, off, 64), o1 = __shfl_up(e1, off, 64);
                if (lane >= off) {
                    e0 += o0;
                    e1 += o1;
                }
            }
            e0 -= r0;
            e1 -= r1;
#pragma unroll
            for (int j = 0; j < TPL; j++) {
                const int tau = g0 + j;
                const float x0 = a0[j] + e0, x1 = a1[j] + e1;
                float s0, c0v, s1, c1v;
                __sincosf(x0, &s0, &c0v);
                __sincosf(x1, &s1, &c1v);
                *(Tab4 *)(cstw + tau * K + k) = Tab4{(TabEl)c0v, (TabEl)s0, (TabEl)c1v, (TabEl)s1};
                if (tau == Q - 1) {   // angles past the end are zero: Phi[Q-1] = Phi[nq-1]
                    if constexpr (!CF::YO) {
                        sum_ph0 += x0;
                        sum_ph1 += x1;
                    }
                    sincos_state(x0, &s0, &c0v);
                    sincos_state(x1, &s1, &c1v);
                    *(f32x4 *)(PHC + k) = f32x4{c0v, s0, c1v, s1};
                }
            }
        }
        __syncthreads();

        if constexpr (!CF::YO) {
            if (tid == 0) sum_s2 += MISC[1];
        }

        // ---- rotated C~ rows of this wave's t-blocks, from the prefetched (or just loaded) raw rows
        bf16x8 creg[TPA][NKK];
        f32x4 yacc[TPA][NPT];
        if constexpr (CF::YO) {
        if constexpr (!CF::PFC) load_crows(c0, tq);
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int tau = (task_tb[u] * 16 + l16) / R;
            // prologue: the row's N values sit in lanes l16 + 16 q4, NKK pieces each
            float cinv = 1.f;
            if constexpr (CF::EPI) {
                if (pr.norm) {
                    float ss = 0.f;
#pragma unroll
                    for (int kk = 0; kk < NKK; kk++) ss += sumsq8(h_c[u][kk]);
                    ss = sum_across_rows(ss);   // the row's 4 lanes l16 + 16 q4
                    cinv = rsqrtf(ss * (1.f / N) + pr.eps);
                }
            }
#pragma unroll
            for (int kk = 0; kk < NKK; kk++) {
                const Tab8 cs = *(const Tab8 *)(cst + tau * K + 16 * kk + 4 * q4);
                bf16x8 o;
                if constexpr (CF::EPI) {
                    float in[8], of[8];
                    prologue_piece(h_c[u][kk], cinv, BIA + N + 32 * kk + 8 * q4, in);
                    rot_piece_f(in, cs, of);
                    o = pack8(of);
                } else {
                    o = rot_pack_bf(h_c[u][kk], cs);
                }
                creg[u][kk] = (FULL || tau < nq) ? o : bf16x8{};
            }
        }

        // ---- inter-chunk term: Y = e^{S_t} C~ H'   (H' bf16 in LDS, [p][n])
        // each H' operand is read once and used for every t-block of the wave
#pragma unroll
        for (int pt = 0; pt < NPT; pt++) {
            const int p = pt * 16 + l16;
#pragma unroll
            for (int u = 0; u < TPW; u++) yacc[u][pt] = f32x4{};
#pragma unroll
            for (int kk = 0; kk < NKK; kk++) {
                const bf16x8 hop = *(const bf16x8 *)(HB + p * NS + 32 * kk + 8 * q4);
#pragma unroll
                for (int u = 0; u < TPW; u++) yacc[u][pt] = mfma16(creg[u][kk], hop, yacc[u][pt]);
            }
        }
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; i++) sc[i] = exp2_neg(S2[(task_tb[u] * 16 + 4 * q4 + i) / R]);
#pragma unroll
            for (int pt = 0; pt < NPT; pt++)
#pragma unroll
                for (int i = 0; i < 4; i++) yacc[u][pt][i] *= sc[i];
        }
        }   // CF::YO
        {
            const float eS = exp2_neg(MISC[1]);
#pragma unroll
            for (int v = 0; v < UPW; v++)
#pragma unroll
                for (int r = 0; r < UR_; r++) hreg[v][r] *= eS;
        }
        // the header registers are consumed: prefetch the next chunk's header now
        load_header(c0 + Q, tq);

        // ---- s-block sweep
        // lane coordinates made opaque per chunk: the mask indices derived from them are
        // recomputed in every chunk instead of being hoisted out of the chunk loop (and spilled)
        unsigned l16c = l16, q4c = q4;
        if constexpr (CF::NSB <= 8) asm volatile("" : "+v"(l16c), "+v"(q4c));   // fully unrolled sweeps
        if constexpr (!CF::EPI) {   // (their ranges, for the index math; see tq above)
            l16c &= 15;
            q4c &= 3;
        }
        const bool fastmask = __builtin_amdgcn_readfirstlane(__float_as_int(MISC[2])) != 0;
        float S2t[TPA];
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
            Tab8 csb[CF::NLB];
            float wxv[CF::NLX];
#pragma unroll
            for (int i = 0; i < CF::NLB; i++) {
                const int c = min(tq + i * NTHR, CF::BCH - 1);
                csb[i] = *(const Tab8 *)(cst + (sb * TOKS + (c / (N / 8)) / R) * K + (c % (N / 8)) * 4);
            }
#pragma unroll
            for (int i = 0; i < CF::NLX; i++) {
                const int c = min(tq + i * NTHR, CF::XCH - 1);
                wxv[i] = WU[sb * TOKS + (c / (P / 8)) / R];
            }
            // prologue: a row's pieces are N/8 consecutive lanes, and every piece of this thread
            // covers the same columns (NTHR is a multiple of N/8), so one bias slice serves all
            float binv[CF::NLB];
            const float *bslice = BIA + (tq % (N / 8)) * 8;
#pragma unroll
            for (int i = 0; i < CF::NLB; i++) binv[i] = 1.f;
            if constexpr (CF::EPI) {
                if (pr.norm) {
#pragma unroll
                    for (int i = 0; i < CF::NLB; i++) {
                        // the row's N / 8 lanes are one aligned group of 8 or 16: sums by DPP lane
                        // moves (quad swaps, then the half-row and row mirrors)
                        static_assert(N / 8 == 8 || N / 8 == 16, "a B row's lanes form a DPP row or half");
                        float ss = sumsq8(rawB[i]);
                        ss += dpp_move<0xB1>(ss);   // quad_perm [1, 0, 3, 2]
                        ss += dpp_move<0x4E>(ss);   // quad_perm [2, 3, 0, 1]
                        ss += dpp_move<0x141>(ss);  // row_half_mirror
                        if constexpr (N / 8 == 16) ss += dpp_move<0x140>(ss);   // row_mirror
                        binv[i] = rsqrtf(ss * (1.f / N) + pr.eps);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < CF::NLB; i++) {
                const int c = tq + i * NTHR;
                if (c < CF::BCH) {
                    const int row = c / (N / 8), col = (c % (N / 8)) * 8;
                    const int tau = sb * TOKS + row / R;
                    bf16x8 o;
                    if constexpr (CF::EPI) {
                        float in[8], of[8];
                        prologue_piece(rawB[i], binv[i], bslice, in);
                        rot_piece_f(in, csb[i], of);
                        o = pack8(of);
                    } else {
                        o = rot_pack_bf(rawB[i], csb[i]);
                    }
                    *(bf16x8 *)(bt + row * NS + col) = (FULL || tau < nq) ? o : bf16x8{};
                }
            }
#pragma unroll
            for (int i = 0; i < CF::NLX; i++) {
                const int c = tq + i * NTHR;
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
            const char *stg = UR + ((CF::NST == 1) ? 0 : (sb & 1)) * CF::STAGE;
            const bf16 *bt = (const bf16 *)(stg + CF::SB_BT);
            const bf16 *xs = (const bf16 *)(stg + CF::SB_X);
            const bf16 *wx = (const bf16 *)(stg + CF::SB_WX);
            // Per 32-row tile, t-blocks in groups of (up to) two: the group's t-blocks that reach
            // the tile share its B~ and X operands; the score MFMAs of both are issued before their
            // masks, and the masks before the output MFMAs, so their dependent chains overlap.
            constexpr int UG = TPW < 2 ? TPA : 2;
#pragma unroll
            for (int ug = 0; ug < (CF::YO ? TPW : 0); ug += UG)
#pragma unroll
            for (int j = 0; j < CF::NSUB; j++) {
                const int sbj = sb * CF::NSUB + j;              // 32-row tile of the chunk
                if (!FULL && 32 * sbj >= nq * R) continue;      // tile past the end of the sequence
                bool act[UG], up[UG];
                bool any = false, anyup = false, anydiag = false;
#pragma unroll
                for (int u = 0; u < UG; u++) {
                    act[u] = 2 * sbj <= task_tb[ug + u];        // t-block reaches this tile
                    up[u] = 2 * sbj + 1 <= task_tb[ug + u];     // second 16-row half of the tile is causal
                    any |= act[u];
                    anyup |= up[u];
                    anydiag |= act[u] && task_tb[ug + u] < 2 * sbj + 2;
                }
                if (!any) continue;
                const int rb = 32 * j;                          // first row of the tile in the stage
                f32x4 g0[UG], g1[UG];
#pragma unroll
                for (int u = 0; u < UG; u++) g0[u] = g1[u] = f32x4{};
#pragma unroll
                for (int kk = 0; kk < NKK; kk++) {
                    const bf16x8 b0 = *(const bf16x8 *)(bt + (rb + l16) * NS + 32 * kk + 8 * q4);
#pragma unroll
                    for (int u = 0; u < UG; u++)
                        if (act[u]) g0[u] = mfma16(b0, creg[ug + u][kk], g0[u]);
                    if (anyup) {
                        const bf16x8 b1 = *(const bf16x8 *)(bt + (rb + 16 + l16) * NS + 32 * kk + 8 * q4);
#pragma unroll
                        for (int u = 0; u < UG; u++)
                            if (up[u]) g1[u] = mfma16(b1, creg[ug + u][kk], g1[u]);
                    }
                }
                // decay/trapezoid mask: column (t, i) = lane's t-row, rows (s, j) of the two halves.
                // Row 16 h + 4 q4 + i of the tile (e = 4 h + i) is token tok_h + i / R.
                const unsigned tok0 = ((unsigned)(sbj * 32) + 4 * q4c) / R, tok1 = tok0 + 16 / R;
                auto sidx = [&](int e) { return (int)(((e < 4) ? tok0 : tok1) + (unsigned)(e % 4) / R); };
                // the distinct per-token values of a tabulated column array for the 8 rows
                auto col8 = [&](const float *tab, float (&o)[8]) {
                    if constexpr (R == 1) {
                        const f32x4 a = *(const f32x4 *)(tab + tok0), b = *(const f32x4 *)(tab + tok1);
#pragma unroll
                        for (int e = 0; e < 4; e++) { o[e] = a[e]; o[e + 4] = b[e]; }
                    } else if constexpr (R == 2) {
                        const float2 a = *(const float2 *)(tab + tok0), b = *(const float2 *)(tab + tok1);
                        o[0] = o[1] = a.x; o[2] = o[3] = a.y; o[4] = o[5] = b.x; o[6] = o[7] = b.y;
                    } else {
                        const float a = tab[tok0], b = tab[tok1];
#pragma unroll
                        for (int e = 0; e < 4; e++) { o[e] = a; o[e + 4] = b; }
                    }
                };
                bf16x8 mop[UG];
                if (fastmask) {
                    // e^{S_t - S_s} w_s = 2^{S2_t - S2_ref} * (2^{S2_ref - S2_s} w_s), ref = first
                    // token of the tile; the second factor is tabulated per chunk
                    const float s2ref = S2[sbj * TOKS32];
                    float fc[8], f0[8];
                    col8(F1, fc);
                    if (anydiag) col8(F0, f0);
#pragma unroll
                    for (int u = 0; u < UG; u++) {
                        if (!act[u]) continue;
                        const int tb = task_tb[ug + u];
                        const float rf = exp2_neg(S2t[ug + u] - s2ref);
                        if (tb >= 2 * sbj + 2) {                // every s of the tile precedes every t
#pragma unroll
                            for (int e = 0; e < 8; e++)
                                mop[u][e] = (bf16)(rf * fc[e] * ((e < 4) ? g0[u][e] : g1[u][e - 4]));
                        } else {
                            const int tt = (int)((unsigned)(tb * 16) + l16c) / R;
#pragma unroll
                            for (int e = 0; e < 8; e++) {
                                // masks as 0/1 factors rather than selects of loaded values, which
                                // the compiler would turn into branches around the loads
                                const int ss = sidx(e);
                                const float m1 = (ss < tt) ? 1.f : 0.f, m0 = (ss == tt) ? 1.f : 0.f;
                                float coef = fc[e] * m1 + f0[e] * m0;
                                if (!(e < 4 || up[u])) coef = 0.f;
                                mop[u][e] = (bf16)(rf * coef * ((e < 4) ? g0[u][e] : g1[u][e - 4]));
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < UG; u++) {
                        if (!act[u]) continue;
                        const int tt = (int)((unsigned)(task_tb[ug + u] * 16) + l16c) / R;
                        const float S2tt = S2[tt];
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            const int ss = sidx(e);
                            const float m1 = (ss < tt) ? 1.f : 0.f, m0 = (ss == tt) ? 1.f : 0.f;
                            float coef = exp2_neg(fminf(S2tt - S2[ss], 0.f)) * (G1[ss] * m1 + GM[ss] * m0);
                            if (!(e < 4 || up[u])) coef = 0.f;
                            mop[u][e] = (bf16)(coef * ((e < 4) ? g0[u][e] : g1[u][e - 4]));
                        }
                    }
                }
#pragma unroll
                for (int pt = 0; pt < NPT; pt++) {
                    // X rows 4 q4 .. and 16 + 4 q4 .. of column 16 pt + l16 (K permuted like mop)
                    const bf16x8 xop = tr_operand(xs, PS, rb + 4 * q4, rb + 16 + 4 * q4, pt * 16, l16);
#pragma unroll
                    for (int u = 0; u < UG; u++)
                        if (act[u]) yacc[ug + u][pt] = mfma16(mop[u], xop, yacc[ug + u][pt]);
                }
                // skip term D x_t of the t-block's own rows (one-stage shapes add it after the sweep)
                if constexpr (CF::NST == 2) {
#pragma unroll
                    for (int u = 0; u < UG; u++) {
                        const int dblk = task_tb[ug + u] - 2 * sbj;   // 0/1: the t-block's rows are in this tile
                        if (dblk != 0 && dblk != 1) continue;
#pragma unroll
                        for (int pt = 0; pt < NPT; pt++) {
                            const bf16x4 xv =
                                ds_read_tr(xs + (rb + 16 * dblk + 4 * q4 + l16 / 4) * PS + pt * 16 + 4 * (l16 % 4));
#pragma unroll
                            for (int i = 0; i < 4; i++) yacc[ug + u][pt][i] += Dh * (float)xv[i];
                        }
                    }
                }
            }
            // chunk-state update on the owned state tiles: H += B~^T (wU X), K = the s-block's rows
#pragma unroll
            for (int j = 0; j < CF::NSUB; j++) {
                if (!FULL && 32 * (sb * CF::NSUB + j) >= nq * R) continue;
                const int rb = 32 * j;
#pragma unroll
                for (int v = 0; v < UPW; v++) {
                    if constexpr (UT == 32) {
                        // lane groups: column half c0 = 16 (group % 2), K rows 8 (group / 2) ..
                        const int grp = lane >> 4;
                        const int cn = ut_n0[v] + 16 * (grp & 1), cp = ut_p0[v] + 16 * (grp & 1);
#pragma unroll
                        for (int ks = 0; ks < 2; ks++) {
                            const int r0 = rb + 16 * ks + 8 * (grp >> 1);
                            hreg[v] = mfma32(tr_operand(bt, NS, r0, r0 + 4, cn, l16),
                                             tr_operand(wx, PS, r0, r0 + 4, cp, l16), hreg[v]);
                        }
                    } else {
                        hreg[v] = mfma16(tr_operand(bt, NS, rb + 8 * q4, rb + 8 * q4 + 4, ut_n0[v], l16),
                                         tr_operand(wx, PS, rb + 8 * q4, rb + 8 * q4 + 4, ut_p0[v], l16), hreg[v]);
                    }
                }
            }
        };

        // block sb of this chunk: set sb % 2 receives block sb + 2 of the stream, then the
        // block is computed and block sb + 1 is staged from the other set
        auto step = [&](auto SETC, int sb) {
            constexpr int ST = decltype(SETC)::value;
            if constexpr (ST == 0) load_block_into(rb0, rx0, ld_c0, ld_sb, tq);
            else load_block_into(rb1, rx1, ld_c0, ld_sb, tq);
            advance(ld_c0, ld_sb);
            compute_block(sb);
            if (sb + 1 < nbs) {
                if constexpr (ST == 0) store_block(rb1, rx1, sb + 1, (sb + 1) & 1);
                else store_block(rb0, rx0, sb + 1, (sb + 1) & 1);
            }
            __syncthreads();
        };
        if constexpr (CF::NST == 1) {
            // the whole chunk is one s-block: stage it, then reuse the register set for the
            // next chunk's block while this one is computed
            store_block(rb0, rx0, 0, 0);
            load_block_into(rb0, rx0, ld_c0, ld_sb, tq);
            advance(ld_c0, ld_sb);
            __syncthreads();
            compute_block(0);
            // skip term D x_t, off the MFMA chains: the stage still holds the chunk's X rows
            const bf16 *xs = (const bf16 *)(UR + CF::SB_X);
#pragma unroll
            for (int u = 0; u < (CF::YO ? TPW : 0); u++)
#pragma unroll
                for (int pt = 0; pt < NPT; pt++) {
                    const bf16x4 xv = ds_read_tr(xs + (task_tb[u] * 16 + 4 * q4 + l16 / 4) * PS + pt * 16 + 4 * (l16 % 4));
#pragma unroll
                    for (int i = 0; i < 4; i++) yacc[u][pt][i] += Dh * (float)xv[i];
                }
        } else if constexpr (FULL && CF::NSB <= 8) {
            store_block(rb0, rx0, 0, 0);
            __syncthreads();
#pragma unroll
            for (int sb = 0; sb < CF::NSB; sb += 2) {
                step(std::integral_constant<int, 0>{}, sb);
                step(std::integral_constant<int, 1>{}, sb + 1);
            }
        } else if constexpr (FULL) {
            store_block(rb0, rx0, 0, 0);
            __syncthreads();
#pragma nounroll
            for (int sb = 0; sb < CF::NSB; sb += 2) {
                step(std::integral_constant<int, 0>{}, sb);
                step(std::integral_constant<int, 1>{}, sb + 1);
            }
        } else {
            store_block(rb0, rx0, 0, 0);
            __syncthreads();
            for (int sb = 0; sb < nbs; sb += 2) {
                step(std::integral_constant<int, 0>{}, sb);
                if (sb + 1 < nbs) step(std::integral_constant<int, 1>{}, sb + 1);
            }
        }

        // ---- epilogue: outputs through a per-wave LDS transpose, 16-byte row stores
        if constexpr (!CF::YO) {
        } else if constexpr (CF::EPI) {
            // fp32 transpose, then y * SiLU(z) in fp32 and one rounding to bf16
            constexpr int NPC = 16 * P / 8 / 64;   // 16-byte pieces per lane and t-block
            static_assert((16 * P / 8) % 64 == 0, "output pieces");
            float *ysf = (float *)(smem + CF::OFF_Y + wave * CF::YST);   // [16 rows][YPS], own region
            const bool has_z = pr.z != nullptr;
            const bf16 *gZ = (has_z ? pr.z : pr.x) + h * (int64_t)R * P;
#pragma unroll
            for (int u = 0; u < TPW; u++) {
                const int tb = task_tb[u];
                bf16x8 zr[NPC];
                if (has_z) {
#pragma unroll
                    for (int k = 0; k < NPC; k++) {
                        const int c = (tq & 63) + 64 * k, row = c / (P / 8), col = (c % (P / 8)) * 8;
                        const int rr = tb * 16 + row, tau = min(rr / R, nq - 1);   // in bounds; unused past the end
                        zr[k] = ld_off<bf16x8>(gZ + tok0 * strX, ((uint32_t)tau * (uint32_t)strX + (uint32_t)((rr % R) * P + col)) * 2u);
                    }
                }
#pragma unroll
                for (int pt = 0; pt < NPT; pt++)
#pragma unroll
                    for (int i = 0; i < 4; i++) ysf[(4 * q4 + i) * CF::YPS + pt * 16 + l16] = yacc[u][pt][i];
                lds_wait();
#pragma unroll
                for (int k = 0; k < NPC; k++) {
                    const int c = (tq & 63) + 64 * k, row = c / (P / 8), col = (c % (P / 8)) * 8;
                    const int rr = tb * 16 + row, tau = rr / R;
                    const f32x4 a = *(const f32x4 *)(ysf + row * CF::YPS + col);
                    const f32x4 b = *(const f32x4 *)(ysf + row * CF::YPS + col + 4);
                    float o[8];
#pragma unroll
                    for (int e = 0; e < 8; e++) o[e] = (e < 4) ? a[e] : b[e - 4];
                    if (has_z) {
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            const float v = (float)zr[k][e];
                            o[e] *= v / (1.f + __expf(-v));
                        }
                    }
                    if (FULL || tau < nq)
                        st_off<bf16x8>(gY + tok0 * strX, ((uint32_t)tau * (uint32_t)strX + (uint32_t)((rr % R) * P + col)) * 2u, pack8(o));
                }
                lds_wait();
            }
        } else {
            bf16 *ys = (bf16 *)(smem + CF::OFF_Y + wave * CF::YST);   // [16 rows][PS], own region
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
                    if (FULL || tau < nq)
                        st_off<bf16x8>(gY + tok0 * strX, ((uint32_t)tau * (uint32_t)strX + (uint32_t)((rr % R) * P + col)) * 2u,
                                       *(const bf16x8 *)(ys + row * PS + col));
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
    if constexpr (!CF::YO) {
        if (pr.seg_sums) {
            float *o = pr.seg_sums + ((int64_t)s * H + h) * (int64_t)N * P;
            if (tid == 0) o[0] = sum_s2 / kLog2e;
            if (lane / CF::KP == CF::TG - 1) {   // the lanes holding the chunks' last token
                const int k = wave * CF::KW + 2 * (lane % CF::KP);
                o[1 + k] = sum_ph0;
                o[2 + k] = sum_ph1;
            }
        }
    }

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
mamba3_status launch_cfg(const mamba3_scan_args *a, hipStream_t st, bf16 *ws_state = nullptr,
                         float *seg_sums = nullptr) {
    BfParams p;
    p.ws_state = ws_state;
    p.seg_sums = seg_sums;
    p.x = (const bf16 *)a->x; p.dt = (const bf16 *)a->dt; p.lam = (const bf16 *)a->lam;
    p.theta = (const bf16 *)a->theta; p.B = (const bf16 *)a->B; p.C = (const bf16 *)a->C;
    p.Bprev = (const bf16 *)a->Bprev; p.xprev = (const bf16 *)a->xprev;
    p.A = a->A; p.D = a->D; p.h_in = a->h_in; p.y = (bf16 *)a->y; p.h_out = a->h_out;
    p.cu = a->cu_seqlens; p.seqlen = a->seqlen; p.H = a->nheads; p.G = a->ngroups;
    p.nseq = a->cu_seqlens ? a->nseq : a->batch;
    p.Bb = a->B_bias; p.Cb = a->C_bias; p.z = (const bf16 *)a->z; p.norm = a->bc_norm; p.eps = a->bc_eps;
    p.Atk = (const bf16 *)(a->A_tok ? a->A_tok : a->dt); p.atok_on = a->A_tok != nullptr;
    p.lam = (const bf16 *)(a->lam ? a->lam : a->dt); p.lam_on = a->lam != nullptr; p.lam_fixed = a->lam_fixed;
    p.Gth = a->theta_groups ? a->theta_groups : a->nheads;
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

// (N, P, R, Q) -> waves per workgroup, state tile size, rows per s-block
#define M3_BF16_SHAPES(X)          \
    X(128, 64, 1, 64, 4, 32, 64)   \
    X(64, 64, 4, 64, 8, 16, 256)   \
    X(128, 64, 4, 128, 8, 16, 32)  \
    X(64, 64, 1, 64, 4, 32, 64)    \
    X(64, 64, 4, 32, 8, 16, 128)   \
    X(128, 64, 2, 64, 8, 32, 128)  \
    X(128, 64, 4, 64, 8, 32, 64)

// state-only shapes at the backward's chunks (N, P, R, Q) -> waves, state tile, rows per s-block
#define M3_BF16_STATE_SHAPES(X)    \
    X(128, 64, 1, 32, 4, 32, 32)   \
    X(64, 64, 4, 16, 4, 16, 64)

bool scan_bf16_supported(int N, int P, int R, int Q) {
#define X(n, p, r, q, w, ut, sbr) if (N == n && P == p && R == r && Q == q) return true;
    M3_BF16_SHAPES(X)
#undef X
    return false;
}

bool scan_bf16_states_supported(int N, int P, int R, int Q) {
#define X(n, p, r, q, w, ut, sbr) if (N == n && P == p && R == r && Q == q) return true;
    M3_BF16_SHAPES(X)
    M3_BF16_STATE_SHAPES(X)
#undef X
    return false;
}

mamba3_status launch_scan_bf16_states(const mamba3_scan_args *a, bf16 *ws_state, float *seg_sums, hipStream_t st) {
    if (a->y) return MAMBA3_EINVAL;
    if (ws_state && a->cu_seqlens) return MAMBA3_EUNSUPPORTED;
    const int N = a->dstate, P = a->headdim, R = a->rank, Q = a->chunk;
    // the EPI instantiations also carry the variants (per-token A, fixed lambda); the gate and
    // the C bias act on outputs only
    const bool epi = a->bc_norm || a->B_bias || a->A_tok || !a->lam;
#define X(n, p, r, q, w, ut, sbr)                                                        \
    if (N == n && P == p && R == r && Q == q)                                            \
        return epi ? launch_cfg<Cfg<n, p, r, q, w, ut, sbr, true, false>>(a, st, ws_state, seg_sums) \
                   : launch_cfg<Cfg<n, p, r, q, w, ut, sbr, false, false>>(a, st, ws_state, seg_sums);
    M3_BF16_SHAPES(X)
    M3_BF16_STATE_SHAPES(X)
#undef X
    return MAMBA3_EUNSUPPORTED;
}

mamba3_status launch_scan_bf16(const mamba3_scan_args *a, hipStream_t st) {
    const int N = a->dstate, P = a->headdim, R = a->rank, Q = a->chunk;
    // y NULL: a state-only scan (the first pass of a segmented scan)
    if (!a->y) return launch_scan_bf16_states(a, nullptr, nullptr, st);
    // the rank-4 shapes of the plain path run in panels
    if (scan_mimo_supported(a)) return launch_scan_mimo(a, st);
    // the EPI instantiations also carry the variants (per-token A, fixed lambda)
    const bool epi = a->bc_norm || a->B_bias || a->C_bias || a->z || a->A_tok || !a->lam;
#define X(n, p, r, q, w, ut, sbr)                                                       \
    if (N == n && P == p && R == r && Q == q)                                           \
        return epi ? launch_cfg<Cfg<n, p, r, q, w, ut, sbr, true>>(a, st)               \
                   : launch_cfg<Cfg<n, p, r, q, w, ut, sbr, false>>(a, st);
    M3_BF16_SHAPES(X)
#undef X
    return MAMBA3_EUNSUPPORTED;
}

}  // namespace m3
