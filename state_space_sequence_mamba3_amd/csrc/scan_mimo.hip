// bf16 chunked MIMO scan on gfx950 MFMA in token panels, fp32 state.
//
// One workgroup (NW waves) owns one (sequence, head) slab and walks it chunk
// by chunk with the state in registers, like the general bf16 scan; the
// chunked form is the same (the three-term update of Proposition 4,
// "Complex-Valued State Space Models", in the matrix form of "Parallel
// representation under SSD", with chunk-local decay S_t and angles Phi_t and
// the RoPE trick of Proposition 3 inside a chunk; the rank-R update of "MIMO
// Formulation"):
//   y_t = e^{S_t} C~_t^T H' + sum_{s<=t} e^{S_t-S_s} w_ts (C~_t.B~_s) X_s + D X_t,
//     w_ts = gamma_s + delta_{s+1} for s < t, gamma_s for s = t
//   H'  <- R(Phi_e) ( e^{S_e} H' + sum_s e^{S_e-S_s} (gamma_s + delta_{s+1}) B~_s X_s^T )
// What differs is how a chunk's work is laid out, for the rank-4 shapes whose
// chunk has Q*R = 256 or 512 rank-expanded rows:
//   * Panels. The chunk's rows are taken PT tokens (32 NW rows) at a time.
//     Only one panel of rotated B rows and X rows sits in LDS, and each wave
//     holds the C~ rows and output accumulators of two 16-row t-blocks of one
//     panel: round p is panel p against itself.
//   * Earlier panels reach later ones through the state. After round p's state
//     update the registers hold
//       H' + sum_{s in panels 0..p} 2^{-S2_s} (gamma_s + delta_{s+1}) B~_s X_s^T,
//     still in the chunk-start frame and decay reference; every s of those
//     panels precedes every t of panel p+1 (weight gamma_s + delta_{s+1}), so
//     panel p+1's inter-chunk term 2^{S2_t} C~_t^T of that sum's bf16 copy is its
//     carried term plus all of the earlier panels'. This is the same sum
//     regrouped (C~_t^T B~_s X_s^T taken as C~_t^T (B~_s X_s^T)), exact up to the
//     bf16 rounding of the summed state, like the carried state's own copy; for
//     two panels it replaces the 256 x 256 score block of panel 1 against panel
//     0 (37 % of a chunk's matrix work at N = 128) by nothing beyond the state
//     update the rounds already do. Each panel is staged behind one barrier and
//     its round ends at another; inside a round each wave runs its score, mask
//     and output MFMAs straight through. The state's bf16 copy is written at the
//     start of the panel that reads it, behind the barrier that ends the
//     previous round's reads of the old copy.
//   * Decay folded into the operands. With the chunk-start reference,
//     e^{S_t-S_s} = 2^{S2_t} 2^{-S2_s} (S2 = S / ln 2), so C~ rows are staged as
//     2^{S2_t} C~_t and B~ rows as 2^{-S2_s} (gamma_s + delta_{s+1}) B~_s. A score
//     tile below the diagonal is then the masked matrix itself (one bf16
//     conversion per element); on a diagonal tile the own-token elements take
//     gamma_s / (gamma_s + delta_{s+1}) and later tokens zero. The inter-chunk
//     term is (2^{S2_t} C~_t)^T H' and the chunk state is
//     2^{S2_e} (H' + sum_s B~'_s X_s^T). A chunk whose total log2 decay is
//     beyond 100 (where the factors could leave the fp32 range), or whose
//     trapezoid weights have gamma_s + delta_{s+1} = 0 with gamma_s != 0, runs
//     unscaled operands with the per-element mask e^{S_t-S_s} w_ts, keeps its
//     state referenced to the start of the current panel, and after each round
//     scales its staged B~ rows in LDS by e^{S_ref'-S_s} (gamma_s + delta_{s+1})
//     and the state by e^{S_ref'-S_ref} (S_ref' of the panel's last token)
//     before the state update: every factor is at most 1.
//   * Operand reads of a tile are all issued before its MFMAs (no per-MFMA
//     conditions), and the next panel's raw B and X rows and the next round's
//     raw C rows are loaded into registers one phase ahead.
//   * Outputs accumulate transposed (the X / H' operand goes first into the
//     MFMA), so each lane ends with four adjacent outputs of one row and stores
//     them from registers; no LDS staging of y. The LDS row strides are padded
//     so that every operand read of the score, output and inter-chunk products
//     is free of bank conflicts.
//   * The rotation R(-Phi) of the B and C rows runs on the bf16 dot-product
//     instruction: the panel's (cos, sin) table holds bf16 pairs, and each
//     rotated element is one two-term dot product of the raw bf16 pair, summed
//     in fp32 (no widening of rows or table). Rounding cos and sin to bf16 adds
//     at most 2^-8 of |u| + |v| per element before the element's own bf16
//     rounding; against the fp64 oracle the outputs moved by under 1e-3 of
//     their slab maximum.
//   * The EPI instantiations fuse the block prologue and epilogue ("Architectural
//     Integration"): every B, C and Bprev column is scaled to unit RMS and gets
//     the head's bias before its rotation (then in fp32), and y is multiplied by
//     SiLU(z) in fp32 before its rounding.
#include "mfma_ops.h"

namespace m3 {

namespace {

// 24-bit unsigned product (full-rate v_mul_u32_u24; a 32-bit v_mul_lo_u32 is quarter rate): a
// token index within a chunk (< 2^7) times a token stride, which the host keeps below 2^24
__device__ __forceinline__ uint32_t mul24(uint32_t a, uint32_t b) { return __umul24(a, b); }

struct MimoParams {
    const bf16 *x, *dt, *lam, *theta, *B, *C, *Bprev, *xprev;
    const float *A, *D, *h_in;
    bf16 *y;
    float *h_out;
    const int32_t *cu;
    int32_t seqlen, H, G, nseq, Gth;
    // fused block prologue / epilogue (EPI instantiations): B, C and Bprev columns scaled to unit
    // RMS (norm) and given the head's bias rows [H, N] (or none), y multiplied by SiLU(z)
    const float *Bb, *Cb;
    const bf16 *z;
    int32_t norm;
    float eps;
};

// Prologue of an 8-element piece of a B or C column (scale by inv, add the bias slice b: 8 fp32 in
// LDS), then the rotation by -Phi against the bf16 (cos, sin) pairs of the piece's 4 angle pairs,
// in fp32, and the operand scale sc; rounded to bf16 once.
__device__ __forceinline__ bf16x8 epi_rot_scale_pack(const bf16x8 raw, float inv, const float *b, const bf16x8 cs,
                                                    float sc) {
    const f32x4 b0 = *(const f32x4 *)b, b1 = *(const f32x4 *)(b + 4);
    float o[8];
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const float u = (float)raw[2 * m] * inv + ((m < 2) ? b0[2 * m] : b1[2 * m - 4]);
        const float v = (float)raw[2 * m + 1] * inv + ((m < 2) ? b0[2 * m + 1] : b1[2 * m - 3]);
        const float c = (float)cs[2 * m], sn = (float)cs[2 * m + 1];
        o[2 * m] = (c * u + sn * v) * sc;
        o[2 * m + 1] = (c * v - sn * u) * sc;
    }
    return pack8(o);
}
__device__ __forceinline__ float epi_sumsq8(const bf16x8 v) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) ss += (float)v[e] * (float)v[e];
    return ss;
}

// NW_ waves per workgroup, PT_ tokens per panel (PT_ R = 32 NW_ rows: two 16-row t-blocks a wave);
// PAD_: LDS rows padded against bank conflicts (below)
template <int N_, int P_, int R_, int Q_, int NW_, int PT_, bool PAD_ = true, int WPE_ = 2, bool EPI_ = false>
struct MCfg {
    static constexpr int N = N_, P = P_, R = R_, Q = Q_;
    static constexpr bool EPI = EPI_;               // the fused block prologue / epilogue
    static constexpr int WPE = WPE_;                // waves per SIMD the registers are sized for
    static constexpr int NW = NW_, NTHR = 64 * NW_;
    static constexpr int K = N / 2;                 // angles per token (state pairs)
    static constexpr int PT = PT_, PR = PT * R;     // tokens and rank-expanded rows per panel
    static constexpr int NPAN = Q / PT;             // panels per chunk
    static constexpr int NTBP = PR / 16;            // 16-row t-blocks per panel
    static constexpr int TPW = NTBP / NW;           // t-blocks per wave and round
    static constexpr int NSTL = PR / 32;            // 32-row s-tiles per panel
    static constexpr int TOKS32 = 32 / R;           // tokens per s-tile
    static constexpr int NKK = N / 32;              // K-steps over N (16x16x32)
    static constexpr int NPT = P / 16;              // 16-column tiles of P
    // padded row strides (bf16, f16x2 elements). On gfx950's 64 four-byte LDS banks (16 lanes a
    // cycle for 16-byte reads, 32 for the transposing 8-byte reads) they make the 16-byte reads
    // of 16 consecutive rows (score operands, H', the angle table) and the transposing reads of 8
    // consecutive X rows free of bank conflicts, with constant offsets between a lane's reads
    static constexpr int NS = N + (PAD_ ? 16 : 0), PS = P + (PAD_ ? 16 : 0), KS = K + (PAD_ ? 8 : 0);
    // the N x P state: 32 x 32 tiles (32x32x16 MFMA) when every wave gets a whole one, else 16 x 16
    static constexpr int UT = ((N / 32) * (P / 32) % NW == 0) ? 32 : 16;
    static constexpr int NUT = (N / UT) * (P / UT), UPW = NUT / NW, URG = (UT == 32) ? 16 : 4;
    // angle prefix of a panel: wave w owns angles [w KW, (w+1) KW); lane = (angle pair, token group)
    static constexpr int KW = K / NW, KP = KW / 2, TG = 64 / KP, TPL = PT / TG;
    // raw 16-byte pieces of a panel per thread
    static constexpr int NLB = PR * N / 8 / NTHR, NLX = PR * P / 8 / NTHR;
    static_assert(R == 4 && P % 32 == 0 && N % 32 == 0 && Q % PT == 0 && NPAN >= 1, "shape");
    static_assert(NTBP == 2 * NW && TPW == 2, "a balanced pair of t-blocks per wave and round");
    static_assert(NUT % NW == 0, "state tiles");
    static_assert(K % NW == 0 && KW % 2 == 0 && 64 % KP == 0 && PT % TG == 0, "angle split");
    static_assert(PR * N / 8 % NTHR == 0 && PR * P / 8 % NTHR == 0, "panel pieces");
    static_assert(NTHR % (N / 8) == 0 && NTHR % (P / 8) == 0, "every piece of a thread has the same columns");
    static_assert(Q <= NTHR && Q % 64 == 0, "prologue");
    // LDS layout (bytes)
    static constexpr int OFF_BS = 0;                              // bf16 [PR][NS]  B~' rows of the panel
    static constexpr int OFF_XS = OFF_BS + PR * NS * 2;           // bf16 [PR][PS]  X rows of the panel
    static constexpr int OFF_HB = OFF_XS + PR * PS * 2;           // bf16 [P][NS]   carried state H'
    static constexpr int OFF_TAB = OFF_HB + P * NS * 2;           // bf16x2 [PT][KS] (cos, sin) of the panel's Phi
    static constexpr int OFF_PHC = OFF_TAB + PT * KS * 4;         // float2 [2][K] chunk total angle
    // per-chunk tables in two copies, by chunk parity: the next chunk's prologue fills its copy
    // during this chunk's last round, which still reads this chunk's
    static constexpr int OFF_S2 = OFF_PHC + 2 * K * 8;            // float [2][Q] log2-decay prefix S2_t
    static constexpr int OFF_G1 = OFF_S2 + 2 * Q * 4;             // float [2][Q] gamma_s + delta_{s+1}
    static constexpr int OFF_GM = OFF_G1 + 2 * Q * 4;             // float [2][Q] gamma_s
    static constexpr int OFF_RR = OFF_GM + 2 * Q * 4;             // float [2][Q] gamma_s / (gamma_s + delta_{s+1})
    static constexpr int OFF_EB = OFF_RR + 2 * Q * 4;             // float [Q] staged B row scale
    static constexpr int OFF_EC = OFF_EB + Q * 4;                 // float [Q] C row scale
    static constexpr int OFF_DT = OFF_EC + Q * 4;                 // float [Q] dt (0 past the end)
    static constexpr int OFF_DL = OFF_DT + Q * 4;                 // float [Q] (1 - lambda) dt
    // the prologue's per-token log2 decay shares S2 (the chunk's copy): wave 0 reads each entry
    // before it writes the entry's new value
    static constexpr int OFF_MISC = OFF_DL + Q * 4;               // float [2][4] per chunk, then A log2 e of the head
    static constexpr int OFF_BIA = (OFF_MISC + 48 + 15) / 16 * 16;  // float [2][N] B, C bias rows (EPI)
    static constexpr int LDS = OFF_BIA + (EPI ? 2 * N * 4 : 0);
    static_assert(LDS <= 160 * 1024, "LDS");
};

template <class CF>
__global__ __launch_bounds__(CF::NTHR) __attribute__((amdgpu_waves_per_eu(CF::WPE))) void k_scan_mimo(MimoParams pr) {
    constexpr int N = CF::N, P = CF::P, R = CF::R, Q = CF::Q, NW = CF::NW, K = CF::K, PT = CF::PT;
    constexpr int PR = CF::PR, NPAN = CF::NPAN, TPW = CF::TPW, NKK = CF::NKK, NPT = CF::NPT;
    constexpr int NS = CF::NS, PS = CF::PS, KS = CF::KS, UT = CF::UT, UPW = CF::UPW, URG = CF::URG, NTHR = CF::NTHR;
    constexpr int KP = CF::KP, TG = CF::TG, TPL = CF::TPL, NLB = CF::NLB, NLX = CF::NLX;
    using UAcc = std::conditional_t<UT == 32, f32x16, f32x4>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16 *BS = (bf16 *)(smem + CF::OFF_BS);
    bf16 *XS = (bf16 *)(smem + CF::OFF_XS);
    bf16 *HB = (bf16 *)(smem + CF::OFF_HB);
    bf16x2 *TAB = (bf16x2 *)(smem + CF::OFF_TAB);
    float2 *const PHC0 = (float2 *)(smem + CF::OFF_PHC);   // copy of chunk parity q at + q K (S2 .. RR: + q Q)
    float *const S20 = (float *)(smem + CF::OFF_S2);
    float *const G10 = (float *)(smem + CF::OFF_G1);
    float *const GM0 = (float *)(smem + CF::OFF_GM);
    float *const RR0 = (float *)(smem + CF::OFF_RR);
    float *EB = (float *)(smem + CF::OFF_EB);
    float *EC = (float *)(smem + CF::OFF_EC);
    float *DT = (float *)(smem + CF::OFF_DT);
    float *DL = (float *)(smem + CF::OFF_DL);
    float *const MISC0 = (float *)(smem + CF::OFF_MISC);   // [4 q + 0..3] of chunk parity q; [8]: A log2 e

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4, l32 = lane & 31, hi = lane >> 5;
    const int H = pr.H, G = pr.G;
    const int h = blockIdx.x % H, g = h / (H / G);
    // packed batches of at most 64 sequences run longest first (workgroup rank r = blockIdx / H
    // takes the sequence of rank r by length, ties by index)
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
        const int64_t a = min(max((int64_t)pr.cu[s], (int64_t)0), (int64_t)pr.seqlen);
        const int64_t b = min(max((int64_t)pr.cu[s + 1], a), (int64_t)pr.seqlen);
        start = a;
        len = b - a;
    } else {
        start = (int64_t)s * pr.seqlen;
        len = pr.seqlen;
    }
    const float A2h = pr.A[h] * kLog2e;
    const float Dh = pr.D ? pr.D[h] : 0.f;
    const bf16 *gB = pr.B + g * (int64_t)R * N;
    const bf16 *gC = pr.C + g * (int64_t)R * N;
    const bf16 *gX = pr.x + h * (int64_t)R * P;
    bf16 *gY = pr.y + h * (int64_t)R * P;
    const bf16 *gTh = pr.theta + (h / (H / pr.Gth)) * (int64_t)K;
    const int64_t strBC = (int64_t)G * R * N, strX = (int64_t)H * R * P, strTh = (int64_t)pr.Gth * K;

    // this wave's state tiles; accumulator register r of a tile is row urow(r), column ucol
    int ut_n0[UPW], ut_p0[UPW];
#pragma unroll
    for (int v = 0; v < UPW; v++) {
        const int ut = wave * UPW + v;
        ut_n0[v] = (ut / (P / UT)) * UT;
        ut_p0[v] = (ut % (P / UT)) * UT;
    }
    auto urow = [&](int r) __attribute__((always_inline)) { return (UT == 32) ? 8 * (r / 4) + 4 * hi + (r % 4) : 4 * q4 + r; };
    const int ucol = (UT == 32) ? l32 : l16;

    // prologue bias rows of the head (zeros for an absent bias): [0, N) for B, [N, 2N) for C
    float *const BIA = (float *)(smem + CF::OFF_BIA);
    if constexpr (CF::EPI) {
        for (int e = tid; e < 2 * N; e += NTHR) {
            const float *src = (e < N) ? pr.Bb : pr.Cb;
            BIA[e] = src ? src[(int64_t)h * N + e % N] : 0.f;
        }
        __syncthreads();
    }

    // ---- the state entering the slab: h_in (+ delta_0 Bprev xprev^T), and its bf16 copy
    UAcc hreg[UPW];
    {
        const int64_t so = ((int64_t)s * H + h) * N * P;
        float d0 = 0.f;
        if (pr.Bprev && len > 0) {
            const float dt0 = to_f(pr.dt[start * H + h]), l0 = to_f(pr.lam[start * H + h]);
            d0 = (1.f - l0) * dt0;
        }
        // the prologue of Bprev's columns: inverse RMS per column (every wave computes its own)
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
            for (int r = 0; r < URG; r++) {
                const int n = ut_n0[v] + urow(r);
                float val = pr.h_in ? pr.h_in[so + (int64_t)n * P + p] : 0.f;
                if (pr.Bprev) {
                    const bf16 *bp = pr.Bprev + ((int64_t)s * G + g) * R * N + n;
                    const bf16 *xp = pr.xprev + ((int64_t)s * H + h) * R * P + p;
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < R; j++) {
                        const float bv = CF::EPI ? to_f(bp[j * N]) * invp[j] + BIA[n] : to_f(bp[j * N]);
                        acc += bv * to_f(xp[j * P]);
                    }
                    val += d0 * acc;
                }
                hreg[v][r] = val;
            }
#pragma unroll
            for (int r = 0; r < URG; r += 2) {
                const int n = ut_n0[v] + urow(r);
                *(bf16x2 *)(HB + p * NS + n) = bf16x2{(bf16)hreg[v][r], (bf16)hreg[v][r + 1]};
            }
        }
    }

    // ---- prefetch registers. Every prefetch load is unconditional: a token past the end of the
    // sequence is clamped to the last valid one (a chunk past the end reads the sequence start),
    // and the consumer zeroes what lies past the end.
    bf16 h_dt = {}, h_lam = {}, h_dtn = {}, h_lamn = {};   // token tid of the chunk; the token after it
    bf16x2 h_th[NPAN][TPL];                                // theta of the lane's angle pair, per panel
    bf16x8 RB[NLB], RX[NLX];                               // raw B and X pieces of the next panel
    bf16x8 HC[TPW][NKK];                                   // raw C rows of the next round's t-blocks
    // Addressing: every load of a chunk is a wave-uniform base (the chunk's first token; SGPRs)
    // plus a 32-bit per-lane element offset (a chunk spans at most Q tokens, far below 2^31
    // elements), so a lane holds one 32-bit offset per load instead of a 64-bit address, and the
    // loads take the scalar-base form. c0c: the chunk's start (a chunk past the end reads the
    // sequence start); ltok: the clamp of chunk-local token indices to the last valid one.
    auto chunk_start = [&](int64_t c0h) __attribute__((always_inline)) { return c0h < len ? c0h : (int64_t)0; };
    auto ltok = [&](int64_t c0c, int tau) __attribute__((always_inline)) {
        return (uint32_t)min(tau, (int)min((int64_t)Q, len - c0c - 1));   // tau <= Q always
    };
    // tq: the thread index the offset math uses (tid, or an opaque copy inside the chunk loop, so
    // that the per-thread terms are recomputed at each load instead of being hoisted out of the
    // loop and spilled)
    auto load_header = [&](int64_t c0h, int tq) __attribute__((always_inline)) {
        const int64_t c0c = chunk_start(c0h);
        const int nqh = (int)min((int64_t)Q, len - c0c);
        const bf16 *bdt = pr.dt + (start + c0c) * H + h, *blam = pr.lam + (start + c0c) * H + h;
        {
            const uint32_t tk = ltok(c0c, min(tq, Q - 1)), tn = ltok(c0c, nqh);
            h_dt = ld_off<bf16>(bdt, mul24(tk, (uint32_t)H) * 2u);
            h_lam = ld_off<bf16>(blam, mul24(tk, (uint32_t)H) * 2u);
            h_dtn = ld_off<bf16>(bdt, mul24(tn, (uint32_t)H) * 2u);
            h_lamn = ld_off<bf16>(blam, mul24(tn, (uint32_t)H) * 2u);
        }
        const int lq = tq & 63;
        const int k = wave * CF::KW + 2 * (lq % KP), g0 = (lq / KP) * TPL;
        const bf16 *bth = gTh + (start + c0c) * strTh;
#pragma unroll
        for (int p = 0; p < NPAN; p++)
#pragma unroll
            for (int j = 0; j < TPL; j++)
                h_th[p][j] = ld_off<bf16x2>(bth, (mul24(ltok(c0c, p * PT + g0 + j), (uint32_t)strTh) + (uint32_t)k) * 2u);
    };
    auto load_panel = [&](int64_t c0h, int pan, int tq) __attribute__((always_inline)) {
        const int64_t c0c = chunk_start(c0h);
        const bf16 *bB = gB + (start + c0c) * strBC, *bX = gX + (start + c0c) * strX;
#pragma unroll
        for (int i = 0; i < NLB; i++) {
            const int c = tq + i * NTHR, row = c / (N / 8), col = (c % (N / 8)) * 8;
            RB[i] = ld_off<bf16x8>(bB, (mul24(ltok(c0c, pan * PT + row / R), (uint32_t)strBC) + (uint32_t)((row % R) * N + col)) * 2u);
        }
#pragma unroll
        for (int i = 0; i < NLX; i++) {
            const int c = tq + i * NTHR, row = c / (P / 8), col = (c % (P / 8)) * 8;
            RX[i] = ld_off<bf16x8>(bX, (mul24(ltok(c0c, pan * PT + row / R), (uint32_t)strX) + (uint32_t)((row % R) * P + col)) * 2u);
        }
    };
    // t-blocks of a round: a balanced pair along the causal triangle of the panel, rotated by the
    // chunk index so the heavy blocks move across the SIMDs
    auto tb_of = [&](int u, int64_t c0h) __attribute__((always_inline)) {
        const int w = (wave + (int)(c0h / Q)) % NW;
        return (u == 0) ? w : 2 * NW - 1 - w;
    };
    auto load_crows = [&](int64_t c0h, int pan, int tq) __attribute__((always_inline)) {
        const int l16q = tq & 15, q4q = (tq & 63) >> 4;
        const int64_t c0c = chunk_start(c0h);
        const bf16 *bC = gC + (start + c0c) * strBC;
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int row = tb_of(u, c0h) * 16 + l16q;
            const uint32_t o = mul24(ltok(c0c, pan * PT + row / R), (uint32_t)strBC) + (uint32_t)((row % R) * N + 8 * q4q);
#pragma unroll
            for (int kk = 0; kk < NKK; kk++) HC[u][kk] = ld_off<bf16x8>(bC, (o + 32 * kk) * 2u);
        }
    };
    if (len > 0) {
        load_header(0, tid);
        load_panel(0, 0, tid);
        load_crows(0, 0, tid);
    }
    // ---- a chunk's prologue, in two parts separated by a barrier: (a) its per-token scalars
    // from the prefetched header, (b) the decay prefix, weights and operand scales (wave 0) and
    // the angle table of panel 0 (every wave). Tables of chunk parity par.
    float car0 = 0.f, car1 = 0.f;   // the angle sums of panel 0, carried into panel 1's table
    // cumulative angles of the wave's angle pairs over panel pan, continuing from the carry
    // (r0, r1: the lane's running sums; the lanes of the panel's last token group hold the
    // panel totals afterwards); phc: the chunk's total-angle table
    auto angle_table = [&](int pan, bool last, float2 *phc) __attribute__((always_inline)) {
        const int lane = opaque<true>(tid) & 63;
        const int k = wave * CF::KW + 2 * (lane % KP), g0 = (lane / KP) * TPL;
        float a0[TPL], a1[TPL];
        float r0 = 0.f, r1 = 0.f;
#pragma unroll
        for (int j = 0; j < TPL; j++) {
            const float dt = DT[pan * PT + g0 + j];
            r0 += dt * (float)h_th[pan][j][0];
            r1 += dt * (float)h_th[pan][j][1];
            a0[j] = r0;
            a1[j] = r1;
        }
        float e0 = r0, e1 = r1;
#pragma unroll
        for (int off = KP; off < 64; off <<= 1) {
            const float o0 = __shfl_up(e0, off, 64), o1 = __shfl_up(e1, off, 64);
            if (lane >= off) {
                e0 += o0;
                e1 += o1;
            }
        }
        // e0, e1: inclusive over the token groups; the panel total sits in the last group
        const float tot0 = __shfl(e0, (TG - 1) * KP + lane % KP, 64), tot1 = __shfl(e1, (TG - 1) * KP + lane % KP, 64);
        e0 += car0 - r0;
        e1 += car1 - r1;
#pragma unroll
        for (int j = 0; j < TPL; j++) {
            const int tau = g0 + j;
            const float x0 = a0[j] + e0, x1 = a1[j] + e1;
            float sn0, cs0, sn1, cs1;
            __sincosf(x0, &sn0, &cs0);
            __sincosf(x1, &sn1, &cs1);
            *(bf16x4 *)(TAB + tau * KS + k) = bf16x4{(bf16)cs0, (bf16)sn0, (bf16)cs1, (bf16)sn1};
            if (last && tau == PT - 1) {   // the chunk's last panel; angles past the end are zero
                sincos_state(x0, &sn0, &cs0);
                sincos_state(x1, &sn1, &cs1);
                *(f32x4 *)(phc + k) = f32x4{cs0, sn0, cs1, sn1};
            }
        }
        car0 += tot0;
        car1 += tot1;
    };
    auto prologue_scalars = [&](int64_t c0x, int nqx, int par) __attribute__((always_inline)) {
        const int tq = opaque<true>(tid) & (NTHR - 1);
        float *A2 = S20 + par * Q, *GM = GM0 + par * Q, *MISC = MISC0 + 4 * par;
        if (tq < Q) {
            const bool ok = tq < nqx;
            const float dt = ok ? to_f(h_dt) : 0.f, lm = ok ? to_f(h_lam) : 0.f;
            DT[tq] = dt;
            // (A log2 e re-read from LDS in every chunk: a register copy held across the loop was
            // spilled, and its reload here waited for every store and load in flight, since
            // memory operations complete in order)
            A2[tq] = dt * *(volatile __attribute__((address_space(3))) const float *)(MISC0 + 8);
            GM[tq] = lm * dt;
            DL[tq] = (1.f - lm) * dt;
        }
        if (tq == 0) MISC[0] = (c0x + nqx < len) ? (1.f - to_f(h_lamn)) * to_f(h_dtn) : 0.f;
    };
    auto prologue_tables = [&](int nqx, int par) __attribute__((always_inline)) {
        const int lane = opaque<true>(tid) & 63;
        float *A2 = S20 + par * Q, *S2 = S20 + par * Q, *G1 = G10 + par * Q, *GM = GM0 + par * Q, *RR = RR0 + par * Q;
        float *MISC = MISC0 + 4 * par;
        const int nq = nqx;
    if (wave == 0) {
        // S2_t = sum_{tau <= t} dt A / ln 2 over the chunk; weights and operand scales
        constexpr int PER = Q / 64;
        float loc[PER];
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            run += A2[lane * PER + i];
            loc[i] = run;
        }
        const float excl = wave_incl_scan(run, lane) - run;
        float s2v[PER];
#pragma unroll
        for (int i = 0; i < PER; i++) s2v[i] = excl + loc[i];
        const float s2e = wave_bcast(s2v[PER - 1], 63);   // S2 of the chunk's last token (dt = 0 past the end)
        const float dn = MISC[0];
        // the fast form needs bounded scale factors and a finite gamma / (gamma + delta) ratio
        bool bad = false;
        float mx = 0.f;
        float g1v[PER];
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int t = lane * PER + i;
            const float next = (t + 1 < nq) ? DL[t + 1] : ((t + 1 == nq) ? dn : 0.f);
            g1v[i] = (t < nq) ? GM[t] + next : 0.f;
            bad |= g1v[i] == 0.f && GM[t] != 0.f;
            mx = fmaxf(mx, fabsf(s2v[i]));
        }
        mx = wave_max_nonneg(mx);
        const bool fast = __ballot(bad) == 0 && mx <= 100.f;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int t = lane * PER + i;
            S2[t] = s2v[i];
            G1[t] = g1v[i];
            RR[t] = (g1v[i] != 0.f) ? GM[t] / g1v[i] : 0.f;
            EB[t] = fast ? exp2_neg(-s2v[i]) * g1v[i] : 1.f;
            EC[t] = fast ? exp2_neg(s2v[i]) : 1.f;
        }
        if (lane == 0) {
            MISC[1] = s2e;
            MISC[2] = fast ? 1.f : 0.f;
        }
    }
        car0 = car1 = 0.f;
        angle_table(0, (nqx + PT - 1) / PT == 1, PHC0 + par * K);
    };
    if (tid == 0) MISC0[8] = A2h;
    __syncthreads();
    if constexpr (NPAN >= 2) {   // the first chunk's prologue; every later one runs in the chunk before
        if (len > 0) {
            prologue_scalars(0, (int)min((int64_t)Q, len), 0);
            __syncthreads();
            prologue_tables((int)min((int64_t)Q, len), 0);
            __syncthreads();
        }
    }

    for (int64_t c0 = 0; c0 < len; c0 += Q) {
        const int nq = (int)min((int64_t)Q, len - c0);
        const int64_t tok0 = start + c0;
        const int npan = (nq + PT - 1) / PT;   // panels holding valid tokens (the last chunk may have fewer)
        // Every lane-derived index inside the loop comes from an opaque copy of the thread index
        // (these names shadow the ones above), so none of it is hoisted out of the loop and held
        // (or spilled) across chunks; it is recomputed where it is used.
        const int tq = opaque<true>(tid) & (NTHR - 1);
        const int lane = tq & 63, l16 = tq & 15, q4 = lane >> 4, l32 = tq & 31, hi = lane >> 5;
        auto urow = [&](int r) __attribute__((always_inline)) { return (UT == 32) ? 8 * (r / 4) + 4 * hi + (r % 4) : 4 * q4 + r; };
        const int ucol = (UT == 32) ? l32 : l16;

        // this chunk's copies of the per-chunk tables (the next chunk's prologue fills the others)
        const int par = (int)((c0 / Q) & 1);
        float2 *PHC = PHC0 + par * K;
        float *S2 = S20 + par * Q, *G1 = G10 + par * Q, *GM = GM0 + par * Q, *RR = RR0 + par * Q;
        float *MISC = MISC0 + 4 * par;
        if constexpr (NPAN == 1) {   // one panel per chunk: the prologue at the chunk's start
            prologue_scalars(c0, nq, par);
            __syncthreads();
            prologue_tables(nq, par);
            __syncthreads();
        }
        const bool fast = __builtin_amdgcn_readfirstlane(__float_as_int(MISC[2])) != 0;
        const float s2e = MISC[1];

        // The slow form keeps the state referenced to the start of the panel in hand (S2 of the
        // previous panel's last token; 0 at the chunk start) and moves it to the next panel's
        // reference at each panel's state update; the fast one keeps the chunk-start reference
        // and applies e^{S_e} at the end of the chunk.
        auto s2ref = [&](int pan) __attribute__((always_inline)) { return pan == 0 ? 0.f : S2[pan * PT - 1]; };

        // ---- staging of panel pan from the prefetched raw rows: B~' = R(-Phi) B * EB, X as is.
        // Rows past the end hold the last token's (finite) values: a zero scale clears their B~'
        // rows, which zeroes every score and state term that would read their X rows.
        auto stage_panel = [&](int pan) __attribute__((always_inline)) {
            const int tq = opaque<true>(tid) & (NTHR - 1);
            if constexpr (CF::EPI) {
                // the fused prologue: a row's N / 8 pieces sit in N / 8 consecutive lanes, whose
                // butterfly sums its squares; every piece of a thread covers the same columns. The
                // pieces go two at a time (their table reads before their stores): fewer values live
                // at once than with every piece's reads first (packed shape: 105 VGPRs spilled, not 158).
                const float *bslice = BIA + (tq % (N / 8)) * 8;
                constexpr int HB2 = (NLB >= 2) ? 2 : 1;
#pragma unroll
                for (int i0 = 0; i0 < NLB; i0 += HB2) {
                    bf16x8 csh[HB2];
                    float ebh[HB2];
#pragma unroll
                    for (int k = 0; k < HB2; k++) {
                        const int c = tq + (i0 + k) * NTHR, row = c / (N / 8), col = (c % (N / 8)) * 8;
                        csh[k] = *(const bf16x8 *)(TAB + (row / R) * KS + col / 2);
                        const float e = EB[pan * PT + row / R];
                        ebh[k] = (pan * PT + row / R < nq) ? e : 0.f;
                    }
#pragma unroll
                    for (int k = 0; k < HB2; k++) {
                        const int i = i0 + k;
                        const int c = tq + i * NTHR, row = c / (N / 8), col = (c % (N / 8)) * 8;
                        float inv = 1.f;
                        if (pr.norm) {
                            // the row's N / 8 lanes are one aligned group of 8 or 16 lanes: sums by
                            // DPP (quad swaps, then the half-row and row mirrors), no LDS round trip
                            static_assert(N / 8 == 8 || N / 8 == 16, "a B row's lanes form a DPP row or half");
                            float ss = epi_sumsq8(RB[i]);
                            ss += dpp_move<0xB1>(ss);   // quad_perm [1, 0, 3, 2]
                            ss += dpp_move<0x4E>(ss);   // quad_perm [2, 3, 0, 1]
                            ss += dpp_move<0x141>(ss);  // row_half_mirror
                            if constexpr (N / 8 == 16) ss += dpp_move<0x140>(ss);   // row_mirror
                            inv = rsqrtf(ss * (1.f / N) + pr.eps);
                        }
                        *(bf16x8 *)(BS + row * NS + col) = epi_rot_scale_pack(RB[i], inv, bslice, csh[k], ebh[k]);
                    }
                }
            } else {
                bf16x8 cs[NLB];
                float eb[NLB];
#pragma unroll
                for (int i = 0; i < NLB; i++) {
                    const int c = tq + i * NTHR, row = c / (N / 8), col = (c % (N / 8)) * 8;
                    cs[i] = *(const bf16x8 *)(TAB + (row / R) * KS + col / 2);
                    const float e = EB[pan * PT + row / R];
                    eb[i] = (pan * PT + row / R < nq) ? e : 0.f;
                }
#pragma unroll
                for (int i = 0; i < NLB; i++) {
                    const int c = tq + i * NTHR, row = c / (N / 8), col = (c % (N / 8)) * 8;
                    *(bf16x8 *)(BS + row * NS + col) = rot_scale_pack_bf(RB[i], cs[i], eb[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < NLX; i++) {
                const int c = tq + i * NTHR, row = c / (P / 8), col = (c % (P / 8)) * 8;
                *(bf16x8 *)(XS + row * PS + col) = RX[i];
            }
        };
        // ---- C~' rows of the round's t-blocks from the prefetched raw rows: R(-Phi) C * EC
        bf16x8 creg[TPW][NKK];
        int tbr[TPW];
        auto rotate_crows = [&](int pan) __attribute__((always_inline)) {
            // lane indices made opaque here: the phase's address math is recomputed in it rather
            // than precomputed for every phase of the chunk and held across them
            const int tqp = opaque<true>(tid) & (NTHR - 1);
            const int lane = tqp & 63, l16 = tqp & 15, q4 = lane >> 4;
#pragma unroll
            for (int u = 0; u < TPW; u++) {
                tbr[u] = tb_of(u, c0);
                const int tau = (tbr[u] * 16 + l16) / R;
                const float e = EC[pan * PT + tau];
                const float ec = (pan * PT + tau < nq) ? e : 0.f;   // (rows past the end: zero)
                if constexpr (CF::EPI) {
                    // the fused prologue: the row's N values sit in lanes l16 + 16 q4, NKK pieces each
                    float inv = 1.f;
                    if (pr.norm) {
                        float ss = 0.f;
#pragma unroll
                        for (int kk = 0; kk < NKK; kk++) ss += epi_sumsq8(HC[u][kk]);
                        ss = sum_across_rows(ss);   // the row's 4 lanes l16 + 16 q4
                        inv = rsqrtf(ss * (1.f / N) + pr.eps);
                    }
#pragma unroll
                    for (int kk = 0; kk < NKK; kk++) {
                        const bf16x8 cs = *(const bf16x8 *)(TAB + tau * KS + 16 * kk + 4 * q4);
                        creg[u][kk] = epi_rot_scale_pack(HC[u][kk], inv, BIA + N + 32 * kk + 8 * q4, cs, ec);
                    }
                } else {
#pragma unroll
                    for (int kk = 0; kk < NKK; kk++) {
                        const bf16x8 cs = *(const bf16x8 *)(TAB + tau * KS + 16 * kk + 4 * q4);
                        creg[u][kk] = rot_scale_pack_bf(HC[u][kk], cs, ec);
                    }
                }
            }
        };
        // ---- output accumulators of the round, transposed: yacc[u][pt] of lane (l16, q4) holds
        // y at t-row 16 tbr[u] + l16, columns 16 pt + 4 q4 .. + 3 (the MFMAs take the X / H'
        // operand first), so a lane stores four adjacent outputs of one row straight from its
        // registers. Here the inter-chunk term e^{S_t} C~_t^T H'.
        f32x4 yacc[TPW][NPT];
        auto inter = [&](int pan) __attribute__((always_inline)) {
            // lane indices made opaque here: the phase's address math is recomputed in it rather
            // than precomputed for every phase of the chunk and held across them
            const int tqp = opaque<true>(tid) & (NTHR - 1);
            const int lane = tqp & 63, l16 = tqp & 15, q4 = lane >> 4;
#pragma unroll
            for (int u = 0; u < TPW; u++)
#pragma unroll
                for (int pt = 0; pt < NPT; pt++) yacc[u][pt] = f32x4{};
#pragma unroll
            for (int pt = 0; pt < NPT; pt++) {
                bf16x8 hop[NKK];
#pragma unroll
                for (int kk = 0; kk < NKK; kk++) hop[kk] = *(const bf16x8 *)(HB + (pt * 16 + l16) * NS + 32 * kk + 8 * q4);
#pragma unroll
                for (int kk = 0; kk < NKK; kk++)
#pragma unroll
                    for (int u = 0; u < TPW; u++) yacc[u][pt] = mfma16(hop[kk], creg[u][kk], yacc[u][pt]);
            }
            if (!fast) {   // unscaled C~ rows: the decay of the lane's output row from the panel reference
                const float ref = s2ref(pan);
#pragma unroll
                for (int u = 0; u < TPW; u++) {
                    const float sc = exp2_neg(S2[pan * PT + (tbr[u] * 16 + l16) / R] - ref);
#pragma unroll
                    for (int pt = 0; pt < NPT; pt++)
#pragma unroll
                        for (int i = 0; i < 4; i++) yacc[u][pt][i] *= sc;
                }
            }
        };
        // ---- one 32-row s-tile j of the staged panel (s-panel spn) for the NA t-blocks u0 ..
        // of the round (t-panel tpn); diag: the s-panel is the t-panel (causal tiles)
        auto tile = [&](auto NAC, int u0, int j, int tpn, int spn) __attribute__((always_inline)) {
            // lane indices made opaque here: the phase's address math is recomputed in it rather
            // than precomputed for every phase of the chunk and held across them
            const int tqp = opaque<true>(tid) & (NTHR - 1);
            const int lane = tqp & 63, l16 = tqp & 15, q4 = lane >> 4;
            constexpr int NA = decltype(NAC)::value;
            // score operands in two halves of the K steps (fewer registers live at once)
            f32x4 g0[NA], g1[NA];
#pragma unroll
            for (int u = 0; u < NA; u++) g0[u] = g1[u] = f32x4{};
            constexpr int KH = (NKK >= 2) ? NKK / 2 : 1;
#pragma unroll
            for (int kh = 0; kh < NKK; kh += KH) {
                bf16x8 b0[KH], b1[KH];
#pragma unroll
                for (int k2 = 0; k2 < KH; k2++) {
                    b0[k2] = *(const bf16x8 *)(BS + (32 * j + l16) * NS + 32 * (kh + k2) + 8 * q4);
                    b1[k2] = *(const bf16x8 *)(BS + (32 * j + 16 + l16) * NS + 32 * (kh + k2) + 8 * q4);
                }
#pragma unroll
                for (int k2 = 0; k2 < KH; k2++)
#pragma unroll
                    for (int u = 0; u < NA; u++) {
                        g0[u] = mfma16(b0[k2], creg[u0 + u][kh + k2], g0[u]);
                        g1[u] = mfma16(b1[k2], creg[u0 + u][kh + k2], g1[u]);
                    }
            }
            // Gt tile: lane holds s-rows 32 j + 4 q4 + i (g0) and 32 j + 16 + 4 q4 + i (g1) of t-row
            // 16 tb + l16. With R = 4 the four rows of a half are one token.
            const int ss0 = spn * PT + (32 * j + 4 * q4) / R, ss1 = ss0 + 16 / R;   // chunk tokens of the halves
            bf16x8 mop[NA];
#pragma unroll
            for (int u = 0; u < NA; u++) {
                const int tb = tbr[u0 + u];
                const int tt = tpn * PT + (tb * 16 + l16) / R;                        // chunk token of the t-row
                const bool full = tpn > spn || tb >= 2 * j + 2;                         // every s precedes every t
                if (fast) {
                    if (full) {
#pragma unroll
                        for (int e = 0; e < 8; e++) mop[u][e] = (bf16)((e < 4) ? g0[u][e] : g1[u][e - 4]);
                    } else {
                        const float r0 = RR[ss0], r1 = RR[ss1];
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            const int ss = (e < 4) ? ss0 : ss1;
                            const float v = (e < 4) ? g0[u][e] : g1[u][e - 4];
                            const float m = (ss < tt) ? v : ((ss == tt) ? v * ((e < 4) ? r0 : r1) : 0.f);
                            mop[u][e] = (bf16)m;
                        }
                    }
                } else {
                    const float s2t = S2[tt];
                    // e^{S_t - S_s}; later tokens (whose factor may overflow) are selected away
                    const float c0v = exp2_neg(s2t - S2[ss0]), c1v = exp2_neg(s2t - S2[ss1]);
                    const float w0 = (ss0 < tt) ? G1[ss0] : GM[ss0], w1 = (ss1 < tt) ? G1[ss1] : GM[ss1];
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const int ss = (e < 4) ? ss0 : ss1;
                        const float v = (e < 4) ? g0[u][e] * c0v * w0 : g1[u][e - 4] * c1v * w1;
                        mop[u][e] = (bf16)((ss <= tt) ? v : 0.f);
                    }
                }
            }
            // X rows 4 q4 .. and 16 + 4 q4 .. of column 16 pt + l16 (K permuted like the score tile)
#pragma unroll
            for (int pt = 0; pt < NPT; pt++) {
                const bf16x8 xop = tr_operand(XS, PS, 32 * j + 4 * q4, 32 * j + 16 + 4 * q4, pt * 16, l16);
#pragma unroll
                for (int u = 0; u < NA; u++) yacc[u0 + u][pt] = mfma16(xop, mop[u], yacc[u0 + u][pt]);
            }
        };
        // every s-tile of the staged panel spn that holds valid tokens, against the round's t-blocks
        auto sweep = [&](int tpn, int spn) __attribute__((always_inline)) {
            const int ntl = min(CF::NSTL, (nq - spn * PT) * R / 32 + (((nq - spn * PT) * R) % 32 != 0));
            if (tpn > spn) {
                for (int j = 0; j < ntl; j++) tile(std::integral_constant<int, 2>{}, 0, j, tpn, spn);
            } else {
                // t-blocks (tb_lo < tb_hi): the tiles j <= tb_lo / 2 reach both, those up to tb_hi / 2
                // only the higher one. Two loops with one tile form each: in one loop with both forms
                // the accumulators took different registers in the two branches and were copied
                // back at every iteration.
                const int j0 = min(ntl, tbr[0] / 2 + 1), j1 = min(ntl, tbr[1] / 2 + 1);
                for (int j = 0; j < j0; j++) tile(std::integral_constant<int, 2>{}, 0, j, tpn, spn);
                for (int j = j0; j < j1; j++) tile(std::integral_constant<int, 1>{}, 1, j, tpn, spn);
                // skip term D x_t of the t-blocks' own rows (their X rows are in this panel)
#pragma unroll
                for (int u = 0; u < TPW; u++)
#pragma unroll
                    for (int pt = 0; pt < NPT; pt++) {
                        const bf16x4 xv = *(const bf16x4 *)(XS + (tbr[u] * 16 + l16) * PS + pt * 16 + 4 * q4);
#pragma unroll
                        for (int i = 0; i < 4; i++) yacc[u][pt][i] += Dh * (float)xv[i];
                    }
            }
        };
        // chunk-state update over the staged panel: H += B~'^T X (K = the panel's rows)
        auto state_update = [&](int spn) __attribute__((always_inline)) {
            // lane indices made opaque here: the phase's address math is recomputed in it rather
            // than precomputed for every phase of the chunk and held across them
            const int tqp = opaque<true>(tid) & (NTHR - 1);
            const int lane = tqp & 63, l16 = tqp & 15, q4 = lane >> 4;
            const int nrow = min(PR, (nq - spn * PT) * R);
            for (int rb = 0; rb < nrow; rb += 32) {
#pragma unroll
                for (int v = 0; v < UPW; v++) {
                    if constexpr (UT == 32) {
                        const int grp = lane >> 4;
                        const int cn = ut_n0[v] + 16 * (grp & 1), cp = ut_p0[v] + 16 * (grp & 1);
#pragma unroll
                        for (int ks = 0; ks < 2; ks++) {
                            const int r0 = rb + 16 * ks + 8 * (grp >> 1);
                            hreg[v] = mfma32(tr_operand(BS, NS, r0, r0 + 4, cn, l16), tr_operand(XS, PS, r0, r0 + 4, cp, l16),
                                             hreg[v]);
                        }
                    } else {
                        hreg[v] = mfma16(tr_operand(BS, NS, rb + 8 * q4, rb + 8 * q4 + 4, ut_n0[v], l16),
                                         tr_operand(XS, PS, rb + 8 * q4, rb + 8 * q4 + 4, ut_p0[v], l16), hreg[v]);
                    }
                }
            }
        };
        // the slow form: staged B~ rows scaled in place by e^{S_ref - S_s} (gamma_s + delta_{s+1}),
        // S_ref that of the panel's last token (the chunk's S_e for the last panel: dt is 0 past the
        // end), and the state moved to that reference
        auto slow_rescale = [&](int spn) __attribute__((always_inline)) {
            const int tq = opaque<true>(tid) & (NTHR - 1);
            const float ref = S2[spn * PT + PT - 1];
            const float eS = exp2_neg(ref - s2ref(spn));
#pragma unroll
            for (int v = 0; v < UPW; v++)
#pragma unroll
                for (int r = 0; r < URG; r++) hreg[v][r] *= eS;
#pragma unroll
            for (int i = 0; i < NLB; i++) {
                const int c = tq + i * NTHR, row = c / (N / 8), col = (c % (N / 8)) * 8;
                const int t = spn * PT + row / R;
                const float f = exp2_neg(ref - S2[t]) * G1[t];
                const bf16x8 v = *(const bf16x8 *)(BS + row * NS + col);
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; e++) o[e] = (float)v[e] * f;
                *(bf16x8 *)(BS + row * NS + col) = pack8(o);
            }
        };
        // bf16 copy of the registers' state for the inter-chunk products (each wave its tiles)
        auto write_hb = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int v = 0; v < UPW; v++) {
                const int p = ut_p0[v] + ucol;
#pragma unroll
                for (int r = 0; r < URG; r += 2) {
                    const int n = ut_n0[v] + urow(r);
                    *(bf16x2 *)(HB + p * NS + n) = bf16x2{(bf16)hreg[v][r], (bf16)hreg[v][r + 1]};
                }
            }
        };
        // outputs of the round straight from the accumulators: four adjacent columns of one row
        // per lane and store (a t-block's 16 rows are 4 tokens' rank rows, 2 KB in all)
        bf16 *yb = gY + tok0 * strX;   // the chunk's first output row (a uniform base)
        // the fused epilogue's gate z at the outputs' addresses (rows past the end read the last
        // token's, unused), loaded once the round's tile work is done
        bf16x4 zr[TPW][NPT];
        const bool has_z = CF::EPI && pr.z != nullptr;
        auto load_z = [&](int tpn) __attribute__((always_inline)) {
            if constexpr (CF::EPI) {
                if (has_z) {
                    const int tqp = opaque<true>(tid) & (NTHR - 1);
                    const int lane = tqp & 63, l16 = tqp & 15, q4 = lane >> 4;
                    const bf16 *zb = pr.z + h * (int64_t)R * P + tok0 * strX;
#pragma unroll
                    for (int u = 0; u < TPW; u++) {
                        const int rr = tbr[u] * 16 + l16, tau = min(tpn * PT + rr / R, nq - 1);
                        const uint32_t o = mul24((uint32_t)tau, (uint32_t)strX) + (uint32_t)((rr % R) * P + 4 * q4);
#pragma unroll
                        for (int pt = 0; pt < NPT; pt++) zr[u][pt] = ld_off<bf16x4>(zb, (o + 16 * pt) * 2u);
                    }
                }
            }
        };
        auto store_y = [&](int tpn) __attribute__((always_inline)) {
            // lane indices made opaque here: the phase's address math is recomputed in it rather
            // than precomputed for every phase of the chunk and held across them
            const int tqp = opaque<true>(tid) & (NTHR - 1);
            const int lane = tqp & 63, l16 = tqp & 15, q4 = lane >> 4;
            if (has_z) {   // y SiLU(z) in fp32, before the single rounding
#pragma unroll
                for (int u = 0; u < TPW; u++)
#pragma unroll
                    for (int pt = 0; pt < NPT; pt++)
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const float v = (float)zr[u][pt][i];
                            yacc[u][pt][i] *= v / (1.f + __expf(-v));
                        }
            }
#pragma unroll
            for (int u = 0; u < TPW; u++) {
                const int rr = tbr[u] * 16 + l16, tau = tpn * PT + rr / R;
                if (tau < nq) {
                    const uint32_t o = mul24((uint32_t)tau, (uint32_t)strX) + (uint32_t)((rr % R) * P + 4 * q4);
#pragma unroll
                    for (int pt = 0; pt < NPT; pt++)
                        st_off<bf16x4>(yb, (o + 16 * pt) * 2u,
                                       bf16x4{(bf16)yacc[u][pt][0], (bf16)yacc[u][pt][1], (bf16)yacc[u][pt][2], (bf16)yacc[u][pt][3]});
                }
            }
        };

        // ---- the panels of the chunk, one round each. Panel p is staged from the prefetched rows
        // with its round's C~' rows, after the state in the registers is copied to HB for its
        // inter-chunk term: the carried state at p = 0, plus every earlier panel's terms after
        // (see above).
        // Round p: panel p against itself; meanwhile the next panel's angle table, the next
        // panel's (or chunk's) raw rows, and in the last round the next chunk's prologue.
        const bool has_next = c0 + Q < len;
        const int nq_next = (int)min((int64_t)Q, len - c0 - Q);
#pragma unroll
        for (int pan = 0; pan < NPAN; pan++) {
            if (pan > 0 && pan >= npan) break;   // (uniform) panels past the sequence's end
            if (pan > 0) {
                rotate_crows(pan);
                __builtin_amdgcn_sched_barrier(0);
            }
            write_hb();
            stage_panel(pan);
            if (pan == 0) rotate_crows(0);
            // the prefetch registers are consumed: no load that refills them may be scheduled into
            // the staging above (old and new contents would be live together)
            __builtin_amdgcn_sched_barrier(0);
            if (pan + 1 < NPAN) {
                load_panel(c0, pan + 1, tq);
            } else {
                if (NPAN == 1) load_header(c0 + Q, tq);
                load_panel(c0 + Q, 0, tq);
                // the next chunk's prologue, part (a): its per-token scalars (this chunk no longer
                // reads dt, DL or the other copy of the tables)
                if (NPAN > 1 && has_next) prologue_scalars(c0 + Q, nq_next, par ^ 1);
            }
            __syncthreads();
            inter(pan);
            sweep(pan, pan);
            // the next round's raw C rows are loaded once the sweep is done (no prefetch beyond
            // the panel rows is live during tile work)
            __builtin_amdgcn_sched_barrier(0);
            if (pan + 1 < NPAN) load_crows(c0, pan + 1, tq);
            else load_crows(c0 + Q, 0, tq);
            load_z(pan);
            if (fast) state_update(pan);
            store_y(pan);
            if (pan + 1 < npan) {
                angle_table(pan + 1, pan + 2 == npan, PHC);
                if (pan + 2 == NPAN) {
                    // the lane's angles of this chunk are consumed: the next chunk's header may load
                    __builtin_amdgcn_sched_barrier(0);
                    load_header(c0 + Q, tq);
                }
            }
            if (!fast) {
                __syncthreads();
                slow_rescale(pan);
                __syncthreads();
                state_update(pan);
            }
            if (pan + 1 == NPAN) {
                // part (b): the decay prefix, the weights and scales, the angle table of panel 0
                // (the angle table and the scales are no longer read by this chunk; the loop's last
                // barrier orders them before the next chunk)
                if (NPAN > 1 && has_next) prologue_tables(nq_next, par ^ 1);
            } else if (pan + 1 < npan) {
                __syncthreads();
            }
        }
        // ---- state epilogue: e^{S_e} (fast form) and the rotation by the chunk's total angle. Its
        // bf16 copy is written at the next chunk's start: other waves may still be reading HB in
        // the last round's inter-chunk product, and the loop's last barrier orders them first.
        {
            const float eS = fast ? exp2_neg(s2e) : 1.f;
            f32x4 rot4[UPW][URG / 4];
#pragma unroll
            for (int v = 0; v < UPW; v++)
#pragma unroll
                for (int q = 0; q < URG / 4; q++) rot4[v][q] = *(const f32x4 *)(PHC + (ut_n0[v] + urow(4 * q)) / 2);
#pragma unroll
            for (int v = 0; v < UPW; v++) {
#pragma unroll
                for (int r = 0; r < URG; r += 2) {
                    const float cs = rot4[v][r / 4][r % 4], sn = rot4[v][r / 4][r % 4 + 1];
                    const float u0 = hreg[v][r] * eS, u1 = hreg[v][r + 1] * eS;
                    hreg[v][r] = cs * u0 - sn * u1;
                    hreg[v][r + 1] = sn * u0 + cs * u1;
                }
            }
        }
        __syncthreads();
    }

    if (pr.h_out) {
        const int64_t so = ((int64_t)s * H + h) * N * P;
#pragma unroll
        for (int v = 0; v < UPW; v++) {
            const int p = ut_p0[v] + ucol;
#pragma unroll
            for (int r = 0; r < URG; r++) pr.h_out[so + (int64_t)(ut_n0[v] + urow(r)) * P + p] = hreg[v][r];
        }
    }
}

template <class CF>
mamba3_status launch_mimo_cfg(const mamba3_scan_args *a, hipStream_t st) {
    MimoParams p;
    p.x = (const bf16 *)a->x; p.dt = (const bf16 *)a->dt; p.lam = (const bf16 *)a->lam;
    p.theta = (const bf16 *)a->theta; p.B = (const bf16 *)a->B; p.C = (const bf16 *)a->C;
    p.Bprev = (const bf16 *)a->Bprev; p.xprev = (const bf16 *)a->xprev;
    p.A = a->A; p.D = a->D; p.h_in = a->h_in; p.y = (bf16 *)a->y; p.h_out = a->h_out;
    p.cu = a->cu_seqlens; p.seqlen = a->seqlen; p.H = a->nheads; p.G = a->ngroups;
    p.nseq = a->cu_seqlens ? a->nseq : a->batch;
    p.Gth = a->theta_groups ? a->theta_groups : a->nheads;
    p.Bb = a->B_bias; p.Cb = a->C_bias; p.z = (const bf16 *)a->z; p.norm = a->bc_norm; p.eps = a->bc_eps;
    const int64_t nblk = (int64_t)p.nseq * a->nheads;
    if (nblk == 0) return MAMBA3_OK;
    if (hipFuncSetAttribute((const void *)k_scan_mimo<CF>, hipFuncAttributeMaxDynamicSharedMemorySize, CF::LDS) !=
        hipSuccess)
        return MAMBA3_EHIP;
    hipLaunchKernelGGL(k_scan_mimo<CF>, dim3((unsigned)nblk), dim3(CF::NTHR), CF::LDS, st, p);
    return hipGetLastError() == hipSuccess ? MAMBA3_OK : MAMBA3_EHIP;
}

}  // namespace

// The panel kernel serves two rank-4 shapes, plain or with the fused block prologue / epilogue
// (EPI), without the variants (a per-token decay rate, a fixed trapezoid weight):
// (N, P, R, Q) = (128, 64, 4, 128), whose chunk (512 rank-expanded rows) does not fit the general
// kernel's per-wave registers, in 8-wave workgroups over two 64-token panels; and (64, 64, 4, 64)
// in 4-wave workgroups over two 32-token panels (58.6 KB of LDS and about 200 VGPRs: two
// workgroups per CU, where the general kernel fits one). The general bf16 kernel runs everything
// else.
bool scan_mimo_supported(const mamba3_scan_args *a) {
    const int N = a->dstate, P = a->headdim, R = a->rank, Q = a->chunk;
    if (a->dtype != MAMBA3_BF16 || !a->y || !a->A || a->A_tok || !a->lam) return false;
    if (!(P == 64 && R == 4 && ((N == 128 && Q == 128) || (N == 64 && Q == 64)))) return false;
    // token strides (in elements) enter 24-bit products
    const int64_t Gth = a->theta_groups ? a->theta_groups : a->nheads;
    const int64_t lim = (int64_t)1 << 24;
    return (int64_t)a->ngroups * R * N < lim && (int64_t)a->nheads * R * P < lim && Gth * (N / 2) < lim &&
           a->nheads < lim;
}

mamba3_status launch_scan_mimo(const mamba3_scan_args *a, hipStream_t st) {
    const bool epi = a->bc_norm || a->B_bias || a->C_bias || a->z;
    if (a->dstate == 128 && a->chunk == 128)
        return epi ? launch_mimo_cfg<MCfg<128, 64, 4, 128, 8, 64, true, 2, true>>(a, st)
                   : launch_mimo_cfg<MCfg<128, 64, 4, 128, 8, 64>>(a, st);
    if (a->dstate == 64 && a->chunk == 64)
        return epi ? launch_mimo_cfg<MCfg<64, 64, 4, 64, 4, 32, true, 2, true>>(a, st)
                   : launch_mimo_cfg<MCfg<64, 64, 4, 64, 4, 32>>(a, st);
    return MAMBA3_EUNSUPPORTED;
}

}  // namespace m3
