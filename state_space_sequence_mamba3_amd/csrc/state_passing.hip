// State passing between the segments of long sequences.
//
// Across a segment the recurrence of Proposition 4 ("Complex-Valued State
// Space Models") is affine in the state that enters it. Folding the segment's
// first previous-token term into that state, H_start = H_in + delta_0 Bprev
// xprev^T, the segment leaves
//   H_end = exp(S) R(Phi) H_start + U,  S = sum_t dt_t A_t,  Phi[k] = sum_t dt_t theta_t[k],
// where U is the segment scanned from a zero state with no previous token: the
// per-token transitions alpha_t R_t are a scalar decay times rotations of the
// same state pairs, so they commute and multiply to exp(S) R(Phi). This is the
// chunk-state recurrence of the chunked form (section "Parallel
// representation under SSD") taken over segments instead of chunks.
//
// Two kernels. k_segment_sums reduces dt A and dt theta over every segment's
// tokens, all (segment, head) pairs in parallel (fixed order: strided
// per-thread partial sums, then the partials in index order). k_state_passing
// then walks each (sequence, head)'s segments in order with the fp32 state in
// LDS: per segment it writes the entering state and the token before the
// segment, and applies the affine map. The state update is elementwise
// per (pair, column), one thread per element; U and the states are read and
// written as whole rows of P consecutive floats.
//
// Packed batches: sequence s (tokens [cu[s], cu[s+1])) is cut into
// max(1, ceil(len / L)) segments of L tokens, and its segments are the rows
// base_s .. base_s + n_s - 1, base_s counting the segments of the sequences
// before it. k_segment_table writes the rows' token ranges as a cu table (so
// the scans can take the rows as a packed batch); k_state_passing finds
// base_s itself from cu and reduces each segment's sums in the walk unless
// the state-only scan staged them.
#include "m3_common.h"

namespace m3 {

struct SPParams {
    const void *x, *dt, *lam, *theta, *B, *Bprev, *xprev, *A_tok;
    const float *A, *h_in, *Bb, *U;
    float *seg_h, *h_out;
    void *seg_B, *seg_x;
    int32_t seqlen, nseg, H, G, P, N, R, Gth;
    int32_t norm;
    float eps, lam_fixed;
    // packed batches: the sequence table, its length, tokens per segment, the segment rows
    const int32_t *cu;
    int32_t nseq, seg_tokens, rows;
    int32_t sums_inline;   // 1: k_state_passing reduces each segment's sums itself
};

constexpr int kSPThreads = 256;

// LDS layout (floats)
struct SPLayout {
    int hs, phi, bl, xl, misc, sums, total;
};
__host__ __device__ inline SPLayout sp_layout(int N, int P, int R) {
    SPLayout L;
    const int K = N / 2;
    int o = 0;
    L.hs = o; o += N * P;
    L.phi = o; o += 2 * K;   // cos, sin of the segment's total angles
    L.bl = o; o += R * N;
    L.xl = o; o += R * P;
    L.misc = o; o += 4;
    L.sums = o; o += K + 1;   // the segment's sum of dt A, then its angle sums
    L.total = o;
    return L;
}

size_t state_passing_lds_bytes(int N, int P, int R) { return (size_t)sp_layout(N, P, R).total * sizeof(float); }

// S = sum_t dt_t A_t and Phi[k] = sum_t dt_t theta_t[k] over tokens [t0, t0 + Ls) of head h, into
// out[0] and out[1 + k] (global memory or LDS). The whole block of kSPThreads takes part and
// every thread must call it: each thread sums a strided set of tokens, then the partials are
// added in index order (a fixed order).
template <typename T>
__device__ void segment_sums_block(const SPParams &p, int64_t t0, int Ls, int h, float *out) {
    __shared__ float part[kSPThreads], spart[kSPThreads];
    const int H = p.H, K = p.N / 2, tid = threadIdx.x, NT = kSPThreads;
    const int TL = K >= NT ? 1 : NT / K;
    const int gq = h / (H / p.Gth);
    const T *dt = (const T *)p.dt, *th = (const T *)p.theta;
    float a = 0.f;
#pragma unroll 8
    for (int t = tid; t < Ls; t += NT) {
        const int64_t i = (t0 + t) * H + h;
        a += to_f(dt[i]) * (p.A_tok ? to_f(((const T *)p.A_tok)[i]) : p.A[h]);
    }
    spart[tid] = a;
    // angles: with K a multiple of the 16-byte vector (VW elements), thread (token lane j, group q)
    // reads VW consecutive angles of a token per load and keeps VW partial sums
    constexpr int VW = 16 / sizeof(T);
    typedef T vec_t __attribute__((ext_vector_type(VW)));
    __shared__ float vpart[kSPThreads * VW];
    if (K % VW == 0 && K / VW <= NT) {
        const int KG = K / VW, TLV = NT / KG, q = tid % KG, j = tid / KG;
        float acc[VW];
#pragma unroll
        for (int m = 0; m < VW; m++) acc[m] = 0.f;
        if (j < TLV) {
#pragma unroll 4
            for (int t = j; t < Ls; t += TLV) {
                const int64_t tok = t0 + t;
                const float d = to_f(dt[tok * H + h]);
                const vec_t v = *(const vec_t *)(th + (tok * p.Gth + gq) * K + q * VW);
#pragma unroll
                for (int m = 0; m < VW; m++) acc[m] += d * to_f(v[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < VW; m++) vpart[tid * VW + m] = acc[m];   // [j][q][m] = [j][angle]
        __syncthreads();
        if (tid < K) {
            float c = 0.f;
            for (int jj = 0; jj < TLV; jj++) c += vpart[jj * K + tid];
            out[1 + tid] = c;
        }
        __syncthreads();
    } else
    for (int kk = 0; kk < K; kk += NT / TL) {   // pairs [kk, kk + NT / TL) per pass (K > NT only)
        const int i = kk + tid % (NT / TL), j = tid / (NT / TL);
        float b = 0.f;
        if (i < K) {
#pragma unroll 8
            for (int t = j; t < Ls; t += TL) {
                const int64_t tok = t0 + t;
                b += to_f(dt[tok * H + h]) * to_f(th[(tok * p.Gth + gq) * K + i]);
            }
        }
        part[tid] = b;
        __syncthreads();
        if (tid < NT / TL && kk + tid < K) {
            float c = 0.f;
            for (int jj = 0; jj < TL; jj++) c += part[jj * (NT / TL) + tid];
            out[1 + kk + tid] = c;
        }
        __syncthreads();
    }
    if (tid == 0) {
        float c = 0.f;
        for (int jj = 0; jj < NT; jj++) c += spart[jj];
        out[0] = c;
    }
    __syncthreads();   // the partial buffers may be reused at once
}

// Per (segment row, head) of a padded batch: the segment's sums, staged in the first K + 1 floats
// of the segment's seg_h_in block (which k_state_passing reads before it writes the entering
// state there). Every (row, head) runs in parallel.
template <typename T>
__global__ __launch_bounds__(kSPThreads) void k_segment_sums(SPParams p) {
    const int64_t rh = blockIdx.x;                  // row * H + h
    const int h = (int)(rh % p.H);
    const int64_t row = rh / p.H, s = row / p.nseg, k = row % p.nseg;
    const int Ls = p.seqlen / p.nseg;
    segment_sums_block<T>(p, s * p.seqlen + k * Ls, Ls, h, p.seg_h + rh * (int64_t)p.N * p.P);
}

// Tokens [a, b) of packed sequence i, entries clamped to [0, seqlen] as the scans clamp them.
__device__ __forceinline__ void seq_bounds(const int32_t *cu, int i, int seqlen, int &a, int &b) {
    a = min(max(cu[i], 0), seqlen);
    b = min(max(cu[i + 1], a), seqlen);
}
// Segments of a packed sequence of len tokens (one, empty, for an empty sequence).
__device__ __forceinline__ int seq_segments(int len, int L) { return max(1, (int)(((int64_t)len + L - 1) / L)); }

// The segment table of a packed batch: seg_cu[r] = first token of segment row r, for the rows of
// every sequence in order, then the end of the last sequence up to seg_cu[rows] (empty rows). One
// workgroup: the sequences in blocks of 1024, a block-wide scan of their segment counts, and a
// running carry. A write is skipped past the rows' bound (reachable only with entries that are not
// non-decreasing).
constexpr int kTabThreads = 1024;
__global__ __launch_bounds__(kTabThreads) void k_segment_table(const int32_t *cu, int nseq, int seqlen, int L,
                                                               int32_t *seg_cu, int rows) {
    __shared__ int wsum[kTabThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0;
    for (int i0 = 0; i0 < nseq; i0 += kTabThreads) {
        const int i = i0 + tid;
        int a = 0, b = 0, n = 0;
        if (i < nseq) {
            seq_bounds(cu, i, seqlen, a, b);
            n = seq_segments(b - a, L);
        }
        int incl = n;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int woff = 0, tot = 0;
        for (int w = 0; w < kTabThreads / 64; w++) {
            woff += (w < wave) ? wsum[w] : 0;
            tot += wsum[w];
        }
        const int64_t first = (int64_t)carry + woff + incl - n;
        for (int k = 0; k < n; k++)
            if (first + k < rows) seg_cu[first + k] = a + k * L;   // a + k L < b <= seqlen
        carry = (int)min((int64_t)carry + tot, (int64_t)rows);
        __syncthreads();   // wsum is rewritten by the next block
    }
    int endv = 0;
    if (nseq > 0) {
        int a, b;
        seq_bounds(cu, nseq - 1, seqlen, a, b);
        endv = b;
    }
    for (int r = carry + tid; r <= rows; r += kTabThreads) seg_cu[r] = endv;
}

// One workgroup per (sequence, head): the chain over the sequence's segments. With PREF (at most
// PREF_MAX (pair, column) elements per thread) each thread loads its elements of U into registers
// at the start of a segment, so that one memory latency per segment overlaps the staging.
constexpr int PREF_MAX = 16;
template <typename T, int PREF>
__global__ __launch_bounds__(kSPThreads) void k_state_passing(SPParams p) {
    extern __shared__ float smem[];
    const int N = p.N, P = p.P, R = p.R, H = p.H, G = p.G, K = N / 2;
    const SPLayout L = sp_layout(N, P, R);
    float *Hs = smem + L.hs, *PHI = smem + L.phi, *BL = smem + L.bl, *XL = smem + L.xl, *MISC = smem + L.misc;
    float *SUMS = smem + L.sums;
    const int tid = threadIdx.x, NT = kSPThreads;
    const int s = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / G);
    const int64_t NP = (int64_t)N * P;
    const T *dt = (const T *)p.dt;

    // the sequence's tokens, segment length and count, and first segment row
    int64_t a0, len, base;
    int Ls, nsg;
    if (p.cu) {
        int a, b;
        seq_bounds(p.cu, s, p.seqlen, a, b);
        a0 = a;
        len = b - a;
        Ls = p.seg_tokens;
        nsg = seq_segments(b - a, Ls);
        // base: the segments of the sequences before s (per-thread strided counts, then a
        // block reduction)
        __shared__ int cnt[kSPThreads];
        int c = 0;
        for (int j = tid; j < s; j += NT) {
            int aj, bj;
            seq_bounds(p.cu, j, p.seqlen, aj, bj);
            c += seq_segments(bj - aj, Ls);
        }
        cnt[tid] = c;
        __syncthreads();
        int64_t tot = 0;
        for (int j = 0; j < NT; j++) tot += cnt[j];
        base = tot;
    } else {
        a0 = (int64_t)s * p.seqlen;
        len = p.seqlen;
        Ls = p.seqlen / p.nseg;
        nsg = p.nseg;
        base = (int64_t)s * p.nseg;
    }
    // rows past the bound (reachable only with a sequence table that is not non-decreasing) are
    // neither read nor written
    if (p.cu) nsg = (int)max((int64_t)0, min((int64_t)nsg, (int64_t)p.rows - base));

    for (int64_t e = tid; e < NP; e += NT) Hs[e] = p.h_in ? p.h_in[((int64_t)s * H + h) * NP + e] : 0.f;

    for (int k = 0; k < nsg; k++) {
        const int64_t t0 = a0 + (int64_t)k * Ls;                       // first token of the segment
        const int tl = (int)min((int64_t)Ls, len - (int64_t)k * Ls);   // its tokens (0: empty sequence)
        const int64_t row = base + k;                                  // segment row
        float *out = p.seg_h + (row * H + h) * NP;
        const float *Uk = p.U + (row * H + h) * NP;
        float u0r[PREF ? PREF_MAX : 1], u1r[PREF ? PREF_MAX : 1];
        if constexpr (PREF) {
#pragma unroll
            for (int j = 0; j < PREF_MAX; j++) {
                const int e = tid + j * NT;
                if (e < K * P) {
                    const int64_t o0 = (int64_t)(2 * (e / P)) * P + e % P;
                    u0r[j] = Uk[o0];
                    u1r[j] = Uk[o0 + P];
                }
            }
        }
        // the segment's sums: reduced here, or staged in this block of seg_h_in (by k_segment_sums
        // or the state-only scan)
        if (p.sums_inline) {
            segment_sums_block<T>(p, t0, tl, h, SUMS);
        } else {
            for (int i = tid; i <= K; i += NT) SUMS[i] = out[i];
            __syncthreads();
        }
        for (int i = tid; i < K; i += NT) sincosf(SUMS[1 + i], &PHI[K + i], &PHI[i]);
        // the token before the segment: the previous segment's last token, or the sequence's own
        const bool has_prev = k > 0 || p.Bprev;
        const T *bsrc = k > 0 ? (const T *)p.B + ((t0 - 1) * G + g) * R * N
                              : (p.Bprev ? (const T *)p.Bprev + ((int64_t)s * G + g) * R * N : nullptr);
        const T *xsrc = k > 0 ? (const T *)p.x + ((t0 - 1) * H + h) * R * P
                              : (p.xprev ? (const T *)p.xprev + ((int64_t)s * H + h) * R * P : nullptr);
        for (int e = tid; e < R * N; e += NT) {
            const T v = has_prev ? bsrc[e] : from_f<T>(0.f);
            BL[e] = to_f(v);
            if (h % (H / G) == 0) ((T *)p.seg_B)[(row * G + g) * R * N + e] = v;   // one head per group writes
        }
        for (int e = tid; e < R * P; e += NT) {
            const T v = has_prev ? xsrc[e] : from_f<T>(0.f);
            XL[e] = to_f(v);
            ((T *)p.seg_x)[(row * H + h) * R * P + e] = v;
        }
        if (tid == 0) {
            MISC[0] = expf(SUMS[0]);
            // delta of the first token (none in an empty segment, which leaves the state as it is)
            float d0 = 0.f;
            if (has_prev && tl > 0) {
                const float lam = p.lam ? to_f(((const T *)p.lam)[t0 * H + h]) : p.lam_fixed;
                d0 = (1.f - lam) * to_f(dt[t0 * H + h]);
            }
            MISC[1] = d0;
        }
        __syncthreads();   // the sums are read: the block of seg_h_in may now be overwritten
        // prologue on the folded previous token: unit-RMS columns and the head's bias, as the scan does
        if (has_prev && (p.norm || p.Bb)) {
            if (tid < R) {
                float *col = BL + tid * N;
                float inv = 1.f;
                if (p.norm) {
                    float ss = 0.f;
                    for (int n = 0; n < N; n++) ss += col[n] * col[n];
                    inv = 1.f / sqrtf(ss / N + p.eps);
                }
                for (int n = 0; n < N; n++) col[n] = col[n] * inv + (p.Bb ? p.Bb[(int64_t)h * N + n] : 0.f);
            }
            __syncthreads();
        }
        // entering state out, then H <- exp(S) R(Phi) (H + delta_0 Bprev xprev^T) + U
        const float decay = MISC[0], d0 = MISC[1];
        auto update = [&](int e, float U0, float U1) {
            const int i = e / P, c = e % P;
            const int64_t o0 = (int64_t)(2 * i) * P + c, o1 = o0 + P;
            float u0 = Hs[o0], u1 = Hs[o1];
            out[o0] = u0;
            out[o1] = u1;
            float f0 = 0.f, f1 = 0.f;
            for (int r = 0; r < R; r++) {
                f0 += BL[r * N + 2 * i] * XL[r * P + c];
                f1 += BL[r * N + 2 * i + 1] * XL[r * P + c];
            }
            u0 += d0 * f0;
            u1 += d0 * f1;
            const float cs = PHI[i], sn = PHI[K + i];
            Hs[o0] = decay * (cs * u0 - sn * u1) + U0;
            Hs[o1] = decay * (sn * u0 + cs * u1) + U1;
        };
        if constexpr (PREF) {
#pragma unroll
            for (int j = 0; j < PREF_MAX; j++)
                if (tid + j * NT < K * P) update(tid + j * NT, u0r[j], u1r[j]);
        } else {
            for (int e = tid; e < K * P; e += NT) {
                const int64_t o0 = (int64_t)(2 * (e / P)) * P + e % P;
                update(e, Uk[o0], Uk[o0 + P]);
            }
        }
        __syncthreads();   // PHI, BL, XL, MISC are rewritten by the next segment
    }
    if (p.h_out)
        for (int64_t e = tid; e < NP; e += NT) p.h_out[((int64_t)s * H + h) * NP + e] = Hs[e];
}

mamba3_status launch_state_passing(const mamba3_state_passing_args *a, hipStream_t st, bool sums_staged) {
    const mamba3_scan_args *f = &a->fwd;
    SPParams p;
    p.x = f->x; p.dt = f->dt; p.lam = f->lam; p.theta = f->theta; p.B = f->B;
    p.Bprev = f->Bprev; p.xprev = f->xprev; p.A_tok = f->A_tok;
    p.A = f->A; p.h_in = f->h_in; p.Bb = f->B_bias; p.U = a->U;
    p.seg_h = a->seg_h_in; p.h_out = a->h_out; p.seg_B = a->seg_Bprev; p.seg_x = a->seg_xprev;
    p.seqlen = f->seqlen; p.nseg = a->nseg; p.H = f->nheads; p.G = f->ngroups; p.P = f->headdim;
    p.N = f->dstate; p.R = f->rank; p.Gth = f->theta_groups ? f->theta_groups : f->nheads;
    p.norm = f->bc_norm; p.eps = f->bc_eps; p.lam_fixed = f->lam_fixed;
    const bool packed = f->cu_seqlens != nullptr;
    p.cu = f->cu_seqlens; p.nseq = packed ? f->nseq : 0; p.seg_tokens = packed ? a->seg_tokens : 0;
    p.rows = packed ? (int32_t)segment_rows_packed(f->nseq, f->seqlen, a->seg_tokens) : f->batch * a->nseg;
    // packed batches reduce the segment sums in the walk (their rows are not known on the host)
    p.sums_inline = packed && !sums_staged;
    const int64_t nblk = (int64_t)(packed ? f->nseq : f->batch) * f->nheads;
    if (nblk == 0) return MAMBA3_OK;
    const size_t lds = state_passing_lds_bytes(p.N, p.P, p.R);
    const bool pref = (int64_t)(p.N / 2) * p.P <= (int64_t)PREF_MAX * kSPThreads;
    const int64_t nrow = packed ? 0 : nblk * a->nseg;   // (segment row, head) pairs of k_segment_sums
    auto chain = [&](auto kern) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return false;
        hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(kSPThreads), lds, st, p);
        return true;
    };
    bool ok;
    if (f->dtype == MAMBA3_BF16) {
        if (nrow && !sums_staged) hipLaunchKernelGGL(k_segment_sums<bf16>, dim3((unsigned)nrow), dim3(kSPThreads), 0, st, p);
        ok = pref ? chain(k_state_passing<bf16, 1>) : chain(k_state_passing<bf16, 0>);
    } else {
        if (nrow && !sums_staged) hipLaunchKernelGGL(k_segment_sums<float>, dim3((unsigned)nrow), dim3(kSPThreads), 0, st, p);
        ok = pref ? chain(k_state_passing<float, 1>) : chain(k_state_passing<float, 0>);
    }
    if (!ok) return MAMBA3_EHIP;
    return hipGetLastError() == hipSuccess ? MAMBA3_OK : MAMBA3_EHIP;
}

int64_t segment_rows_packed(int64_t nseq, int64_t seqlen, int64_t seg_tokens) {
    return seg_tokens >= 1 ? nseq + (seqlen + seg_tokens - 1) / seg_tokens : 0;
}

mamba3_status launch_segment_table(const int32_t *cu, int32_t nseq, int32_t seqlen, int32_t seg_tokens,
                                   int32_t *seg_cu, hipStream_t st) {
    const int64_t rows = segment_rows_packed(nseq, seqlen, seg_tokens);
    hipLaunchKernelGGL(k_segment_table, dim3(1), dim3(kTabThreads), 0, st, cu, nseq, seqlen, seg_tokens, seg_cu,
                       (int)rows);
    return hipGetLastError() == hipSuccess ? MAMBA3_OK : MAMBA3_EHIP;
}

}  // namespace m3
