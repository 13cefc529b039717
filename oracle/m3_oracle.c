/*
 * Mamba-3 SSM recurrence: plain, slow, fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and
 * its Python binding) may link, load or call this file. Only the tests, the
 * smoke check and the CPU-baseline leg of the bench use it. It shares no code,
 * header, table or helper with the GPU path.
 *
 * What it computes (the pages' statement of the layer, written out directly):
 *
 *   per sequence s, head h (group g = h / (H/G)), token t of that sequence:
 *     alpha_t = exp(dt_t A_h)                       (discretised decay)
 *     delta_t = (1 - lam_t) dt_t,  beta_t = delta_t alpha_t,  gamma_t = lam_t dt_t
 *     angle_t[k] = dt_t theta_t[k]  for k < N/2     (rotation of state pair k)
 *     h_t = alpha_t R_t h_{t-1} + beta_t R_t B_{t-1} X_{t-1}^T + gamma_t B_t X_t^T
 *     y_t = H_t^T C_t + D_h X_t                      (P x R output)
 *   "Mamba-3" paper summary, sections "Exponential-Trapezoidal Discretization"
 *   (Proposition 1: the three-term update and its alpha, beta, gamma),
 *   "Complex-Valued State Space Models" (Proposition 2: complex diagonal
 *   transition = real block-diagonal rotation; Proposition 4: the
 *   exponential-trapezoidal complex recurrence), "MIMO Formulation"
 *   (B_t in R^{N x R}, X_t in R^{P x R}, rank-R update B_t X_t^T, output
 *   y_t = H_t^T C_t in R^{P x R}).
 *
 * Three independent forms are provided; the tests pin them against each other
 * and against closed forms:
 *   O1  m3o_scan_o1   : complex state in C^{N/2 x P}, physical frame, the
 *                       transition exp(dt (A + i theta)) applied directly.
 *   O2  m3o_scan_o2   : Proposition 4 literally - real state in the rotated
 *                       frame, cumulative rotations from the sequence start
 *                       absorbed into B and C ("RoPE trick", Proposition 3).
 *   O3  m3o_scan_o3   : the SSD matrix form Y = (L o C~ B~^T) X with
 *                       L = L1 L2 materialised (1-semiseparable decay times
 *                       the 2-band trapezoid matrix), section "Parallel
 *                       representation under SSD", Figure 1.
 *   O3C m3o_scan_chunked : the same matrix form inside chunks of Q tokens,
 *                       with the state carried from chunk to chunk (the
 *                       parallel-within, recurrent-across-chunks reading of
 *                       that section): per chunk, B and C are rotated by the
 *                       chunk-local cumulative angle, L = L1 L2 is the
 *                       chunk's own, the state entering the chunk (with the
 *                       previous token's term folded in) decays into every
 *                       output and into the chunk's final state, which is
 *                       rotated back to the physical frame.
 *
 * Readings taken where the pages leave a step open:
 *   - State pair k is rows (2k, 2k+1) of the real state; the complex value is
 *     h[2k] + i h[2k+1]; B's complex entry is B[2k] + i B[2k+1]; since the real
 *     form stacks C as [C; -C^], C's complex entry is C[2k] - i C[2k+1].
 *   - theta is the raw per-token frequency; the applied angle is dt * theta.
 *   - A sequence start has a zero state and no previous-token term unless a
 *     state h_in and a previous token (Bprev, xprev) are given (resume).
 *   - D is a per-head skip term y += D_h X_t (absent from the pages).
 *   - MIMO: the rotation acts on the N axis identically for every rank column.
 *
 * Optional block prologue and epilogue (section "Architectural Integration"):
 * every B and C column (N values of one token, group and rank) may be scaled
 * to unit root-mean-square and then get its head's per-channel bias added,
 * before the rotation, for the current and the previous token alike; the
 * output may be gated, y <- y * SiLU(z). Readings: the norm has no gain and
 * normalizes each rank column of B_t, C_t separately; the bias is [H, N],
 * shared by the rank columns; the skip term D x is added before the gate.
 *
 * Variants (section "The Complex-Valued A Parameterization", Remark 1; Table 8
 * of the paper listing): a per-token decay rate A_t [T, H] replaces the head's
 * A (alpha_t = exp(dt_t A_t)), and a fixed trapezoid weight replaces the
 * per-token lam (lam = 1/2 is the classical trapezoid, lam = 1 exponential-
 * Euler). The angle rows may also be shared by groups of heads (th_groups
 * rows per token, head h reading row h / (H / th_groups), as B and C are
 * shared by groups); the pages state no angle sharing, so this is a layout
 * option only, and with one row per head it is the per-head form above.
 *
 * Inputs are read through a dtype tag (f64, f32, bf16 bits) and converted
 * exactly to double; all arithmetic is in double / double complex.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { M3O_F64 = 0, M3O_F32 = 1, M3O_BF16 = 2 };

typedef struct {
    int32_t nseq;              /* number of sequences */
    const int64_t *seq_start;  /* [nseq] first token of each sequence (flat token axis) */
    const int64_t *seq_len;    /* [nseq] tokens in each sequence */
    int32_t H, G, P, N, R;     /* heads, B/C groups, head dim, state dim (even), rank */
    int32_t in_dtype;          /* dtype tag of x, dt, lam, theta, B, C, Bprev, xprev */
    const void *x;             /* [T, H, R, P] */
    const void *dt;            /* [T, H] (post-softplus step) */
    const void *lam;           /* [T, H] (trapezoid weight in [0,1]) */
    const void *theta;         /* [T, Gth, N/2] (rotation frequency; Gth = H unless th_groups says) */
    const void *B;             /* [T, G, R, N] */
    const void *C;             /* [T, G, R, N] */
    const double *A;           /* [H], negative */
    const double *D;           /* [H] or NULL */
    const double *h_in;        /* [nseq, H, N, P] or NULL (zero state) */
    const void *Bprev;         /* [nseq, G, R, N] or NULL (no previous token) */
    const void *xprev;         /* [nseq, H, R, P] or NULL */
    /* Block prologue and epilogue around the recurrence (section "Architectural
     * Integration": BC normalization, BC biases, output gating): */
    const double *B_bias;      /* [H, N] per-head bias added to B after the norm, or NULL */
    const double *C_bias;      /* [H, N] per-head bias added to C after the norm, or NULL */
    const void *z;             /* [T, H, R, P] gate (dtype in_dtype), or NULL: y <- y * SiLU(z) */
    int32_t bc_norm;           /* 1: every B and C column (N values) is scaled to unit RMS */
    double bc_eps;             /* added to the mean square under the root */
    /* Variants: */
    const void *A_tok;         /* [T, H] per-token decay rate A_t (dtype in_dtype), or NULL: A[h] */
    double lam_fixed;          /* the trapezoid weight of every token when lam is NULL */
    int32_t th_groups;         /* angle rows per token, Gth (0 = H): heads h*Gth/H share one, as B/C groups do */
} m3o_args;

static inline double ld(const void *p, int dt, int64_t i) {
    if (dt == M3O_F64) return ((const double *)p)[i];
    if (dt == M3O_F32) return (double)((const float *)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Flat index of angle k of head h at token t: head h reads the angle row of
 * its group h / (H / Gth), exactly as it reads the B/C row of group h / (H / G). */
static inline int64_t th_at(const m3o_args *a, int64_t t, int h, int k) {
    const int Gth = a->th_groups ? a->th_groups : a->H, K = a->N / 2;
    return (t * Gth + h / (a->H / Gth)) * K + k;
}

/* One N-vector of B or C as the recurrence sees it: the raw column at src[off ..
 * off + N), scaled to unit root-mean-square when bc_norm is set (RMSNorm without a
 * gain), then the head's bias added (section "Architectural Integration": BC
 * normalization after the projection, then learned per-head, per-channel biases). */
static void bc_row(const m3o_args *a, const void *src, int64_t off, int h, const double *bias, double *out) {
    const int N = a->N;
    double ss = 0.0;
    for (int n = 0; n < N; n++) {
        out[n] = ld(src, a->in_dtype, off + n);
        ss += out[n] * out[n];
    }
    if (a->bc_norm) {
        const double inv = 1.0 / sqrt(ss / N + a->bc_eps);
        for (int n = 0; n < N; n++) out[n] *= inv;
    }
    if (bias)
        for (int n = 0; n < N; n++) out[n] += bias[(int64_t)h * N + n];
}

/* The token's trapezoid weight lam_t, or the fixed one when no lam array is given
 * (the fixed-lambda variants, Table 8 of the paper listing: lam = 1/2, lam = 1). */
static inline double lam_of(const m3o_args *a, int64_t i) {
    return a->lam ? ld(a->lam, a->in_dtype, i) : a->lam_fixed;
}
/* The token's decay rate A_t (data-dependent A, Remark 1, section "The Complex-Valued A
 * Parameterization"), or the head's A when no per-token array is given. i = t * H + h. */
static inline double A_of(const m3o_args *a, int64_t i, int h) {
    return a->A_tok ? ld(a->A_tok, a->in_dtype, i) : a->A[h];
}

/* Output gating: y * SiLU(z) with SiLU(v) = v / (1 + e^{-v}) (section
 * "Architectural Integration", output gating); y itself when there is no gate. */
static inline double gate(const m3o_args *a, double y, int64_t zi) {
    if (!a->z) return y;
    const double v = ld(a->z, a->in_dtype, zi);
    return y * v / (1.0 + exp(-v));
}

/* ---------------------------------------------------------------- O1 ---- */
/* Complex physical-frame recurrence for one (sequence, head) slab.
 * y_slab: [len, R, P]; h_slab: [N, P] (may be NULL). */
static void o1_slab(const m3o_args *a, int s, int h, double *y_slab, double *h_slab) {
    const int H = a->H, G = a->G, P = a->P, N = a->N, R = a->R, K = N / 2;
    const int g = h / (H / G);
    const int dtp = a->in_dtype;
    const int64_t t0 = a->seq_start[s], len = a->seq_len[s];
    double complex *hc = calloc((size_t)K * P, sizeof *hc);   /* state   [K][P] */
    double complex *bp = calloc((size_t)K * R, sizeof *bp);   /* prev b  [K][R] */
    double *xp = calloc((size_t)P * R, sizeof *xp);           /* prev x  [P][R] */
    double complex *bc = malloc((size_t)K * R * sizeof *bc);  /* cur b   [K][R] */
    double complex *cc = malloc((size_t)K * R * sizeof *cc);  /* cur c   [K][R] */
    double *xc = malloc((size_t)P * R * sizeof *xc);          /* cur x   [P][R] */
    double complex *z = malloc((size_t)K * sizeof *z);
    double *row = malloc((size_t)N * sizeof *row), *row2 = malloc((size_t)N * sizeof *row2);
    int has_prev = 0;

    if (a->h_in) {
        const double *hi = a->h_in + ((int64_t)s * H + h) * N * P;
        for (int k = 0; k < K; k++)
            for (int p = 0; p < P; p++)
                hc[k * P + p] = hi[(2 * k) * P + p] + I * hi[(2 * k + 1) * P + p];
    }
    if (a->Bprev && a->xprev) {
        has_prev = 1;
        int64_t ob = ((int64_t)s * G + g) * N * R, ox = ((int64_t)s * H + h) * P * R;
        for (int j = 0; j < R; j++) {
            bc_row(a, a->Bprev, ob + j * N, h, a->B_bias, row);
            for (int k = 0; k < K; k++) bp[k * R + j] = row[2 * k] + I * row[2 * k + 1];
        }
        for (int p = 0; p < P; p++)
            for (int j = 0; j < R; j++) xp[p * R + j] = ld(a->xprev, dtp, ox + j * P + p);
    }
    const double Dh = a->D ? a->D[h] : 0.0;

    for (int64_t tt = 0; tt < len; tt++) {
        const int64_t t = t0 + tt;
        const double dt = ld(a->dt, dtp, t * H + h);
        const double lam = lam_of(a, t * H + h);
        const double delta = (1.0 - lam) * dt, gamma = lam * dt;
        const double decay = exp(dt * A_of(a, t * H + h, h));
        for (int k = 0; k < K; k++) {
            double ang = dt * ld(a->theta, dtp, th_at(a, t, h, k));
            z[k] = decay * (cos(ang) + I * sin(ang));
        }
        const int64_t ob = (t * G + g) * N * R, ox = (t * H + h) * P * R;
        for (int j = 0; j < R; j++) {
            bc_row(a, a->B, ob + j * N, h, a->B_bias, row);
            bc_row(a, a->C, ob + j * N, h, a->C_bias, row2);
            for (int k = 0; k < K; k++) {
                bc[k * R + j] = row[2 * k] + I * row[2 * k + 1];
                cc[k * R + j] = row2[2 * k] - I * row2[2 * k + 1];
            }
        }
        for (int p = 0; p < P; p++)
            for (int j = 0; j < R; j++) xc[p * R + j] = ld(a->x, dtp, ox + j * P + p);

        /* h <- z (h + delta b_prev x_prev^T) + gamma b x^T */
        for (int k = 0; k < K; k++)
            for (int p = 0; p < P; p++) {
                double complex prev = 0, cur = 0;
                for (int j = 0; j < R; j++) {
                    if (has_prev) prev += bp[k * R + j] * xp[p * R + j];
                    cur += bc[k * R + j] * xc[p * R + j];
                }
                hc[k * P + p] = z[k] * (hc[k * P + p] + delta * prev) + gamma * cur;
            }
        /* y[i][p] = Re sum_k c[k][i] h[k][p] + D x[p][i] */
        double *yt = y_slab + tt * P * R;
        for (int p = 0; p < P; p++)
            for (int i = 0; i < R; i++) {
                double complex acc = 0;
                for (int k = 0; k < K; k++) acc += cc[k * R + i] * hc[k * P + p];
                yt[i * P + p] = gate(a, creal(acc) + Dh * xc[p * R + i], ox + i * P + p);
            }
        memcpy(bp, bc, (size_t)K * R * sizeof *bp);
        memcpy(xp, xc, (size_t)P * R * sizeof *xp);
        has_prev = 1;
    }
    if (h_slab)
        for (int k = 0; k < K; k++)
            for (int p = 0; p < P; p++) {
                h_slab[(2 * k) * P + p] = creal(hc[k * P + p]);
                h_slab[(2 * k + 1) * P + p] = cimag(hc[k * P + p]);
            }
    free(hc); free(bp); free(xp); free(bc); free(cc); free(xc); free(z); free(row); free(row2);
}

/* ---------------------------------------------------------------- O2 ---- */
/* Proposition 4 literally: real state h~ in the frame rotated by the
 * cumulative angle Psi_t = sum_{i<=t} dt_i theta_i (the product of R_i^T over
 * i = 0..t), B and C rotated by R(-Psi_t), a real scalar transition alpha_t;
 * the previous-token input carries the previous token's rotation R(-Psi_{t-1}).
 * The physical state is recovered at the end as h = R(Psi_T) h~. */
static void rot_vec(double *dst, const double *src, const double *psi, int K, int R, int sign) {
    /* dst[2k][j], dst[2k+1][j] = R(sign*psi[k]) applied to (src[2k][j], src[2k+1][j]) */
    for (int k = 0; k < K; k++) {
        double c = cos(psi[k]), sn = sign * sin(psi[k]);
        for (int j = 0; j < R; j++) {
            double u = src[(2 * k) * R + j], v = src[(2 * k + 1) * R + j];
            dst[(2 * k) * R + j] = c * u - sn * v;
            dst[(2 * k + 1) * R + j] = sn * u + c * v;
        }
    }
}

static void o2_slab(const m3o_args *a, int s, int h, double *y_slab, double *h_slab) {
    const int H = a->H, G = a->G, P = a->P, N = a->N, R = a->R, K = N / 2;
    const int g = h / (H / G);
    const int dtp = a->in_dtype;
    const int64_t t0 = a->seq_start[s], len = a->seq_len[s];
    double *hr = calloc((size_t)N * P, sizeof *hr);      /* rotated-frame state [N][P] */
    double *psi = calloc((size_t)K, sizeof *psi);        /* cumulative angle */
    double *braw = malloc((size_t)N * R * sizeof *braw), *craw = malloc((size_t)N * R * sizeof *craw);
    double *brot = malloc((size_t)N * R * sizeof *brot), *crot = malloc((size_t)N * R * sizeof *crot);
    double *bprot = calloc((size_t)N * R, sizeof *bprot); /* previous token's rotated B */
    double *xp = calloc((size_t)P * R, sizeof *xp), *xc = malloc((size_t)P * R * sizeof *xc);
    double *rowb = malloc((size_t)N * sizeof *rowb), *rowc = malloc((size_t)N * sizeof *rowc);
    int has_prev = 0;

    /* Before the first token the cumulative product is empty: h~ = h_in. */
    if (a->h_in) memcpy(hr, a->h_in + ((int64_t)s * H + h) * N * P, (size_t)N * P * sizeof *hr);
    if (a->Bprev && a->xprev) {
        has_prev = 1;
        int64_t ob = ((int64_t)s * G + g) * N * R, ox = ((int64_t)s * H + h) * P * R;
        double *row = malloc((size_t)N * sizeof *row);
        for (int j = 0; j < R; j++) {
            bc_row(a, a->Bprev, ob + j * N, h, a->B_bias, row);
            for (int n = 0; n < N; n++) bprot[n * R + j] = row[n];
        }
        free(row);
        for (int p = 0; p < P; p++)
            for (int j = 0; j < R; j++) xp[p * R + j] = ld(a->xprev, dtp, ox + j * P + p);
    }
    const double Dh = a->D ? a->D[h] : 0.0;

    for (int64_t tt = 0; tt < len; tt++) {
        const int64_t t = t0 + tt;
        const double dt = ld(a->dt, dtp, t * H + h);
        const double lam = lam_of(a, t * H + h);
        const double alpha = exp(dt * A_of(a, t * H + h, h));
        const double beta = (1.0 - lam) * dt * alpha, gamma = lam * dt;
        for (int k = 0; k < K; k++) psi[k] += dt * ld(a->theta, dtp, th_at(a, t, h, k));
        const int64_t ob = (t * G + g) * N * R, ox = (t * H + h) * P * R;
        for (int j = 0; j < R; j++) {
            bc_row(a, a->B, ob + j * N, h, a->B_bias, rowb);
            bc_row(a, a->C, ob + j * N, h, a->C_bias, rowc);
            for (int n = 0; n < N; n++) {
                braw[n * R + j] = rowb[n];
                craw[n * R + j] = rowc[n];
            }
        }
        for (int p = 0; p < P; p++)
            for (int j = 0; j < R; j++) xc[p * R + j] = ld(a->x, dtp, ox + j * P + p);
        rot_vec(brot, braw, psi, K, R, -1);
        rot_vec(crot, craw, psi, K, R, -1);
        for (int n = 0; n < N; n++)
            for (int p = 0; p < P; p++) {
                double prev = 0, cur = 0;
                for (int j = 0; j < R; j++) {
                    if (has_prev) prev += bprot[n * R + j] * xp[p * R + j];
                    cur += brot[n * R + j] * xc[p * R + j];
                }
                hr[n * P + p] = alpha * hr[n * P + p] + beta * prev + gamma * cur;
            }
        double *yt = y_slab + tt * P * R;
        for (int p = 0; p < P; p++)
            for (int i = 0; i < R; i++) {
                double acc = 0;
                for (int n = 0; n < N; n++) acc += crot[n * R + i] * hr[n * P + p];
                yt[i * P + p] = gate(a, acc + Dh * xc[p * R + i], ox + i * P + p);
            }
        memcpy(bprot, brot, (size_t)N * R * sizeof *bprot);
        memcpy(xp, xc, (size_t)P * R * sizeof *xp);
        has_prev = 1;
    }
    if (h_slab) {
        /* h = R(Psi_T) h~ on every state pair and column */
        for (int k = 0; k < K; k++) {
            double c = cos(psi[k]), sn = sin(psi[k]);
            for (int p = 0; p < P; p++) {
                double u = hr[(2 * k) * P + p], v = hr[(2 * k + 1) * P + p];
                h_slab[(2 * k) * P + p] = c * u - sn * v;
                h_slab[(2 * k + 1) * P + p] = sn * u + c * v;
            }
        }
    }
    free(hr); free(psi); free(braw); free(craw); free(brot); free(crot); free(rowb); free(rowc);
    free(bprot); free(xp); free(xc);
}

/* ---------------------------------------------------------------- O3 ---- */
/* SSD matrix form for one slab starting from a zero state with no previous
 * token (the pages unroll from h_0 = gamma_0 B_0 x_0):
 *   L1[t][s] = prod_{k=s+1..t} alpha_k (s <= t), L2 = diag(gamma) + subdiag(beta)
 *   L = L1 L2,   Y[t][p][i] = sum_s sum_j L[t][s] (C~_t[:,i] . B~_s[:,j]) X_s[p][j]
 * with B~, C~ rotated by the cumulative angle of their own token. O(len^2). */
static void o3_slab(const m3o_args *a, int s, int h, double *y_slab) {
    const int H = a->H, G = a->G, P = a->P, N = a->N, R = a->R, K = N / 2;
    const int g = h / (H / G);
    const int dtp = a->in_dtype;
    const int64_t t0 = a->seq_start[s], T = a->seq_len[s];
    double *alpha = malloc(T * sizeof *alpha), *beta = malloc(T * sizeof *beta), *gamma = malloc(T * sizeof *gamma);
    double *L1 = calloc(T * T, sizeof *L1), *L2 = calloc(T * T, sizeof *L2), *L = calloc(T * T, sizeof *L);
    double *Bt = malloc(T * N * R * sizeof *Bt), *Ct = malloc(T * N * R * sizeof *Ct);
    double *X = malloc(T * P * R * sizeof *X);
    double *psi = calloc(K, sizeof *psi), *tmp = malloc((size_t)N * R * sizeof *tmp);
    double *row = malloc((size_t)N * sizeof *row);
    const double Dh = a->D ? a->D[h] : 0.0;

    for (int64_t t = 0; t < T; t++) {
        const int64_t tg = t0 + t;
        double dt = ld(a->dt, dtp, tg * H + h), lam = lam_of(a, tg * H + h);
        alpha[t] = exp(dt * A_of(a, tg * H + h, h));
        beta[t] = (1.0 - lam) * dt * alpha[t];
        gamma[t] = lam * dt;
        for (int k = 0; k < K; k++) psi[k] += dt * ld(a->theta, dtp, th_at(a, tg, h, k));
        const int64_t ob = (tg * G + g) * N * R, ox = (tg * H + h) * P * R;
        for (int j = 0; j < R; j++) {
            bc_row(a, a->B, ob + j * N, h, a->B_bias, row);
            for (int n = 0; n < N; n++) tmp[n * R + j] = row[n];
        }
        rot_vec(Bt + t * N * R, tmp, psi, K, R, -1);
        for (int j = 0; j < R; j++) {
            bc_row(a, a->C, ob + j * N, h, a->C_bias, row);
            for (int n = 0; n < N; n++) tmp[n * R + j] = row[n];
        }
        rot_vec(Ct + t * N * R, tmp, psi, K, R, -1);
        for (int p = 0; p < P; p++)
            for (int j = 0; j < R; j++) X[t * P * R + p * R + j] = ld(a->x, dtp, ox + j * P + p);
    }
    for (int64_t t = 0; t < T; t++) {
        double prod = 1.0;
        for (int64_t s2 = t; s2 >= 0; s2--) {
            L1[t * T + s2] = prod;
            prod *= alpha[s2];
        }
        L2[t * T + t] = gamma[t];
        if (t > 0) L2[t * T + t - 1] = beta[t];
    }
    for (int64_t t = 0; t < T; t++)
        for (int64_t s2 = 0; s2 < T; s2++) {
            double acc = 0;
            for (int64_t k = 0; k < T; k++) acc += L1[t * T + k] * L2[k * T + s2];
            L[t * T + s2] = acc;
        }
    for (int64_t t = 0; t < T; t++)
        for (int p = 0; p < P; p++)
            for (int i = 0; i < R; i++) {
                double acc = 0;
                for (int64_t s2 = 0; s2 < T; s2++) {
                    if (L[t * T + s2] == 0.0) continue;
                    for (int j = 0; j < R; j++) {
                        double cb = 0;
                        for (int n = 0; n < N; n++) cb += Ct[t * N * R + n * R + i] * Bt[s2 * N * R + n * R + j];
                        acc += L[t * T + s2] * cb * X[s2 * P * R + p * R + j];
                    }
                }
                y_slab[t * P * R + i * P + p] =
                    gate(a, acc + Dh * X[t * P * R + p * R + i], ((t0 + t) * H + h) * P * R + i * P + p);
            }
    free(alpha); free(beta); free(gamma); free(L1); free(L2); free(L);
    free(Bt); free(Ct); free(X); free(psi); free(tmp); free(row);
}

/* --------------------------------------------------------------- O3C ---- */
/* Chunked SSD form for one slab, chunk size Q >= 1. In a chunk of tokens c0 .. e, with
 * Phi_t = sum_{k=c0..t} dt_k theta_k (chunk-local, the frame before c0 being the physical one),
 * B~_t = R(-Phi_t) B_t, C~_t = R(-Phi_t) C_t and the chunk's own L = L1 L2 (L1[t][s] = prod_{k=s+1..t}
 * alpha_k, L2 = diag(gamma) + subdiag(beta), both over the chunk's tokens only), Proposition 4
 * unrolls to
 *   H_start = H_{c0-1} + delta_{c0} B_{c0-1} X_{c0-1}^T      (the previous token, if any)
 *   y_t     = C~_t^T (prod_{k=c0..t} alpha_k) H_start + sum_{s=c0..t} L[t][s] (C~_t . B~_s) X_s + D X_t
 *   H_e     = R(Phi_e) [ (prod_{k=c0..e} alpha_k) H_start + sum_{s=c0..e} L[e][s] B~_s X_s^T ]
 * H is the real physical-frame state [N][P]; the gate applies to y as in the other forms. */
static void o3c_slab(const m3o_args *a, int Q, int s, int h, double *y_slab, double *h_slab) {
    const int H = a->H, G = a->G, P = a->P, N = a->N, R = a->R, K = N / 2;
    const int g = h / (H / G);
    const int dtp = a->in_dtype;
    const int64_t t0 = a->seq_start[s], len = a->seq_len[s];
    double *Hs = calloc((size_t)N * P, sizeof *Hs);                      /* state entering the chunk */
    double *Bprev = calloc((size_t)N * R, sizeof *Bprev), *Xprev = calloc((size_t)P * R, sizeof *Xprev);
    double *alpha = malloc((size_t)Q * sizeof *alpha), *beta = malloc((size_t)Q * sizeof *beta);
    double *gamma = malloc((size_t)Q * sizeof *gamma), *delta = malloc((size_t)Q * sizeof *delta);
    double *L1 = malloc((size_t)Q * Q * sizeof *L1), *L2 = malloc((size_t)Q * Q * sizeof *L2), *L = malloc((size_t)Q * Q * sizeof *L);
    double *Braw = malloc((size_t)Q * N * R * sizeof *Braw), *Bt = malloc((size_t)Q * N * R * sizeof *Bt);
    double *Ct = malloc((size_t)Q * N * R * sizeof *Ct), *X = malloc((size_t)Q * P * R * sizeof *X);
    double *psi = malloc((size_t)K * sizeof *psi), *tmp = malloc((size_t)N * R * sizeof *tmp);
    double *row = malloc((size_t)N * sizeof *row), *Hn = malloc((size_t)N * P * sizeof *Hn);
    int has_prev = 0;
    const double Dh = a->D ? a->D[h] : 0.0;

    if (a->h_in) memcpy(Hs, a->h_in + ((int64_t)s * H + h) * N * P, (size_t)N * P * sizeof *Hs);
    if (a->Bprev && a->xprev) {
        has_prev = 1;
        const int64_t ob = ((int64_t)s * G + g) * N * R, ox = ((int64_t)s * H + h) * P * R;
        for (int j = 0; j < R; j++) {
            bc_row(a, a->Bprev, ob + j * N, h, a->B_bias, row);
            for (int n = 0; n < N; n++) Bprev[n * R + j] = row[n];
        }
        for (int p = 0; p < P; p++)
            for (int j = 0; j < R; j++) Xprev[p * R + j] = ld(a->xprev, dtp, ox + j * P + p);
    }
    for (int64_t c0 = 0; c0 < len; c0 += Q) {
        const int nq = (int)((len - c0 < Q) ? len - c0 : Q);
        for (int k = 0; k < K; k++) psi[k] = 0.0;
        for (int t = 0; t < nq; t++) {
            const int64_t tg = t0 + c0 + t;
            const double dt = ld(a->dt, dtp, tg * H + h), lam = lam_of(a, tg * H + h);
            alpha[t] = exp(dt * A_of(a, tg * H + h, h));
            delta[t] = (1.0 - lam) * dt;
            beta[t] = delta[t] * alpha[t];
            gamma[t] = lam * dt;
            for (int k = 0; k < K; k++) psi[k] += dt * ld(a->theta, dtp, th_at(a, tg, h, k));
            const int64_t ob = (tg * G + g) * N * R, ox = (tg * H + h) * P * R;
            for (int j = 0; j < R; j++) {
                bc_row(a, a->B, ob + j * N, h, a->B_bias, row);
                for (int n = 0; n < N; n++) Braw[t * N * R + n * R + j] = row[n];
            }
            rot_vec(Bt + t * N * R, Braw + t * N * R, psi, K, R, -1);
            for (int j = 0; j < R; j++) {
                bc_row(a, a->C, ob + j * N, h, a->C_bias, row);
                for (int n = 0; n < N; n++) tmp[n * R + j] = row[n];
            }
            rot_vec(Ct + t * N * R, tmp, psi, K, R, -1);
            for (int p = 0; p < P; p++)
                for (int j = 0; j < R; j++) X[t * P * R + p * R + j] = ld(a->x, dtp, ox + j * P + p);
        }
        /* the previous token's term folded into the state entering the chunk */
        if (has_prev)
            for (int n = 0; n < N; n++)
                for (int p = 0; p < P; p++) {
                    double acc = 0;
                    for (int j = 0; j < R; j++) acc += Bprev[n * R + j] * Xprev[p * R + j];
                    Hs[n * P + p] += delta[0] * acc;
                }
        /* the chunk's own L = L1 L2 */
        for (int t = 0; t < nq; t++)
            for (int u = 0; u < nq; u++) {
                double prod = 0.0;
                if (u <= t) {
                    prod = 1.0;
                    for (int k = u + 1; k <= t; k++) prod *= alpha[k];
                }
                L1[t * Q + u] = prod;
                L2[t * Q + u] = (u == t) ? gamma[t] : ((u == t - 1) ? beta[t] : 0.0);
            }
        for (int t = 0; t < nq; t++)
            for (int u = 0; u < nq; u++) {
                double acc = 0;
                for (int k = 0; k < nq; k++) acc += L1[t * Q + k] * L2[k * Q + u];
                L[t * Q + u] = acc;
            }
        /* outputs */
        for (int t = 0; t < nq; t++) {
            double decay = 1.0;
            for (int k = 0; k <= t; k++) decay *= alpha[k];
            const int64_t tg = t0 + c0 + t;
            for (int p = 0; p < P; p++)
                for (int i = 0; i < R; i++) {
                    double acc = 0;
                    for (int n = 0; n < N; n++) acc += Ct[t * N * R + n * R + i] * decay * Hs[n * P + p];
                    for (int u = 0; u <= t; u++) {
                        if (L[t * Q + u] == 0.0) continue;
                        for (int j = 0; j < R; j++) {
                            double cb = 0;
                            for (int n = 0; n < N; n++) cb += Ct[t * N * R + n * R + i] * Bt[u * N * R + n * R + j];
                            acc += L[t * Q + u] * cb * X[u * P * R + p * R + j];
                        }
                    }
                    y_slab[(c0 + t) * P * R + i * P + p] =
                        gate(a, acc + Dh * X[t * P * R + p * R + i], (tg * H + h) * P * R + i * P + p);
                }
        }
        /* the chunk's final state, rotated back to the physical frame */
        const int e = nq - 1;
        double decay = 1.0;
        for (int k = 0; k <= e; k++) decay *= alpha[k];
        for (int n = 0; n < N; n++)
            for (int p = 0; p < P; p++) {
                double acc = decay * Hs[n * P + p];
                for (int u = 0; u <= e; u++)
                    for (int j = 0; j < R; j++) acc += L[e * Q + u] * Bt[u * N * R + n * R + j] * X[u * P * R + p * R + j];
                Hn[n * P + p] = acc;
            }
        for (int k = 0; k < K; k++) {
            const double c = cos(psi[k]), sn = sin(psi[k]);
            for (int p = 0; p < P; p++) {
                const double u = Hn[(2 * k) * P + p], v = Hn[(2 * k + 1) * P + p];
                Hs[(2 * k) * P + p] = c * u - sn * v;
                Hs[(2 * k + 1) * P + p] = sn * u + c * v;
            }
        }
        /* the chunk's last token is the next chunk's previous token (raw, physical frame) */
        memcpy(Bprev, Braw + e * N * R, (size_t)N * R * sizeof *Bprev);
        memcpy(Xprev, X + e * P * R, (size_t)P * R * sizeof *Xprev);
        has_prev = 1;
    }
    if (h_slab) memcpy(h_slab, Hs, (size_t)N * P * sizeof *Hs);
    free(Hs); free(Bprev); free(Xprev); free(alpha); free(beta); free(gamma); free(delta);
    free(L1); free(L2); free(L); free(Braw); free(Bt); free(Ct); free(X); free(psi); free(tmp); free(row); free(Hn);
}

/* ---------------------------------------------------------------- OB ---- */
/* Gradient of the layer (reverse mode), one (sequence, head) slab at a time.
 *
 * Given dL/dy for every output and dL/dh_out for the final state, it returns
 * dL/d(every input). It is the chain rule taken backwards through the plain
 * real-form recurrence of the physical frame (the statement in the header):
 *   U_t = H_{t-1} + delta_t Bp_t Xp_t^T      (Bp, Xp: the previous token, or Bprev, xprev)
 *   H_t = alpha_t R(dt_t theta_t) U_t + gamma_t B_t X_t^T
 *   y_t = gate(H_t^T C_t + D X_t, z_t)
 * Backwards, with G = dL/dH_t carried from the future (dh_out at the end):
 *   G      += C_t dy0_t^T                   (dy0: dy through the gate)
 *   dC_t    = H_t dy0_t,   dX_t += D dy0_t + gamma_t G^T B_t,   dB_t += gamma_t G X_t
 *   dgamma  = <G, B_t X_t^T>,  dalpha = <G, R U_t>,  dphi_k = alpha <G_k, R'(phi_k) U_k>
 *   V       = alpha R^T G                   (= dL/dU_t)
 *   ddelta  = <V, Bp Xp^T>,  dBp += delta V Xp,  dXp += delta V^T Bp,  and G <- V
 * then alpha = e^{dt A}, delta = (1 - lam) dt, gamma = lam dt, phi = dt theta
 * give dA, ddt, dlam, dtheta; the prologue's norm and bias and the gate are
 * differentiated as written in bc_row and gate. No chunking, no reordering.
 * (The pins compare every gradient with central differences of O1.) */
typedef struct {
    const double *dy;      /* [T, H, R, P] */
    const double *dh_out;  /* [nseq, H, N, P] or NULL */
    /* outputs, accumulated into caller-zeroed arrays (NULL: not wanted) */
    double *dx;            /* [T, H, R, P] */
    double *ddt, *dlam;    /* [T, H] */
    double *dtheta;        /* [T, H, N/2] */
    double *dB, *dC;       /* [T, G, R, N] */
    double *dA, *dD;       /* [H] */
    double *dh_in;         /* [nseq, H, N, P] */
    double *dBprev;        /* [nseq, G, R, N] */
    double *dxprev;        /* [nseq, H, R, P] */
    double *dB_bias, *dC_bias;   /* [H, N] */
    double *dz;            /* [T, H, R, P] */
    double *dA_tok;        /* [T, H] (with a per-token A) */
} m3o_grads;

/* Backward of bc_row: gout = dL/d(out) for the N outputs; adds dL/d(raw column)
 * to graw and dL/d(bias) to gbias (if not NULL). out = v inv + bias with
 * inv = (mean(v^2) + eps)^(-1/2) when the norm is on (else inv = 1), so
 * d out_n / d v_m = inv [n = m] - v_n v_m inv^3 / N. */
static void bc_row_bwd(const m3o_args *a, const void *src, int64_t off, const double *gout, double *graw,
                       double *gbias) {
    const int N = a->N;
    double *v = malloc((size_t)N * sizeof *v);
    double ss = 0.0, dot = 0.0;
    for (int n = 0; n < N; n++) {
        v[n] = ld(src, a->in_dtype, off + n);
        ss += v[n] * v[n];
        dot += gout[n] * v[n];
    }
    if (gbias)
        for (int n = 0; n < N; n++) gbias[n] += gout[n];
    if (a->bc_norm) {
        const double inv = 1.0 / sqrt(ss / N + a->bc_eps);
        for (int m = 0; m < N; m++) graw[m] += gout[m] * inv - dot * inv * inv * inv * v[m] / N;
    } else {
        for (int m = 0; m < N; m++) graw[m] += gout[m];
    }
    free(v);
}

static void ob_slab(const m3o_args *a, const m3o_grads *gr, int s, int h, double *dA_h, double *dD_h,
                    double *dBb_h, double *dCb_h) {
    const int H = a->H, G = a->G, P = a->P, N = a->N, R = a->R, K = N / 2;
    const int g = h / (H / G);
    const int dtp = a->in_dtype;
    const int64_t t0 = a->seq_start[s], L = a->seq_len[s];
    const size_t NP = (size_t)N * P, RN = (size_t)R * N, RP = (size_t)R * P;
    const double Dh = a->D ? a->D[h] : 0.0;
    const int has_prev = a->Bprev && a->xprev;
    const int64_t Lm = L > 0 ? L : 1;

    /* the recurrence's B, C (after the prologue) and x, rank-major [R][N] / [R][P] per token */
    double *Be = malloc(Lm * RN * sizeof *Be), *Ce = malloc(Lm * RN * sizeof *Ce);
    double *X = malloc(Lm * RP * sizeof *X), *Bpe = calloc(RN, sizeof *Bpe), *Xp0 = calloc(RP, sizeof *Xp0);
    for (int64_t t = 0; t < L; t++) {
        const int64_t ob = ((t0 + t) * G + g) * RN, ox = ((t0 + t) * H + h) * RP;
        for (int j = 0; j < R; j++) {
            bc_row(a, a->B, ob + j * N, h, a->B_bias, Be + t * RN + j * N);
            bc_row(a, a->C, ob + j * N, h, a->C_bias, Ce + t * RN + j * N);
        }
        for (size_t e = 0; e < RP; e++) X[t * RP + e] = ld(a->x, dtp, ox + e);
    }
    if (has_prev) {
        for (int j = 0; j < R; j++) bc_row(a, a->Bprev, ((int64_t)s * G + g) * RN + j * N, h, a->B_bias, Bpe + j * N);
        for (size_t e = 0; e < RP; e++) Xp0[e] = ld(a->xprev, dtp, ((int64_t)s * H + h) * RP + e);
    }
    /* forward: every state H_t kept ([L][N][P]), plus the initial one */
    double *Hall = malloc((Lm + 1) * NP * sizeof *Hall);   /* Hall[0] = H_{-1}, Hall[t+1] = H_t */
    for (size_t e = 0; e < NP; e++) Hall[e] = a->h_in ? a->h_in[((int64_t)s * H + h) * NP + e] : 0.0;
    double *U = malloc(NP * sizeof *U);
    for (int64_t t = 0; t < L; t++) {
        const int64_t tg = t0 + t;
        const double dt = ld(a->dt, dtp, tg * H + h), lam = lam_of(a, tg * H + h);
        const double Ah = A_of(a, tg * H + h, h);
        const double alpha = exp(dt * Ah), delta = (1.0 - lam) * dt, gamma = lam * dt;
        const double *Hp = Hall + t * NP;
        double *Hn = Hall + (t + 1) * NP;
        const double *Bp = t > 0 ? Be + (t - 1) * RN : Bpe, *Xp = t > 0 ? X + (t - 1) * RP : Xp0;
        const int prev = t > 0 || has_prev;
        for (int n = 0; n < N; n++)
            for (int p = 0; p < P; p++) {
                double v = 0.0;
                if (prev)
                    for (int j = 0; j < R; j++) v += Bp[j * N + n] * Xp[j * P + p];
                U[n * P + p] = Hp[n * P + p] + delta * v;
            }
        for (int k = 0; k < K; k++) {
            const double ang = dt * ld(a->theta, dtp, th_at(a, tg, h, k));
            const double c = cos(ang), sn = sin(ang);
            for (int p = 0; p < P; p++) {
                const double u0 = U[(2 * k) * P + p], u1 = U[(2 * k + 1) * P + p];
                double w0 = 0.0, w1 = 0.0;
                for (int j = 0; j < R; j++) {
                    w0 += Be[t * RN + j * N + 2 * k] * X[t * RP + j * P + p];
                    w1 += Be[t * RN + j * N + 2 * k + 1] * X[t * RP + j * P + p];
                }
                Hn[(2 * k) * P + p] = alpha * (c * u0 - sn * u1) + gamma * w0;
                Hn[(2 * k + 1) * P + p] = alpha * (sn * u0 + c * u1) + gamma * w1;
            }
        }
    }
    /* reverse */
    double *Gm = calloc(NP, sizeof *Gm), *V = malloc(NP * sizeof *V);
    double *dBe = calloc(Lm * RN, sizeof *dBe), *dCe = calloc(Lm * RN, sizeof *dCe);
    double *dX = calloc(Lm * RP, sizeof *dX), *dBpe = calloc(RN, sizeof *dBpe), *dXp0 = calloc(RP, sizeof *dXp0);
    double *dy0 = malloc(RP * sizeof *dy0), *dphi = malloc((size_t)K * sizeof *dphi);
    if (gr->dh_out)
        for (size_t e = 0; e < NP; e++) Gm[e] = gr->dh_out[((int64_t)s * H + h) * NP + e];
    for (int64_t t = L - 1; t >= 0; t--) {
        const int64_t tg = t0 + t;
        const double dt = ld(a->dt, dtp, tg * H + h), lam = lam_of(a, tg * H + h);
        const double Ah = A_of(a, tg * H + h, h);
        const double alpha = exp(dt * Ah), delta = (1.0 - lam) * dt, gamma = lam * dt;
        const double *Ht = Hall + (t + 1) * NP, *Hp = Hall + t * NP;
        const double *Bt = Be + t * RN, *Ct = Ce + t * RN, *Xt = X + t * RP;
        const int64_t oy = (tg * H + h) * RP;
        /* output and gate */
        for (int i = 0; i < R; i++)
            for (int p = 0; p < P; p++) {
                double y0 = Dh * Xt[i * P + p];
                for (int n = 0; n < N; n++) y0 += Ht[n * P + p] * Ct[i * N + n];
                const double d = gr->dy[oy + i * P + p];
                if (a->z) {
                    const double v = ld(a->z, dtp, oy + i * P + p), sg = 1.0 / (1.0 + exp(-v));
                    dy0[i * P + p] = d * v * sg;
                    if (gr->dz) gr->dz[oy + i * P + p] += d * y0 * (sg + v * sg * (1.0 - sg));
                } else {
                    dy0[i * P + p] = d;
                }
                dX[t * RP + i * P + p] += Dh * dy0[i * P + p];
                *dD_h += dy0[i * P + p] * Xt[i * P + p];
            }
        for (int i = 0; i < R; i++)
            for (int n = 0; n < N; n++) {
                double acc = 0.0;
                for (int p = 0; p < P; p++) acc += Ht[n * P + p] * dy0[i * P + p];
                dCe[t * RN + i * N + n] += acc;
            }
        for (int n = 0; n < N; n++)
            for (int p = 0; p < P; p++)
                for (int i = 0; i < R; i++) Gm[n * P + p] += Ct[i * N + n] * dy0[i * P + p];
        /* H_t = alpha R U + gamma B X^T */
        double dgamma = 0.0, dalpha = 0.0, ddelta = 0.0;
        for (int n = 0; n < N; n++)
            for (int p = 0; p < P; p++)
                for (int j = 0; j < R; j++) {
                    dgamma += Gm[n * P + p] * Bt[j * N + n] * Xt[j * P + p];
                    dBe[t * RN + j * N + n] += gamma * Gm[n * P + p] * Xt[j * P + p];
                    dX[t * RP + j * P + p] += gamma * Gm[n * P + p] * Bt[j * N + n];
                }
        const double *Bp = t > 0 ? Be + (t - 1) * RN : Bpe, *Xp = t > 0 ? X + (t - 1) * RP : Xp0;
        const int prev = t > 0 || has_prev;
        for (int n = 0; n < N; n++)
            for (int p = 0; p < P; p++) {
                double v = 0.0;
                if (prev)
                    for (int j = 0; j < R; j++) v += Bp[j * N + n] * Xp[j * P + p];
                U[n * P + p] = Hp[n * P + p] + delta * v;
            }
        for (int k = 0; k < K; k++) {
            const double ang = dt * ld(a->theta, dtp, th_at(a, tg, h, k));
            const double c = cos(ang), sn = sin(ang);
            double acc = 0.0;
            for (int p = 0; p < P; p++) {
                const double u0 = U[(2 * k) * P + p], u1 = U[(2 * k + 1) * P + p];
                const double g0 = Gm[(2 * k) * P + p], g1 = Gm[(2 * k + 1) * P + p];
                dalpha += g0 * (c * u0 - sn * u1) + g1 * (sn * u0 + c * u1);
                acc += g0 * (-sn * u0 - c * u1) + g1 * (c * u0 - sn * u1);
                V[(2 * k) * P + p] = alpha * (c * g0 + sn * g1);
                V[(2 * k + 1) * P + p] = alpha * (-sn * g0 + c * g1);
            }
            dphi[k] = alpha * acc;
        }
        /* U = H_{t-1} + delta Bp Xp^T */
        if (prev) {
            double *dBp = t > 0 ? dBe + (t - 1) * RN : dBpe, *dXp = t > 0 ? dX + (t - 1) * RP : dXp0;
            for (int n = 0; n < N; n++)
                for (int p = 0; p < P; p++)
                    for (int j = 0; j < R; j++) {
                        ddelta += V[n * P + p] * Bp[j * N + n] * Xp[j * P + p];
                        dBp[j * N + n] += delta * V[n * P + p] * Xp[j * P + p];
                        dXp[j * P + p] += delta * V[n * P + p] * Bp[j * N + n];
                    }
        }
        memcpy(Gm, V, NP * sizeof *Gm);
        /* scalars: alpha = e^{dt A}, delta = (1 - lam) dt, gamma = lam dt, phi_k = dt theta_k */
        double ddt = Ah * alpha * dalpha + (1.0 - lam) * ddelta + lam * dgamma;
        for (int k = 0; k < K; k++) {
            const double th = ld(a->theta, dtp, th_at(a, tg, h, k));
            ddt += th * dphi[k];
            if (gr->dtheta) gr->dtheta[th_at(a, tg, h, k)] += dt * dphi[k];
        }
        if (gr->ddt) gr->ddt[tg * H + h] += ddt;
        if (gr->dlam && a->lam) gr->dlam[tg * H + h] += dt * (dgamma - ddelta);
        if (a->A_tok) {
            if (gr->dA_tok) gr->dA_tok[tg * H + h] += dt * alpha * dalpha;
        } else {
            *dA_h += dt * alpha * dalpha;
        }
    }
    if (gr->dh_in)
        for (size_t e = 0; e < NP; e++) gr->dh_in[((int64_t)s * H + h) * NP + e] += Gm[e];
    /* back through the prologue to the raw B, C columns (shared by the heads of a group) */
    for (int64_t t = 0; t < L; t++) {
        const int64_t ob = ((t0 + t) * G + g) * RN, ox = ((t0 + t) * H + h) * RP;
        for (int j = 0; j < R; j++) {
            if (gr->dB) bc_row_bwd(a, a->B, ob + j * N, dBe + t * RN + j * N, gr->dB + ob + j * N, a->B_bias ? dBb_h : NULL);
            if (gr->dC) bc_row_bwd(a, a->C, ob + j * N, dCe + t * RN + j * N, gr->dC + ob + j * N, a->C_bias ? dCb_h : NULL);
        }
        if (gr->dx)
            for (size_t e = 0; e < RP; e++) gr->dx[ox + e] += dX[t * RP + e];
    }
    if (has_prev) {
        const int64_t ob = ((int64_t)s * G + g) * RN, ox = ((int64_t)s * H + h) * RP;
        for (int j = 0; j < R; j++)
            if (gr->dBprev) bc_row_bwd(a, a->Bprev, ob + j * N, dBpe + j * N, gr->dBprev + ob + j * N, a->B_bias ? dBb_h : NULL);
        if (gr->dxprev)
            for (size_t e = 0; e < RP; e++) gr->dxprev[ox + e] += dXp0[e];
    }
    free(Be); free(Ce); free(X); free(Bpe); free(Xp0); free(Hall); free(U); free(Gm); free(V);
    free(dBe); free(dCe); free(dX); free(dBpe); free(dXp0); free(dy0); free(dphi);
}

/* ------------------------------------------------------------ exports ---- */
static int check(const m3o_args *a) {
    if (!a || a->nseq < 0 || a->H <= 0 || a->G <= 0 || a->P <= 0 || a->N <= 0 || a->R <= 0) return 1;
    if (a->N % 2 || a->H % a->G) return 1;
    if (!a->x || !a->dt || !a->theta || !a->B || !a->C || (!a->A && !a->A_tok)) return 1;
    if (a->bc_norm && !(a->bc_eps >= 0.0)) return 1;
    if (a->th_groups < 0 || (a->th_groups && a->H % a->th_groups)) return 1;
    return 0;
}

/* Which form: 1 = O1 (complex), 2 = O2 (rotated frame). y: [T, H, R, P] on the
 * flat token axis, h_out: [nseq, H, N, P] (may be NULL). OpenMP over slabs. */
int m3o_scan(const m3o_args *a, int form, double *y, double *h_out, int nthreads) {
    if (check(a) || !y || (form != 1 && form != 2)) return 1;
    const int H = a->H, P = a->P, N = a->N, R = a->R;
    const int64_t nslab = (int64_t)a->nseq * H;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t sl = 0; sl < nslab; sl++) {
        int s = (int)(sl / H), h = (int)(sl % H);
        int64_t len = a->seq_len[s];
        double *ys = malloc((size_t)(len > 0 ? len : 1) * P * R * sizeof *ys);
        double *hs = h_out ? h_out + ((int64_t)s * H + h) * N * P : NULL;
        if (form == 1) o1_slab(a, s, h, ys, hs); else o2_slab(a, s, h, ys, hs);
        for (int64_t tt = 0; tt < len; tt++)
            memcpy(y + ((a->seq_start[s] + tt) * H + h) * P * R, ys + tt * P * R, (size_t)P * R * sizeof *ys);
        free(ys);
    }
    return 0;
}

/* The chunked SSD form (O3C) over every slab, chunk size Q >= 1. y: [T, H, R, P] on the flat
 * token axis, h_out: [nseq, H, N, P] (may be NULL). OpenMP over slabs. */
int m3o_scan_chunked(const m3o_args *a, int Q, double *y, double *h_out, int nthreads) {
    if (check(a) || !y || Q < 1) return 1;
    const int H = a->H, P = a->P, N = a->N, R = a->R;
    const int64_t nslab = (int64_t)a->nseq * H;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t sl = 0; sl < nslab; sl++) {
        int s = (int)(sl / H), h = (int)(sl % H);
        int64_t len = a->seq_len[s];
        double *ys = malloc((size_t)(len > 0 ? len : 1) * P * R * sizeof *ys);
        double *hs = h_out ? h_out + ((int64_t)s * H + h) * N * P : NULL;
        o3c_slab(a, Q, s, h, ys, hs);
        for (int64_t tt = 0; tt < len; tt++)
            memcpy(y + ((a->seq_start[s] + tt) * H + h) * P * R, ys + tt * P * R, (size_t)P * R * sizeof *ys);
        free(ys);
    }
    return 0;
}

/* One (sequence, head) slab. y_slab: [len, R, P]; h_slab: [N, P] or NULL.
 * form 1 = O1, 2 = O2, 3 = O3 (zero initial state / no previous token only). */
int m3o_scan_slab(const m3o_args *a, int form, int s, int h, double *y_slab, double *h_slab) {
    if (check(a) || !y_slab || s < 0 || s >= a->nseq || h < 0 || h >= a->H) return 1;
    if (form == 1) o1_slab(a, s, h, y_slab, h_slab);
    else if (form == 2) o2_slab(a, s, h, y_slab, h_slab);
    else if (form == 3) {
        if (a->h_in || a->Bprev || a->xprev || h_slab) return 1;
        o3_slab(a, s, h, y_slab);
    } else return 1;
    return 0;
}

/* One decode step = one token of the O1 recurrence from a given state and
 * previous token, for every (batch row, head): batch rows are sequences of
 * length one. h_io: [batch, H, N, P] in/out; y: [batch, H, R, P]. */
int m3o_decode(const m3o_args *a_in, double *h_io, double *y, int nthreads) {
    if (check(a_in) || !h_io || !y) return 1;
    m3o_args a = *a_in;
    const int H = a.H, P = a.P, N = a.N, R = a.R;
    double *hcopy = malloc((size_t)a.nseq * H * N * P * sizeof *hcopy);
    memcpy(hcopy, h_io, (size_t)a.nseq * H * N * P * sizeof *hcopy);
    a.h_in = hcopy;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t sl = 0; sl < (int64_t)a.nseq * H; sl++) {
        int s = (int)(sl / H), h = (int)(sl % H);
        o1_slab(&a, s, h, y + ((int64_t)s * H + h) * P * R, h_io + ((int64_t)s * H + h) * N * P);
    }
    free(hcopy);
    return 0;
}

/* Gradient of the whole scan (OB). Sequences run in parallel; the heads of a
 * sequence run in order, so the heads of a group add into dB, dC, dBprev (and
 * the heads sharing an angle row into dtheta) one after another. The per-head sums dA, dD and the bias gradients are added
 * in sequence order. */
int m3o_scan_bwd(const m3o_args *a, const m3o_grads *gr, int nthreads) {
    if (check(a) || !gr || !gr->dy) return 1;
    const int H = a->H, N = a->N;
    double *pA = calloc((size_t)a->nseq * H + 1, sizeof *pA), *pD = calloc((size_t)a->nseq * H + 1, sizeof *pD);
    double *pBb = calloc((size_t)a->nseq * H * N + 1, sizeof *pBb), *pCb = calloc((size_t)a->nseq * H * N + 1, sizeof *pCb);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < a->nseq; s++)
        for (int h = 0; h < H; h++) {
            const int64_t sh = (int64_t)s * H + h;
            ob_slab(a, gr, s, h, pA + sh, pD + sh, pBb + sh * N, pCb + sh * N);
        }
    for (int s = 0; s < a->nseq; s++)
        for (int h = 0; h < H; h++) {
            const int64_t sh = (int64_t)s * H + h;
            if (gr->dA) gr->dA[h] += pA[sh];
            if (gr->dD) gr->dD[h] += pD[sh];
            for (int n = 0; n < N; n++) {
                if (gr->dB_bias) gr->dB_bias[h * N + n] += pBb[sh * N + n];
                if (gr->dC_bias) gr->dC_bias[h * N + n] += pCb[sh * N + n];
            }
        }
    free(pA); free(pD); free(pBb); free(pCb);
    return 0;
}

int m3o_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
