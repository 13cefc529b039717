/*
 * mamba3.h - C ABI of the Mamba-3 SSM layer recurrence on AMD MI355X (gfx950).
 *
 * The operation (per sequence s, head h, B/C group g = h / (H/G), token t):
 *   alpha_t = exp(dt_t A_h),  delta_t = (1 - lam_t) dt_t,  gamma_t = lam_t dt_t
 *   R_t     = block-diagonal 2x2 rotations R(dt_t theta_t[k]) on state rows
 *             (2k, 2k+1), R(a) = [[cos a, -sin a], [sin a, cos a]]
 *   H_t     = alpha_t R_t (H_{t-1} + delta_t B_{t-1} X_{t-1}^T) + gamma_t B_t X_t^T
 *   y_t     = H_t^T C_t + D_h X_t
 * with H_t in R^{N x P} (fp32), B_t, C_t in R^{N x R}, X_t, y_t in R^{P x R}.
 * This is the exponential-trapezoidal three-term update ("Mamba-3" paper
 * summary, section "Exponential-Trapezoidal Discretization", Proposition 1:
 * alpha, beta = delta * alpha, gamma) with the complex-valued transition of
 * Propositions 2-4 ("Complex-Valued State Space Models": exp(dt(A + i theta))
 * as a scalar decay times block-diagonal rotations, realised by the RoPE trick
 * of cumulative rotation angles on B and C) and the rank-R MIMO state update
 * B_t X_t^T = sum_r B_t^(r) X_t^(r)T ("MIMO Formulation"). The state is kept in
 * the physical frame (no cumulative angle is carried across calls).
 *
 * Layouts (row-major, innermost last; T = tokens). Rank-major: the R columns
 * of B_t, C_t (length N) and of X_t, y_t (length P) are stored one after
 * another, i.e. B_t^T, C_t^T, X_t^T, y_t^T row-major.
 *   x, y        [batch, seqlen, H, R, P]        token inputs / outputs
 *   dt, lam     [batch, seqlen, H]              step (post-softplus), trapezoid weight in [0,1]
 *   theta       [batch, seqlen, H, N/2]         rotation frequency; the angle is dt*theta
 *                                               (or [batch, seqlen, Gth, N/2]: theta_groups)
 *   B, C        [batch, seqlen, G, R, N]
 *   A, D        [H] fp32                         decay (A < 0) and skip; D may be NULL (= 0);
 *                                               A may be NULL with a per-token A_tok
 *   states      [S, H, N, P] fp32                S = batch (padded) or nseq (packed)
 *   Bprev       [S, G, R, N],  xprev [S, H, R, P]   token before position 0 of each sequence
 * Token inputs x, dt, lam, theta, B, C, Bprev, xprev and the output y share
 * one dtype (fp32 or bf16); states, A and D are fp32; arithmetic accumulates
 * in fp32.
 *
 * Conventions:
 *   - All pointers are device pointers, owned by the caller. The library
 *     allocates nothing, keeps no pointer after returning, holds no global
 *     mutable state and is reentrant.
 *   - Calls enqueue work on the given HIP stream (a hipStream_t passed as
 *     void*, NULL = default stream) and return without synchronising.
 *   - Every argument is validated on the host before anything is enqueued: a
 *     status other than MAMBA3_OK means nothing was launched. Device data
 *     (values of A, cu_seqlens, ...) is not inspected.
 *   - A launch failure reported by the HIP runtime returns MAMBA3_EHIP.
 *   - y must not alias any input. h_out may alias h_in (same slab layout).
 *   - x, theta, B, C, Bprev, xprev, y and the states must be 16-byte aligned;
 *     dt and lam need element alignment, A, D and cu_seqlens 4 bytes.
 *   - Callers zero-initialise the argument structs, so that fields added in a
 *     later minor version (all of which default to "off" at zero) stay off.
 *
 * Block prologue and epilogue (ABI 1.1, fields B_bias, C_bias, z, bc_norm,
 * bc_eps of both argument structs; all zero = off). The paper summary's
 * section "Architectural Integration" places a normalization on B and C right
 * after their projection, adds learned per-head, per-channel biases to B and
 * C after it, and gates the layer output. The library fuses these steps into
 * the scan and the decode step:
 *   bc_norm = 1  every column of B and C (the N values of one token, group and
 *                rank column; Bprev's columns too) is divided by
 *                sqrt(mean of its squares + bc_eps): an RMS norm without a
 *                gain. bc_norm must be 0 or 1; with bc_norm = 1, bc_eps must be
 *                finite and >= 0.
 *   B_bias, C_bias  [H, N] fp32 (16-byte aligned) or NULL: row h is added to
 *                every (normalised) column of B, C (and Bprev) that head h
 *                reads, for every rank column. With G < H the heads of a group
 *                then see different B and C.
 *   z            gate in the token dtype with the layout of x (16-byte
 *                aligned) or NULL: y <- y * SiLU(z), SiLU(v) = v / (1 + e^-v),
 *                applied after the D x term.
 * The normalisation and biases act before the rotation; the recurrence is
 * otherwise unchanged. y must not alias z or a bias; the states must not
 * alias them either.
 *
 * Variants (ABI 1.3, fields A_tok and lam_fixed of both argument structs):
 *   A_tok        per-token decay rate in the token dtype, layout of dt, or NULL.
 *                When given, alpha_t = exp(dt_t A_tok_t) and A is not read (it
 *                may be NULL): the data-dependent A of Remark 1 (section "The
 *                Complex-Valued A Parameterization"), which the pages make the
 *                default of Mamba-3.
 *   lam == NULL  every token uses the trapezoid weight lam_fixed (finite): the
 *                fixed-lambda variants of the pages' ablation (Table 8 of the
 *                paper listing: 1/2 is the classical trapezoid rule, 1 the
 *                exponential-Euler rule of Mamba-2).
 *
 * Shared angle rows (ABI 1.4, field theta_groups of both argument structs):
 *   theta_groups 0 (= nheads: one angle row per head, the layout above) or a
 *                divisor Gth of nheads: theta is [batch, seqlen, Gth, N/2]
 *                (decode: [batch, Gth, N/2]) and head h uses row
 *                h / (nheads / Gth), the mapping of B/C groups. Gth = 1 shares
 *                one set of angles across all heads, as B and C are shared
 *                across heads (section "MIMO Formulation"; the pages do not say
 *                whether the angles are shared, so both layouts are offered).
 *                The backward's dtheta has theta's layout and sums the shares
 *                of the heads that read a row.
 */
#ifndef MAMBA3_H
#define MAMBA3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MAMBA3_OK = 0,
    MAMBA3_EINVAL = 1,        /* bad size, NULL required pointer, inconsistent shape */
    MAMBA3_EUNSUPPORTED = 2,  /* valid but no kernel for this (N, P, R, chunk, dtype) */
    MAMBA3_EALIGN = 3,        /* a pointer lacks its required alignment */
    MAMBA3_EHIP = 4,          /* HIP runtime error (no device, launch failure) */
    MAMBA3_EWORKSPACE = 5     /* workspace missing or too small */
} mamba3_status;

typedef enum { MAMBA3_F32 = 0, MAMBA3_BF16 = 1 } mamba3_dtype;

/* Whole-sequence chunked scan.
 *
 * Padded mode (cu_seqlens == NULL): batch sequences of seqlen tokens each.
 * Packed mode (cu_seqlens != NULL): batch must be 1; the seqlen tokens hold
 * nseq sequences back to back, sequence s occupying tokens
 * [cu_seqlens[s], cu_seqlens[s+1]) (device int32 array of nseq+1 entries,
 * non-decreasing, cu_seqlens[0] = 0, cu_seqlens[nseq] = seqlen; entries are
 * clamped to [0, seqlen] on the device). Every sequence start resets the
 * recurrence: the state is h_in[s] (or zero) and the previous-token term uses
 * Bprev[s], xprev[s] (or is zero).
 *
 * chunk: tokens per chunk of the chunked algorithm (intra-chunk quadratic
 * form, inter-chunk recurrence: section "Parallel representation under SSD").
 * The result does not depend on it beyond rounding.
 *
 * h_in  NULL: zero initial state.
 * Bprev/xprev NULL (both): no previous-token term at the sequence start.
 * h_out NULL: final state not written.
 */
typedef struct {
    int32_t batch, seqlen, nheads, headdim /* P */, dstate /* N, even */, rank /* R */;
    int32_t ngroups /* G, divides nheads */, chunk /* Q */;
    int32_t dtype;               /* mamba3_dtype of the token inputs and y */
    const int32_t *cu_seqlens;   /* packed mode sequence table, or NULL */
    int32_t nseq;                /* packed mode: number of sequences */
    const void *x, *dt, *lam, *theta, *B, *C;
    const float *A, *D;
    const float *h_in;
    const void *Bprev, *xprev;
    void *y;
    float *h_out;
    void *workspace;             /* reserved: pass NULL / 0 when the size query returns 0 */
    size_t workspace_bytes;
    /* Block prologue and epilogue fused into the scan (ABI 1.1; see below). */
    const float *B_bias, *C_bias;
    const void *z;
    int32_t bc_norm;
    float bc_eps;
    /* Variants (ABI 1.3; see below). */
    const void *A_tok;
    float lam_fixed;
    /* Shared angle rows (ABI 1.4; see below). */
    int32_t theta_groups;
} mamba3_scan_args;

/* Pure host check of every argument (no HIP call). */
mamba3_status mamba3_scan_validate(const mamba3_scan_args *args);

/* Workspace bytes mamba3_scan_fwd needs for these arguments (currently 0 for
 * every supported configuration). */
size_t mamba3_scan_workspace_size(const mamba3_scan_args *args);

/* Enqueue the scan on `stream`. Writes y (every token) and h_out (if given). */
mamba3_status mamba3_scan_fwd(const mamba3_scan_args *args, void *stream);

/* Backward of the scan: the gradient of a loss L with respect to every input
 * of mamba3_scan_fwd, given dL/dy and dL/dh_out: the chain rule taken
 * backwards through the recurrence above, in the same chunked form. Training
 * runs the layer chunk-parallel (sections "Parallel representation under SSD"
 * and "MIMO Formulation") and needs this gradient.
 *
 * fwd       the forward call's arguments, unchanged (its y, h_out and
 *           workspace fields are ignored). Every input the forward read is
 *           read again; nothing of the forward pass needs to be kept.
 * dy        dL/dy, layout and dtype of x (required when there are tokens).
 * dh_out    [S, H, N, P] fp32 dL/dh_out, or NULL (zero).
 * Outputs, overwritten, in the layout and dtype of the matching input:
 *   dx, ddt, dtheta, dB, dC (required when there are tokens);
 *   dA [H] fp32 (required unless fwd.A_tok is given: then dA_tok is, and
 *   dA is not written); dD [H] fp32 or NULL;
 *   dlam is required only when fwd.lam is given (a fixed weight has none);
 *   dh_in [S, H, N, P] fp32 or NULL;
 *   dBprev, dxprev: both or neither, and only with Bprev/xprev;
 *   dB_bias, dC_bias [H, N] fp32, each only with its bias (or NULL);
 *   dz: only with z (or NULL).
 * No output may overlap any input or another output. Alignment as for the
 * matching inputs. The fused prologue / epilogue settings of fwd apply.
 *
 * workspace: device memory of at least mamba3_scan_bwd_workspace_size(args)
 * bytes, owned by the caller, 256-byte aligned. It holds the state entering
 * every chunk (the backward walks the chunks in reverse; a bf16 copy on the
 * matrix-core path of bf16 inputs, fp32 otherwise) and per-(sequence,
 * head) partial sums (per head also for dB, dC with G < H and for dtheta with
 * theta_groups < H), so that every sum is formed in a fixed order: the
 * results are bitwise reproducible. Its contents are scratch on return. The
 * size depends on the shapes, the chunk the backward picks and which inputs
 * are present, so query it for every distinct argument set. */
typedef struct {
    mamba3_scan_args fwd;
    const void *dy;
    const float *dh_out;
    void *dx, *ddt, *dlam, *dtheta, *dB, *dC;
    float *dA, *dD;
    float *dh_in;
    void *dBprev, *dxprev;
    float *dB_bias, *dC_bias;
    void *dz;
    void *workspace;
    size_t workspace_bytes;
    void *dA_tok;    /* ABI 1.3: with fwd.A_tok, dL/dA_tok (layout and dtype of A_tok) */
} mamba3_scan_bwd_args;

mamba3_status mamba3_scan_bwd_validate(const mamba3_scan_bwd_args *args);
size_t mamba3_scan_bwd_workspace_size(const mamba3_scan_bwd_args *args);
mamba3_status mamba3_scan_bwd(const mamba3_scan_bwd_args *args, void *stream);

/* State passing between the segments of long sequences (ABI 1.4): the
 * combine step of a context-parallel scan, and on one GPU a way to run a few
 * long sequences as many independent segments.
 *
 * The chunked form hands each chunk the state that enters it (section
 * "Parallel representation under SSD": chunk-local quadratic work plus a
 * recurrence over chunk states). Across a segment of tokens t the recurrence
 * is affine in its entering state: with the previous-token term of the
 * segment's first token folded in, H_start = H_in + delta_0 Bprev xprev^T,
 *   H_end = exp(S) R(Phi) H_start + U,   S = sum_t dt_t A_t,
 *   Phi[k] = sum_t dt_t theta_t[k],
 * where U is the segment's final state scanned from a zero state with no
 * previous token (the rotations R_t are block-diagonal on the same pairs and
 * commute, so their product is R(Phi)).
 *
 * Padded mode: every sequence of fwd is cut into nseg segments of seqlen /
 * nseg tokens; segment k of sequence s is "segment row" s * nseg + k, which
 * is how the token arrays [batch, seqlen, ...] read as [batch * nseg,
 * seqlen / nseg, ...]. Packed mode (ABI 1.5; fwd.cu_seqlens set, nseg = 0):
 * sequence s is cut into max(1, ceil(len_s / seg_tokens)) segments of
 * seg_tokens tokens (the last one shorter; one empty segment for an empty
 * sequence), numbered in sequence order: the segment rows, at most
 * mamba3_segment_rows(fwd, 0, seg_tokens) of them. mamba3_segment_table
 * writes their token ranges as a cu_seqlens table, which makes the segment
 * rows a packed batch of their own (rows past the last segment are empty).
 * The intended use:
 *   0. packed mode: mamba3_segment_table, and the segment rows' scans below
 *      take its table as cu_seqlens and its row count as nseq;
 *   1. mamba3_scan_fwd on the segment rows with h_in, Bprev, xprev NULL:
 *      its h_out is U [rows, H, N, P] (its y is not needed);
 *   2. mamba3_state_passing: writes seg_h_in, seg_Bprev, seg_xprev;
 *   3. mamba3_scan_fwd on the segment rows with h_in = seg_h_in,
 *      Bprev = seg_Bprev, xprev = seg_xprev: y equals the whole-sequence
 *      scan's y (up to rounding), and the h_out row of a sequence's last
 *      segment is its final state.
 * Here rows = batch * nseg (padded) or mamba3_segment_rows(fwd, 0,
 * seg_tokens) (packed), and S = batch (padded) or nseq (packed).
 *
 * fwd        the whole-sequence arguments as for mamba3_scan_fwd (padded or
 *            packed; y, h_out, workspace, z and D are not read; h_in, Bprev
 *            and xprev are those of the sequences).
 * nseg       padded: segments per sequence, >= 1, dividing seqlen; packed: 0.
 * U          [rows, H, N, P] fp32, step 1's final states.
 * seg_h_in   [rows, H, N, P] fp32 out: the state entering each segment
 *            (fwd.h_in, or zero, for a sequence's first segment).
 * seg_Bprev  [rows, G, R, N], seg_xprev [rows, H, R, P] out, token dtype: the
 *            token before each segment (the last token of the previous
 *            segment; fwd.Bprev/xprev, or zeros, for a first segment), raw as
 *            read (the prologue, if any, is applied by the scan).
 * h_out      [S, H, N, P] fp32 out or NULL: the final state of every
 *            sequence (it may be fwd.h_in exactly).
 * seg_tokens packed: tokens per segment, >= 1; padded: 0.
 * Rows past the packed batch's last segment are neither read nor written.
 * The outputs must not overlap each other or any input. Alignment: 16 bytes
 * for U and every output. The prologue settings of fwd (bc_norm, biases)
 * apply to the folded previous token, as in the scan. Deterministic. */
typedef struct {
    mamba3_scan_args fwd;
    int32_t nseg;
    const float *U;
    float *seg_h_in;
    void *seg_Bprev, *seg_xprev;
    float *h_out;
    int32_t seg_tokens;   /* ABI 1.5 */
} mamba3_state_passing_args;

mamba3_status mamba3_state_passing_validate(const mamba3_state_passing_args *args);
mamba3_status mamba3_state_passing(const mamba3_state_passing_args *args, void *stream);

/* Segment rows of a batch (ABI 1.5): batch * nseg in padded mode (nseg >= 1,
 * seg_tokens = 0); in packed mode (nseg = 0, seg_tokens >= 1) the bound
 * nseq + ceil(seqlen / seg_tokens) on the number of segments, the row count
 * of the packed segment arrays. 0 for any other combination. */
int64_t mamba3_segment_rows(const mamba3_scan_args *fwd, int32_t nseg, int32_t seg_tokens);

/* Segment table of a packed batch (ABI 1.5): writes rows + 1 entries of
 * seg_cu (device int32, rows = nseq + ceil(seqlen / seg_tokens)) such that
 * segment row r holds tokens [seg_cu[r], seg_cu[r+1]): the segments of
 * state passing's packed mode in order, then empty rows at the end of the
 * last sequence. Entries of cu_seqlens are clamped as the scan clamps them.
 * cu_seqlens [nseq + 1] and seg_cu are device arrays, 4-byte aligned, not
 * overlapping; nseq >= 0, seqlen >= 0, seg_tokens >= 1, rows + 1 <=
 * INT32_MAX (MAMBA3_EINVAL otherwise). One kernel of one workgroup. */
mamba3_status mamba3_segment_table(const int32_t *cu_seqlens, int32_t nseq, int32_t seqlen, int32_t seg_tokens,
                                   int32_t *seg_cu, void *stream);

/* The whole-sequence scan run as independent segments (ABI 1.4; packed
 * batches ABI 1.5): steps 0-3 above, enqueued in order on one stream. Step 1
 * runs as a state-only scan (the chunk-state updates alone: no C rows read,
 * no scores or y formed). The result equals mamba3_scan_fwd's up to
 * rounding; it costs about one and a half scans but multiplies the
 * workgroups, which pays for a few long sequences.
 *
 * fwd        as for mamba3_scan_fwd, padded or packed (fwd.workspace must be
 *            NULL / 0). y and h_out (if given) are written as by
 *            mamba3_scan_fwd; h_in, Bprev and xprev are honoured.
 * nseg       padded: segments per sequence, >= 1, dividing seqlen; seqlen
 *            >= 1. Packed: 0.
 * seg_tokens packed: tokens per segment, >= 1 (each sequence is cut as in
 *            state passing's packed mode). Padded: 0.
 * workspace  device memory of at least mamba3_scan_segmented_workspace_size
 *            bytes, 256-byte aligned, owned by the caller: the segments' zero-
 *            state final states and entering states (fp32), their previous
 *            tokens and (packed) the segment table. Its contents are scratch
 *            on return. It must not overlap any input or output.
 * Errors as for mamba3_scan_fwd and mamba3_state_passing; MAMBA3_EUNSUPPORTED
 * also when no kernel exists for the segments' shape (chunk as in fwd). */
typedef struct {
    mamba3_scan_args fwd;
    int32_t nseg;
    void *workspace;
    size_t workspace_bytes;
    int32_t seg_tokens;   /* ABI 1.5 */
} mamba3_scan_segmented_args;

size_t mamba3_scan_segmented_workspace_size(const mamba3_scan_segmented_args *args);
mamba3_status mamba3_scan_segmented_validate(const mamba3_scan_segmented_args *args);
mamba3_status mamba3_scan_segmented(const mamba3_scan_segmented_args *args, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): mamba3_scan_segmented
 * with a library-owned workspace, so the call allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine). Same kernels and results as
 * mamba3_scan_segmented.
 *
 * args       as for mamba3_scan_segmented, with workspace NULL and
 *            workspace_bytes 0 (MAMBA3_EINVAL otherwise).
 * stream     a stream of the current device (MAMBA3_EINVAL for another's).
 * Workspace  a device array of MAMBA3_NOALLOC_SCRATCH_BYTES (64 MiB), 256-byte
 *            aligned, held by every GPU the library runs on from the loading of
 *            its code until the process ends. MAMBA3_EWORKSPACE when
 *            mamba3_scan_segmented_workspace_size(args) exceeds it (about
 *            rows * H * N * P * 8 bytes).
 * Races      every call on one GPU uses that GPU's one array: calls that may run
 *            at the same time on one GPU (different streams, or the same stream
 *            from host threads without ordering) race and give wrong results.
 *            Calls enqueued in order on one stream are safe: the array holds the
 *            last call's contents and each call writes all it reads.
 * Errors     as for mamba3_scan_segmented (nothing is enqueued on any error);
 *            MAMBA3_EHIP also when the array's device address cannot be taken. */
#define MAMBA3_NOALLOC_SCRATCH_BYTES (64u << 20)
mamba3_status mamba3_scan_segmented_noalloc(const mamba3_scan_segmented_args *args, void *stream);

/* One decode step for a batch of independent sequences, state updated in
 * place: h <- alpha R (h + delta Bprev xprev^T) + gamma B x^T, y = h^T C + D x
 * (the same update as one token of the scan; section "MIMO Formulation" gives
 * the decode-time form H_t = alpha_t H_{t-1} + dt B_t x_t^T, y_t = H_t^T C_t).
 * Layouts: x, y [batch, H, R, P]; dt, lam [batch, H]; theta [batch, H, N/2];
 * B, C [batch, G, R, N]; Bprev [batch, G, R, N] and xprev [batch, H, R, P]
 * (both NULL = no previous-token term); h [batch, H, N, P] fp32 in/out.
 *
 * Slot-indexed states for continuous batching (ABI 1.4, fields slots and
 * nslots): with slots == NULL, batch row i updates h[i]. With slots given
 * (device int32 [batch], 4-byte aligned), h is a pool of nslots states
 * [nslots, H, N, P] and row i updates h[slots[i]] in place; a row whose slot
 * is negative or >= nslots is inactive: its state and its y row are left
 * untouched (a serving loop keeps one batch shape while sequences join and
 * leave). Token inputs, y, Bprev and xprev stay indexed by batch row. Two
 * active rows naming the same slot race (undefined result); slot values are
 * device data and are not inspected on the host. */
typedef struct {
    int32_t batch, nheads, headdim, dstate, rank, ngroups;
    int32_t dtype;
    const void *x, *dt, *lam, *theta, *B, *C;
    const void *Bprev, *xprev;
    const float *A, *D;
    float *h;
    void *y;
    /* Block prologue and epilogue (ABI 1.1; see below). */
    const float *B_bias, *C_bias;
    const void *z;
    int32_t bc_norm;
    float bc_eps;
    /* Variants (ABI 1.3; see below). */
    const void *A_tok;
    float lam_fixed;
    /* ABI 1.4: shared angle rows (see the scan) and slot-indexed states. */
    int32_t theta_groups;
    const int32_t *slots;
    int32_t nslots;
} mamba3_decode_args;

mamba3_status mamba3_decode_validate(const mamba3_decode_args *args);
mamba3_status mamba3_decode_step(const mamba3_decode_args *args, void *stream);

/* Static description of a status code. */
const char *mamba3_status_string(mamba3_status status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t mamba3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA3_H */
