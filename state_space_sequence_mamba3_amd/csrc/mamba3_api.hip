// C ABI of the library: host-side validation and dispatch. Every check runs
// before any HIP call, so an error status means nothing was enqueued.
#include <string.h>

#include <cmath>

#include "m3_common.h"

namespace {

constexpr size_t kMaxLds = 160 * 1024;  // gfx950 LDS per workgroup

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
bool aligned_elem(const void *p, int32_t dtype) { return ((uintptr_t)p & (dtype == MAMBA3_BF16 ? 1u : 3u)) == 0; }

struct Range {
    const char *lo, *hi;
};

bool overlaps(Range a, Range b) { return a.lo && b.lo && a.lo < b.hi && b.lo < a.hi; }

Range span(const void *p, int64_t elems, int64_t esize) {
    if (!p || elems <= 0) return {nullptr, nullptr};
    return {(const char *)p, (const char *)p + elems * esize};
}

// The fused block prologue / epilogue fields shared by both argument structs.
mamba3_status check_prologue(int32_t bc_norm, float bc_eps, const float *B_bias, const float *C_bias,
                             const void *z) {
    if (bc_norm != 0 && bc_norm != 1) return MAMBA3_EINVAL;
    if (bc_norm && !(bc_eps >= 0.f && std::isfinite(bc_eps))) return MAMBA3_EINVAL;   // NaN fails >= 0
    const void *al16[] = {B_bias, C_bias, z};
    for (const void *p : al16)
        if (p && !aligned16(p)) return MAMBA3_EALIGN;
    return MAMBA3_OK;
}

}  // namespace

extern "C" {

const char *mamba3_status_string(mamba3_status s) {
    switch (s) {
        case MAMBA3_OK: return "ok";
        case MAMBA3_EINVAL: return "invalid argument";
        case MAMBA3_EUNSUPPORTED: return "unsupported configuration";
        case MAMBA3_EALIGN: return "pointer not aligned";
        case MAMBA3_EHIP: return "HIP runtime error";
        case MAMBA3_EWORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

int32_t mamba3_version(void) { return 10500; }

// Segment rows: batch * nseg (padded, nseg >= 1, seg_tokens = 0) or the packed bound (nseg = 0,
// seg_tokens >= 1); 0 for anything else.
static int64_t seg_rows(const mamba3_scan_args *f, int32_t nseg, int32_t seg_tokens) {
    if (!f) return 0;
    if (f->cu_seqlens) {
        if (nseg != 0 || seg_tokens < 1 || f->nseq < 0 || f->seqlen < 0) return 0;
        return m3::segment_rows_packed(f->nseq, f->seqlen, seg_tokens);
    }
    if (seg_tokens != 0 || nseg < 1 || f->batch < 0) return 0;
    return (int64_t)f->batch * nseg;
}

int64_t mamba3_segment_rows(const mamba3_scan_args *fwd, int32_t nseg, int32_t seg_tokens) {
    return seg_rows(fwd, nseg, seg_tokens);
}

mamba3_status mamba3_segment_table(const int32_t *cu_seqlens, int32_t nseq, int32_t seqlen, int32_t seg_tokens,
                                   int32_t *seg_cu, void *stream) {
    if (!cu_seqlens || !seg_cu || nseq < 0 || seqlen < 0 || seg_tokens < 1) return MAMBA3_EINVAL;
    if (!aligned4(cu_seqlens) || !aligned4(seg_cu)) return MAMBA3_EALIGN;
    const int64_t rows = m3::segment_rows_packed(nseq, seqlen, seg_tokens);
    if (rows + 1 > INT32_MAX) return MAMBA3_EINVAL;
    if (overlaps(span(cu_seqlens, (int64_t)nseq + 1, 4), span(seg_cu, rows + 1, 4))) return MAMBA3_EINVAL;
    return m3::launch_segment_table(cu_seqlens, nseq, seqlen, seg_tokens, seg_cu, (hipStream_t)stream);
}

// Every check of the scan arguments except the availability of a forward kernel. need_y = false
// for callers that do not write y (y must then be NULL).
static mamba3_status scan_args_check(const mamba3_scan_args *a, bool need_y = true) {
    if (!a) return MAMBA3_EINVAL;
    if (a->dtype != MAMBA3_F32 && a->dtype != MAMBA3_BF16) return MAMBA3_EINVAL;
    if (a->batch < 0 || a->seqlen < 0 || a->nheads < 1 || a->headdim < 1 || a->dstate < 2 ||
        (a->dstate & 1) || a->rank < 1 || a->ngroups < 1 || a->chunk < 1)
        return MAMBA3_EINVAL;
    if (a->nheads % a->ngroups) return MAMBA3_EINVAL;
    if (a->theta_groups < 0 || (a->theta_groups && a->nheads % a->theta_groups)) return MAMBA3_EINVAL;
    const bool packed = a->cu_seqlens != nullptr;
    if (packed && (a->batch != 1 || a->nseq < 1)) return MAMBA3_EINVAL;
    const int64_t S = packed ? a->nseq : a->batch;
    const int64_t T = (int64_t)a->batch * a->seqlen;
    if (S * a->nheads > INT32_MAX) return MAMBA3_EINVAL;
    if ((a->Bprev == nullptr) != (a->xprev == nullptr)) return MAMBA3_EINVAL;
    if (T > 0 && (!a->x || !a->dt || !a->theta || !a->B || !a->C || (need_y && !a->y))) return MAMBA3_EINVAL;
    if (!need_y && a->y) return MAMBA3_EINVAL;
    if (!a->A && !a->A_tok) return MAMBA3_EINVAL;
    if (!a->lam && !std::isfinite(a->lam_fixed)) return MAMBA3_EINVAL;
    if (a->A_tok && !aligned_elem(a->A_tok, a->dtype)) return MAMBA3_EALIGN;
    if (a->workspace_bytes > 0 && !a->workspace) return MAMBA3_EWORKSPACE;
    const void *al16[] = {a->x, a->theta, a->B, a->C, a->y, a->h_in, a->h_out, a->Bprev, a->xprev};
    for (const void *p : al16)
        if (p && !aligned16(p)) return MAMBA3_EALIGN;
    if (!aligned_elem(a->dt, a->dtype) || !aligned_elem(a->lam, a->dtype)) return MAMBA3_EALIGN;
    if ((a->A && !aligned4(a->A)) || (a->D && !aligned4(a->D)) || (a->cu_seqlens && !aligned4(a->cu_seqlens)))
        return MAMBA3_EALIGN;
    mamba3_status pst = check_prologue(a->bc_norm, a->bc_eps, a->B_bias, a->C_bias, a->z);
    if (pst != MAMBA3_OK) return pst;
    // y must not overlap any input
    const int64_t es = a->dtype == MAMBA3_BF16 ? 2 : 4;
    const int64_t H = a->nheads, G = a->ngroups, P = a->headdim, N = a->dstate, R = a->rank;
    const int64_t Gth = a->theta_groups ? a->theta_groups : H;
    Range y = span(a->y, T * H * P * R, es);
    Range ins[] = {span(a->x, T * H * P * R, es), span(a->dt, T * H, es), span(a->lam, T * H, es),
                   span(a->theta, T * Gth * (N / 2), es), span(a->B, T * G * N * R, es),
                   span(a->C, T * G * N * R, es), span(a->h_in, S * H * N * P, 4),
                   span(a->Bprev, S * G * N * R, es), span(a->xprev, S * H * P * R, es),
                   span(a->h_out, S * H * N * P, 4), span(a->B_bias, H * N, 4), span(a->C_bias, H * N, 4),
                   span(a->z, T * H * P * R, es), span(a->A_tok, T * H, es)};
    for (Range r : ins)
        if (overlaps(y, r)) return MAMBA3_EINVAL;
    // h_out may be h_in exactly, but no other overlap with an input
    Range ho = span(a->h_out, S * H * N * P, 4);
    Range ins2[] = {ins[0], ins[1], ins[2], ins[3], ins[4], ins[5], ins[7], ins[8], ins[10], ins[11], ins[12], ins[13]};
    for (Range r : ins2)
        if (overlaps(ho, r)) return MAMBA3_EINVAL;
    if (a->h_in && a->h_out && a->h_in != a->h_out && overlaps(ins[6], ho)) return MAMBA3_EINVAL;
    return MAMBA3_OK;
}

// The scan's checks; need_y = false admits the state-only scan (y NULL, final states alone) that
// the segmented scan runs as its first pass.
static mamba3_status scan_validate_impl(const mamba3_scan_args *a, bool need_y) {
    const mamba3_status st = scan_args_check(a, need_y);
    if (st != MAMBA3_OK) return st;
    // kernel availability
    if (a->dtype == MAMBA3_F32) {
        if (m3::scan_f32_lds_bytes(a->dstate, a->headdim, a->rank, a->chunk) > kMaxLds) return MAMBA3_EUNSUPPORTED;
    } else if (!m3::scan_bf16_supported(a->dstate, a->headdim, a->rank, a->chunk)) {
        return MAMBA3_EUNSUPPORTED;
    }
    return MAMBA3_OK;
}

static mamba3_status scan_run(const mamba3_scan_args *a, void *stream, bool need_y) {
    mamba3_status st = scan_validate_impl(a, need_y);
    if (st != MAMBA3_OK) return st;
    const int64_t S = a->cu_seqlens ? a->nseq : a->batch;
    if (S == 0) return MAMBA3_OK;
    if ((int64_t)a->batch * a->seqlen == 0 && !a->h_out) return MAMBA3_OK;
    hipStream_t hs = (hipStream_t)stream;
    return a->dtype == MAMBA3_F32 ? m3::launch_scan_f32(a, hs) : m3::launch_scan_bf16(a, hs);
}

mamba3_status mamba3_scan_validate(const mamba3_scan_args *a) { return scan_validate_impl(a, true); }

size_t mamba3_scan_workspace_size(const mamba3_scan_args *a) {
    (void)a;
    return 0;
}

mamba3_status mamba3_scan_fwd(const mamba3_scan_args *a, void *stream) { return scan_run(a, stream, true); }

mamba3_status mamba3_scan_bwd_validate(const mamba3_scan_bwd_args *b) {
    if (!b) return MAMBA3_EINVAL;
    // the forward arguments, with dy in the place of y (same layout, must not overlap an input)
    mamba3_scan_args f = b->fwd;
    f.y = (void *)b->dy;
    f.h_out = nullptr;
    f.workspace = nullptr;
    f.workspace_bytes = 0;
    mamba3_status st = scan_args_check(&f);
    if (st != MAMBA3_OK) return st;
    const mamba3_scan_args *a = &b->fwd;
    const int64_t S = a->cu_seqlens ? a->nseq : a->batch, T = (int64_t)a->batch * a->seqlen;
    const int64_t H = a->nheads, G = a->ngroups, P = a->headdim, N = a->dstate, R = a->rank;
    const int64_t Gth = a->theta_groups ? a->theta_groups : H;
    if (T > 0 && (!b->dx || !b->ddt || !b->dtheta || !b->dB || !b->dC)) return MAMBA3_EINVAL;
    if (T > 0 && a->lam && !b->dlam) return MAMBA3_EINVAL;
    if (!a->A_tok && !b->dA) return MAMBA3_EINVAL;
    if (a->A_tok && T > 0 && !b->dA_tok) return MAMBA3_EINVAL;
    if (b->dA_tok && !a->A_tok) return MAMBA3_EINVAL;
    if (b->dA_tok && !aligned_elem(b->dA_tok, a->dtype)) return MAMBA3_EALIGN;
    if ((b->dBprev == nullptr) != (b->dxprev == nullptr)) return MAMBA3_EINVAL;
    if (b->dBprev && !a->Bprev) return MAMBA3_EINVAL;
    if ((b->dB_bias && !a->B_bias) || (b->dC_bias && !a->C_bias) || (b->dz && !a->z)) return MAMBA3_EINVAL;
    const void *al16[] = {b->dx, b->dtheta, b->dB, b->dC, b->dBprev, b->dxprev, b->dz, b->dh_in, b->dh_out,
                          b->dB_bias, b->dC_bias};
    for (const void *q : al16)
        if (q && !aligned16(q)) return MAMBA3_EALIGN;
    if ((b->ddt && !aligned_elem(b->ddt, a->dtype)) || (b->dlam && !aligned_elem(b->dlam, a->dtype)) ||
        (b->dA && !aligned4(b->dA)) || (b->dD && !aligned4(b->dD)))
        return MAMBA3_EALIGN;
    const int64_t es = a->dtype == MAMBA3_BF16 ? 2 : 4;
    // every output against every input and every other output
    Range outs[] = {span(b->dx, T * H * P * R, es), span(b->ddt, T * H, es), span(b->dlam, T * H, es),
                    span(b->dtheta, T * Gth * (N / 2), es), span(b->dB, T * G * N * R, es),
                    span(b->dC, T * G * N * R, es), span(b->dA, H, 4), span(b->dD, H, 4),
                    span(b->dh_in, S * H * N * P, 4), span(b->dBprev, S * G * N * R, es),
                    span(b->dxprev, S * H * P * R, es), span(b->dB_bias, H * N, 4), span(b->dC_bias, H * N, 4),
                    span(b->dz, T * H * P * R, es), span(b->dA_tok, T * H, es)};
    Range ins[] = {span(a->x, T * H * P * R, es), span(a->dt, T * H, es), span(a->lam, T * H, es),
                   span(a->theta, T * Gth * (N / 2), es), span(a->B, T * G * N * R, es),
                   span(a->C, T * G * N * R, es), span(a->h_in, S * H * N * P, 4),
                   span(a->Bprev, S * G * N * R, es), span(a->xprev, S * H * P * R, es), span(a->A, H, 4),
                   span(a->D, H, 4), span(a->B_bias, H * N, 4), span(a->C_bias, H * N, 4),
                   span(a->z, T * H * P * R, es), span(a->cu_seqlens, a->cu_seqlens ? a->nseq + 1 : 0, 4),
                   span(a->A_tok, T * H, es),
                   span(b->dy, T * H * P * R, es), span(b->dh_out, S * H * N * P, 4)};
    const int nout = sizeof outs / sizeof outs[0];
    for (int i = 0; i < nout; i++) {
        for (Range r : ins)
            if (overlaps(outs[i], r)) return MAMBA3_EINVAL;
        for (int j = i + 1; j < nout; j++)
            if (overlaps(outs[i], outs[j])) return MAMBA3_EINVAL;
    }
    if (!m3::scan_bwd_chunk(a->dstate, a->headdim, a->rank)) return MAMBA3_EUNSUPPORTED;
    const size_t need = m3::scan_bwd_workspace_bytes(b);
    if (b->workspace_bytes < need || (need > 0 && !b->workspace)) return MAMBA3_EWORKSPACE;
    if (b->workspace && ((uintptr_t)b->workspace & 255u)) return MAMBA3_EALIGN;
    const Range wsr = span(b->workspace, (int64_t)b->workspace_bytes, 1);
    for (Range r : ins)
        if (overlaps(wsr, r)) return MAMBA3_EINVAL;
    for (Range r : outs)
        if (overlaps(wsr, r)) return MAMBA3_EINVAL;
    return MAMBA3_OK;
}

size_t mamba3_scan_bwd_workspace_size(const mamba3_scan_bwd_args *b) {
    if (!b || !m3::scan_bwd_chunk(b->fwd.dstate, b->fwd.headdim, b->fwd.rank)) return 0;
    return m3::scan_bwd_workspace_bytes(b);
}

mamba3_status mamba3_scan_bwd(const mamba3_scan_bwd_args *b, void *stream) {
    const mamba3_status st = mamba3_scan_bwd_validate(b);
    if (st != MAMBA3_OK) return st;
    return m3::launch_scan_bwd(b, (hipStream_t)stream);
}

mamba3_status mamba3_state_passing_validate(const mamba3_state_passing_args *sp) {
    if (!sp) return MAMBA3_EINVAL;
    // the sequences' arguments: y, h_out, workspace, z and D are not read
    mamba3_scan_args f = sp->fwd;
    f.y = nullptr;
    f.h_out = nullptr;
    f.workspace = nullptr;
    f.workspace_bytes = 0;
    f.z = nullptr;
    f.D = nullptr;
    mamba3_status st = scan_args_check(&f, false);
    if (st != MAMBA3_OK) return st;
    const bool packed = f.cu_seqlens != nullptr;
    if (packed) {
        if (sp->nseg != 0 || sp->seg_tokens < 1) return MAMBA3_EINVAL;
    } else if (sp->seg_tokens != 0 || sp->nseg < 1 || f.seqlen < 1 || f.seqlen % sp->nseg) {
        return MAMBA3_EINVAL;
    }
    // S: sequences; SR: segment rows
    const int64_t b = packed ? f.nseq : f.batch, T = (int64_t)f.batch * f.seqlen;
    const int64_t SR = seg_rows(&f, sp->nseg, sp->seg_tokens);
    if (SR * f.nheads > INT32_MAX || SR + 1 > INT32_MAX) return MAMBA3_EINVAL;
    if (b > 0 && (!sp->U || !sp->seg_h_in || !sp->seg_Bprev || !sp->seg_xprev)) return MAMBA3_EINVAL;
    const void *al16[] = {sp->U, sp->seg_h_in, sp->seg_Bprev, sp->seg_xprev, sp->h_out};
    for (const void *q : al16)
        if (q && !aligned16(q)) return MAMBA3_EALIGN;
    const int64_t es = f.dtype == MAMBA3_BF16 ? 2 : 4;
    const int64_t H = f.nheads, G = f.ngroups, P = f.headdim, N = f.dstate, R = f.rank;
    const int64_t Gth = f.theta_groups ? f.theta_groups : H;
    Range outs[] = {span(sp->seg_h_in, SR * H * N * P, 4), span(sp->seg_Bprev, SR * G * N * R, es),
                    span(sp->seg_xprev, SR * H * P * R, es), span(sp->h_out, b * H * N * P, 4)};
    Range ins[] = {span(f.x, T * H * P * R, es), span(f.dt, T * H, es), span(f.lam, T * H, es),
                   span(f.theta, T * Gth * (N / 2), es), span(f.B, T * G * N * R, es), span(f.A, H, 4),
                   span(f.h_in, b * H * N * P, 4), span(f.Bprev, b * G * N * R, es),
                   span(f.xprev, b * H * P * R, es), span(f.B_bias, H * N, 4), span(f.A_tok, T * H, es),
                   span(sp->U, SR * H * N * P, 4), span(f.cu_seqlens, packed ? f.nseq + 1 : 0, 4)};
    const int nout = sizeof outs / sizeof outs[0];
    for (int i = 0; i < nout; i++) {
        for (Range r : ins) {
            // h_out may be h_in exactly (each workgroup reads its slab's h_in before it writes h_out)
            if (i == 3 && sp->h_out && sp->h_out == f.h_in && r.lo == (const char *)f.h_in) continue;
            if (overlaps(outs[i], r)) return MAMBA3_EINVAL;
        }
        for (int j = i + 1; j < nout; j++)
            if (overlaps(outs[i], outs[j])) return MAMBA3_EINVAL;
    }
    if (m3::state_passing_lds_bytes(f.dstate, f.headdim, f.rank) > kMaxLds) return MAMBA3_EUNSUPPORTED;
    return MAMBA3_OK;
}

mamba3_status mamba3_state_passing(const mamba3_state_passing_args *sp, void *stream) {
    const mamba3_status st = mamba3_state_passing_validate(sp);
    if (st != MAMBA3_OK) return st;
    return m3::launch_state_passing(sp, (hipStream_t)stream);
}

// Segmented scan: the workspace holds U and the entering states [rows, H, N, P] fp32, then the
// previous tokens [rows, G, R, N] and [rows, H, R, P] in the token dtype, then (packed batches) the
// segment table [rows + 1] int32 (each region 256-byte aligned).
namespace {
struct SegWs {
    size_t U, h, B, x, cu, total;
};
SegWs seg_ws(const mamba3_scan_segmented_args *a) {
    const mamba3_scan_args &f = a->fwd;
    const int64_t SR = seg_rows(&f, a->nseg, a->seg_tokens);
    const int64_t H = f.nheads, G = f.ngroups, P = f.headdim, N = f.dstate, R = f.rank;
    const int64_t es = f.dtype == MAMBA3_BF16 ? 2 : 4;
    auto al = [](int64_t v) { return (size_t)((v + 255) / 256 * 256); };
    SegWs w;
    size_t o = 0;
    w.U = o; o += al(SR * H * N * P * 4);
    w.h = o; o += al(SR * H * N * P * 4);
    w.B = o; o += al(SR * G * R * N * es);
    w.x = o; o += al(SR * H * R * P * es);
    w.cu = o; o += f.cu_seqlens ? al((SR + 1) * 4) : 0;
    w.total = o;
    return w;
}
// The three calls' arguments, built over the workspace.
void seg_calls(const mamba3_scan_segmented_args *a, mamba3_scan_args *pass1, mamba3_state_passing_args *sp,
               mamba3_scan_args *pass2) {
    const mamba3_scan_args &f = a->fwd;
    const SegWs w = seg_ws(a);
    char *ws = (char *)a->workspace;
    float *U = (float *)(ws + w.U), *segh = (float *)(ws + w.h);
    void *segB = ws + w.B, *segx = ws + w.x;
    mamba3_scan_args rows = f;
    if (f.cu_seqlens) {           // the segments as a packed batch of their own (the segment table)
        rows.cu_seqlens = (const int32_t *)(ws + w.cu);
        rows.nseq = (int32_t)seg_rows(&f, a->nseg, a->seg_tokens);
    } else {                      // the segments as independent rows of seqlen / nseg tokens
        rows.batch = f.batch * a->nseg;
        rows.seqlen = a->nseg > 0 ? f.seqlen / a->nseg : 0;
    }
    rows.workspace = nullptr;
    rows.workspace_bytes = 0;
    *pass1 = rows;                // from zero states, no previous token, state only: U in h_out
    pass1->y = nullptr;
    pass1->h_in = nullptr;
    pass1->Bprev = pass1->xprev = nullptr;
    pass1->z = nullptr;
    pass1->h_out = U;
    *sp = mamba3_state_passing_args{};
    sp->fwd = f;
    sp->fwd.y = nullptr;
    sp->fwd.h_out = nullptr;
    sp->fwd.z = nullptr;
    sp->fwd.D = nullptr;
    sp->nseg = a->nseg;
    sp->seg_tokens = a->seg_tokens;
    sp->U = U;
    sp->seg_h_in = segh;
    sp->seg_Bprev = segB;
    sp->seg_xprev = segx;
    sp->h_out = f.h_out;
    *pass2 = rows;                // from the entering states, with the previous tokens
    pass2->h_in = segh;
    pass2->Bprev = segB;
    pass2->xprev = segx;
    pass2->h_out = nullptr;
}
}  // namespace

size_t mamba3_scan_segmented_workspace_size(const mamba3_scan_segmented_args *a) {
    if (!a || a->fwd.batch < 0 || a->fwd.nheads < 1 || a->fwd.headdim < 1 || a->fwd.dstate < 2 ||
        a->fwd.rank < 1 || a->fwd.ngroups < 1)
        return 0;
    if (seg_rows(&a->fwd, a->nseg, a->seg_tokens) < 1) return 0;
    return seg_ws(a).total;
}

mamba3_status mamba3_scan_segmented_validate(const mamba3_scan_segmented_args *a) {
    if (!a) return MAMBA3_EINVAL;
    const mamba3_scan_args &f = a->fwd;
    if (f.workspace || f.workspace_bytes) return MAMBA3_EINVAL;
    mamba3_status st = scan_args_check(&f);
    if (st != MAMBA3_OK) return st;
    if (f.cu_seqlens) {
        if (a->nseg != 0 || a->seg_tokens < 1) return MAMBA3_EINVAL;
        const int64_t SR = seg_rows(&f, 0, a->seg_tokens);
        if (SR * f.nheads > INT32_MAX || SR + 1 > INT32_MAX) return MAMBA3_EINVAL;
    } else if (a->seg_tokens != 0 || a->nseg < 1 || f.seqlen < 1 || f.seqlen % a->nseg) {
        return MAMBA3_EINVAL;
    }
    const size_t need = seg_ws(a).total;
    if (a->workspace_bytes < need || !a->workspace) return MAMBA3_EWORKSPACE;
    if ((uintptr_t)a->workspace & 255u) return MAMBA3_EALIGN;
    // the workspace against every input and output of the whole-sequence call
    const int64_t es = f.dtype == MAMBA3_BF16 ? 2 : 4;
    const int64_t S = f.cu_seqlens ? f.nseq : f.batch, T = (int64_t)f.batch * f.seqlen;
    const int64_t H = f.nheads, G = f.ngroups, P = f.headdim, N = f.dstate, R = f.rank;
    const int64_t Gth = f.theta_groups ? f.theta_groups : H;
    const Range wsr = span(a->workspace, (int64_t)a->workspace_bytes, 1);
    Range all[] = {span(f.x, T * H * P * R, es), span(f.dt, T * H, es), span(f.lam, T * H, es),
                   span(f.theta, T * Gth * (N / 2), es), span(f.B, T * G * N * R, es), span(f.C, T * G * N * R, es),
                   span(f.h_in, S * H * N * P, 4), span(f.Bprev, S * G * N * R, es), span(f.xprev, S * H * P * R, es),
                   span(f.h_out, S * H * N * P, 4), span(f.B_bias, H * N, 4), span(f.C_bias, H * N, 4),
                   span(f.z, T * H * P * R, es), span(f.A_tok, T * H, es), span(f.y, T * H * P * R, es),
                   span(f.A, H, 4), span(f.D, H, 4), span(f.cu_seqlens, f.cu_seqlens ? f.nseq + 1 : 0, 4)};
    for (Range r : all)
        if (overlaps(wsr, r)) return MAMBA3_EINVAL;
    // each call's own checks (kernel availability for the segment rows included)
    mamba3_scan_args p1, p2;
    mamba3_state_passing_args sp;
    seg_calls(a, &p1, &sp, &p2);
    if ((st = scan_validate_impl(&p1, false)) != MAMBA3_OK) return st;
    if ((st = mamba3_state_passing_validate(&sp)) != MAMBA3_OK) return st;
    return mamba3_scan_validate(&p2);
}

mamba3_status mamba3_scan_segmented(const mamba3_scan_segmented_args *a, void *stream) {
    mamba3_status st = mamba3_scan_segmented_validate(a);
    if (st != MAMBA3_OK) return st;
    if (a->fwd.batch == 0) return MAMBA3_OK;
    mamba3_scan_args p1, p2;
    mamba3_state_passing_args sp;
    seg_calls(a, &p1, &sp, &p2);
    // packed: the segment rows' token ranges first
    if (a->fwd.cu_seqlens &&
        (st = m3::launch_segment_table(a->fwd.cu_seqlens, a->fwd.nseq, a->fwd.seqlen, a->seg_tokens,
                                       (int32_t *)p1.cu_seqlens, (hipStream_t)stream)) != MAMBA3_OK)
        return st;
    // bf16: the state-only first pass also stages the segment sums that state passing reads
    const bool staged = p1.dtype == MAMBA3_BF16;
    if (staged) {
        if ((st = scan_validate_impl(&p1, false)) != MAMBA3_OK) return st;
        if ((st = m3::launch_scan_bf16_states(&p1, nullptr, sp.seg_h_in, (hipStream_t)stream)) != MAMBA3_OK)
            return st;
    } else if ((st = scan_run(&p1, stream, false)) != MAMBA3_OK) {
        return st;
    }
    if ((st = mamba3_state_passing_validate(&sp)) != MAMBA3_OK) return st;
    if ((st = m3::launch_state_passing(&sp, (hipStream_t)stream, staged)) != MAMBA3_OK) return st;
    return mamba3_scan_fwd(&p2, stream);
}

mamba3_status mamba3_decode_validate(const mamba3_decode_args *a) {
    if (!a) return MAMBA3_EINVAL;
    if (a->dtype != MAMBA3_F32 && a->dtype != MAMBA3_BF16) return MAMBA3_EINVAL;
    if (a->batch < 0 || a->nheads < 1 || a->headdim < 1 || a->dstate < 2 || (a->dstate & 1) || a->rank < 1 ||
        a->ngroups < 1 || a->nheads % a->ngroups)
        return MAMBA3_EINVAL;
    if (a->theta_groups < 0 || (a->theta_groups && a->nheads % a->theta_groups)) return MAMBA3_EINVAL;
    if (a->nslots < 0 || (a->slots && (int64_t)a->nslots * a->nheads > INT32_MAX)) return MAMBA3_EINVAL;
    if (a->slots && !aligned4(a->slots)) return MAMBA3_EALIGN;
    if ((int64_t)a->batch * a->nheads > INT32_MAX) return MAMBA3_EINVAL;
    if ((a->Bprev == nullptr) != (a->xprev == nullptr)) return MAMBA3_EINVAL;
    if (a->batch > 0 && (!a->x || !a->dt || !a->theta || !a->B || !a->C || !a->h || !a->y)) return MAMBA3_EINVAL;
    if (a->batch > 0 && !a->A && !a->A_tok) return MAMBA3_EINVAL;
    if (!a->lam && !std::isfinite(a->lam_fixed)) return MAMBA3_EINVAL;
    if (a->A_tok && !aligned_elem(a->A_tok, a->dtype)) return MAMBA3_EALIGN;
    const void *al16[] = {a->x, a->theta, a->B, a->C, a->Bprev, a->xprev, a->h, a->y};
    for (const void *p : al16)
        if (p && !aligned16(p)) return MAMBA3_EALIGN;
    if (!aligned_elem(a->dt, a->dtype) || !aligned_elem(a->lam, a->dtype)) return MAMBA3_EALIGN;
    if ((a->A && !aligned4(a->A)) || (a->D && !aligned4(a->D))) return MAMBA3_EALIGN;
    mamba3_status pst = check_prologue(a->bc_norm, a->bc_eps, a->B_bias, a->C_bias, a->z);
    if (pst != MAMBA3_OK) return pst;
    const int64_t es = a->dtype == MAMBA3_BF16 ? 2 : 4;
    const int64_t b = a->batch, H = a->nheads, G = a->ngroups, P = a->headdim, N = a->dstate, R = a->rank;
    const int64_t Gth = a->theta_groups ? a->theta_groups : H;
    // with slots, h is the pool of nslots states; slots is an input like the token arrays
    Range y = span(a->y, b * H * P * R, es);
    Range hh = span(a->h, (a->slots ? a->nslots : b) * H * N * P, 4);
    Range ins[] = {span(a->x, b * H * P * R, es), span(a->dt, b * H, es), span(a->lam, b * H, es),
                   span(a->theta, b * Gth * (N / 2), es), span(a->B, b * G * N * R, es),
                   span(a->C, b * G * N * R, es), span(a->Bprev, b * G * N * R, es),
                   span(a->xprev, b * H * P * R, es), span(a->B_bias, H * N, 4), span(a->C_bias, H * N, 4),
                   span(a->z, b * H * P * R, es), span(a->A_tok, b * H, es), span(a->slots, b, 4), hh};
    for (Range r : ins)
        if (overlaps(y, r)) return MAMBA3_EINVAL;
    for (int i = 0; i < 13; i++)
        if (overlaps(hh, ins[i])) return MAMBA3_EINVAL;
    if (!m3::decode_supported(a->dstate, a->headdim, a->rank, a->dtype)) return MAMBA3_EUNSUPPORTED;
    return MAMBA3_OK;
}

mamba3_status mamba3_decode_step(const mamba3_decode_args *a, void *stream) {
    mamba3_status st = mamba3_decode_validate(a);
    if (st != MAMBA3_OK) return st;
    if (a->batch == 0) return MAMBA3_OK;
    return m3::launch_decode(a, (hipStream_t)stream);
}

}  // extern "C"
