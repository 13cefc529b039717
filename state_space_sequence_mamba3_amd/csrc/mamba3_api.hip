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

int32_t mamba3_version(void) { return 10100; }

mamba3_status mamba3_scan_validate(const mamba3_scan_args *a) {
    if (!a) return MAMBA3_EINVAL;
    if (a->dtype != MAMBA3_F32 && a->dtype != MAMBA3_BF16) return MAMBA3_EINVAL;
    if (a->batch < 0 || a->seqlen < 0 || a->nheads < 1 || a->headdim < 1 || a->dstate < 2 ||
        (a->dstate & 1) || a->rank < 1 || a->ngroups < 1 || a->chunk < 1)
        return MAMBA3_EINVAL;
    if (a->nheads % a->ngroups) return MAMBA3_EINVAL;
    const bool packed = a->cu_seqlens != nullptr;
    if (packed && (a->batch != 1 || a->nseq < 1)) return MAMBA3_EINVAL;
    const int64_t S = packed ? a->nseq : a->batch;
    const int64_t T = (int64_t)a->batch * a->seqlen;
    if (S * a->nheads > INT32_MAX) return MAMBA3_EINVAL;
    if ((a->Bprev == nullptr) != (a->xprev == nullptr)) return MAMBA3_EINVAL;
    if (T > 0 && (!a->x || !a->dt || !a->lam || !a->theta || !a->B || !a->C || !a->y)) return MAMBA3_EINVAL;
    if (!a->A) return MAMBA3_EINVAL;
    if (a->workspace_bytes > 0 && !a->workspace) return MAMBA3_EWORKSPACE;
    const void *al16[] = {a->x, a->theta, a->B, a->C, a->y, a->h_in, a->h_out, a->Bprev, a->xprev};
    for (const void *p : al16)
        if (p && !aligned16(p)) return MAMBA3_EALIGN;
    if (!aligned_elem(a->dt, a->dtype) || !aligned_elem(a->lam, a->dtype)) return MAMBA3_EALIGN;
    if (!aligned4(a->A) || (a->D && !aligned4(a->D)) || (a->cu_seqlens && !aligned4(a->cu_seqlens)))
        return MAMBA3_EALIGN;
    mamba3_status pst = check_prologue(a->bc_norm, a->bc_eps, a->B_bias, a->C_bias, a->z);
    if (pst != MAMBA3_OK) return pst;
    // y must not overlap any input
    const int64_t es = a->dtype == MAMBA3_BF16 ? 2 : 4;
    const int64_t H = a->nheads, G = a->ngroups, P = a->headdim, N = a->dstate, R = a->rank;
    Range y = span(a->y, T * H * P * R, es);
    Range ins[] = {span(a->x, T * H * P * R, es), span(a->dt, T * H, es), span(a->lam, T * H, es),
                   span(a->theta, T * H * (N / 2), es), span(a->B, T * G * N * R, es),
                   span(a->C, T * G * N * R, es), span(a->h_in, S * H * N * P, 4),
                   span(a->Bprev, S * G * N * R, es), span(a->xprev, S * H * P * R, es),
                   span(a->h_out, S * H * N * P, 4), span(a->B_bias, H * N, 4), span(a->C_bias, H * N, 4),
                   span(a->z, T * H * P * R, es)};
    for (Range r : ins)
        if (overlaps(y, r)) return MAMBA3_EINVAL;
    // h_out may be h_in exactly, but no other overlap with an input
    Range ho = span(a->h_out, S * H * N * P, 4);
    Range ins2[] = {ins[0], ins[1], ins[2], ins[3], ins[4], ins[5], ins[7], ins[8], ins[10], ins[11], ins[12]};
    for (Range r : ins2)
        if (overlaps(ho, r)) return MAMBA3_EINVAL;
    if (a->h_in && a->h_out && a->h_in != a->h_out && overlaps(ins[6], ho)) return MAMBA3_EINVAL;
    // kernel availability
    if (a->dtype == MAMBA3_F32) {
        if (m3::scan_f32_lds_bytes(a->dstate, a->headdim, a->rank, a->chunk) > kMaxLds) return MAMBA3_EUNSUPPORTED;
    } else if (!m3::scan_bf16_supported(a->dstate, a->headdim, a->rank, a->chunk)) {
        return MAMBA3_EUNSUPPORTED;
    }
    return MAMBA3_OK;
}

size_t mamba3_scan_workspace_size(const mamba3_scan_args *a) {
    (void)a;
    return 0;
}

mamba3_status mamba3_scan_fwd(const mamba3_scan_args *a, void *stream) {
    mamba3_status st = mamba3_scan_validate(a);
    if (st != MAMBA3_OK) return st;
    const int64_t S = a->cu_seqlens ? a->nseq : a->batch;
    if (S == 0) return MAMBA3_OK;
    if ((int64_t)a->batch * a->seqlen == 0 && !a->h_out) return MAMBA3_OK;
    hipStream_t hs = (hipStream_t)stream;
    return a->dtype == MAMBA3_F32 ? m3::launch_scan_f32(a, hs) : m3::launch_scan_bf16(a, hs);
}

mamba3_status mamba3_decode_validate(const mamba3_decode_args *a) {
    if (!a) return MAMBA3_EINVAL;
    if (a->dtype != MAMBA3_F32 && a->dtype != MAMBA3_BF16) return MAMBA3_EINVAL;
    if (a->batch < 0 || a->nheads < 1 || a->headdim < 1 || a->dstate < 2 || (a->dstate & 1) || a->rank < 1 ||
        a->ngroups < 1 || a->nheads % a->ngroups)
        return MAMBA3_EINVAL;
    if ((int64_t)a->batch * a->nheads > INT32_MAX) return MAMBA3_EINVAL;
    if ((a->Bprev == nullptr) != (a->xprev == nullptr)) return MAMBA3_EINVAL;
    if (a->batch > 0 && (!a->x || !a->dt || !a->lam || !a->theta || !a->B || !a->C || !a->A || !a->h || !a->y))
        return MAMBA3_EINVAL;
    const void *al16[] = {a->x, a->theta, a->B, a->C, a->Bprev, a->xprev, a->h, a->y};
    for (const void *p : al16)
        if (p && !aligned16(p)) return MAMBA3_EALIGN;
    if (!aligned_elem(a->dt, a->dtype) || !aligned_elem(a->lam, a->dtype)) return MAMBA3_EALIGN;
    if ((a->A && !aligned4(a->A)) || (a->D && !aligned4(a->D))) return MAMBA3_EALIGN;
    mamba3_status pst = check_prologue(a->bc_norm, a->bc_eps, a->B_bias, a->C_bias, a->z);
    if (pst != MAMBA3_OK) return pst;
    const int64_t es = a->dtype == MAMBA3_BF16 ? 2 : 4;
    const int64_t b = a->batch, H = a->nheads, G = a->ngroups, P = a->headdim, N = a->dstate, R = a->rank;
    Range y = span(a->y, b * H * P * R, es);
    Range hh = span(a->h, b * H * N * P, 4);
    Range ins[] = {span(a->x, b * H * P * R, es), span(a->dt, b * H, es), span(a->lam, b * H, es),
                   span(a->theta, b * H * (N / 2), es), span(a->B, b * G * N * R, es),
                   span(a->C, b * G * N * R, es), span(a->Bprev, b * G * N * R, es),
                   span(a->xprev, b * H * P * R, es), span(a->B_bias, H * N, 4), span(a->C_bias, H * N, 4),
                   span(a->z, b * H * P * R, es), hh};
    for (Range r : ins)
        if (overlaps(y, r)) return MAMBA3_EINVAL;
    for (int i = 0; i < 11; i++)
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
