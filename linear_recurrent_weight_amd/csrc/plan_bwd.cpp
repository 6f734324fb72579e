// Argument validation and workspace carve-up for falcon_bwd (Falcon-1
// backward).  Pure host code: nothing here calls into HIP.
#include <cmath>
#include <cstdint>

#include "plan.h"

namespace falcon {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool is_head_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool finite_nonneg(float x) { return std::isfinite(x) && x >= 0.f; }

struct Span {
    const void *p;
    size_t n;
};
bool overlap(const Span &a, const Span &b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    auto x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
    return x < y + b.n && y < x + a.n;
}

}  // namespace

int build_bwd_plan(const falcon_bwd_args *a, BwdPlan *p, bool check_pointers) {
    if (!a || !p) return FALCON_ERR_INVALID_ARG;
    *p = BwdPlan{};
    if (a->abi_version != FALCON_ABI_VERSION) return FALCON_ERR_INVALID_ARG;
    const int var = a->variant;
    if (var != FALCON_V1 && var != FALCON_V2 && var != FALCON_V3 && var != FALCON_V1A &&
        var != FALCON_V2A && var != FALCON_V3A)
        return FALCON_ERR_INVALID_ARG;
    if (a->dtype != FALCON_BF16 && a->dtype != FALCON_F32) return FALCON_ERR_INVALID_ARG;
    if (a->phi != FALCON_PHI_RMSNORM && a->phi != FALCON_PHI_IDENTITY) return FALCON_ERR_INVALID_ARG;
    if (a->batch < 1 || a->heads < 1 || a->seqlen < 0 || a->dk < 1 || a->dv < 1)
        return FALCON_ERR_INVALID_ARG;
    if (!finite_nonneg(a->eps) || !finite_nonneg(a->eps_rms)) return FALCON_ERR_INVALID_ARG;
    if (!(a->eps_gamma > 0.f && a->eps_gamma < 1.f)) return FALCON_ERR_INVALID_ARG;
    if (var != FALCON_V1) return FALCON_ERR_UNSUPPORTED;
    if (!is_head_dim(a->dk) || !is_head_dim(a->dv)) return FALCON_ERR_UNSUPPORTED;
    const long long bh = static_cast<long long>(a->batch) * a->heads;
    if (bh > (1LL << 30)) return FALCON_ERR_UNSUPPORTED;
    const falcon_state *si = a->state_in;
    if (si) {
        if (si->n_tail != 0) return FALCON_ERR_INVALID_ARG;
        p->fresh = si->fresh != 0;
    }

    p->dtype = a->dtype;
    p->phi = a->phi;
    p->BH = static_cast<int>(bh);
    p->T = a->seqlen;
    p->dk = a->dk;
    p->dv = a->dv;
    p->eps = a->eps;
    p->eps_gamma = a->eps_gamma;
    p->eps_rms = a->eps_rms;

    const size_t T = static_cast<size_t>(a->seqlen), ub = static_cast<size_t>(bh);
    const size_t dk = static_cast<size_t>(a->dk), dv = static_cast<size_t>(a->dv);
    size_t off = 0;
    p->chunked = bwd_chunked(a->seqlen, a->dk, a->dv);
    if (p->chunked) {
        // workspace: per chunk the records A [d_k][d_k], B and G^T dO
        // [d_k][d_v]; the entry state of every chunk and S_T; the state
        // gradient at every chunk's end; <H, S_end> per 16 value columns
        const size_t nck = (T + kBwdChunk - 1) / kBwdChunk;
        p->nchunks = static_cast<int>(nck);
        p->off_ops = off; off = align_up(off + ub * nck * (dk * dk + 2 * dk * dv) * 4);
        p->off_cst = off; off = align_up(off + ub * (nck + 1) * dk * dv * 4);
        p->off_hg = off; off = align_up(off + ub * nck * dk * dv * 4);
        p->off_phip = off; off = align_up(off + ub * nck * (dv / 16) * 4);
    } else {
        // workspace: fp32 features and step scalars, the states before every
        // kBwdCheckpoint-th token, the residuals r_t, and the partial sums of
        // the reverse sweep
        p->off_xn = off; off = align_up(off + ub * T * dk * 4);
        p->off_qn = off; off = align_up(off + ub * T * dk * 4);
        p->off_eta = off; off = align_up(off + ub * T * 4);
        p->off_alpha = off; off = align_up(off + ub * T * 4);
        p->off_states = off; off = align_up(off + ub * bwd_checkpoints(a->seqlen) * dk * dv * 4);
        p->off_res = off; off = align_up(off + ub * T * dv * 4);   // residuals r_t
        p->off_part = off; off = align_up(off + ub * T * (dv / 16) * bwd_part_floats(a->dk) * 4);
    }
    p->ws_bytes = off;

    if (!check_pointers) return FALCON_OK;

    const size_t esz = a->dtype == FALCON_BF16 ? 2 : 4;
    const size_t nk = ub * T * a->dk * esz, nv = ub * T * a->dv * esz, ns = ub * T * 4;
    const size_t nS = ub * a->dk * a->dv * 4, nX = ub * a->dk * 4;
    if (T > 0) {
        const void *need[] = {a->q, a->k, a->v, a->beta, a->lambda, a->d_o,
                              a->d_q, a->d_k, a->d_v, a->d_beta, a->d_lambda};
        for (const void *ptr : need)
            if (!ptr || !aligned16(ptr)) return FALCON_ERR_INVALID_ARG;
    }
    if (si) {
        if (!si->S || !aligned16(si->S)) return FALCON_ERR_INVALID_ARG;
        if (!p->fresh && (!si->x_next || !aligned16(si->x_next))) return FALCON_ERR_INVALID_ARG;
        p->S_in = si->S;
        p->xnext_in = p->fresh ? nullptr : si->x_next;
    }
    const void *opt[] = {a->d_S_out, a->d_x_next_out, a->d_S_in, a->d_x_next_in};
    for (const void *ptr : opt)
        if (ptr && !aligned16(ptr)) return FALCON_ERR_INVALID_ARG;
    const Span ins[] = {{a->q, T ? nk : 0}, {a->k, T ? nk : 0}, {a->v, T ? nv : 0},
                        {a->beta, T ? ns : 0}, {a->lambda, T ? ns : 0}, {a->d_o, T ? nv : 0},
                        {a->d_S_out, nS}, {a->d_x_next_out, nX}, {p->S_in, nS}, {p->xnext_in, nX}};
    const Span outs[] = {{a->d_q, T ? nk : 0}, {a->d_k, T ? nk : 0}, {a->d_v, T ? nv : 0},
                         {a->d_beta, T ? ns : 0}, {a->d_lambda, T ? ns : 0},
                         {a->d_S_in, nS}, {a->d_x_next_in, nX}};
    for (const Span &o : outs) {
        for (const Span &i : ins)
            if (overlap(o, i)) return FALCON_ERR_INVALID_ARG;
        for (const Span &o2 : outs)
            if (&o2 != &o && overlap(o, o2)) return FALCON_ERR_INVALID_ARG;
    }
    if (p->ws_bytes > 0) {
        if (!a->workspace || a->workspace_bytes < p->ws_bytes) return FALCON_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(a->workspace) % kAlign) return FALCON_ERR_WORKSPACE;
    }
    p->ws = a->workspace;
    return FALCON_OK;
}

}  // namespace falcon

extern "C" {

size_t falcon_bwd_workspace_size(const falcon_bwd_args *args) {
    falcon::BwdPlan p;
    if (falcon::build_bwd_plan(args, &p, false) != FALCON_OK) return 0;
    return p.ws_bytes;
}

int falcon_bwd_validate(const falcon_bwd_args *args) {
    falcon::BwdPlan p;
    return falcon::build_bwd_plan(args, &p, true);
}

}  // extern "C"
