// Argument validation, path selection and workspace carve-up for falcon_fwd.
// Pure host code: nothing here calls into HIP, so the whole file can be
// exercised on a machine without a GPU.
#include "plan.h"

#include <cmath>
#include <cstring>

#include "chunk_layout.h"

namespace falcon {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_head_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool finite_nonneg(float x) { return std::isfinite(x) && x >= 0.f; }

}  // namespace

int build_plan(const falcon_fwd_args *a, Plan *p, bool check_pointers) {
    if (!a || !p) return FALCON_ERR_INVALID_ARG;
    *p = Plan{};
    if (a->abi_version != FALCON_ABI_VERSION) return FALCON_ERR_INVALID_ARG;
    const int var = a->variant;
    if (var != FALCON_V1 && var != FALCON_V2 && var != FALCON_V3 && var != FALCON_V1A &&
        var != FALCON_V2A && var != FALCON_V3A)
        return FALCON_ERR_INVALID_ARG;
    if (a->dtype != FALCON_BF16 && a->dtype != FALCON_F32) return FALCON_ERR_INVALID_ARG;
    if (a->phi != FALCON_PHI_RMSNORM && a->phi != FALCON_PHI_IDENTITY) return FALCON_ERR_INVALID_ARG;
    if (a->batch < 1 || a->heads < 1 || a->seqlen < 0 || a->dk < 1 || a->dv < 1)
        return FALCON_ERR_INVALID_ARG;
    if (a->window < 1 || a->chunk < 0) return FALCON_ERR_INVALID_ARG;
    const bool windowed = (var == FALCON_V3 || var == FALCON_V3A);
    if (!windowed && a->window != 1) return FALCON_ERR_INVALID_ARG;
    if (!finite_nonneg(a->eps) || !finite_nonneg(a->eps_rms)) return FALCON_ERR_INVALID_ARG;
    if (!(a->eps_gamma > 0.f && a->eps_gamma < 1.f)) return FALCON_ERR_INVALID_ARG;
    if (!is_head_dim(a->dk) || !is_head_dim(a->dv)) return FALCON_ERR_UNSUPPORTED;
    if (a->window > FALCON_MAX_WINDOW) return FALCON_ERR_UNSUPPORTED;
    const long long bh = static_cast<long long>(a->batch) * a->heads;
    if (bh > (1LL << 30)) return FALCON_ERR_UNSUPPORTED;
    // per-head element offsets are kept in 32 bits inside the kernels
    if (static_cast<long long>(a->seqlen + 64) * (a->dk > a->dv ? a->dk : a->dv) >= (1LL << 31))
        return FALCON_ERR_UNSUPPORTED;

    p->variant = var;
    p->dtype = a->dtype;
    p->phi = a->phi;
    p->B = a->batch;
    p->H = a->heads;
    p->T = a->seqlen;
    p->dk = a->dk;
    p->dv = a->dv;
    p->chunk = a->chunk;
    p->window = a->window;
    p->BH = static_cast<int>(bh);
    p->eps = a->eps;
    p->eps_gamma = a->eps_gamma;
    p->eps_rms = a->eps_rms;

    // path selection
    if (a->chunk == 0) {
        p->path = Path::kRecurrent;
    } else if (a->chunk == kChunk) {
        if (var == FALCON_V1 && chunk_f1_xfer_supported(a->dtype == FALCON_BF16, a->dk, a->dv)) {
            p->path = Path::kChunkF1Xfer;
            p->slice = f1_xfer_slice(a->dv);
        } else if (var == FALCON_V1 && chunk_f1_supported(a->dk, a->dv)) {
            p->path = Path::kChunkF1;
        } else if (var == FALCON_V2 && chunk_f2_supported(a->dtype == FALCON_BF16, a->dk, a->dv)) {
            p->path = Path::kChunkF2;
        } else if (var == FALCON_V2A && chunk_f2a_supported(a->dk, a->dv)) {
            p->path = Path::kChunkF2A;
        } else if (var == FALCON_V3 && chunk_f3_xfer_supported(a->dtype == FALCON_BF16, a->dk, a->dv, a->window)) {
            p->path = Path::kChunkF3X;
        } else if (var == FALCON_V3 && chunk_f3_supported(a->dk, a->dv)) {
            p->path = Path::kChunkF3;
        } else if (chunk_a1_supported(a->dtype == FALCON_BF16, var, a->window, a->dk, a->dv)) {
            p->path = Path::kChunkA1;
        } else if ((var == FALCON_V1A || var == FALCON_V3A) && chunk_a_supported(a->dk, a->dv)) {
            p->path = Path::kChunkA;
        } else {
            return FALCON_ERR_UNSUPPORTED;
        }
    } else {
        return FALCON_ERR_UNSUPPORTED;
    }
    if (a->seqlen == 0) p->path = Path::kEmpty;
    if (a->seqlen == 1) p->path = Path::kDecode;   // one token: both forms are one step


    // boundary state rules (host fields are always readable)
    const falcon_state *si = a->state_in;
    p->fresh = true;
    p->n_tail_in = 0;
    if (si) {
        p->fresh = si->fresh != 0;
        if (si->n_tail < 0 || si->n_tail > a->window - 1) return FALCON_ERR_INVALID_ARG;
        if (p->fresh && si->n_tail != 0) return FALCON_ERR_INVALID_ARG;
        p->n_tail_in = si->n_tail;
    }
    {
        long long pairs = static_cast<long long>(p->n_tail_in) + a->seqlen;
        p->n_tail_out = static_cast<int>(pairs < a->window - 1 ? pairs : a->window - 1);
    }

    // workspace carve-up: normalised features and step scalars (padded to
    // whole chunks on the chunk paths), then the per-chunk operators
    const int T = a->seqlen;
    size_t off = 0;
    if (p->path == Path::kDecode) {
        // no workspace: the step reads the inputs and the state directly
    } else if (p->path == Path::kChunkF2 || p->path == Path::kChunkF2A) {
        p->nchunks = (T + kChunk - 1) / kChunk;
    } else if (p->path == Path::kChunkF1Xfer) {
        p->nchunks = (T + kChunk - 1) / kChunk;
        p->seg_chunks = f1_xfer_segment_chunks(bh, a->dv, p->nchunks);
        p->nseg = (p->nchunks + p->seg_chunks - 1) / p->seg_chunks;
        p->off_chunk = off;
        off = align_up(off + static_cast<size_t>(bh) * p->nchunks * f1_xfer_bytes(a->dv));
        if (p->nseg > 1) {   // composed maps [A~ | beta], their gamma, entry states
            const size_t ns = static_cast<size_t>(bh) * p->nseg;
            p->off_seg_m = off; off = align_up(off + ns * f1_segmap_bytes(a->dv));
            p->off_seg_g = off; off = align_up(off + ns * 4);
            p->off_seg_s = off; off = align_up(off + ns * a->dk * a->dv * 4);
        }
    } else if (p->path == Path::kChunkA1) {
        p->nchunks = (T + kChunk - 1) / kChunk;
        p->Tpad = p->nchunks * kChunk;
        p->seg_chunks = chunk_a1_segment_chunks(bh, p->nchunks);
        p->nseg = (p->nchunks + p->seg_chunks - 1) / p->seg_chunks;
        const size_t st = static_cast<size_t>(bh) * p->nseg * a->dk * a->dv * 4;
        if (a->window > 1) {   // per-token w_t and log2 gamma_t from the window pass
            const size_t rows = static_cast<size_t>(bh) * p->Tpad;
            p->off_eta = off; off = align_up(off + rows * 4);
            p->off_alpha = off; off = align_up(off + rows * 4);
        }
        p->off_chunk = off; off = align_up(off + st);           // segment writes [d][j]
        p->off_seg_g = off; off = align_up(off + static_cast<size_t>(bh) * p->nseg * 4);
        p->off_seg_s = off; off = align_up(off + st);           // segment entry states [d][j]
    } else if (p->path == Path::kChunkF3X) {
        // per-token w_t and log2 gamma_t from the window pass, then the
        // Falcon-1 records of every 64-token chunk and the Falcon-1 walk
        // (split into segments as for Falcon-1)
        p->nchunks = (T + kChunk - 1) / kChunk;
        p->Tpad = p->nchunks * kChunk;
        const size_t rows = static_cast<size_t>(bh) * p->Tpad;
        p->off_eta = off; off = align_up(off + rows * 4);
        p->off_alpha = off; off = align_up(off + rows * 4);
        p->chunk_bytes = f1_xfer_bytes(a->dv);
        p->off_chunk = off; off = align_up(off + static_cast<size_t>(bh) * p->nchunks * p->chunk_bytes);
        p->seg_chunks = f1_xfer_segment_chunks(bh, a->dv, p->nchunks);
        p->nseg = (p->nchunks + p->seg_chunks - 1) / p->seg_chunks;
        if (p->nseg > 1) {
            const size_t ns = static_cast<size_t>(bh) * p->nseg;
            p->off_seg_m = off; off = align_up(off + ns * f1_segmap_bytes(a->dv));
            p->off_seg_g = off; off = align_up(off + ns * 4);
            p->off_seg_s = off; off = align_up(off + ns * a->dk * a->dv * 4);
        }
    } else if (p->path == Path::kChunkA) {
        p->nchunks = (T + kChunk - 1) / kChunk;
        p->Tpad = p->nchunks * kChunk;
        p->seg_chunks = chunk_a_segment_chunks(bh, p->nchunks);
        p->nseg = (p->nchunks + p->seg_chunks - 1) / p->seg_chunks;
        const size_t rows = static_cast<size_t>(bh) * p->Tpad;
        const size_t st = static_cast<size_t>(bh) * p->nseg * a->dk * a->dv * 4;
        p->off_eta = off; off = align_up(off + rows * 4);       // eta_t / B_t
        p->off_alpha = off; off = align_up(off + rows * 4);     // log gamma_t
        p->off_chunk = off; off = align_up(off + st);           // segment writes
        p->off_seg_g = off; off = align_up(off + static_cast<size_t>(bh) * p->nseg * 4);
        p->off_seg_s = off; off = align_up(off + st);           // segment entry states
    } else if (p->path != Path::kEmpty) {
        const bool chunked = p->path != Path::kRecurrent;
        if (p->path == Path::kChunkF3) {
            // stacked rows: 64 / W tokens per chunk; the feature buffers get
            // one extra tile so that the last chunk's 64-row reads stay inside
            p->ct = chunk_f3_tokens(a->window);
            p->nchunks = (T + p->ct - 1) / p->ct;
            p->Tpad = (p->nchunks * p->ct + kChunk - 1) / kChunk * kChunk + kChunk;
        } else {
            p->nchunks = chunked ? (T + kChunk - 1) / kChunk : 0;
            p->Tpad = chunked ? p->nchunks * kChunk : T;
        }
        p->feat_f32 = !chunked || a->dtype == FALCON_F32;
        const size_t rows = static_cast<size_t>(bh) * p->Tpad;
        const size_t fsz = p->feat_f32 ? 4 : 2;
        p->off_xn = off; off = align_up(off + rows * a->dk * fsz);
        p->off_qn = off; off = align_up(off + rows * a->dk * fsz);
        const size_t ncol = (var == FALCON_V2 || var == FALCON_V2A) ? a->dv : 1;
        p->off_eta = off; off = align_up(off + rows * ncol * 4);
        p->off_alpha = off; off = align_up(off + rows * ncol * 4);
        if (p->path == Path::kChunkF1 || p->path == Path::kChunkF3) {
            const size_t nch = static_cast<size_t>(bh) * p->nchunks;
            p->chunk_bytes = p->path == Path::kChunkF1 ? chunk_f1_bytes(a->dk, a->dv, a->dtype == FALCON_F32)
                                                       : chunk_f3_bytes(a->dk, a->dtype == FALCON_F32);
            p->off_chunk = off;
            off = align_up(off + nch * p->chunk_bytes);
        }
    }
    p->ws_bytes = off;

    if (!check_pointers) return FALCON_OK;

    // pointers
    const size_t nk = static_cast<size_t>(bh) * T * a->dk;
    const size_t nv = static_cast<size_t>(bh) * T * a->dv;
    const size_t esz = a->dtype == FALCON_BF16 ? 2 : 4;
    if (T > 0) {
        if (!a->q || !a->k || !a->v || !a->beta || !a->lambda || !a->o) return FALCON_ERR_INVALID_ARG;
        if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) ||
            !aligned16(a->beta) || !aligned16(a->lambda))
            return FALCON_ERR_INVALID_ARG;
        // the output may not alias any input
        const size_t nb = static_cast<size_t>(bh) * T * ((var == FALCON_V2 || var == FALCON_V2A) ? a->dv : 1);
        const size_t ot = nv * esz;
        if (overlap(a->o, ot, a->q, nk * esz) || overlap(a->o, ot, a->k, nk * esz) ||
            overlap(a->o, ot, a->v, nv * esz) || overlap(a->o, ot, a->beta, nb * 4) ||
            overlap(a->o, ot, a->lambda, static_cast<size_t>(bh) * T * 4))
            return FALCON_ERR_INVALID_ARG;
    }
    const size_t nS = static_cast<size_t>(bh) * a->dk * a->dv * 4;
    const size_t nX = static_cast<size_t>(bh) * a->dk * 4;
    const size_t nTx = static_cast<size_t>(bh) * (a->window - 1) * a->dk * 4;
    const size_t nTy = static_cast<size_t>(bh) * (a->window - 1) * a->dv * 4;
    if (si) {
        if (!si->S || !aligned16(si->S)) return FALCON_ERR_INVALID_ARG;
        if (!p->fresh && (!si->x_next || !aligned16(si->x_next))) return FALCON_ERR_INVALID_ARG;
        if (si->n_tail > 0 && (!si->tail_x || !si->tail_y)) return FALCON_ERR_INVALID_ARG;
        p->S_in = si->S;
        p->xnext_in = p->fresh ? nullptr : si->x_next;
        p->tailx_in = si->n_tail > 0 ? si->tail_x : nullptr;
        p->taily_in = si->n_tail > 0 ? si->tail_y : nullptr;
    }
    falcon_state *so = a->state_out;
    if (so) {
        if (!so->S || !so->x_next || !aligned16(so->S) || !aligned16(so->x_next))
            return FALCON_ERR_INVALID_ARG;
        if (a->window > 1 && (!so->tail_x || !so->tail_y)) return FALCON_ERR_INVALID_ARG;
        p->S_out = so->S;
        p->xnext_out = so->x_next;
        p->tailx_out = a->window > 1 ? so->tail_x : nullptr;
        p->taily_out = a->window > 1 ? so->tail_y : nullptr;
        if (si) {
            const void *ins[4] = {p->S_in, p->xnext_in, p->tailx_in, p->taily_in};
            const size_t ni[4] = {nS, nX, nTx, nTy};
            const void *outs[4] = {p->S_out, p->xnext_out, p->tailx_out, p->taily_out};
            const size_t no[4] = {nS, nX, nTx, nTy};
            for (int i = 0; i < 4; ++i)
                for (int j = 0; j < 4; ++j)
                    if (overlap(ins[i], ni[i], outs[j], no[j])) return FALCON_ERR_INVALID_ARG;
        }
    }
    if (p->ws_bytes > 0) {
        if (!a->workspace || a->workspace_bytes < p->ws_bytes) return FALCON_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(a->workspace) % kAlign) return FALCON_ERR_WORKSPACE;
    }
    p->q = a->q;
    p->k = a->k;
    p->v = a->v;
    p->beta = a->beta;
    p->lambda = a->lambda;
    p->o = a->o;
    p->ws = a->workspace;
    return FALCON_OK;
}

}  // namespace falcon

extern "C" {

size_t falcon_fwd_workspace_size(const falcon_fwd_args *args) {
    falcon::Plan p;
    if (falcon::build_plan(args, &p, false) != FALCON_OK) return 0;
    return p.ws_bytes;
}

int falcon_fwd_validate(const falcon_fwd_args *args) {
    falcon::Plan p;
    return falcon::build_plan(args, &p, true);
}

const char *falcon_status_str(int status) {
    switch (status) {
        case FALCON_OK: return "ok";
        case FALCON_ERR_INVALID_ARG: return "invalid argument";
        case FALCON_ERR_UNSUPPORTED: return "unsupported combination of sizes or options";
        case FALCON_ERR_WORKSPACE: return "workspace missing or too small";
        case FALCON_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

int falcon_abi_version(void) { return FALCON_ABI_VERSION; }

}  // extern "C"
