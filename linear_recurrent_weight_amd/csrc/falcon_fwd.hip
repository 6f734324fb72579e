// falcon_fwd: validate, plan, and enqueue the kernels of the chosen path.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "chunk_layout.h"
#include "kernels.h"
#include "plan.h"

using namespace falcon;

namespace falcon {

int cu_count() {
    static std::atomic<int> cached[64];   // zero-initialised (static storage)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);   // every thread stores the same value
    }
    return n;
}

}  // namespace falcon

namespace falcon {

// FALCON_SYNC_CHECK=1 (debug only): synchronise and check the HIP error
// state after every kernel launch; read once per process
bool sync_check_enabled() {
    static const bool on = [] {
        const char *e = std::getenv("FALCON_SYNC_CHECK");
        return e && e[0] && std::strcmp(e, "0") != 0;
    }();
    return on;
}

}  // namespace falcon

namespace {

const char *const kNamesEmpty[] = {"passthrough"};
const char *const kNamesRecurrent[] = {"feature", "recurrent"};
const char *const kNamesDecode[] = {"decode"};
const char *const kNamesChunkF1[] = {"feature", "chunk_f1_prep", "chunk_f1_scan"};
const char *const kNamesChunkA[] = {"a_segment", "a_segscan", "a_output"};
const char *const kNamesChunkA1[] = {"a1_segment", "a1_segscan", "a1_output"};
const char *const kNamesChunkA3[] = {"a3_window", "a1_segment", "a1_segscan", "a1_output"};
const char *const kNamesChunkA1Fold[] = {"a1_segment", "a1_output"};
const char *const kNamesChunkA3Fold[] = {"a3_window", "a1_segment", "a1_output"};
const char *const kNamesChunkF2[] = {"chunk_f2"};
const char *const kNamesChunkF2A[] = {"chunk_f2a"};
const char *const kNamesChunkF3[] = {"feature", "f3_prep", "f3_scan"};
const char *const kNamesChunkF3X[] = {"a3_window", "f3_xfer", "f1_carry"};
const char *const kNamesChunkF3XSeg[] = {"a3_window", "f3_xfer", "f1_segmap", "f1_segscan", "f1_carry"};
const char *const kNamesChunkF1Xfer[] = {"f1_xfer", "f1_carry"};
const char *const kNamesChunkF1XferSeg[] = {"f1_xfer", "f1_segmap", "f1_segscan", "f1_carry"};

int run(const falcon_fwd_args *args, void *stream, Marks *m) {
    Plan p;
    const int rc = build_plan(args, &p, true);
    if (rc != FALCON_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    m->sync_check = sync_check_enabled();
    m->mark(s);
    if (args->state_out) {
        args->state_out->n_tail = p.n_tail_out;
        args->state_out->fresh = (p.T == 0 && p.fresh) ? 1 : 0;
    }

    if (p.path == Path::kEmpty) {
        if (p.S_out) {
            PassArgs pa{};
            pa.BH = p.BH;
            pa.dk = p.dk;
            pa.dv = p.dv;
            pa.halo = p.window - 1;
            pa.n_tail = p.n_tail_in;
            pa.S_in = p.S_in;
            pa.xnext_in = p.xnext_in;
            pa.tailx_in = p.tailx_in;
            pa.taily_in = p.taily_in;
            pa.S_out = p.S_out;
            pa.xnext_out = p.xnext_out;
            pa.tailx_out = p.tailx_out;
            pa.taily_out = p.taily_out;
            launch_passthrough(pa, s, m);
        }
    } else if (p.path == Path::kDecode) {
        DecodeArgs da{};
        da.variant = p.variant;
        da.phi = p.phi;
        da.BH = p.BH;
        da.dk = p.dk;
        da.dv = p.dv;
        da.window = p.window;
        da.fresh = p.fresh ? 1 : 0;
        da.n_tail_in = p.n_tail_in;
        da.n_tail_out = p.n_tail_out;
        da.eps = p.eps;
        da.eps_gamma = p.eps_gamma;
        da.eps_rms = p.eps_rms;
        da.q = p.q;
        da.k = p.k;
        da.v = p.v;
        da.beta = p.beta;
        da.lambda = p.lambda;
        da.xnext_in = p.xnext_in;
        da.tailx_in = p.tailx_in;
        da.taily_in = p.taily_in;
        da.S_in = p.S_in;
        da.S_out = p.S_out;
        da.xnext_out = p.xnext_out;
        da.tailx_out = p.tailx_out;
        da.taily_out = p.taily_out;
        da.o = p.o;
        launch_decode(da, p.dtype == FALCON_BF16, s, m);
    } else if (p.path == Path::kChunkA || p.path == Path::kChunkA1) {
        ChunkAArgs ca{};
        ca.variant = p.variant;
        ca.phi = p.phi;
        ca.BH = p.BH;
        ca.T = p.T;
        ca.Tpad = p.Tpad;
        ca.nchunks = p.nchunks;
        ca.dk = p.dk;
        ca.dv = p.dv;
        ca.window = p.window;
        ca.fresh = p.fresh ? 1 : 0;
        ca.n_tail_in = p.n_tail_in;
        ca.n_tail_out = p.n_tail_out;
        ca.seg_chunks = p.seg_chunks;
        ca.nseg = p.nseg;
        ca.eps = p.eps;
        ca.eps_gamma = p.eps_gamma;
        ca.eps_rms = p.eps_rms;
        ca.q = p.q;
        ca.k = p.k;
        ca.v = p.v;
        ca.beta = p.beta;
        ca.lambda = p.lambda;
        ca.xnext_in = p.xnext_in;
        ca.tailx_in = p.tailx_in;
        ca.taily_in = p.taily_in;
        ca.S_in = p.S_in;
        ca.S_out = p.S_out;
        ca.xnext_out = p.xnext_out;
        ca.tailx_out = p.tailx_out;
        ca.taily_out = p.taily_out;
        ca.o = p.o;
        ca.Dseg = p.ws_at<float>(p.off_chunk);
        ca.Gseg = p.ws_at<float>(p.off_seg_g);
        ca.Sseg = p.ws_at<float>(p.off_seg_s);
        if (p.path == Path::kChunkA1) {
            if (p.window > 1) {
                ca.etaw = p.ws_at<float>(p.off_eta);
                ca.lg = p.ws_at<float>(p.off_alpha);
            }
            launch_chunk_a1(ca, s, m);
        } else {
            ca.etaw = p.ws_at<float>(p.off_eta);
            ca.lg = p.ws_at<float>(p.off_alpha);
            launch_chunk_a(ca, p.dtype == FALCON_BF16, s, m);
        }
    } else if (p.path == Path::kChunkF2 || p.path == Path::kChunkF2A) {
        ChunkF2Args fa{};
        fa.BH = p.BH;
        fa.T = p.T;
        fa.nchunks = p.nchunks;
        fa.dk = p.dk;
        fa.dv = p.dv;
        fa.phi = p.phi;
        fa.fresh = p.fresh ? 1 : 0;
        fa.eps = p.eps;
        fa.eps_gamma = p.eps_gamma;
        fa.eps_rms = p.eps_rms;
        fa.q = p.q;
        fa.k = p.k;
        fa.v = p.v;
        fa.beta = p.beta;
        fa.lambda = p.lambda;
        fa.xnext_in = p.xnext_in;
        fa.S_in = p.S_in;
        fa.S_out = p.S_out;
        fa.xnext_out = p.xnext_out;
        fa.o = p.o;
        if (p.path == Path::kChunkF2A) launch_chunk_f2a(fa, p.dtype == FALCON_BF16, s, m);
        else launch_chunk_f2(fa, p.dtype == FALCON_BF16, s, m);
    } else if (p.path == Path::kChunkF3X) {
        // the window pass (w_t, log2 gamma_t), the 64-token operators, the walk
        ChunkAArgs wa{};
        wa.variant = p.variant;
        wa.phi = p.phi;
        wa.BH = p.BH;
        wa.T = p.T;
        wa.Tpad = p.Tpad;
        wa.nchunks = p.nchunks;
        wa.dk = p.dk;
        wa.dv = p.dv;
        wa.window = p.window;
        wa.fresh = p.fresh ? 1 : 0;
        wa.n_tail_in = p.n_tail_in;
        wa.n_tail_out = p.n_tail_out;
        wa.eps = p.eps;
        wa.eps_gamma = p.eps_gamma;
        wa.eps_rms = p.eps_rms;
        wa.k = p.k;
        wa.beta = p.beta;
        wa.lambda = p.lambda;
        wa.xnext_in = p.xnext_in;
        wa.tailx_in = p.tailx_in;
        wa.taily_in = p.taily_in;
        wa.etaw = p.ws_at<float>(p.off_eta);
        wa.lg = p.ws_at<float>(p.off_alpha);
        launch_a3_window(wa, s, m);
        F3XferArgs xa{};
        xa.BH = p.BH;
        xa.T = p.T;
        xa.Tpad = p.Tpad;
        xa.nchunks = p.nchunks;
        xa.window = p.window;
        xa.phi = p.phi;
        xa.n_tail_in = p.n_tail_in;
        xa.n_tail_out = p.n_tail_out;
        xa.eps_rms = p.eps_rms;
        xa.q = p.q;
        xa.k = p.k;
        xa.v = p.v;
        xa.w = wa.etaw;
        xa.lg = wa.lg;
        xa.xnext_in = p.xnext_in;
        xa.tailx_in = p.tailx_in;
        xa.taily_in = p.taily_in;
        xa.xnext_out = p.xnext_out;
        xa.tailx_out = p.tailx_out;
        xa.taily_out = p.taily_out;
        xa.ops = p.ws_at<void>(p.off_chunk);
        launch_chunk_f3_xfer(xa, s, m);
        F1XferArgs fa{};   // the walk reads the records (x_next is written above)
        fa.BH = p.BH;
        fa.T = p.T;
        fa.nchunks = p.nchunks;
        fa.dk = p.dk;
        fa.dv = p.dv;
        fa.phi = p.phi;
        fa.eps_rms = p.eps_rms;
        fa.k = p.k;
        fa.S_in = p.S_in;
        fa.S_out = p.S_out;
        fa.o = p.o;
        fa.ops = xa.ops;
        fa.seg_chunks = p.seg_chunks;
        fa.nseg = p.nseg;
        if (p.nseg > 1) {
            fa.Mseg = p.ws_at<void>(p.off_seg_m);
            fa.Gseg = p.ws_at<float>(p.off_seg_g);
            fa.Sseg = p.ws_at<float>(p.off_seg_s);
        }
        launch_f1_walk(fa, s, m);
    } else if (p.path == Path::kChunkF1Xfer) {
        F1XferArgs fa{};
        fa.BH = p.BH;
        fa.T = p.T;
        fa.nchunks = p.nchunks;
        fa.dk = p.dk;
        fa.dv = p.dv;
        fa.phi = p.phi;
        fa.fresh = p.fresh ? 1 : 0;
        fa.eps = p.eps;
        fa.eps_gamma = p.eps_gamma;
        fa.eps_rms = p.eps_rms;
        fa.q = p.q;
        fa.k = p.k;
        fa.v = p.v;
        fa.beta = p.beta;
        fa.lambda = p.lambda;
        fa.xnext_in = p.xnext_in;
        fa.S_in = p.S_in;
        fa.S_out = p.S_out;
        fa.xnext_out = p.xnext_out;
        fa.o = p.o;
        fa.ops = p.ws_at<void>(p.off_chunk);
        fa.seg_chunks = p.seg_chunks;
        fa.nseg = p.nseg;
        if (p.nseg > 1) {
            fa.Mseg = p.ws_at<void>(p.off_seg_m);
            fa.Gseg = p.ws_at<float>(p.off_seg_g);
            fa.Sseg = p.ws_at<float>(p.off_seg_s);
        }
        launch_chunk_f1_xfer(fa, p.slice, s, m);
    } else {
        FeatureArgs fa{};
        fa.variant = p.variant;
        fa.phi = p.phi;
        fa.BH = p.BH;
        fa.T = p.T;
        fa.Tpad = p.Tpad;
        fa.dk = p.dk;
        fa.dv = p.dv;
        fa.window = p.window;
        fa.eps = p.eps;
        fa.eps_gamma = p.eps_gamma;
        fa.eps_rms = p.eps_rms;
        fa.fresh = p.fresh ? 1 : 0;
        fa.n_tail_in = p.n_tail_in;
        fa.n_tail_out = p.n_tail_out;
        fa.q = p.q;
        fa.k = p.k;
        fa.v = p.v;
        fa.beta = p.beta;
        fa.lambda = p.lambda;
        fa.xnext_in = p.xnext_in;
        fa.tailx_in = p.tailx_in;
        fa.taily_in = p.taily_in;
        fa.xnext_out = p.xnext_out;
        fa.tailx_out = p.tailx_out;
        fa.taily_out = p.taily_out;
        fa.xn = p.ws_at<void>(p.off_xn);
        fa.qn = p.ws_at<void>(p.off_qn);
        fa.eta = p.ws_at<float>(p.off_eta);
        fa.alpha = p.ws_at<float>(p.off_alpha);
        const bool io_bf16 = p.dtype == FALCON_BF16;
        launch_features(fa, io_bf16, !p.feat_f32, s, m);

        if (p.path == Path::kRecurrent) {
            RecurrentArgs ra{};
            ra.variant = p.variant;
            ra.BH = p.BH;
            ra.T = p.T;
            ra.dk = p.dk;
            ra.dv = p.dv;
            ra.window = p.window;
            ra.n_tail_in = p.n_tail_in;
            ra.xn = fa.xn ? static_cast<const float *>(fa.xn) : nullptr;
            ra.qn = static_cast<const float *>(fa.qn);
            ra.eta = fa.eta;
            ra.alpha = fa.alpha;
            ra.v = p.v;
            ra.o = p.o;
            ra.S_in = p.S_in;
            ra.tailx_in = p.tailx_in;
            ra.taily_in = p.taily_in;
            ra.S_out = p.S_out;
            launch_recurrent(ra, io_bf16, s, m);
        } else if (p.path == Path::kChunkF1) {
            ChunkF1Args ca{};
            ca.BH = p.BH;
            ca.T = p.T;
            ca.Tpad = p.Tpad;
            ca.nchunks = p.nchunks;
            ca.dk = p.dk;
            ca.dv = p.dv;
            ca.xn = fa.xn;
            ca.qn = fa.qn;
            ca.eta = fa.eta;
            ca.alpha = fa.alpha;
            ca.v = p.v;
            ca.o = p.o;
            ca.S_in = p.S_in;
            ca.S_out = p.S_out;
            ca.ops = p.ws_at<void>(p.off_chunk);
            ca.chunk_bytes = p.chunk_bytes;
            launch_chunk_f1(ca, io_bf16, s, m);
        } else if (p.path == Path::kChunkF3) {
            ChunkF3Args ca{};
            ca.BH = p.BH;
            ca.T = p.T;
            ca.Tpad = p.Tpad;
            ca.nchunks = p.nchunks;
            ca.ct = p.ct;
            ca.window = p.window;
            ca.dk = p.dk;
            ca.dv = p.dv;
            ca.n_tail_in = p.n_tail_in;
            ca.xn = fa.xn;
            ca.qn = fa.qn;
            ca.eta = fa.eta;
            ca.alpha = fa.alpha;
            ca.tailx_in = p.tailx_in;
            ca.taily_in = p.taily_in;
            ca.v = p.v;
            ca.o = p.o;
            ca.S_in = p.S_in;
            ca.S_out = p.S_out;
            ca.ops = p.ws_at<void>(p.off_chunk);
            ca.chunk_bytes = p.chunk_bytes;
            launch_chunk_f3(ca, io_bf16, s, m);
        }
    }
    if (m->failed_at >= 0) {
        std::fprintf(stderr, "falcon_fwd: FALCON_SYNC_CHECK: kernel %d of the call failed\n", m->failed_at);
        return FALCON_ERR_HIP;
    }
    if (hipGetLastError() != hipSuccess) return FALCON_ERR_HIP;
    return m->count - 1;
}

}  // namespace

extern "C" int falcon_fwd(const falcon_fwd_args *args, void *stream) {
    Marks m;
    const int rc = run(args, stream, &m);
    return rc < 0 ? rc : FALCON_OK;
}

extern "C" int falcon_fwd_profile(const falcon_fwd_args *args, void *stream, void *const *events,
                                  int n_events) {
    Marks m;
    m.ev = events;
    m.n = n_events < 0 ? 0 : n_events;
    return run(args, stream, &m);
}

extern "C" const char *falcon_kernel_name(const falcon_fwd_args *args, int i) {
    Plan p;
    if (build_plan(args, &p, false) != FALCON_OK || i < 0) return nullptr;
    switch (p.path) {
        case Path::kEmpty: return i < 1 ? kNamesEmpty[i] : nullptr;
        case Path::kRecurrent: return i < 2 ? kNamesRecurrent[i] : nullptr;
        case Path::kDecode: return i < 1 ? kNamesDecode[i] : nullptr;
        case Path::kChunkF1: return i < 3 ? kNamesChunkF1[i] : nullptr;
        case Path::kChunkA: return i < 3 ? kNamesChunkA[i] : nullptr;
        case Path::kChunkA1:
            if (p.nseg <= chunk_a1_fold_segments) {
                if (p.window > 1) return i < 3 ? kNamesChunkA3Fold[i] : nullptr;
                return i < 2 ? kNamesChunkA1Fold[i] : nullptr;
            }
            if (p.window > 1) return i < 4 ? kNamesChunkA3[i] : nullptr;
            return i < 3 ? kNamesChunkA1[i] : nullptr;
        case Path::kChunkF2: return i < 1 ? kNamesChunkF2[i] : nullptr;
        case Path::kChunkF2A: return i < 1 ? kNamesChunkF2A[i] : nullptr;
        case Path::kChunkF3: return i < 3 ? kNamesChunkF3[i] : nullptr;
        case Path::kChunkF3X:
            if (p.nseg > 1) return i < 5 ? kNamesChunkF3XSeg[i] : nullptr;
            return i < 3 ? kNamesChunkF3X[i] : nullptr;
        case Path::kChunkF1Xfer:
            if (p.nseg > 1) return i < 4 ? kNamesChunkF1XferSeg[i] : nullptr;
            return i < 2 ? kNamesChunkF1Xfer[i] : nullptr;
        default: return nullptr;
    }
}

// ---------------------------------------------------------------------------
// falcon_fwd_noalloc: falcon_fwd with the workspace taken from a fixed device
// array of this library instead of the caller's buffer.
// ---------------------------------------------------------------------------
namespace {

// One array per device (a __device__ object exists once on every GPU the
// library runs on and stays allocated until the process ends).  Host code
// never uses its name as an address: scratch_ptr() looks the address up.
static __device__ __align__(256) unsigned char scratch[FALCON_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// device address of the current device's copy of `scratch`, looked up once
// per device with that device current; nullptr on failure
void *scratch_ptr(int dev) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int falcon_fwd_noalloc(const falcon_fwd_args *args, void *stream) {
    if (!args) return FALCON_ERR_INVALID_ARG;
    const size_t need = falcon_fwd_workspace_size(args);
    falcon_fwd_args a = *args;
    if (need == 0) {
        // malformed or unsupported arguments, or a path without workspace
        a.workspace = nullptr;
        a.workspace_bytes = 0;
    } else {
        if (need > FALCON_NOALLOC_SCRATCH_BYTES) return FALCON_ERR_WORKSPACE;
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FALCON_ERR_HIP;
        void *p = scratch_ptr(dev);
        if (!p) return FALCON_ERR_HIP;
        a.workspace = p;
        a.workspace_bytes = FALCON_NOALLOC_SCRATCH_BYTES;
    }
    Marks m;
    const int rc = run(&a, stream, &m);
    return rc < 0 ? rc : FALCON_OK;
}
