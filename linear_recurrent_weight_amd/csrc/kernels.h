// Launch interfaces of the Falcon kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/falcon.h"

namespace falcon {

struct FeatureArgs {
    int variant, phi, BH, T, Tpad, dk, dv, window;
    float eps, eps_gamma, eps_rms;
    int fresh, n_tail_in, n_tail_out;
    const void *q, *k, *v;
    const float *beta, *lambda;
    const float *xnext_in, *tailx_in, *taily_in;
    float *xnext_out, *tailx_out, *taily_out;
    void *xn, *qn;          // [BH, Tpad, dk] features (fp32 or bf16)
    float *eta, *alpha;     // [BH, Tpad] ([BH, Tpad, dv] for Falcon-2)
};

struct PassArgs {
    int BH, dk, dv, halo, n_tail;
    const float *S_in, *xnext_in, *tailx_in, *taily_in;
    float *S_out, *xnext_out, *tailx_out, *taily_out;
};

struct RecurrentArgs {
    int variant, BH, T, dk, dv, window, n_tail_in;
    const float *xn, *qn;   // fp32 features [BH, T, dk]
    const float *eta, *alpha;
    const void *v;          // [BH, T, dv] in the io dtype
    void *o;
    const float *S_in;      // nullptr => 0
    const float *tailx_in, *taily_in;
    float *S_out;           // nullptr => not written
};

struct ChunkF1Args {
    int BH, T, Tpad, nchunks, dk, dv;
    const void *xn, *qn;    // features [BH, Tpad, dk] (bf16 or fp32)
    const float *eta, *alpha;
    const void *v;          // [BH, T, dv]
    void *o;
    const float *S_in;
    float *S_out;
    void *ops;              // per-chunk operators
    size_t chunk_bytes;
};

// Called after every kernel launch: optional event marks between launches
// (measurement entry point), and the debug check of FALCON_SYNC_CHECK=1
// (synchronise the stream and read the HIP error state after each launch).
struct Marks {
    void *const *ev = nullptr;
    int n = 0;
    int count = 0;
    bool sync_check = false;
    int failed_at = -1;      // index of the first launch that failed the debug check
    void mark(hipStream_t s) {
        if (ev && count < n) (void)hipEventRecord(static_cast<hipEvent_t>(ev[count]), s);
        if (sync_check && count > 0 && failed_at < 0) {
            const hipError_t e = hipStreamSynchronize(s);
            const hipError_t l = hipGetLastError();
            if (e != hipSuccess || l != hipSuccess) failed_at = count - 1;
        }
        ++count;
    }
};

// compute units of the current device (queried once per device, thread-safe)
int cu_count();

// the FALCON_SYNC_CHECK debug switch (read once per process)
bool sync_check_enabled();

// Falcon-1 backward (token-recurrent): fp32 features and step scalars from
// the feature pass, the states before tokens 0, 4, 8, ..
// [BH][ceil(T/4)][d_v/4][d_k][4], the residuals, and the partial sums of the
// reverse sweep [BH][T][d_v/16][bwd_part_floats(d_k)]
struct BwdArgs {
    int phi, BH, T, dk, dv, fresh;
    float eps, eps_gamma, eps_rms;
    const void *q, *k, *v, *d_o;          // io dtype
    const float *beta, *lambda;
    const float *S_in, *d_S_out, *d_x_next_out;
    const float *xn, *qn, *eta, *alpha;   // [BH, T, d_k], [BH, T]
    float *states, *res, *part;             // res: r_t = y_t - S_{t-1}^T x_t [BH][T][d_v]
    void *d_q, *d_k, *d_v;                // io dtype
    float *d_beta, *d_lambda, *d_S_in, *d_x_next_in;
    // chunk-parallel form
    int nchunks;
    const float *xnext_in;                // carried feature (nullptr when fresh)
    float *ops;                           // [BH][nchunks] records: A [d_k][d_k], B, G^T dO [d_k][d_v]
    float *cst;                           // [BH][nchunks + 1][d_k][d_v] chunk entry states, then S_T
    float *hg;                            // [BH][nchunks][d_k][d_v] dL/dS at each chunk's end
    float *phip;                          // [BH][nchunks][d_v / 16] <H, S_end> per 16 value columns
};

struct ChunkAArgs {
    int variant, phi, BH, T, Tpad, nchunks, dk, dv, window, fresh, n_tail_in, n_tail_out;
    int seg_chunks, nseg;    // chunks per segment, segments per head
    float eps, eps_gamma, eps_rms;
    const void *q, *k, *v;
    const float *beta, *lambda;
    const float *xnext_in, *tailx_in, *taily_in;
    const float *S_in;
    float *S_out, *xnext_out, *tailx_out, *taily_out;
    void *o;
    float *etaw, *lg;        // [BH, Tpad] eta_t / B_t and log gamma_t
    float *Dseg, *Gseg;      // [BH, nseg, dv, dk] segment writes, [BH, nseg] carries
    float *Sseg;             // [BH, nseg, dv, dk] segment entry states (transposed)
};

struct ChunkF2Args {
    int BH, T, nchunks, dk, dv, phi, fresh;
    float eps, eps_gamma, eps_rms;
    const void *q, *k, *v;  // [BH, T, d] in the io dtype
    const float *beta;      // [BH, T, dv] per-column gains
    const float *lambda;    // [BH, T]
    const float *xnext_in;  // nullptr when fresh
    const float *S_in;
    float *S_out, *xnext_out;
    void *o;
};

struct F1XferArgs {
    int BH, T, nchunks, dk, dv, phi, fresh;
    float eps, eps_gamma, eps_rms;
    const void *q, *k, *v;  // bf16 [BH, T, d]
    const float *beta, *lambda;
    const float *xnext_in;  // nullptr when fresh
    const float *S_in;
    float *S_out, *xnext_out;
    void *o;
    void *ops;              // per-chunk transfer operators (f1_xfer_bytes(dv) each)
    // segments of seg_chunks chunks whose maps are composed and scanned
    // (nseg == 1: one walk over all chunks)
    int seg_chunks, nseg;
    void *Mseg;             // [BH][nseg] composed maps (f1_segmap_bytes(d_v) each)
    float *Gseg;            // [BH][nseg] scalar part gamma of the composed maps
    float *Sseg;            // [BH][nseg] entry states of the segments, d_k x d_v fp32
                            // in accumulator tiles [row tile][value tile][lane][4]
};

// one token (T = 1) of every variant, continuing from the incoming state
struct DecodeArgs {
    int variant, phi, BH, dk, dv, window, fresh, n_tail_in, n_tail_out;
    float eps, eps_gamma, eps_rms;
    const void *q, *k, *v;      // [BH, 1, d] in the io dtype
    const float *beta, *lambda; // [BH] ([BH, dv] beta for Falcon-2)
    const float *xnext_in, *tailx_in, *taily_in, *S_in;
    float *S_out, *xnext_out, *tailx_out, *taily_out;
    void *o;
};

struct ChunkF3Args {
    int BH, T, Tpad, nchunks, ct, window, dk, dv, n_tail_in;
    const void *xn, *qn;    // features [BH, Tpad, dk] (bf16 or fp32)
    const float *eta, *alpha;
    const float *tailx_in, *taily_in;   // incoming window pairs (nullptr when none)
    const void *v;          // [BH, T, dv]
    void *o;
    const float *S_in;
    float *S_out;
    void *ops;              // per-chunk operators
    size_t chunk_bytes;
};

void launch_features(const FeatureArgs &a, bool in_bf16, bool feat_bf16, hipStream_t s, Marks *m);
void launch_passthrough(const PassArgs &a, hipStream_t s, Marks *m);
void launch_recurrent(const RecurrentArgs &a, bool io_bf16, hipStream_t s, Marks *m);
void launch_decode(const DecodeArgs &a, bool io_bf16, hipStream_t s, Marks *m);
void launch_chunk_f1(const ChunkF1Args &a, bool bf16, hipStream_t s, Marks *m);
void launch_chunk_a(const ChunkAArgs &a, bool bf16, hipStream_t s, Marks *m);
// bf16 Falcon-1A with d_k = d_v = 64 (etaw and lg unused)
void launch_chunk_a1(const ChunkAArgs &a, hipStream_t s, Marks *m);
void launch_chunk_f2(const ChunkF2Args &a, bool bf16, hipStream_t s, Marks *m);
// Falcon-2A (same arguments as Falcon-2: per-column beta), d_k in {32, 64}
void launch_chunk_f2a(const ChunkF2Args &a, bool bf16, hipStream_t s, Marks *m);
void launch_chunk_f3(const ChunkF3Args &a, bool bf16, hipStream_t s, Marks *m);
// bf16 Falcon-1, d_k = 64: transfer operators, then the carry over slices of
// `slice` value columns
void launch_chunk_f1_xfer(const F1XferArgs &a, int slice, hipStream_t s, Marks *m);
// the carry over records already in the workspace (segment maps and scan
// first when a.nseg > 1)
void launch_f1_walk(const F1XferArgs &a, hipStream_t s, Marks *m);
// bf16 Falcon-3, d_k = d_v = 64, W in {2, 4, 8}: per 64-token chunk the
// Falcon-1 transfer operators (f1_xfer_bytes(64) each), from the raw rows
// and the window pass's step scalars; the walk is launch_f1_walk
struct F3XferArgs {
    int BH, T, Tpad, nchunks, window, phi, n_tail_in, n_tail_out;
    float eps_rms;
    const void *q, *k, *v;          // bf16 [BH, T, 64]
    const float *w, *lg;            // [BH, Tpad] eta_t / B_t and log2 gamma_t
    const float *xnext_in, *tailx_in, *taily_in;
    float *xnext_out, *tailx_out, *taily_out;
    void *ops;                      // [BH][nchunks] Falcon-1 records
};
void launch_chunk_f3_xfer(const F3XferArgs &a, hipStream_t s, Marks *m);
// the window pass of the bf16 d = 64 inner-product path: per token w_t =
// eta_t / B_t and log2 gamma_t into a.etaw and a.lg
void launch_a3_window(const ChunkAArgs &a, hipStream_t s, Marks *m);
// Falcon-1 backward after the feature pass: states, reverse sweep, reduction
void launch_bwd(const BwdArgs &a, bool io_bf16, hipStream_t s, Marks *m);
void launch_bwd_chunk(const BwdArgs &a, bool io_bf16, hipStream_t s, Marks *m);

}  // namespace falcon
