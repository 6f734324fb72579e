// Internal host-side plan of one falcon_fwd call: validated sizes, the path
// chosen, and the carve-up of the caller's workspace.  Pure C++ (no HIP
// types) so that argument checking can be built and tested without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/falcon.h"

namespace falcon {

enum class Path : int {
    kEmpty = 0,      // seqlen == 0: only the boundary state is passed through
    kRecurrent = 1,  // token-recurrent form (every variant)
    kChunkF1 = 2,    // chunk-parallel Falcon-1
    kChunkA = 3,     // chunk-parallel Falcon-1A / Falcon-3A (scalar-decay writes)
    kChunkF2 = 4,    // chunk-parallel Falcon-2
    kChunkF3 = 6,    // chunk-parallel Falcon-3 (stacked window rows)
    kChunkF1Xfer = 8,   // chunk-parallel Falcon-1, bf16: per-chunk transfer operators, then the carry
    kChunkA1 = 9,    // chunk-parallel Falcon-1A, bf16, d_k = d_v = 64: register-operand segment kernels
    kDecode = 11,    // seqlen == 1: the single-token step of any variant, one kernel
    kChunkF2A = 12,  // chunk-parallel Falcon-2A (per-column inner-product write)
    kChunkF3X = 13,  // Falcon-3, bf16, d = 64, W in {2, 4, 8}: window pass, 64-token transfer operators, Falcon-1 walk
};

struct Plan {
    // problem
    int variant = 0, dtype = 0, phi = 0;
    int B = 0, H = 0, T = 0, dk = 0, dv = 0, chunk = 0, window = 1;
    int BH = 0;
    int nchunks = 0;         // ceil(T / chunk) for chunk paths (T / tokens per chunk for F3)
    int ct = 0;              // tokens per chunk (Falcon-3 chunk path)
    int Tpad = 0;            // rows of the feature buffers (T, or nchunks * chunk)
    float eps = 0.f, eps_gamma = 0.f, eps_rms = 0.f;
    Path path = Path::kEmpty;

    // boundary
    bool fresh = true;       // input is a fresh sequence
    int n_tail_in = 0;
    int n_tail_out = 0;
    const float *S_in = nullptr, *xnext_in = nullptr, *tailx_in = nullptr, *taily_in = nullptr;
    float *S_out = nullptr, *xnext_out = nullptr, *tailx_out = nullptr, *taily_out = nullptr;

    // tensors
    const void *q = nullptr, *k = nullptr, *v = nullptr;
    const float *beta = nullptr, *lambda = nullptr;
    void *o = nullptr;

    // workspace carve-up (offsets in bytes from the workspace base)
    int slice = 0;           // value columns per workgroup of the state carry
    int seg_chunks = 0, nseg = 0;   // segmentation of the Falcon-1A/3A and bf16 Falcon-1 chunk paths
    bool feat_f32 = true;    // storage type of the normalised features
    size_t off_xn = 0, off_qn = 0, off_eta = 0, off_alpha = 0;
    size_t off_chunk = 0;    // chunk-path operators
    size_t off_seg_g = 0, off_seg_s = 0, off_seg_m = 0;
    size_t chunk_bytes = 0;
    size_t ws_bytes = 0;     // total required
    void *ws = nullptr;

    template <class T>
    T *ws_at(size_t off) const { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }
};

// Validate `a` and fill `p`.  Never touches the GPU.  Returns a falcon status.
// With check_pointers == false, only sizes and scalars are checked (used by
// falcon_fwd_workspace_size, which must not read pointer fields).
int build_plan(const falcon_fwd_args *a, Plan *p, bool check_pointers);

// Plan of one falcon_bwd call: sizes, the state in, and the workspace
// carve-up (features and step scalars, checkpointed states, the residuals,
// per-group partial sums of the reverse sweep).
struct BwdPlan {
    int dtype = 0, phi = 0, BH = 0, T = 0, dk = 0, dv = 0;
    float eps = 0.f, eps_gamma = 0.f, eps_rms = 0.f;
    bool fresh = true;
    const float *S_in = nullptr, *xnext_in = nullptr;
    // chunk-parallel form (T > 0, d_k and d_v at most 64): 64-token chunks
    bool chunked = false;
    int nchunks = 0;
    size_t off_ops = 0, off_cst = 0, off_hg = 0, off_phip = 0;
    // token-recurrent form (the other shapes)
    size_t off_xn = 0, off_qn = 0, off_eta = 0, off_alpha = 0, off_states = 0, off_res = 0, off_part = 0;
    size_t ws_bytes = 0;
    void *ws = nullptr;
    template <class T>
    T *ws_at(size_t off) const { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }
};

// tokens per chunk of the chunk-parallel backward
constexpr int kBwdChunk = 64;
constexpr bool bwd_chunked(long long T, int dk, int dv) { return T > 0 && dk <= 64 && dv <= 64; }

// floats per (head, token, group of 16 value columns) record of the reverse
// sweep's partial sums: dgamma, deta, two pad words, dx [d_k], dqh [d_k]
constexpr int bwd_part_floats(int dk) { return 4 + 2 * dk; }
// the state pass keeps the state before every kBwdCheckpoint-th token; the
// sweep rebuilds the states in between from the stored residuals
constexpr int kBwdCheckpoint = 4;
constexpr long long bwd_checkpoints(long long T) { return (T + kBwdCheckpoint - 1) / kBwdCheckpoint; }

int build_bwd_plan(const falcon_bwd_args *a, BwdPlan *p, bool check_pointers);

}  // namespace falcon
