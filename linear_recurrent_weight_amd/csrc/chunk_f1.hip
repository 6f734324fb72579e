// Chunk-parallel Falcon-1 forward (summary Figure 2/4 "chunk-parallel form",
// §D.1 "Chunk-Local Evaluation", §E.2, §G and §G.1 single-solve kernel).
//
// Within a chunk of C = 64 tokens, with the log-prefix b_i = sum_{s<=i} log
// gamma_s restarted at 0 (log gamma = log1p(-alpha) in fp32), the write
// u_i = eta_i (y_i - S_{i-1}^T x_i) of every token satisfies the unit-lower
// system
//     u_i + eta_i sum_{j<i} e^{b_{i-1}-b_j} (x_i.x_j) u_j
//         = eta_i (y_i - e^{b_{i-1}} S_0^T x_i),
// where S_0 is the chunk-entry state.  With Tp = L^{-1} diag(eta):
//     U   = Tp (Y - diag(e^{b_{i-1}}) X S_0)                  (one solve)
//     O   = diag(e^{b_i}) Qh S_0 + P U,   P_ij = e^{b_i-b_j} qh_i.x_j, j <= i
//     S_C = e^{b_C} S_0 + (diag(e^{b_C-b_i}) X)^T U.
// Every factor is a ratio e^{b_i - b_j} with i >= j, so nothing overflows.
//
// Kernel 1 (chunk_f1_prep), one workgroup per chunk, all chunks in parallel:
//   log-prefix, Gram X X^T and scores Qh X^T on MFMA, the inverse of the
//   unit-lower system in fp32, and the chunk operators Tp and P.
// Kernel 2 (chunk_f1_scan), one workgroup per (head, 16 value columns):
//   walks the chunks in order with the fp32 state slice held in MFMA
//   accumulators; per chunk  XS -> residual -> U = Tp R -> output, state.
#include "chunk_layout.h"
#include "common.h"
#include "kernels.h"
#include "tri_inverse.h"

namespace falcon {
namespace {

constexpr int C = kChunk;

// One 16x16 MFMA tile: acc += A[16 x K] * B[K x 16].  A is row-major with k
// contiguous (row stride lda); B is given transposed, Bt[16 x K] with k
// contiguous (row stride ldb).  Result lane layout: acc[r] holds row
// 4*(lane/16)+r, column lane%16.
template <class E> struct Mma;

template <> struct Mma<bf16_t> {
    static constexpr int KS = 32;
    __device__ static f32x4 run(f32x4 acc, const bf16_t *A, int lda, const bf16_t *Bt, int ldb, int kbeg,
                                int kend) {
        const int lane = threadIdx.x & 63;
        const int row = lane & 15, kq = 8 * (lane >> 4);
        for (int k0 = kbeg; k0 < kend; k0 += KS) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(A + row * lda + k0 + kq);
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(Bt + row * ldb + k0 + kq);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
        return acc;
    }
};

template <> struct Mma<float> {
    static constexpr int KS = 4;
    __device__ static f32x4 run(f32x4 acc, const float *A, int lda, const float *Bt, int ldb, int kbeg,
                                int kend) {
        const int lane = threadIdx.x & 63;
        const int row = lane & 15, kq = lane >> 4;
        for (int k0 = kbeg; k0 < kend; k0 += KS) {
            const float a = A[row * lda + k0 + kq];
            const float b = Bt[row * ldb + k0 + kq];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
        return acc;
    }
};

// end of the k range of a lower-triangular operator for output rows up to
// (16 * tile + 15), rounded up to the MFMA k step
template <class E>
__device__ __forceinline__ int tri_kend(int tile) {
    const int need = 16 * tile + 16;
    return (need + Mma<E>::KS - 1) / Mma<E>::KS * Mma<E>::KS;
}

// ---------------------------------------------------------------------------
// Kernel 1: per-chunk operators
// ---------------------------------------------------------------------------
constexpr int kLs = C + 1;  // fp32 LDS row stride

template <class E, int DK>
__global__ __launch_bounds__(256) void chunk_f1_prep(ChunkF1Args a) {
    __shared__ float Lm[C * kLs];   // strictly-lower part of the system
    __shared__ float Tm[C * kLs];   // its inverse
    __shared__ float Pm[C * kLs];   // decayed scores
    __shared__ float Mt[3 * 16 * 17];
    __shared__ float bs[C], bps[C], etas[C];

    const int c = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t row0 = size_t(bh) * a.Tpad + size_t(c) * C;
    const E *X = static_cast<const E *>(a.xn) + row0 * DK;
    const E *Q = static_cast<const E *>(a.qn) + row0 * DK;
    char *ops = static_cast<char *>(a.ops) + (size_t(bh) * a.nchunks + c) * a.chunk_bytes;
    E *Tp = reinterpret_cast<E *>(ops + chunk_f1_tp_off());
    E *Pg = reinterpret_cast<E *>(ops + chunk_f1_p_off(sizeof(E)));
    float *scal = reinterpret_cast<float *>(ops + chunk_f1_scal_off(sizeof(E)));

    // 1. chunk-local log-prefix (restarted at 0) and decay factors
    if (wave == 0) {
        const float eta = a.eta[row0 + lane];
        const float alpha = a.alpha[row0 + lane];
        const float lg = log1pf(-alpha);
        const float b = wave_inclusive_scan(lg);
        float bp = __shfl_up(b, 1, 64);
        if (lane == 0) bp = 0.f;
        const float bC = __shfl(b, 63, 64);
        bs[lane] = b;
        bps[lane] = bp;
        etas[lane] = eta;
        scal[0 * C + lane] = expf(bp);
        scal[1 * C + lane] = expf(b);
        scal[2 * C + lane] = expf(bC - b);
        scal[3 * C + lane] = lane == 0 ? expf(bC) : 0.f;
    }
    __syncthreads();

    // 2. Gram and score tiles on MFMA (lower triangle of 16x16 tiles)
    for (int job = wave; job < 20; job += 4) {
        const int which = job / 10;  // 0: Gram X X^T, 1: scores Qh X^T
        int t = job % 10, I = 0;
        while (t > I) { t -= I + 1; ++I; }
        const int J = t;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const E *A = (which == 0 ? X : Q) + size_t(16 * I) * DK;
        acc = Mma<E>::run(acc, A, DK, X + size_t(16 * J) * DK, DK, 0, DK);
        const int j = 16 * J + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * (lane >> 4) + r;
            if (which == 0) {
                Lm[i * kLs + j] = j < i ? etas[i] * expf(bps[i] - bs[j]) * acc[r] : 0.f;
            } else {
                Pm[i * kLs + j] = j <= i ? expf(bs[i] - bs[j]) * acc[r] : 0.f;
            }
        }
    }
    // upper tiles are zero
    for (int idx = tid; idx < C * C; idx += 256) {
        const int i = idx / C, j = idx % C;
        if ((j >> 4) > (i >> 4)) {
            Lm[i * kLs + j] = 0.f;
            Pm[i * kLs + j] = 0.f;
            Tm[i * kLs + j] = 0.f;
        }
    }
    __syncthreads();

    // 3. inverse of the unit-lower system I + Lm, by 16x16 blocks
    unit_lower_inverse64(Lm, Tm, Mt, kLs);

    // 4. Tp = L^{-1} diag(eta) and P, in the storage type
    for (int idx = tid; idx < C * C; idx += 256) {
        const int i = idx / C, j = idx % C;
        st(Tp, idx, j <= i ? Tm[i * kLs + j] * etas[j] : 0.f);
        st(Pg, idx, Pm[i * kLs + j]);
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: sequential walk over the chunks of one (head, 16-column slice)
// ---------------------------------------------------------------------------
template <class E> struct Pad;
template <> struct Pad<bf16_t> { static constexpr int v = 8; };   // keeps rows 16-byte aligned
template <> struct Pad<float> { static constexpr int v = 4; };

template <class E>
__device__ __forceinline__ void st4(E *p, const f32x4 &v) {
#pragma unroll
    for (int r = 0; r < 4; ++r) st(p, r, v[r]);
}

template <class E, int DK>
__global__ __launch_bounds__(256) void chunk_f1_scan(ChunkF1Args a, int nslice) {
    constexpr int PD = Pad<E>::v;
    constexpr int LS = DK + PD;   // stride of [j][d] buffers
    constexpr int LT = C + PD;    // stride of [.][token] buffers
    constexpr int NT = DK >= 64 ? DK / 64 : 1;  // state row tiles per wave
    __shared__ __align__(16) E St[2][16 * LS];  // S^T slice (bf16/fp32 copy)
    __shared__ __align__(16) E R0t[16 * LT];    // residual^T
    __shared__ __align__(16) E Ut[16 * LT];     // U^T
    __shared__ __align__(16) E Xht[DK * LT];    // (diag(w) X)^T

    // XCD-aware order: all slices of one head land on the same XCD
    const int id = blockIdx.x;
    const int u = id & 7, rest = id >> 3;
    const int s = rest % nslice, g = rest / nslice;
    const int bh = g * 8 + u;
    if (bh >= a.BH) return;
    const int j0 = 16 * s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dv = a.dv, T = a.T;
    const E *Xall = static_cast<const E *>(a.xn) + size_t(bh) * a.Tpad * DK;
    const E *Qall = static_cast<const E *>(a.qn) + size_t(bh) * a.Tpad * DK;
    const E *V = static_cast<const E *>(a.v) + size_t(bh) * T * dv;
    E *O = static_cast<E *>(a.o) + size_t(bh) * T * dv;
    const char *opsb = static_cast<const char *>(a.ops) + size_t(bh) * a.nchunks * a.chunk_bytes;

    // state slice S[d][j0 + j] in accumulators: tile m of this wave covers
    // rows 16 * (wave * NT + m) .. + 15
    const bool owns = 16 * wave * NT < DK;
    f32x4 S[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
        const int dbase = 16 * (wave * NT + m);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = dbase + 4 * (lane >> 4) + r;
            S[m][r] = (owns && a.S_in) ? a.S_in[(size_t(bh) * DK + d) * dv + j0 + (lane & 15)] : 0.f;
        }
        if (owns) {
            // S^T copy: row j = lane % 16, columns d .. d+3
            E *dst = St[0] + (lane & 15) * LS + dbase + 4 * (lane >> 4);
            st4(dst, S[m]);
        }
    }
    int cur = 0;
    __syncthreads();

    for (int c = 0; c < a.nchunks; ++c) {
        const int t0 = c * C;
        const E *X = Xall + size_t(t0) * DK;
        const E *Qh = Qall + size_t(t0) * DK;
        const char *ops = opsb + size_t(c) * a.chunk_bytes;
        const E *Tp = reinterpret_cast<const E *>(ops + chunk_f1_tp_off());
        const E *Pg = reinterpret_cast<const E *>(ops + chunk_f1_p_off(sizeof(E)));
        const float *scal = reinterpret_cast<const float *>(ops + chunk_f1_scal_off(sizeof(E)));

        // phase 1: R0 = Y - diag(Gamma_{i-1}) X S_0 for tokens 16w..16w+15
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = Mma<E>::run(acc, X + size_t(16 * wave) * DK, DK, St[cur], LS, 0, DK);
            const int j = lane & 15;
            f32x4 r0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * wave + 4 * (lane >> 4) + r;
                const float y = (t0 + i < T) ? ld(V, size_t(t0 + i) * dv + j0 + j) : 0.f;
                r0[r] = y - scal[i] * acc[r];
            }
            st4(R0t + j * LT + 16 * wave + 4 * (lane >> 4), r0);
        }
        __syncthreads();

        // phase 2: U = Tp R0 (rows 16w..16w+15); build (diag(w) X)^T
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = Mma<E>::run(acc, Tp + 16 * wave * C, C, R0t, LT, 0, tri_kend<E>(wave));
            st4(Ut + (lane & 15) * LT + 16 * wave + 4 * (lane >> 4), acc);
            for (int idx = tid; idx < C * DK; idx += 256) {
                const int i = idx / DK, d = idx % DK;
                st(Xht, d * LT + i, scal[2 * C + i] * ld(X, idx));
            }
        }
        __syncthreads();

        // phase 3a: O^T = diag-scaled S^T Qh^T + U^T P^T (tokens 16w..16w+15)
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = Mma<E>::run(acc, St[cur], LS, Qh + size_t(16 * wave) * DK, DK, 0, DK);
            const int i = 16 * wave + (lane & 15);
            const float gi = scal[C + i];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= gi;
            acc = Mma<E>::run(acc, Ut, LT, Pg + size_t(16 * wave) * C, C, 0, tri_kend<E>(wave));
            if (t0 + i < T) st4(O + size_t(t0 + i) * dv + j0 + 4 * (lane >> 4), acc);
        }
        // phase 3b: S = Gamma_C S + (diag(w) X)^T U
        {
            const float gC = scal[3 * C];
            if (owns) {
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    const int dbase = 16 * (wave * NT + m);
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[m][r] *= gC;
                    S[m] = Mma<E>::run(S[m], Xht + dbase * LT, LT, Ut, LT, 0, C);
                    st4(St[cur ^ 1] + (lane & 15) * LS + dbase + 4 * (lane >> 4), S[m]);
                }
            }
        }
        cur ^= 1;
        __syncthreads();
    }

    if (a.S_out && owns) {
#pragma unroll
        for (int m = 0; m < NT; ++m) {
            const int dbase = 16 * (wave * NT + m);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = dbase + 4 * (lane >> 4) + r;
                a.S_out[(size_t(bh) * DK + d) * dv + j0 + (lane & 15)] = S[m][r];
            }
        }
    }
}

template <class E, int DK>
void launch_dk(const ChunkF1Args &a, hipStream_t s, Marks *m) {
    chunk_f1_prep<E, DK><<<dim3(a.nchunks, a.BH), 256, 0, s>>>(a);
    m->mark(s);
    const int nslice = a.dv / 16;
    const int groups = (a.BH + 7) / 8;
    chunk_f1_scan<E, DK><<<groups * nslice * 8, 256, 0, s>>>(a, nslice);
    m->mark(s);
}

template <class E>
void launch_e(const ChunkF1Args &a, hipStream_t s, Marks *m) {
    if (a.dk == 32) launch_dk<E, 32>(a, s, m);
    else if (a.dk == 64) launch_dk<E, 64>(a, s, m);
    else launch_dk<E, 128>(a, s, m);
}

}  // namespace

void launch_chunk_f1(const ChunkF1Args &a, bool bf16, hipStream_t s, Marks *m) {
    if (bf16) launch_e<bf16_t>(a, s, m);
    else launch_e<float>(a, s, m);
}

}  // namespace falcon
