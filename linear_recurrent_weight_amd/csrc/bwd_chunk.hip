// Falcon-1 backward pass, chunk-parallel (summary §E.3 "Chunk-Parallel
// Backward Pass", §G.3 "Forward and Backward Algorithms", §H.1 "Affine Chunk
// Map"), in fp32 on the matrix cores (v_mfma_f32_16x16x4_f32), for
// d_k, d_v <= 64.
//
// Chunks of C = 64 tokens, local index t = 0..63, log-decay prefix
// b_t = sum_{i<=t} log2 gamma_i (b_{-1} = 0), D0_tj = 2^{b_t - b_j} (j <= t),
// D1_tj = 2^{b_{t-1} - b_j} (j < t).  With L = D1 o (X X^T) (strictly lower),
// N = diag(eta) L and T = (I + N)^{-1}, the forward of one chunk is affine in
// its entry state S_0:
//   S_end = A S_0 + B,   O = G S_0 + (terms free of S_0), where
//   A = 2^{b_63} I - X^T diag(2^{b_63 - b_t}) T diag(eta_t 2^{b_{t-1}}) X,
//   B = X^T diag(2^{b_63 - b_t}) T diag(eta) V,
//   G = diag(2^{b_t}) Qh - M T diag(eta_t 2^{b_{t-1}}) X,  M = D0 o (Qh X^T).
// The state gradient therefore crosses a chunk backwards as H <- A^T H +
// G^T dO (the transposed affine map).  Within a chunk, with S_0 and H (= dL/dS
// at the chunk's end, from the later chunks) known:
//   R = V - diag(2^{b_{t-1}}) X S_0 - L U,  U = diag(eta) R = T diag(eta)(V - diag(2^{b_{t-1}}) X S_0)
//       (u_t = eta_t r_t, r_t the residuals at S_{t-1});
//   W = T^T (M^T dO + diag(2^{b_63 - b_t}) X H)      (w_t = G_t^T x_t);
//   dqh = diag(2^{b_t}) dO S_0^T + (D0 o (dO U^T)) X;
//   dx / eta = diag(2^{b_63 - b_t}) R H^T + (D0^T o (R dO^T)) Qh
//              - (D1^T o (R W^T)) diag(eta) X - diag(2^{b_{t-1}}) W S_0^T - (D1 o (W U^T)) X;
//   deta_t = w_t . r_t,  dv_t = eta_t w_t;
//   gamma_t dgamma_t = <G_t, gamma_t S_{t-1}> = Phi_t - eta_t deta_t, where
//   Phi_t = <G_t, S_t> = <H, S_end> + sum_{s>=t} qh_s . dqh_s - sum_{s>t} eta_s w_s . v_s
//   (o_s . do_s = qh_s . dqh_s, and each step changes <G, S> by those terms).
// Kernels:
//   bwd_ops        per chunk: A, B and G^T dO, as fp32 records;
//   bwd_carry_fwd  per (head, 16 value columns): the entry state of every chunk, and S_T;
//   bwd_carry_rev  per (head, 16 value columns): H of every chunk, <H, S_end>
//                  per 16 columns, and dL/dS_0;
//   bwd_grads      per chunk: the token gradients above, the decay and step
//                  chain, and phi's vector-Jacobian products.
//
// Every matrix in LDS is fp32 with a row stride of 68 floats.  MFMA operands
// come in 16-index blocks of the contraction, lane (g = lane / 16, l16 = lane
// % 16) supplying k = k0 + 4 g + r in the r-th of four 16x16x4 steps, in A and
// B alike: an accumulator tile (lane holds rows 4 g + r, column l16) is then
// directly the B operand of a product over its rows, and the A operand of a
// product with its transpose.  A stored row with k contiguous gives one
// 16-byte read per lane; a matrix stored k-major gives four 4-byte reads
// whose banks 16 g + l16 are distinct.
#include <cstdio>

#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace falcon {
namespace {

constexpr int kC = 64;            // tokens per chunk
constexpr int kLd = 68;           // LDS row stride (floats)
constexpr int kMat = kC * kLd;    // floats of one 64-row LDS matrix

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// A-operand block of rows row0.. of M (k contiguous): M[row0 + l16][k0 + 4 g + r]
__device__ __forceinline__ f32x4 frag_kc(const float *M, int row0, int k0) {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const f32x4 *>(M + (row0 + (lane & 15)) * kLd + k0 + 4 * (lane >> 4));
}
// operand block read k-major: M[k0 + 4 g + r][col0 + l16]
__device__ __forceinline__ f32x4 frag_km(const float *M, int col0, int k0) {
    const int lane = threadIdx.x & 63;
    const float *p = M + (k0 + 4 * (lane >> 4)) * kLd + col0 + (lane & 15);
    return f32x4{p[0], p[kLd], p[2 * kLd], p[3 * kLd]};
}
// acc += A_blk * B_blk over one block of 16 contraction indices
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const f32x4 &a, const f32x4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
}
// the tile at rows row0.., columns col0.. of an LDS matrix in accumulator
// layout (lane holds rows row0 + 4 g + r, column col0 + l16)
__device__ __forceinline__ f32x4 get_tile(const float *M, int row0, int col0) {
    const int lane = threadIdx.x & 63;
    const float *p = M + (row0 + 4 * (lane >> 4)) * kLd + col0 + (lane & 15);
    return f32x4{p[0], p[kLd], p[2 * kLd], p[3 * kLd]};
}
// an accumulator tile stored transposed: element (row0 + 4 g + r, col0 + l16)
// at M[col0 + l16][row0 + 4 g + r] (one 16-byte write per lane)
__device__ __forceinline__ void put_tile_t(float *M, int row0, int col0, const f32x4 &v) {
    const int lane = threadIdx.x & 63;
    *reinterpret_cast<f32x4 *>(M + (col0 + (lane & 15)) * kLd + row0 + 4 * (lane >> 4)) = v;
}
// arr[row0 + 4 g + r], r = 0..3: per-token values of this lane's accumulator rows
__device__ __forceinline__ f32x4 rows4(const float *arr, int row0) {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const f32x4 *>(arr + row0 + 4 * (lane >> 4));
}
// an accumulator tile stored as rows row0.. / columns col0.. of an LDS matrix
__device__ __forceinline__ void put_tile(float *M, int row0, int col0, const f32x4 &v) {
    const int lane = threadIdx.x & 63;
    float *p = M + (row0 + 4 * (lane >> 4)) * kLd + col0 + (lane & 15);
    p[0] = v[0];
    p[kLd] = v[1];
    p[2 * kLd] = v[2];
    p[3 * kLd] = v[3];
}

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its global loads, so prefetched rows stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// per-token scalars of one chunk
struct __attribute__((aligned(16))) Tok {
    float eta[kC], alpha[kC], lam[kC], den[kC];
    float bl[kC], bm[kC];       // b_t and b_{t-1}
    float sq[kC], sk[kC];       // phi's scale of q_t and of k_{t-1}
    float xx[kC];               // ||x_t||^2
    float dden[kC], qdq[kC];    // the denominator's gradient; qh_t . dqh_t
};

// n consecutive elements of one row (16-byte aligned) into fp32, or zeros
template <class E, int n>
__device__ __forceinline__ void load_row(const E *p, bool valid, float (&z)[n]) {
    if constexpr (sizeof(E) == 2) {
        static_assert(n % 8 == 0, "16-byte pieces");
#pragma unroll
        for (int c = 0; c < n / 8; ++c) {
            const uint4 u = valid ? reinterpret_cast<const uint4 *>(p)[c] : make_uint4(0, 0, 0, 0);
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z[8 * c + 2 * e] = __uint_as_float(wd[e] << 16);
                z[8 * c + 2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
            }
        }
    } else {
        static_assert(n % 4 == 0, "16-byte pieces");
#pragma unroll
        for (int c = 0; c < n / 4; ++c) {
            const float4 u = valid ? reinterpret_cast<const float4 *>(p)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
            z[4 * c] = u.x;
            z[4 * c + 1] = u.y;
            z[4 * c + 2] = u.z;
            z[4 * c + 3] = u.w;
        }
    }
}

template <class E, int DK>
__device__ void rows_features(const BwdArgs &a, int bh, int t0, float *X, float *Q, Tok &tk) {
    constexpr int HALF = DK / 2;
    const int tid = threadIdx.x;
    const int mq = tid >> 7, t = (tid >> 1) & 63, h = tid & 1;   // matrix (0: q, 1: k), row, half
    const int gt = t0 + t, T = a.T;
    float z[HALF];
    bool valid, carried = false;
    if (mq == 0) {
        valid = gt < T;
        load_row<E, HALF>(static_cast<const E *>(a.q) + (size_t(bh) * T + (valid ? gt : 0)) * DK + h * HALF,
                          valid, z);
    } else if (gt == 0) {
        carried = true;
        valid = T > 0 && !a.fresh && a.xnext_in;
        load_row<float, HALF>(a.xnext_in ? a.xnext_in + size_t(bh) * DK + h * HALF : nullptr, valid, z);
    } else {
        valid = gt < T;
        load_row<E, HALF>(static_cast<const E *>(a.k) + (size_t(bh) * T + (valid ? gt - 1 : 0)) * DK + h * HALF,
                          valid, z);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < HALF; ++e) ss += z[e] * z[e];
    ss += dpp<kDppQuadXor1>(ss);   // the row's other half (lanes 2t, 2t + 1)
    const float s = !valid ? 0.f : carried ? 1.f : phi_scale(ss, DK, a.eps_rms, a.phi);
    float *dst = (mq == 0 ? Q : X) + t * kLd + h * HALF;
    float xs = 0.f;
#pragma unroll
    for (int e = 0; e < HALF; ++e) {
        const float f = s * z[e];
        dst[e] = f;
        xs += f * f;
    }
    xs += dpp<kDppQuadXor1>(xs);
    if (h == 0) {
        if (mq == 0) tk.sq[t] = s;
        else {
            tk.sk[t] = s;
            tk.xx[t] = xs;
        }
    }
}

// eta, alpha, lambda, the denominator and the log-decay prefix (wave 0, lane =
// token), after the rows
__device__ void step_scalars(const BwdArgs &a, int t0, Tok &tk, const float2 &beta_lam) {
    const int tid = threadIdx.x, T = a.T;
    if (tid < 64) {
        const int tt = tid, gtt = t0 + tid;
        const bool in = gtt < T;
        const float beta = beta_lam.x, lam = beta_lam.y;
        const float den = tk.xx[tt] + lam + a.eps;
        float eta = step_eta(beta, den), alpha = step_alpha(eta, lam, a.eps_gamma);
        if (!in || (a.fresh && gtt == 0)) {
            eta = 0.f;
            alpha = 0.f;
        }
        const float lg = log2_1m(alpha);
        const float b = wave_inclusive_scan(lg);
        float bp = __shfl_up(b, 1, 64);
        if (tt == 0) bp = 0.f;
        tk.eta[tt] = eta;
        tk.alpha[tt] = alpha;
        tk.lam[tt] = lam;
        tk.den[tt] = den;
        tk.bl[tt] = b;
        tk.bm[tt] = bp;
    }
}

// beta_t and lambda_t of token t0 + lane (wave 0 only; 0 past T), requested
// at kernel entry so that their latency overlaps the rows'
__device__ __forceinline__ float2 load_beta_lam(const BwdArgs &a, int bh, int t0) {
    float2 v = make_float2(0.f, 0.f);
    const int gt = t0 + (threadIdx.x & 63);
    if (threadIdx.x < 64 && gt < a.T) {
        const size_t row = size_t(bh) * a.T + gt;
        v = make_float2(a.beta[row], a.lambda[row]);
    }
    return v;
}

// Features and step scalars of chunk c of head bh into LDS: Qh rows
// phi(q_t), X rows x_t = phi(k_{t-1}) (x of the sequence's first token: the
// carried feature, or 0 for a fresh sequence), rows past T zero, and the
// per-token eta, alpha (0 past T and for the fresh first step), lambda, the
// denominator, b_t, b_{t-1} and phi's scales.  The rows take the first 256
// threads (two per row); called by all threads of the workgroup, ends with a
// barrier.
template <class E, int DK>
__device__ void chunk_features(const BwdArgs &a, int bh, int t0, float *X, float *Q, Tok &tk,
                               const float2 &beta_lam) {
    if (threadIdx.x < 256) rows_features<E, DK>(a, bh, t0, X, Q, tk);
    __syncthreads();
    step_scalars(a, t0, tk, beta_lam);
    __syncthreads();
}

__device__ void inverse_diagonal(const float *Nm, float *Tm, float *Tt) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
    float *scr = w < 3 ? Tm + 16 * (w + 1) : Tm + 16 * kLd + 32;
    const float *Lw = Nm + 16 * w * kLd + 16 * w;   // diagonal block w of N (strictly lower part read)
    auto sync = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));   // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    };
    // L as operands: A rows from Lw (k contiguous), B k-major; entries on or
    // above the diagonal are zero by construction of N
    f32x4 z1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        z1[r] = (i == l16 ? 1.f : 0.f) - (l16 < i ? Lw[i * kLd + l16] : 0.f);
    }
    f32x4 la = frag_kc(Lw, 0, 0), lb = frag_km(Lw, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {   // zero the diagonal and above (not part of L)
        const int i = l16, k = 4 * g + r;
        if (k >= i) la[r] = 0.f;
        if (i >= k) lb[r] = 0.f;
    }
    f32x4 p = mma16(zero4(), la, lb);   // L^2
    put_tile(scr, 0, 0, p);
    sync();
    f32x4 z = z1 + mma16(zero4(), frag_kc(scr, 0, 0), z1);   // (I + L^2)(I - L)
    f32x4 p4 = mma16(zero4(), frag_kc(scr, 0, 0), p);         // L^4
    sync();
    put_tile(scr, 0, 0, p4);
    sync();
    z = z + mma16(zero4(), frag_kc(scr, 0, 0), z);            // (I + L^4) ...
    f32x4 p8 = mma16(zero4(), frag_kc(scr, 0, 0), p4);        // L^8
    sync();
    put_tile(scr, 0, 0, p8);
    sync();
    z = z + mma16(zero4(), frag_kc(scr, 0, 0), z);            // (I + L^8) ...
    put_tile(Tm, 16 * w, 16 * w, z);
    if (Tt) put_tile_t(Tt, 16 * w, 16 * w, z);
}

// column block w of T below the diagonal, from the diagonal blocks in Tm
__device__ void inverse_columns(const float *Nm, float *Tm, float *Tt) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
    (void)g;
    (void)l16;
    const f32x4 z = get_tile(Tm, 16 * w, 16 * w);
    f32x4 col[4];
#pragma unroll
    for (int K = 0; K < 4; ++K) col[K] = K == w ? z : zero4();
#pragma unroll
    for (int I = 1; I < 4; ++I) {
        if (I <= w) continue;
        f32x4 acc = zero4();
#pragma unroll
        for (int K = 0; K < 4; ++K)
            if (K >= w && K < I) acc = mma16(acc, frag_kc(Nm, 16 * I, 16 * K), col[K]);
        f32x4 t = mma16(zero4(), frag_kc(Tm, 16 * I, 16 * I), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = -t[r];
        col[I] = t;
        put_tile(Tm, 16 * I, 16 * w, t);
        if (Tt) put_tile_t(Tt, 16 * I, 16 * w, t);
    }
}

// T = (I + N)^{-1} for N strictly lower (64 x 64 in LDS), into the lower
// tiles of Tm (and transposed into Tt when given); all 256 threads, N complete before the call, ends with a
// barrier.  Wave w inverts diagonal block w as (I - L)(I + L^2)(I + L^4)(I +
// L^8) (L = N_ww, exact because L^16 = 0), with upper tile (0,1), (0,2),
// (0,3) or (1,2) of Tm (never read as part of T) as its scratch; then column
// block w by substitution, T_IJ = -T_II sum_{K=J}^{I-1} N_IK T_KJ.
__device__ void unit_lower_inverse_mfma(const float *Nm, float *Tm, float *Tt = nullptr) {
    const int w = threadIdx.x >> 6;
    if (w < 4) inverse_diagonal(Nm, Tm, Tt);
    __syncthreads();
    if (w < 3) inverse_columns(Nm, Tm, Tt);
    __syncthreads();
}

// the ten lower 16x16 tiles (m >= n) of a 64 x 64 matrix, in order
__device__ __forceinline__ void lower_tile(int idx, int &m, int &n) {
    m = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    n = idx - m * (m + 1) / 2;
}

// The Grams of a chunk: L = D1 o (X X^T) (into Lm when given) and N =
// diag(eta) L (into Nm), lower tiles; the raw lower tiles of Qh X^T stay in
// qk (this wave's tiles w and w + 8 of eight waves).  The caller puts a
// barrier after.
template <int NK>
__device__ void chunk_grams(const float *X, const float *Q, const Tok &tk, float *Lm, float *Nm, f32x4 (&qk)[2]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = w + 8 * q;
        qk[q] = zero4();
        if (idx >= 10) continue;
        int m, n;
        lower_tile(idx, m, n);
        f32x4 kk = zero4(), qq = zero4();
#pragma unroll
        for (int s = 0; s < NK; ++s) {
            const f32x4 fb = frag_kc(X, 16 * n, 16 * s);
            kk = mma16(kk, frag_kc(X, 16 * m, 16 * s), fb);
            qq = mma16(qq, frag_kc(Q, 16 * m, 16 * s), fb);
        }
        qk[q] = qq;
        f32x4 lv, nv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * m + 4 * g + r, j = 16 * n + l16;
            lv[r] = j < t ? ex2(tk.bm[t] - tk.bl[j]) * kk[r] : 0.f;
            nv[r] = tk.eta[t] * lv[r];
        }
        if (Lm) put_tile(Lm, 16 * m, 16 * n, lv);
        put_tile(Nm, 16 * m, 16 * n, nv);
    }
}

// M = D0 o (Qh X^T) from the raw tiles of chunk_grams, stored transposed
// into Mm (Mm[j][t] = M_tj; the lower tiles of M)
__device__ void chunk_put_m(const Tok &tk, const f32x4 (&qk)[2], float *Mm) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = w + 8 * q;
        if (idx >= 10) continue;
        int m, n;
        lower_tile(idx, m, n);
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * m + 4 * g + r, j = 16 * n + l16;
            v[r] = j <= t ? ex2(tk.bl[t] - tk.bl[j]) * qk[q][r] : 0.f;
        }
        put_tile_t(Mm, 16 * m, 16 * n, v);
    }
}

// rows 16 m + 4 g + r, columns c0 + l16 of a [rows x ld] global matrix (rows
// at or past `nrows` read 0)
template <class E>
__device__ __forceinline__ f32x4 load_tile(const E *p, int stride, int row0, int c0, int nrows) {
    const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = row0 + 4 * g + r;
        v[r] = row < nrows ? ld(p, size_t(row) * stride + c0 + l16) : 0.f;
    }
    return v;
}

// ---------------------------------------------------------------------------
// bwd_ops: per chunk, the forward's transfer A, B and the reverse term G^T dO
// ---------------------------------------------------------------------------
template <class E, int NK, int NV>
__global__ __launch_bounds__(512, 4) void bwd_ops(BwdArgs a) {
    constexpr int DK = 16 * NK, DV = 16 * NV;
    __shared__ __attribute__((aligned(16))) float lds[4 * kMat];
    __shared__ Tok tk;
    float *X = lds, *Q = lds + kMat, *Nm = lds + 2 * kMat, *Tm = lds + 3 * kMat;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
    const int nck = a.nchunks;
    const int bh = blockIdx.x / nck, c = blockIdx.x % nck, t0 = c * kC;
    const int T = a.T;
    // waves 0-3: A (key tile w) and B (value tile w); waves 4-7: G^T dO (value tile w - 4)
    const int n = w & 3;
    const float2 beta_lam = load_beta_lam(a, bh, t0);
    const bool val = n < NV;
    // this wave's value tile of V (waves 0-3) or dO (waves 4-7), requested first
    f32x4 vt[4];
    {
        const E *src = static_cast<const E *>(w < 4 ? a.v : a.d_o) + (size_t(bh) * T + t0) * DV;
#pragma unroll
        for (int s = 0; s < 4; ++s) vt[s] = val ? load_tile(src, DV, 16 * s, 16 * n, T - t0) : zero4();
    }

    chunk_features<E, DK>(a, bh, t0, X, Q, tk, beta_lam);
    f32x4 qk[2];
    chunk_grams<NK>(X, Q, tk, nullptr, Nm, qk);
    __syncthreads();
    unit_lower_inverse_mfma(Nm, Tm);          // ends with a barrier; Nm is free afterwards
    chunk_put_m(tk, qk, Nm);                  // Nm now holds M^T
    __syncthreads();

    float *rec = a.ops + (size_t(bh) * nck + c) * size_t(DK * DK + 2 * DK * DV);
    float *Aop = rec, *Bop = rec + DK * DK, *Bb = Bop + DK * DV;
    const float bC = tk.bl[kC - 1];
    if (w < 4) {
        if (val) {
            // Z = T diag(eta) V; B = X^T diag(2^{b_63-b_t}) Z
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) vt[s][r] *= tk.eta[16 * s + 4 * g + r];
            f32x4 z[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s <= m; ++s) acc = mma16(acc, frag_kc(Tm, 16 * m, 16 * s), vt[s]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= ex2(bC - tk.bl[16 * m + 4 * g + r]);
                z[m] = acc;
            }
#pragma unroll
            for (int mm = 0; mm < NK; ++mm) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mma16(acc, frag_km(X, 16 * mm, 16 * s), z[s]);
#pragma unroll
                for (int r = 0; r < 4; ++r) Bop[(16 * mm + 4 * g + r) * DV + 16 * n + l16] = acc[r];
            }
        }
        if (w < NK) {
            // Y = T diag(eta_t 2^{b_{t-1}}) X, column tile w; A = 2^{b_63} I - X^T diag(2^{b_63-b_t}) Y
            f32x4 xb[4], y[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                xb[s] = frag_km(X, 16 * w, 16 * s);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * s + 4 * g + r;
                    xb[s][r] *= tk.eta[t] * ex2(tk.bm[t]);
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s <= m; ++s) acc = mma16(acc, frag_kc(Tm, 16 * m, 16 * s), xb[s]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= ex2(bC - tk.bl[16 * m + 4 * g + r]);
                y[m] = acc;
            }
            const float gC = ex2(bC);
#pragma unroll
            for (int mm = 0; mm < NK; ++mm) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mma16(acc, frag_km(X, 16 * mm, 16 * s), y[s]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i1 = 16 * mm + 4 * g + r, i2 = 16 * w + l16;
                    Aop[i1 * DK + i2] = (i1 == i2 ? gC : 0.f) - acc[r];
                }
            }
        }
    } else if (val) {
        // W_do = T^T M^T dO; G^T dO = Qh^T diag(2^{b_t}) dO - X^T diag(eta_t 2^{b_{t-1}}) W_do
        f32x4 pd[4], wd[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = m; s < 4; ++s) acc = mma16(acc, frag_kc(Nm, 16 * m, 16 * s), vt[s]);
            pd[m] = acc;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = m; s < 4; ++s) acc = mma16(acc, frag_km(Tm, 16 * m, 16 * s), pd[s]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * m + 4 * g + r;
                acc[r] *= tk.eta[t] * ex2(tk.bm[t]);
                vt[m][r] *= ex2(tk.bl[t]);
            }
            wd[m] = acc;
        }
#pragma unroll
        for (int mm = 0; mm < NK; ++mm) {
            f32x4 acc = zero4(), neg = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                acc = mma16(acc, frag_km(Q, 16 * mm, 16 * s), vt[s]);
                neg = mma16(neg, frag_km(X, 16 * mm, 16 * s), wd[s]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Bb[(16 * mm + 4 * g + r) * DV + 16 * n + l16] = acc[r] - neg[r];
        }
    }
}

// ---------------------------------------------------------------------------
// bwd_carry_fwd / bwd_carry_rev: one workgroup per (head, 16 value columns),
// wave w holding rows 16 w .. 16 w + 15 of that column tile
// ---------------------------------------------------------------------------
constexpr int kXs = 20;   // row stride of the exchanged column tile

// (head, 16-column tile) of a carry workgroup.  Workgroup ids go round-robin
// over the 8 XCDs; the tiles of one head take ids 8 apart, so they run on one
// XCD and read each chunk's record through one L2.  The grid is padded to a
// multiple of 8 heads (workgroups past the last head return at once).
__device__ __forceinline__ void carry_tile(int NV, int &bh, int &n) {
    const int id = blockIdx.x, rest = id >> 3;
    n = rest % NV;
    bh = (rest / NV) * 8 + (id & 7);
}
constexpr int kRing = 4;  // chunk records requested ahead of their step

template <int NK>
__global__ __launch_bounds__(64 * NK) void bwd_carry_fwd(BwdArgs a) {
    constexpr int DK = 16 * NK;
    __shared__ float Sx[2][DK * kXs];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
    const int DV = a.dv, NV = DV / 16, nck = a.nchunks;
    int bh, n;
    carry_tile(NV, bh, n);
    if (bh >= a.BH) return;
    const size_t rec = size_t(DK) * DK + 2 * size_t(DK) * DV;
    const int row0 = 16 * w + 4 * g, col = 16 * n + l16;
    f32x4 S;
#pragma unroll
    for (int r = 0; r < 4; ++r) S[r] = a.S_in ? a.S_in[(size_t(bh) * DK + row0 + r) * DV + col] : 0.f;
    float *cst = a.cst + size_t(bh) * (nck + 1) * DK * DV;
    // ring slot u holds chunk c = u (mod kRing): A rows 16 w + l16 as A
    // operands, and B rows row0 + r
    f32x4 fa[kRing][NK], fb[kRing];
    auto load = [&](int c, f32x4 (&ra)[NK], f32x4 &rb) {
        const float *A = a.ops + (size_t(bh) * nck + c) * rec, *B = A + DK * DK;
#pragma unroll
        for (int s = 0; s < NK; ++s)
            ra[s] = *reinterpret_cast<const f32x4 *>(A + (16 * w + l16) * DK + 16 * s + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) rb[r] = B[(row0 + r) * DV + col];
    };
#pragma unroll
    for (int u = 0; u < kRing; ++u)
        if (u < nck) load(u, fa[u], fb[u]);
    for (int c0 = 0; c0 < nck; c0 += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const int c = c0 + u;
            if (c >= nck) break;
            float *sx = Sx[u & 1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                cst[(size_t(c) * DK + row0 + r) * DV + col] = S[r];
                sx[(row0 + r) * kXs + l16] = S[r];
            }
            lds_barrier();
            f32x4 acc = fb[u];
#pragma unroll
            for (int s = 0; s < NK; ++s) {
                const float *p = sx + (16 * s + 4 * g) * kXs + l16;
                acc = mma16(acc, fa[u][s], f32x4{p[0], p[kXs], p[2 * kXs], p[3 * kXs]});
            }
            S = acc;
            if (c + kRing < nck) load(c + kRing, fa[u], fb[u]);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) cst[(size_t(nck) * DK + row0 + r) * DV + col] = S[r];
}

template <int NK>
__global__ __launch_bounds__(64 * NK) void bwd_carry_rev(BwdArgs a) {
    constexpr int DK = 16 * NK;
    __shared__ float Hx[2][DK * kXs];
    __shared__ float red[2][NK];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
    const int DV = a.dv, NV = DV / 16, nck = a.nchunks;
    int bh, n;
    carry_tile(NV, bh, n);
    if (bh >= a.BH) return;
    const size_t rec = size_t(DK) * DK + 2 * size_t(DK) * DV;
    const int row0 = 16 * w + 4 * g, col = 16 * n + l16;
    f32x4 H;
#pragma unroll
    for (int r = 0; r < 4; ++r) H[r] = a.d_S_out ? a.d_S_out[(size_t(bh) * DK + row0 + r) * DV + col] : 0.f;
    const float *cst = a.cst + size_t(bh) * (nck + 1) * DK * DV;
    float *hg = a.hg + size_t(bh) * nck * DK * DV;
    // ring slot u holds the u-th chunk from the end (mod kRing): A^T as A
    // operands (element (i, k) = A[k][i]), the rows of G^T dO, and the rows
    // of the state after the chunk
    f32x4 fa[kRing][NK], fb[kRing], sn[kRing];
    auto load = [&](int c, f32x4 (&ra)[NK], f32x4 &rb, f32x4 &rs) {
        const float *A = a.ops + (size_t(bh) * nck + c) * rec, *Bb = A + DK * DK + DK * DV;
#pragma unroll
        for (int s = 0; s < NK; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) ra[s][r] = A[(16 * s + 4 * g + r) * DK + 16 * w + l16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            rb[r] = Bb[(row0 + r) * DV + col];
            rs[r] = cst[(size_t(c + 1) * DK + row0 + r) * DV + col];
        }
    };
#pragma unroll
    for (int u = 0; u < kRing; ++u)
        if (u < nck) load(nck - 1 - u, fa[u], fb[u], sn[u]);
    for (int e0 = 0; e0 < nck; e0 += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const int e = e0 + u, c = nck - 1 - e;
            if (e >= nck) break;
            float *hx = Hx[u & 1];
            float ph = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hg[(size_t(c) * DK + row0 + r) * DV + col] = H[r];
                hx[(row0 + r) * kXs + l16] = H[r];
                ph += H[r] * sn[u][r];
            }
            ph = wave_sum(ph);
            if (lane == 0) red[u & 1][w] = ph;
            lds_barrier();
            if (w == 0 && lane == 0) {
                float tot = 0.f;
                for (int q = 0; q < NK; ++q) tot += red[u & 1][q];
                a.phip[(size_t(bh) * nck + c) * NV + n] = tot;
            }
            f32x4 acc = fb[u];
#pragma unroll
            for (int s = 0; s < NK; ++s) {
                const float *p = hx + (16 * s + 4 * g) * kXs + l16;
                acc = mma16(acc, fa[u][s], f32x4{p[0], p[kXs], p[2 * kXs], p[3 * kXs]});
            }
            H = acc;
            if (e + kRing < nck) load(c - kRing, fa[u], fb[u], sn[u]);
        }
    }
    if (a.d_S_in)
#pragma unroll
        for (int r = 0; r < 4; ++r) a.d_S_in[(size_t(bh) * DK + row0 + r) * DV + col] = H[r];
}

// ---------------------------------------------------------------------------
// bwd_grads: per chunk, every token gradient
// ---------------------------------------------------------------------------
template <class E, int NK, int NV>
__global__ __launch_bounds__(512) void bwd_grads(BwdArgs a) {
    constexpr int DK = 16 * NK, DV = 16 * NV;
    __shared__ __attribute__((aligned(16))) float lds[6 * kMat];
    __shared__ Tok tk;
    __shared__ float red[4][4][kC];   // partial sums per 16 columns: deta, w.v, qh.dqh, x.dx
    float *X = lds, *Q = lds + kMat, *SL = lds + 2 * kMat, *SN = lds + 3 * kMat, *ST = lds + 4 * kMat,
          *SD = lds + 5 * kMat;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
    const int nck = a.nchunks;
    const int bh = blockIdx.x / nck, c = blockIdx.x % nck, t0 = c * kC;
    const int T = a.T, nin = T - t0;   // rows of this chunk inside the sequence (> 0)
    const float *S0 = a.cst + (size_t(bh) * (nck + 1) + c) * DK * DV;
    const float *Hc = a.hg + (size_t(bh) * nck + c) * DK * DV;
    const size_t rowbase = size_t(bh) * T + t0;
    // Waves w and w + 4 share a SIMD.  Value tile n = w & 3: waves 0-3 the
    // forward solve (U, R), waves 4-7 the backward one (P, W).  Key tile
    // n: waves 0-3 dqh, waves 4-7 dx.
    const int n = w & 3;
    const bool lo = w < 4, val = n < NV, key = n < NK;

    // operands from memory, requested before the chunk's features
    const float2 beta_lam = load_beta_lam(a, bh, t0);
    f32x4 vv[4], dov[4], sb[NK], s0t[NV], ht[NV];
    {
        const E *v = static_cast<const E *>(a.v) + rowbase * DV;
        const E *dO = static_cast<const E *>(a.d_o) + rowbase * DV;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            vv[s] = val ? load_tile(v, DV, 16 * s, 16 * n, nin) : zero4();
            dov[s] = (val && !lo) ? load_tile(dO, DV, 16 * s, 16 * n, nin) : zero4();
        }
        // S_0 (waves 0-3) or H (waves 4-7) as B operands over the key index
#pragma unroll
        for (int s = 0; s < NK; ++s) sb[s] = val ? load_tile(lo ? S0 : Hc, DV, 16 * s, 16 * n, DK) : zero4();
        // S_0^T and H^T blocks: lane (g, i) holds row 16 n + i, columns 16 s + 4 g ..
#pragma unroll
        for (int s = 0; s < NV; ++s) {
            s0t[s] = key ? *reinterpret_cast<const f32x4 *>(S0 + (16 * n + l16) * DV + 16 * s + 4 * g) : zero4();
            ht[s] = (key && !lo) ? *reinterpret_cast<const f32x4 *>(Hc + (16 * n + l16) * DV + 16 * s + 4 * g)
                                 : zero4();
        }
    }

    chunk_features<E, DK>(a, bh, t0, X, Q, tk, beta_lam);
    f32x4 qk[2];
    chunk_grams<NK>(X, Q, tk, SL, SN, qk);
    __syncthreads();
    unit_lower_inverse_mfma(SN, ST, SD);   // SD: T^T until dO is stored there
    chunk_put_m(tk, qk, SN);               // SN: M^T
    __syncthreads();

    const float bC = tk.bl[kC - 1];
    // ---- value tile n: waves 0-3 U = T diag(eta) RHS0, R = RHS0 - L U with
    // RHS0 = V - diag(2^{b_{t-1}}) X S_0; waves 4-7 P = M^T dO + diag(2^{b_63-b_t}) X H,
    // W = T^T P, dv = eta W, w.v
    f32x4 sol[4];
    f32x4 rr[4];
    if (val) {
        if (lo) {
            f32x4 rhs[4], y[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 xs = zero4();
#pragma unroll
                for (int s = 0; s < NK; ++s) xs = mma16(xs, frag_kc(X, 16 * m, 16 * s), sb[s]);
                const f32x4 bm = rows4(tk.bm, 16 * m), et = rows4(tk.eta, 16 * m);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    rhs[m][r] = vv[m][r] - ex2(bm[r]) * xs[r];
                    y[m][r] = et[r] * rhs[m][r];
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s <= m; ++s) acc = mma16(acc, frag_kc(ST, 16 * m, 16 * s), y[s]);
                sol[m] = acc;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s <= m; ++s) acc = mma16(acc, frag_kc(SL, 16 * m, 16 * s), sol[s]);
                rr[m] = rhs[m] - acc;
            }
        } else {
            f32x4 p[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = zero4(), xh = zero4();
#pragma unroll
                for (int s = m; s < 4; ++s) acc = mma16(acc, frag_kc(SN, 16 * m, 16 * s), dov[s]);
#pragma unroll
                for (int s = 0; s < NK; ++s) xh = mma16(xh, frag_kc(X, 16 * m, 16 * s), sb[s]);
                const f32x4 bl = rows4(tk.bl, 16 * m);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += ex2(bC - bl[r]) * xh[r];
                p[m] = acc;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = m; s < 4; ++s) acc = mma16(acc, frag_kc(SD, 16 * m, 16 * s), p[s]);
                sol[m] = acc;
            }
            E *dV = static_cast<E *>(a.d_v) + rowbase * DV;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 et = rows4(tk.eta, 16 * m);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * m + 4 * g + r;
                    const float wvv = group_sum<16>(sol[m][r] * vv[m][r]);
                    if (l16 == 0) red[1][n][t] = wvv;
                    if (t < nin) st(dV, size_t(t) * DV + 16 * n + l16, et[r] * sol[m][r]);
                }
            }
        }
    }
    __syncthreads();   // L, M^T, T and T^T are no longer read
    float *SU = SL, *SR = SN, *SW = ST, *SO = SD;
    if (val) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (lo) {
                put_tile(SU, 16 * m, 16 * n, sol[m]);
                put_tile(SR, 16 * m, 16 * n, rr[m]);
            } else {
                put_tile(SW, 16 * m, 16 * n, sol[m]);
                put_tile(SO, 16 * m, 16 * n, dov[m]);
            }
        }
    }
    __syncthreads();
    // deta_t = w_t . r_t over value tile n (waves 4-7: W in registers, R from LDS)
    if (val && !lo) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 rv = get_tile(SR, 16 * m, 16 * n);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float de = group_sum<16>(sol[m][r] * rv[r]);
                if (l16 == 0) red[0][n][16 * m + 4 * g + r] = de;
            }
        }
    }

    // ---- products over the value index, column tile n of C x C:
    //   waves 0-3: dO U^T and W U^T on lower tiles (m >= n), R W^T on tile (n, n);
    //   waves 4-7: R dO^T on upper tiles (m <= n), R W^T on tiles m < n.
    // Key tile n: waves 0-3 dO S_0^T; waves 4-7 R H^T and W S_0^T.
    // The shared operand blocks are read once per value block s.
    f32x4 fa[4], fb[4], kx[4], ky = zero4();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        fa[m] = zero4();
        fb[m] = zero4();
        kx[m] = zero4();
    }
    if (lo) {
#pragma unroll
        for (int s = 0; s < NV; ++s) {
            const f32x4 bu = frag_kc(SU, 16 * n, 16 * s), bw = frag_kc(SW, 16 * n, 16 * s);
            ky = mma16(ky, frag_kc(SR, 16 * n, 16 * s), bw);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 ado = frag_kc(SO, 16 * m, 16 * s);
                if (key) kx[m] = mma16(kx[m], ado, s0t[s]);
                if (m >= n) {
                    fa[m] = mma16(fa[m], ado, bu);
                    fb[m] = mma16(fb[m], frag_kc(SW, 16 * m, 16 * s), bu);
                }
            }
        }
    } else {
        f32x4 rh[4], ws[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            rh[m] = zero4();
            ws[m] = zero4();
        }
#pragma unroll
        for (int s = 0; s < NV; ++s) {
            const f32x4 bo = frag_kc(SO, 16 * n, 16 * s), bw = frag_kc(SW, 16 * n, 16 * s);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 ar = frag_kc(SR, 16 * m, 16 * s);
                if (key) {
                    rh[m] = mma16(rh[m], ar, ht[s]);
                    ws[m] = mma16(ws[m], frag_kc(SW, 16 * m, 16 * s), s0t[s]);
                }
                if (m <= n) fa[m] = mma16(fa[m], ar, bo);
                if (m < n) fb[m] = mma16(fb[m], ar, bw);
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 bl = rows4(tk.bl, 16 * m), bm = rows4(tk.bm, 16 * m);
#pragma unroll
            for (int r = 0; r < 4; ++r) kx[m][r] = ex2(bC - bl[r]) * rh[m][r] - ex2(bm[r]) * ws[m][r];
        }
    }
    __syncthreads();   // U, R, W, dO are no longer read
    // the masked C x C factors, column tile n:
    //   F1 (SL) = D0 o (dO U^T), lower tiles (waves 0-3);
    //   F2 (SN) = -(D1^T o (R W^T)) diag(eta) - D1 o (W U^T): tiles m >= n by waves 0-3, m < n by waves 4-7;
    //   F3 (ST) = D0^T o (R dO^T), upper tiles (waves 4-7)
    float *F1 = SL, *F2 = SN, *F3 = ST;
    {
        const int uu = 16 * n + l16;
        const float bl_u = tk.bl[uu], bm_u = tk.bm[uu], eta_u = tk.eta[uu];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 bl = rows4(tk.bl, 16 * m), bm = rows4(tk.bm, 16 * m);
            f32x4 v1, v2, v3;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * m + 4 * g + r;
                if (lo) {
                    v1[r] = uu <= t ? ex2(bl[r] - bl_u) * fa[m][r] : 0.f;
                    v2[r] = uu < t ? -ex2(bm[r] - bl_u) * fb[m][r]
                          : uu > t ? -ex2(bm_u - bl[r]) * eta_u * ky[r] : 0.f;
                } else {
                    v3[r] = uu >= t ? ex2(bl_u - bl[r]) * fa[m][r] : 0.f;
                    v2[r] = -ex2(bm_u - bl[r]) * eta_u * fb[m][r];
                }
            }
            if (lo) {
                if (m >= n) {
                    put_tile(F1, 16 * m, 16 * n, v1);
                    put_tile(F2, 16 * m, 16 * n, v2);
                }
            } else {
                if (m <= n) put_tile(F3, 16 * m, 16 * n, v3);
                if (m < n) put_tile(F2, 16 * m, 16 * n, v2);
            }
        }
    }
    __syncthreads();

    // ---- key tile n: waves 0-3 dqh = diag(2^{b_t}) dO S_0^T + F1 X;
    // waves 4-7 dx / eta = (R H^T, W S_0^T terms) + F3 Qh + F2 X
    f32x4 kd[4];
    if (key) {
        f32x4 acc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = zero4();
        if (lo) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const f32x4 bx = frag_km(X, 16 * n, 16 * s);
#pragma unroll
                for (int m = s; m < 4; ++m) acc[m] = mma16(acc[m], frag_kc(F1, 16 * m, 16 * s), bx);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 bl = rows4(tk.bl, 16 * m);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * m + 4 * g + r;
                    kd[m][r] = ex2(bl[r]) * kx[m][r] + acc[m][r];
                    const float qd = group_sum<16>(Q[t * kLd + 16 * n + l16] * kd[m][r]);
                    if (l16 == 0) red[2][n][t] = qd;
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const f32x4 bx = frag_km(X, 16 * n, 16 * s), bq = frag_km(Q, 16 * n, 16 * s);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    acc[m] = mma16(acc[m], frag_kc(F2, 16 * m, 16 * s), bx);
                    if (m <= s) acc[m] = mma16(acc[m], frag_kc(F3, 16 * m, 16 * s), bq);
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) kd[m] = kx[m] + acc[m];
        }
    }
    __syncthreads();

    // ---- per token (wave 0, lane i takes token 63 - i so that suffix sums
    // are prefix scans): Phi_t, the decay and step chain, dbeta, dlambda
    if (tid < 64) {
        const int t = kC - 1 - lane, gt = t0 + t;
        float de = 0.f, wvv = 0.f, qd = 0.f;
        for (int q = 0; q < NV; ++q) {
            de += red[0][q][t];
            wvv += red[1][q][t];
        }
        for (int q = 0; q < NK; ++q) qd += red[2][q][t];
        float phiE = 0.f;
        for (int q = 0; q < NV; ++q) phiE += a.phip[(size_t(bh) * nck + c) * NV + q];
        const float eta = tk.eta[t], alpha = tk.alpha[t], lam = tk.lam[t], den = tk.den[t];
        const float ewv = eta * wvv;
        const float sq_ge = wave_inclusive_scan(qd);          // sum over s >= t
        const float se_gt = wave_inclusive_scan(ewv) - ewv;   // sum over s > t
        const float phi_t = phiE + sq_ge - se_gt;
        const float dgam = (phi_t - eta * de) / (1.f - alpha);
        float dbeta = 0.f, dl = 0.f, dden = 0.f;
        if (!(a.fresh && gt == 0)) {
            const float dalpha = -dgam;
            float de2 = de;
            if (alpha < 1.f - a.eps_gamma) {   // the clamp does not bind
                de2 += dalpha * lam;
                dl = dalpha * eta;
            }
            if (den != 0.f) {
                dbeta = de2 / den;
                dden = -de2 * eta / den;
                dl += dden;
            }
        }
        if (gt < T) {
            a.d_beta[size_t(bh) * T + gt] = dbeta;
            a.d_lambda[size_t(bh) * T + gt] = dl;
        }
        tk.dden[t] = dden;
        tk.qdq[t] = qd;
    }
    __syncthreads();

    // ---- waves 0-3: dq_t through phi.  Waves 4-7: dx_t = eta_t (...) + 2 dden_t x_t
    const float invd = 1.f / float(DK);
    const bool rms = a.phi == FALCON_PHI_RMSNORM;
    if (key) {
        if (lo) {
            E *dQ = static_cast<E *>(a.d_q) + rowbase * DK;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * m + 4 * g + r, i = 16 * n + l16;
                    if (t < nin) {
                        const float val_ = rms ? tk.sq[t] * (kd[m][r] - invd * tk.qdq[t] * Q[t * kLd + i]) : kd[m][r];
                        st(dQ, size_t(t) * DK + i, val_);
                    }
                }
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * m + 4 * g + r, i = 16 * n + l16;
                    const float xh = X[t * kLd + i];
                    kd[m][r] = tk.eta[t] * kd[m][r] + 2.f * tk.dden[t] * xh;
                    const float xd = group_sum<16>(xh * kd[m][r]);
                    if (l16 == 0) red[3][n][t] = xd;
                }
        }
    }
    __syncthreads();
    // x_t = phi(k_{t-1}): d_k of token t - 1; the first token's x is the carried feature
    if (key && !lo) {
        E *dK = static_cast<E *>(a.d_k) + size_t(bh) * T * DK;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * m + 4 * g + r, gt = t0 + t, i = 16 * n + l16;
                if (t >= nin) continue;
                float xd = 0.f;
                for (int q = 0; q < NK; ++q) xd += red[3][q][t];
                if (gt >= 1) {
                    const float val_ = rms ? tk.sk[t] * (kd[m][r] - invd * xd * X[t * kLd + i]) : kd[m][r];
                    st(dK, size_t(gt - 1) * DK + i, val_);
                } else if (a.d_x_next_in) {
                    a.d_x_next_in[size_t(bh) * DK + i] = a.fresh ? 0.f : kd[m][r];
                }
            }
    }
    // k_{T-1} feeds only the next segment's first pair
    if (c == nck - 1 && w == 0) {
        E *dK = static_cast<E *>(a.d_k) + size_t(bh) * T * DK;
        const E *kk = static_cast<const E *>(a.k) + size_t(bh) * T * DK;
        const float z = lane < DK ? ld(kk, size_t(T - 1) * DK + lane) : 0.f;
        const float gx = (a.d_x_next_out && lane < DK) ? a.d_x_next_out[size_t(bh) * DK + lane] : 0.f;
        const float s = phi_scale(wave_sum(z * z), DK, a.eps_rms, a.phi);
        const float xh = s * z;
        const float xg = wave_sum(xh * gx);
        const float val_ = rms ? s * (gx - xg * xh * invd) : gx;
        if (lane < DK) st(dK, size_t(T - 1) * DK + lane, val_);
    }
}

template <class E, int NK, int NV>
void launch_nv(const BwdArgs &a, hipStream_t s, Marks *m) {
    const unsigned chunks = static_cast<unsigned>(a.BH) * static_cast<unsigned>(a.nchunks);
    const unsigned tiles = static_cast<unsigned>((a.BH + 7) / 8) * 8 * NV;
    bwd_ops<E, NK, NV><<<chunks, 512, 0, s>>>(a);
    m->mark(s);
    bwd_carry_fwd<NK><<<tiles, 64 * NK, 0, s>>>(a);
    m->mark(s);
    bwd_carry_rev<NK><<<tiles, 64 * NK, 0, s>>>(a);
    m->mark(s);
    bwd_grads<E, NK, NV><<<chunks, 512, 0, s>>>(a);
    m->mark(s);
}

template <class E, int NK>
void launch_nk(const BwdArgs &a, hipStream_t s, Marks *m) {
    switch (a.dv) {
        case 16: launch_nv<E, NK, 1>(a, s, m); break;
        case 32: launch_nv<E, NK, 2>(a, s, m); break;
        default: launch_nv<E, NK, 4>(a, s, m); break;
    }
}

template <class E>
void launch_io(const BwdArgs &a, hipStream_t s, Marks *m) {
    switch (a.dk) {
        case 16: launch_nk<E, 1>(a, s, m); break;
        case 32: launch_nk<E, 2>(a, s, m); break;
        default: launch_nk<E, 4>(a, s, m); break;
    }
}

}  // namespace

void launch_bwd_chunk(const BwdArgs &a, bool io_bf16, hipStream_t s, Marks *m) {
    if (io_bf16) launch_io<bf16_t>(a, s, m);
    else launch_io<float>(a, s, m);
}

}  // namespace falcon
