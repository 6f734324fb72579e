// Chunk-parallel Falcon-3 forward for bf16 inputs, d_k = d_v = 64 and a
// window W of 2, 4 or 8 pairs (summary §4.4 "Mini-batch Update Rule for
// Regression (Falcon-3)", §C.7, §H.3 "Mapping Falcon-3 to ParallelFlow"),
// through the same per-chunk transfer operators as the bf16 Falcon-1 path.
//
// Token t writes the W pairs of its window, each with the residual at the
// state before t and the weight w_t = eta_t / B_t.  Stacking the W rows of
// every token (row r = (token tau, slot k), pair tau - W + 1 + k) turns a
// chunk into a unit-lower system whose rows of one token do not interact:
// with the chunk-local log-prefix b (base 2, restarted at 0 per chunk),
//     u_r + w_r sum_{r': tau' < tau} 2^{b_{tau-1} - b_tau'} (x_r . x_r') u_r'
//         = w_r (y_r - 2^{b_{tau-1}} S_0^T x_r),
// so that, as for Falcon-1, u = Ut - W S_0 with [-W | Ut] = Z = (I + N)^{-1} R,
// R = [-diag(w 2^{b_{tau-1}}) X | diag(w) Y], and the chunk folds into
//     A = sum_r 2^{b_C - b_tau} x_r Z_W,r,   B = sum_r 2^{b_C - b_tau} x_r Z_U,r,
//     [G | H]_t = [2^{b_t} qh_t | 0] + sum_{r: tau <= t} 2^{b_t - b_tau} (qh_t . x_r) Z_r
// (S_C = 2^{b_C} S_0 + A S_0 + B, o_t = G_t S_0 + H_t).
//
// A chunk of 64 tokens has 64 W stacked rows.  It is worked in W sub-chunks
// of 64 / W tokens (64 rows each, as in Falcon-1).  The rows of earlier
// sub-chunks enter a sub-chunk only through
//     K = sum_{r earlier} 2^{b_e - b_tau} x_r Z_r        [d_k x (d_k + d_v)],
// b_e the log-prefix at the end of the previous sub-chunk (every factor at
// most 1): the residuals lose w_r 2^{b_{tau-1} - b_e} (X K)_r, the outputs
// gain 2^{b_t - b_e} qh_t^T K, and K advances by 2^{b_e' - b_e} and the
// sub-chunk's own rows.  After the last sub-chunk K = [A | B].  The
// sub-chunk's system is solved as in the Falcon-1 kernel: diagonal 16-row
// blocks of I + N inverted in fp32, forward substitution over the blocks on
// MFMA, one column tile of Z per wave, in registers; K stays in the waves'
// accumulators (fp32) with a bf16 copy in LDS for the products that read it.
//
// The rows are the raw q, k_{p-1} and v of the sequence: the RMS scales of
// phi (s_x of a pair, s_q of a query) are formed as the rows are staged and
// folded into the per-row and per-token factors that every product applies
// anyway.  w_t = eta_t / B_t and log2 gamma_t come from the window pass.
// One workgroup per (chunk, head), chunk-major; the records go to the
// workspace in the Falcon-1 layout, and f1_carry walks them.  The workgroup
// holding the last token writes the boundary state's x_next and window pairs.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;       // tokens of a chunk; stacked rows of a sub-chunk
constexpr int D = 64;           // d_k = d_v
constexpr int PK = 72;          // bf16 pitch of LDS rows of 64 elements
constexpr int NBP = 20;         // bf16 pitch of the 16 x 16 solve blocks
constexpr int LFB = 16 * 16 + 4;
constexpr int NTH = 512;        // 8 waves

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pk2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint2 pk4(const f32x4 &v) { return make_uint2(pk2(v[0], v[1]), pk2(v[2], v[3])); }
__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ f32x4 unpk4(const uint2 &u) { return f32x4{lo16(u.x), hi16(u.x), lo16(u.y), hi16(u.y)}; }
__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const s16x4 &a, const s16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 as_s4(const uint2 &u) { return __builtin_bit_cast(s16x4, u); }
template <class P>
__device__ __forceinline__ bf16x8 ld8(const P *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ void put2(void *p, const uint2 &v) { *reinterpret_cast<uint2 *>(p) = v; }
template <int CTRL>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// 8 fp32 values -> 8 bf16 (16 bytes)
__device__ __forceinline__ uint4 pk8(const float *f) {
    return make_uint4(pk2(f[0], f[1]), pk2(f[2], f[3]), pk2(f[4], f[5]), pk2(f[6], f[7]));
}

// per stacked row of a sub-chunk: w_r (the values' factor); with the row's
// RMS scale s_x folded in, w_r 2^{b_{tau-1}} s_x, w_r 2^{b_{tau-1} - b_e} s_x
// (residual cross term and Gram row factor), 2^{b_e - b_tau} s_x (separable
// column factor), 2^{b_e' - b_tau} s_x (weight of the row in K); then
// b_{tau-1} - b_e, b_tau - b_e for the pairwise form, and s_x itself
enum { rW = 0, rXf, rRs, rCs, rEw, rBp, rBt, rSx, kNr };
// per token slot of a sub-chunk: 2^{b_t - b_e} s_q, 2^{b_t} s_q, b_t - b_e, s_q
enum { tQs = 0, tGd, tB, tSq, kNt };

// phi's RMS scale 1 / sqrt(mean(z^2) + eps_rms) (0 when that is 0) from the
// sum of squares over 64 elements
__device__ __forceinline__ float rms_scale(float ss, float eps_rms, int phi_kind) {
    if (phi_kind == FALCON_PHI_IDENTITY) return 1.f;
    const float ms = ss * (1.f / D) + eps_rms;
    return ms > 0.f ? __builtin_amdgcn_rsqf(ms) : 0.f;
}
// sum of squares of 8 bf16 values
__device__ __forceinline__ float sumsq8(const uint4 &u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16x2_t h = __builtin_bit_cast(bf16x2_t, w[e]);
        s = __builtin_amdgcn_fdot2_f32_bf16(h, h, s, false);
    }
    return s;
}

// The raw data of one sub-chunk: for stacked row tid / 8 (pair p) 8
// elements (part tid % 8) of k_{p-1} and of v_p; for token slot tid / 8 its
// query piece.  Loaded unconditionally from rows clamped into [0, T); pairs
// at or before position 0 (the incoming x_0 and tail) are replaced when the
// rows are stored.
struct F3Rows {
    uint4 x, y, q;
    __device__ __forceinline__ void load(const F3XferArgs &a, int bh, int c, int s, int W, int CT, int TR,
                                         int row, int part) {
        const int T = a.T;
        const int tau = row / W, k = row % W;
        const int t = c * C + s * CT + tau, p = t - (W - 1) + k;
        const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * D;
        const bf16_t *qg = static_cast<const bf16_t *>(a.q) + size_t(bh) * T * D;
        const bf16_t *vg = static_cast<const bf16_t *>(a.v) + size_t(bh) * T * D;
        const int pk = p < 1 ? 0 : (p - 1 < T ? p - 1 : T - 1);
        const int py = p < 0 ? 0 : (p < T ? p : T - 1);
        x = *reinterpret_cast<const uint4 *>(kg + size_t(pk) * D + 8 * part);
        y = *reinterpret_cast<const uint4 *>(vg + size_t(py) * D + 8 * part);
        const int tq = c * C + s * CT + (row < TR ? row : 0);
        q = *reinterpret_cast<const uint4 *>(qg + size_t(tq < T ? tq : T - 1) * D + 8 * part);
    }
};

template <int W>
__global__ __launch_bounds__(NTH, 4) void f3_xfer(F3XferArgs a) {
    static_assert(W == 2 || W == 4 || W == 8, "windows whose token blocks tile 16 rows");
    constexpr int CT = C / W;                      // tokens of a sub-chunk
    constexpr int NTT = CT >= 16 ? CT / 16 : 1;    // token tiles of a sub-chunk
    constexpr int TR = 16 * NTT;                   // token slots (rows of QB, PB)
    constexpr size_t RB = f1_xfer_bytes(D);
    __shared__ __align__(16) bf16_t XB[C * PK];     // stacked pair features [r][d]
    __shared__ __align__(16) bf16_t YB[C * PK];     // stacked pair values [r][j]
    __shared__ __align__(16) bf16_t XW[D * PK];     // (diag(2^{b_e' - b_tau}) X)^T [d][r]
    __shared__ __align__(16) bf16_t QB[TR * PK];    // queries of the sub-chunk's tokens [t][d]
    __shared__ __align__(16) bf16_t PB[TR * PK];    // scores [t][r]
    __shared__ __align__(16) bf16_t KT[2 * D * PK]; // K^T [j'][d], bf16
    __shared__ __align__(16) bf16_t NB[6][16 * NBP];   // -N below the diagonal blocks
    __shared__ __align__(16) bf16_t DB[4][16 * NBP];   // inverses of the diagonal blocks of I + N
    __shared__ __align__(16) float LF[4 * LFB];         // the diagonal blocks L_J, fp32 row-major
    __shared__ __align__(16) float rs[kNr][C];
    __shared__ __align__(16) float ts[kNt][TR];
    __shared__ float rsx[C], tsq[TR];                   // RMS scales of the staged rows
    __shared__ float cb[C], cw[C];                      // chunk tokens: b_t, w_t
    __shared__ __align__(16) bf16x8 IDT[2][64];         // column pickers

    const int c = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;   // chunk-major: a head's chunks on one XCD
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4), kq = lane >> 4;
    const int row = tid >> 3, part = tid & 7;
    const int T = a.T, H = W - 1;
    char *rec = static_cast<char *>(a.ops) + (size_t(bh) * a.nchunks + c) * RB;

    if (tid < 128) {
        typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
        const int h = tid >> 6;
        u16x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = (k8 + e == 16 * h + col) ? 0x3F80 : 0;   // bf16 1.0
        IDT[h][lane] = __builtin_bit_cast(bf16x8, u);
    }
    // the chunk's step scalars (wave 0, lane = token): b_t (base 2, restarted
    // at 0) and w_t (padding tokens have w = 0 and log2 gamma = 0)
    if (wave == 0) {
        const size_t ft = size_t(bh) * a.Tpad + c * C + lane;
        const float b = wave_inclusive_scan(a.lg[ft]);
        cb[lane] = b;
        cw[lane] = a.w[ft];
        if (lane == 63) *reinterpret_cast<float *>(rec + f1_xfer_scal_off(D)) = ex2(b);
    }

    F3Rows rows;
    rows.load(a, bh, c, 0, W, CT, TR, row, part);
    f32x4 K[4];   // K tiles (rows d = 16 m + g4 .., columns j' = 16 wave + col), fp32
#pragma unroll
    for (int m = 0; m < 4; ++m) K[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    // rows (pitch PK) of a 16 x 32 block, 16 of whose columns (block n of 16)
    // come back transposed into the accumulator layout
    auto transposed = [&](const bf16_t *src, int m, int n) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        return mfma(ld8(src + (16 * m + col) * PK + 32 * (n >> 1) + k8), IDT[n & 1][lane], z);
    };
    // the products below contract over the 64 stacked rows 32 at a time:
    // lane (col, q) of the 16x16x32 MFMA takes rows 32 p + 4 q .. + 3 and
    // 32 p + 16 + 4 q .. + 3, i.e. its two register pieces of Z side by side,
    // and XW and the scores hold their row index in that order (pair_slot)
    auto tok8 = [&](const bf16_t *base, int r, int p) { return ld8(base + r * PK + 32 * p + k8); };

    for (int s = 0; s < W; ++s) {
        // 1. the sub-chunk's rows to LDS (pairs before position 0 from the
        //    incoming tail, pairs that do not exist zero), then the next
        //    sub-chunk's loads
        {
            const int tau = row / W, k = row % W;
            const int t = c * C + s * CT + tau, p = t - H + k;
            uint4 xr = rows.x, yr = rows.y;
            float ss = sumsq8(xr);
            bool feat = false;   // a boundary pair: features already (scale 1)
            if (p <= 0) {
                xr = make_uint4(0, 0, 0, 0);
                if (p < 0) yr = xr;
                ss = 0.f;
                const float *src = nullptr;
                if (p == 0 && a.xnext_in) src = a.xnext_in + size_t(bh) * D + 8 * part;
                if (p < 0 && p >= -a.n_tail_in) {
                    src = a.tailx_in + (size_t(bh) * H + H + p) * D + 8 * part;
                    yr = pk8(a.taily_in + (size_t(bh) * H + H + p) * D + 8 * part);
                }
                if (src) {
                    xr = pk8(src);
                    feat = true;
                }
            } else if (p >= T) {
                yr = make_uint4(0, 0, 0, 0);
            }
            ss = group_sum<8>(ss);
            const float sx = feat ? 1.f : (p >= 1 && p <= T ? rms_scale(ss, a.eps_rms, a.phi) : 0.f);
            *reinterpret_cast<uint4 *>(XB + row * PK + 8 * part) = xr;
            *reinterpret_cast<uint4 *>(YB + row * PK + 8 * part) = yr;
            if (part == 0) rsx[row] = sx;
            if (row < TR) {
                const bool live = row < CT && c * C + s * CT + row < T;
                float sq = group_sum<8>(sumsq8(rows.q));
                *reinterpret_cast<uint4 *>(QB + row * PK + 8 * part) = live ? rows.q : make_uint4(0, 0, 0, 0);
                if (part == 0) tsq[row] = live ? rms_scale(sq, a.eps_rms, a.phi) : 0.f;
            }
            if (s + 1 < W) rows.load(a, bh, c, s + 1, W, CT, TR, row, part);
        }
        __syncthreads();

        // 2. row and token scalars, formed by wave 0 and published by a
        //    barrier
        const float b_e = s > 0 ? cb[s * CT - 1] : 0.f;
        const float b_e2 = cb[s * CT + CT - 1];
        const bool sep = b_e2 >= b_e - 100.f;
        if (wave == 0) {
            const int tc = s * CT + lane / W;
            const float w = cw[tc], bt = cb[tc], bp = tc > 0 ? cb[tc - 1] : 0.f, sx = rsx[lane];
            rs[rW][lane] = w;
            rs[rXf][lane] = w * ex2(bp) * sx;
            rs[rRs][lane] = w * ex2(bp - b_e) * sx;
            rs[rCs][lane] = sep ? ex2(b_e - bt) * sx : 0.f;
            rs[rEw][lane] = ex2(b_e2 - bt) * sx;
            rs[rBp][lane] = bp - b_e;
            rs[rBt][lane] = bt - b_e;
            rs[rSx][lane] = sx;
            if (lane < TR) {
                const bool live = lane < CT;
                const float btk = live ? cb[s * CT + lane] : b_e2, sq = tsq[lane];
                ts[tQs][lane] = live ? ex2(btk - b_e) * sq : 0.f;
                ts[tGd][lane] = live ? ex2(btk) * sq : 0.f;
                ts[tB][lane] = btk - b_e;
                ts[tSq][lane] = sq;
            }
        }
        __syncthreads();

        // 3. Gram blocks, scores, diagonal inverses, transposes of x
        //    Gram N_ij = w_i 2^{b_{tau_i - 1} - b_tau_j} x_i . x_j for tau_j < tau_i
        //    (rows of different 16-row blocks always belong to different
        //    tokens); scores P_tj = 2^{b_t - b_tau_j} qh_t . x_j for tau_j <= t
        auto gram_scale = [&](int i, int j) {   // factor of entry (i, j), the RMS scales included
            return sep ? rs[rRs][i] * rs[rCs][j]
                       : rs[rW][i] * rs[rSx][i] * ex2(rs[rBp][i] - rs[rBt][j]) * rs[rSx][j];
        };
        auto score_scale = [&](int t, int j) {
            return sep ? ts[tQs][t] * rs[rCs][j] : ex2(ts[tB][t] - rs[rBt][j]) * ts[tSq][t] * rs[rSx][j];
        };
        // job 0-5: Gram block (1,0) (2,0) (2,1) (3,0) (3,1) (3,2); job 6 ..:
        // score tile (token tile, row block J); the tile is formed
        // transposed (rows of x as the A operand): lane (col, g4) gets
        // row i = 16 I + col at columns j = 16 J + g4 .. + 3
        auto job = [&](int jb) {
            const bool isG = jb < 6;
            const int tt = isG ? 0 : (jb - 6) >> 2;
            const int I = isG ? (0xFE9 >> (2 * jb)) & 3 : tt;
            const int J = isG ? (0x910 >> (2 * jb)) & 3 : (jb - 6) & 3;
            const bf16_t *ar = (isG ? XB : QB) + (16 * I + col) * PK + k8;
            const bf16_t *br = XB + (16 * J + col) * PK + k8;
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 acc = mfma(ld8(br), ld8(ar), z);
            acc = mfma(ld8(br + 32), ld8(ar + 32), acc);
            const int i = 16 * I + col, j0 = 16 * J + g4;
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = j0 + r;
                if (isG) {
                    v[r] = -acc[r] * gram_scale(i, j);
                } else {
                    const bool live = i < CT && (j / W) <= i;   // token of row j up to slot i
                    v[r] = live ? acc[r] * score_scale(i, j) : 0.f;
                }
            }
            put2(isG ? NB[jb] + col * NBP + g4 : PB + i * PK + pair_slot(j0), pk4(v));
        };
        constexpr int NJ = 6 + 4 * NTT;   // jobs: 6 Gram blocks, the score tiles
        if (wave < 4) {
            const int J = wave;
            {   // L_J row-major in fp32: the block X_J X_J^T is symmetric, so
                // the accumulator tile also holds row col of L_J at columns
                // g4 .. + 3; entries of a later token than the column's
                const bf16_t *xr = XB + (16 * J + col) * PK + k8;
                f32x4 g = {0.f, 0.f, 0.f, 0.f};
                g = mfma(ld8(xr), ld8(xr), g);
                g = mfma(ld8(xr + 32), ld8(xr + 32), g);
                const int i = 16 * J + col, j0 = 16 * J + g4;
                f32x4 l;
#pragma unroll
                for (int r = 0; r < 4; ++r) l[r] = (j0 + r) / W < i / W ? g[r] * gram_scale(i, j0 + r) : 0.f;
                *reinterpret_cast<f32x4 *>(&LF[J * LFB + col * 16 + g4]) = l;
            }
            wave_lds_sync();
            // lane (r = lane / 4, h = lane % 4): elements 4 h .. + 3 of row r of
            // D_J = (I + L_J)^{-1}, from d (I + L_J) = e_r, right-looking over
            // the columns from the last
            const int r = lane >> 2, h = lane & 3;
            const float *lf = LF + J * LFB + 4 * h;
            f32x4 dq;
#pragma unroll
            for (int e = 0; e < 4; ++e) dq[e] = 4 * h + e == r ? 1.f : 0.f;
#pragma unroll
            for (int k = 15; k > 0; --k) {
                const float x = dq[k & 3];
                const int hk = k >> 2;
                const float dk = hk == 0 ? quad_bcast<0x00>(x) : hk == 1 ? quad_bcast<0x55>(x)
                               : hk == 2 ? quad_bcast<0xAA>(x) : quad_bcast<0xFF>(x);
                dq -= dk * *reinterpret_cast<const f32x4 *>(lf + k * 16);
            }
            put2(DB[J] + r * NBP + 4 * h, pk4(dq));
        }
        // waves 0-3 take the score tiles, waves 4-7 the Gram blocks
        if (wave < 4) {
            for (int jb = 6 + wave; jb < NJ; jb += 4) job(jb);
        } else {
            for (int jb = wave - 4; jb < 6; jb += 4) job(jb);
        }
        {   // (diag(2^{b_e' - b_tau}) x)^T, tile (row block m, d block n): two per wave
            const int m = wave >> 1;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int n = 2 * (wave & 1) + u;
                const f32x4 ew = *reinterpret_cast<const f32x4 *>(&rs[rEw][16 * m + g4]);
                put2(XW + (16 * n + col) * PK + pair_slot(16 * m + g4), pk4(transposed(XB, m, n) * ew));
            }
        }
        __syncthreads();

        // 4. Z = (I + N)^{-1} R, column tile n = wave of R = [x part | value
        //    part], R = [-diag(w 2^{b_{tau-1}}) X | diag(w) Y] - diag(w
        //    2^{b_{tau-1} - b_e}) X K, by forward substitution over 16-row
        //    blocks in registers
        const int n = wave;
        const bool xp = n < 4;
        f32x4 r0[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const f32x4 sc = *reinterpret_cast<const f32x4 *>(&rs[xp ? rXf : rW][16 * I + g4]);
            r0[I] = xp ? transposed(XB, I, n) * -sc : transposed(YB, I, n - 4) * sc;
            if (s > 0) {   // cross term: (X K)[r][j'] with K^T rows j' = 16 n + col
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const bf16_t *xr = XB + (16 * I + col) * PK + k8, *kr = KT + (16 * n + col) * PK + k8;
                f32x4 cr = mfma(ld8(xr), ld8(kr), z);
                cr = mfma(ld8(xr + 32), ld8(kr + 32), cr);
                const f32x4 rr = *reinterpret_cast<const f32x4 *>(&rs[rRs][16 * I + g4]);
                r0[I] -= rr * cr;
            }
        }
        // blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2) of -N: the pieces of
        // (I, 0) and (I, 1) side by side meet Z's blocks 0 and 1 in one
        // 32-deep MFMA (pair order), which block 3 issues before Z block 2;
        // block 3's 16-deep term has an accumulator of its own (an
        // accumulator handed from a 16x16x32 MFMA straight to a 16x16x16
        // one is not safe)
        auto nbp = [&](int blk) { return as_s4(*reinterpret_cast<const uint2 *>(NB[blk] + col * NBP + 4 * kq)); };
        s16x4 zb[4];
        bf16x8 zp01;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 acc = r0[I];
            if (I == 1) acc = mfma16(nbp(0), zb[0], acc);
            if (I >= 2) acc = mfma(cat8(nbp(I == 2 ? 1 : 3), nbp(I == 2 ? 2 : 4)), zp01, acc);
            const f32x4 z0 = {0.f, 0.f, 0.f, 0.f};
            if (I == 3) acc += mfma16(nbp(5), zb[2], z0);
            const f32x4 zz = mfma16(as_s4(*reinterpret_cast<const uint2 *>(DB[I] + col * NBP + 4 * kq)),
                                    as_s4(pk4(acc)), z0);
            zb[I] = as_s4(pk4(zz));
            if (I == 1) zp01 = cat8(zb[0], zb[1]);
        }
        const bf16x8 zp[2] = {cat8(zb[0], zb[1]), cat8(zb[2], zb[3])};

        // 5. outputs of the sub-chunk's tokens: tile (rows j' of tile n,
        //    token slots of tile tt) = 2^{b_t - b_e} K^T qh_t + Z^T P^T (+ 2^{b_t}
        //    qh_t for the x part), to the record's G or H tiles
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const int ts_ = 16 * tt + col;   // this lane's token slot
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (s > 0) {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const bf16_t *kr = KT + (16 * n + col) * PK + k8, *qr = QB + ts_ * PK + k8;
                acc = mfma(ld8(kr), ld8(qr), z);
                acc = mfma(ld8(kr + 32), ld8(qr + 32), acc);
                acc *= ts[tQs][ts_];
            }
            if (xp) acc += unpk4(*reinterpret_cast<const uint2 *>(QB + ts_ * PK + 16 * n + g4)) * ts[tGd][ts_];
#pragma unroll
            for (int p = 0; p < 2; ++p) acc = mfma(zp[p], tok8(PB, ts_, p), acc);
            if (ts_ < CT) {
                const int tr = s * CT + ts_;       // token within the chunk
                const int m = tr >> 4, cl = tr & 15;
                if (xp) {
                    const int xo = ((n >> 1) * 64 + 16 * (2 * (n & 1) + (kq >> 1)) + cl) * 16 + 8 * (kq & 1);
                    put2(rec + kF1XferGOff + xo + m * 2048, pk4(acc));
                } else {
                    put2(rec + f1_xfer_h_off(D) + ((n - 4) * 256 + 16 * kq + cl) * 8 + m * 512, pk4(acc));
                }
            }
        }
        // K <- 2^{b_e' - b_e} K + X^T diag(2^{b_e' - b_tau}) Z (tiles of
        // column tile n)
        {
            const float gk = ex2(b_e2 - b_e);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = K[m] * gk;
#pragma unroll
                for (int p = 0; p < 2; ++p) acc = mfma(tok8(XW, 16 * m + col, p), zp[p], acc);
                K[m] = acc;
            }
        }
        __syncthreads();   // every read of this sub-chunk's buffers and of K^T is done
#pragma unroll
        for (int m = 0; m < 4; ++m) put2(KT + (16 * n + col) * PK + 16 * m + g4, pk4(K[m]));
    }

    // B (value tiles, as the accumulators hold them) and A (from K^T: row d,
    // elements d' .. + 7) in the record's operand lane order
    if (wave >= 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) put2(rec + kF1XferBOff + ((wave - 4) * 256 + lane) * 8 + m * 512, pk4(K[m]));
    }
    __syncthreads();
    {
        const int m = tid >> 7, h = (tid >> 6) & 1;
        const int d = 16 * m + col, d1 = 32 * h + 8 * kq;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = reinterpret_cast<const uint16_t *>(KT)[(d1 + 2 * e) * PK + d];
            const uint32_t hi = reinterpret_cast<const uint16_t *>(KT)[(d1 + 2 * e + 1) * PK + d];
            w[e] = lo | (hi << 16);
        }
        *reinterpret_cast<uint4 *>(rec + m * 2048 + h * 1024 + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
    }

    // the boundary state's x_next = phi(k_{T-1}) and last W - 1 pairs
    // (features, values; right-aligned, the valid ones last), from the
    // workgroup holding the last token
    if (c == (T - 1) / C && wave == 0) {
        const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * D;
        const bf16_t *vg = static_cast<const bf16_t *>(a.v) + size_t(bh) * T * D;
        if (a.xnext_out) {
            const float xv = bf16_to_f32(kg[size_t(T - 1) * D + lane].bits);
            const float sc = phi_scale(wave_sum(xv * xv), D, a.eps_rms, a.phi);
            a.xnext_out[size_t(bh) * D + lane] = xv * sc;
        }
        if (a.tailx_out) {
            for (int sl = 0; sl < H; ++sl) {
                const int tau = T - H + sl;
                const bool valid = sl >= H - a.n_tail_out;
                float x = 0.f, y = 0.f;
                if (tau >= 1) {
                    const float kv = bf16_to_f32(kg[size_t(tau - 1) * D + lane].bits);
                    x = kv * phi_scale(wave_sum(kv * kv), D, a.eps_rms, a.phi);
                } else if (tau == 0) {
                    x = a.xnext_in ? a.xnext_in[size_t(bh) * D + lane] : 0.f;
                } else if (valid) {
                    x = a.tailx_in[(size_t(bh) * H + H + tau) * D + lane];
                }
                if (tau >= 0) y = bf16_to_f32(vg[size_t(tau) * D + lane].bits);
                else if (valid) y = a.taily_in[(size_t(bh) * H + H + tau) * D + lane];
                a.tailx_out[(size_t(bh) * H + sl) * D + lane] = valid ? x : 0.f;
                a.taily_out[(size_t(bh) * H + sl) * D + lane] = valid ? y : 0.f;
            }
        }
    }
}

}  // namespace

void launch_chunk_f3_xfer(const F3XferArgs &a, hipStream_t s, Marks *m) {
    const int blocks = a.nchunks * a.BH;
    if (a.window == 2) f3_xfer<2><<<blocks, NTH, 0, s>>>(a);
    else if (a.window == 4) f3_xfer<4><<<blocks, NTH, 0, s>>>(a);
    else f3_xfer<8><<<blocks, NTH, 0, s>>>(a);
    m->mark(s);
}

}  // namespace falcon
