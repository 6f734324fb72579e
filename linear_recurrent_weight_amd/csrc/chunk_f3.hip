// Chunk-parallel Falcon-3 forward (window of W pairs, regression writes):
// summary §4.4 "Mini-batch Update Rule for Regression (Falcon-3)", §C.7, and
// §H.3 "Mapping Falcon-3 to ParallelFlow" (the window rows stacked into one
// block-strict-causal system; rows of the same step do not interact).
//
// Token t writes the W pairs of its window I_t, each with the residual at the
// pre-update state and the weight w_t = eta_t / B_t:
//     u_{t,j} = w_t (y_j - S_{t-1}^T x_j),   S_t = gamma_t S_{t-1} + sum_j x_j u_{t,j}^T.
// A chunk holds Ct = 64 / W tokens, so its stacked rows r = (t, k) number at
// most 64; row r carries the pair j = t - W + 1 + k.  With the chunk-local
// log-prefix b over tokens (restarted at 0) and S_0 the chunk-entry state:
//     u_r + w_r sum_{r': t' < t} e^{b_{t-1} - b_{t'}} (x_r . x_r') u_r'
//         = w_r (y_r - e^{b_{t-1}} S_0^T x_r)
// (unit lower triangular in r; rows of one token are decoupled), and
//     o_t = e^{b_t} S_0^T qh_t + sum_{r': t' <= t} e^{b_t - b_t'} (qh_t . x_r') u_r',
//     S_C = e^{b_C} S_0 + sum_r e^{b_C - b_t} x_r u_r^T.
// Rows whose pair lies before the sequence start (and is not in the incoming
// tail) have w = 0 and x = 0: they are inert.  The first chunk reads pairs
// before position 0 from the incoming tail.
//
// Kernel f3_prep, one workgroup per chunk, all chunks in parallel: gathers the
// stacked rows, forms the Gram and the token-by-row scores on MFMA, inverts
// the unit-lower system in fp32, and stores Tp = L^{-1} diag(w), the scores
// and the stacked features.
// Kernel f3_scan, one workgroup per (head, 16 value columns): walks the
// chunks in order with the fp32 state slice in MFMA accumulators.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"
#include "tri_inverse.h"

namespace falcon {
namespace {

constexpr int C = kChunk;
constexpr int kLs = C + 1;   // fp32 LDS row stride

struct RowMap {
    int ct, W, halo;
    // local token of stacked row r (rows past ct * W belong to no token)
    __device__ int token(int r) const { return r < ct * W ? r / W : -1; }
    // global pair index of row r of chunk c (may be negative: incoming tail)
    __device__ int pair(int c, int r) const { return c * ct + r / W - halo + r % W; }
};

template <class E, int DK>
__global__ __launch_bounds__(256) void f3_prep(ChunkF3Args a) {
    constexpr int PD = Pad<E>::v;
    constexpr int LK = DK + PD;
    __shared__ __align__(16) E Xs[C * LK];   // stacked write features
    __shared__ __align__(16) E Qs[C * LK];   // token queries (Ct rows used)
    __shared__ float Lm[C * kLs];
    __shared__ float Tm[C * kLs];
    __shared__ float Pm[C * kLs];
    __shared__ float Mt[3 * 16 * 17];
    __shared__ float bt[C], bpt[C];          // per token: b_t, b_{t-1}
    __shared__ float wr[C];                  // per row: eta_t / B_t (0 when inert)
    __shared__ int tr[C];                    // per row: local token, -1 for padding

    const int c = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const RowMap rm{a.ct, a.window, a.window - 1};
    const int T = a.T, ct = a.ct, W = a.window, halo = a.window - 1;
    const size_t frow0 = size_t(bh) * a.Tpad;
    const E *xn = static_cast<const E *>(a.xn) + frow0 * DK;
    const E *qn = static_cast<const E *>(a.qn) + frow0 * DK;
    char *ops = static_cast<char *>(a.ops) + (size_t(bh) * a.nchunks + c) * a.chunk_bytes;
    E *Tp = reinterpret_cast<E *>(ops + chunk_f1_tp_off());
    E *Pg = reinterpret_cast<E *>(ops + chunk_f1_p_off(sizeof(E)));
    E *Xg = reinterpret_cast<E *>(ops + chunk_f3_x_off(sizeof(E)));
    float *scal = reinterpret_cast<float *>(ops + chunk_f3_scal_off(DK, sizeof(E)));

    // 1. per-token log-prefix (wave 0, lane = local token) and per-row weights
    if (wave == 0) {
        const int t = c * ct + lane;   // < Tpad: the feature buffers have a spare tile
        const float alpha = lane < ct ? a.alpha[frow0 + t] : 0.f;
        const float b = wave_inclusive_scan(log1pf(-alpha));
        float bp = __shfl_up(b, 1, 64);
        if (lane == 0) bp = 0.f;
        bt[lane] = b;
        bpt[lane] = bp;
        const float bC = __shfl(b, ct - 1, 64);
        scal[2 * C + lane] = expf(b);
        if (lane == 0) scal[3 * C] = expf(bC);
    } else if (wave == 1) {
        const int r = lane, tl = rm.token(r);
        float w = 0.f;
        if (tl >= 0) {
            const int t = c * ct + tl, p = rm.pair(c, r);
            if (t < T && p >= -a.n_tail_in) {
                const long long pairs = (long long)a.n_tail_in + t + 1;
                const int nb = pairs < W ? int(pairs) : W;
                w = a.eta[frow0 + t] / float(nb);
            }
        }
        wr[r] = w;
        tr[r] = tl;
    }
    // stacked features and token queries, 16 bytes of a row per thread and
    // pass; all passes' loads (only of rows that exist) are issued before the
    // first store
    {
        constexpr int VEC = 16 / int(sizeof(E)), NXV = C * DK / VEC / 256;
        const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
        uint4 xv[NXV], qv[NXV];
#pragma unroll
        for (int u = 0; u < NXV; ++u) {
            const int idx = (tid + 256 * u) * VEC, r = idx / DK, e = idx % DK;
            const int p = rm.pair(c, r);
            xv[u] = z4;
            qv[u] = z4;
            if (rm.token(r) >= 0 && p >= 0) xv[u] = *reinterpret_cast<const uint4 *>(xn + size_t(p) * DK + e);
            if (r < ct) qv[u] = *reinterpret_cast<const uint4 *>(qn + size_t(c * ct + r) * DK + e);
        }
#pragma unroll
        for (int u = 0; u < NXV; ++u) {
            const int idx = (tid + 256 * u) * VEC, r = idx / DK, e = idx % DK;
            const int tl = rm.token(r), p = rm.pair(c, r);
            uint4 x = xv[u];
            if (tl >= 0 && p < 0 && p >= -a.n_tail_in) {   // an incoming tail pair (fp32)
                const float *src = a.tailx_in + (size_t(bh) * halo + halo + p) * DK + e;
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if constexpr (sizeof(E) == 2)
                        w[k] = uint32_t(f32_to_bf16(src[2 * k])) | (uint32_t(f32_to_bf16(src[2 * k + 1])) << 16);
                    else
                        w[k] = __float_as_uint(src[k]);
                }
                x = make_uint4(w[0], w[1], w[2], w[3]);
            }
            *reinterpret_cast<uint4 *>(Xs + size_t(r) * LK + e) = x;
            *reinterpret_cast<uint4 *>(Xg + idx) = x;
            *reinterpret_cast<uint4 *>(Qs + size_t(r) * LK + e) = qv[u];
        }
    }
    __syncthreads();
    {
        const int r = tid & 63, tl = tr[r];
        if (tid < 64) {
            scal[0 * C + r] = tl >= 0 ? expf(bpt[tl]) : 0.f;
            scal[1 * C + r] = tl >= 0 ? expf(bt[ct - 1] - bt[tl]) : 0.f;
        }
    }

    // 2. Gram (lower 16x16 tiles) and token-by-row scores (all tiles of the
    //    token rows) on MFMA, with the decays and the causal masks
    const int nqt = (ct + 15) / 16;
    const int njobs = 10 + 4 * nqt;
    for (int job = wave; job < njobs; job += 4) {
        const bool isG = job < 10;
        int I, J;
        if (isG) {
            int t = job;
            I = 0;
            while (t > I) {
                t -= I + 1;
                ++I;
            }
            J = t;
        } else {
            I = (job - 10) / 4;
            J = (job - 10) % 4;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = Mma<E>::run(acc, (isG ? Xs : Qs) + 16 * I * LK, LK, Xs + 16 * J * LK, LK, 0, DK);
        const int j = 16 * J + (lane & 15), tj = tr[j];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int i = 16 * I + 4 * (lane >> 4) + rr;
            if (isG) {
                const int ti = tr[i];
                const bool live = ti >= 0 && tj >= 0 && tj < ti;
                Lm[i * kLs + j] = live ? wr[i] * expf(bpt[ti] - bt[tj]) * acc[rr] : 0.f;
            } else {
                const bool live = i < ct && tj >= 0 && tj <= i;
                Pm[i * kLs + j] = live ? expf(bt[i] - bt[tj]) * acc[rr] : 0.f;
            }
        }
    }
    for (int idx = tid; idx < C * C; idx += 256) {
        const int i = idx / C, j = idx % C;
        if ((j >> 4) > (i >> 4)) {
            Lm[i * kLs + j] = 0.f;
            Tm[i * kLs + j] = 0.f;
        }
        if ((i >> 4) >= nqt) Pm[i * kLs + j] = 0.f;
    }
    __syncthreads();

    // 3. inverse of the unit-lower system
    unit_lower_inverse64(Lm, Tm, Mt, kLs);

    // 4. Tp = L^{-1} diag(w) and the scores, in the storage type, 16 bytes
    //    per thread and store
    {
        constexpr int VEC = 16 / int(sizeof(E));
#pragma unroll
        for (int u = 0; u < C * C / VEC / 256; ++u) {
            const int idx = (tid + 256 * u) * VEC, i = idx / C, j0 = idx % C;
            float tv[VEC], pv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int j = j0 + e;
                tv[e] = j <= i ? Tm[i * kLs + j] * wr[j] : 0.f;
                pv[e] = Pm[i * kLs + j];
            }
            uint32_t wt[4], wp[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (sizeof(E) == 2) {
                    wt[k] = uint32_t(f32_to_bf16(tv[2 * k])) | (uint32_t(f32_to_bf16(tv[2 * k + 1])) << 16);
                    wp[k] = uint32_t(f32_to_bf16(pv[2 * k])) | (uint32_t(f32_to_bf16(pv[2 * k + 1])) << 16);
                } else {
                    wt[k] = __float_as_uint(tv[k]);
                    wp[k] = __float_as_uint(pv[k]);
                }
            }
            *reinterpret_cast<uint4 *>(Tp + idx) = make_uint4(wt[0], wt[1], wt[2], wt[3]);
            *reinterpret_cast<uint4 *>(Pg + idx) = make_uint4(wp[0], wp[1], wp[2], wp[3]);
        }
    }
}

template <class E, int DK>
__global__ __launch_bounds__(256) void f3_scan(ChunkF3Args a, int nslice) {
    constexpr int PD = Pad<E>::v;
    constexpr int LS = DK + PD;   // stride of [j][d] buffers
    constexpr int LT = C + PD;    // stride of [.][row] buffers
    constexpr int NT = DK >= 64 ? DK / 64 : 1;
    __shared__ __align__(16) E St[2][16 * LS];  // S^T slice copy
    __shared__ __align__(16) E R0t[16 * LT];    // residual^T
    __shared__ __align__(16) E Ut[16 * LT];     // U^T
    __shared__ __align__(16) E Xht[DK * LT];    // (diag(e^{b_C - b_t}) X)^T

    const int id = blockIdx.x;
    const int u8 = id & 7, rest = id >> 3;
    const int s = rest % nslice, g = rest / nslice;
    const int bh = g * 8 + u8;
    if (bh >= a.BH) return;
    const int j0 = 16 * s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dv = a.dv, T = a.T, ct = a.ct, halo = a.window - 1;
    const RowMap rm{a.ct, a.window, a.window - 1};
    const E *Qall = static_cast<const E *>(a.qn) + size_t(bh) * a.Tpad * DK;
    const E *V = static_cast<const E *>(a.v) + size_t(bh) * T * dv;
    E *O = static_cast<E *>(a.o) + size_t(bh) * T * dv;
    const char *opsb = static_cast<const char *>(a.ops) + size_t(bh) * a.nchunks * a.chunk_bytes;

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
        if (owns) st4(St[0] + (lane & 15) * LS + dbase + 4 * (lane >> 4), S[m]);
    }
    int cur = 0;
    __syncthreads();

    // Each chunk's operands from memory (rows of X, Tp, Qh and Pg as MFMA
    // fragments, the transposed-copy pieces of X, the scalars and the values
    // y) are loaded for the next chunk right after their last use in this
    // one, so their latency overlaps the rest of the chunk.
    using F = MmaFrag<E>;
    using FT = typename F::T;
    constexpr int NKD = DK / F::KS, NKC = C / F::KS;
    constexpr int VEC = 16 / int(sizeof(E)), NXV = C * DK / VEC / 256;
    const int kend2 = (16 * wave + 16 + F::KS - 1) / F::KS;   // k steps of Tp's lower rows
    const bool outw = 16 * wave < ct;                          // wave with output rows
    auto chunk_ops = [&](int cc) { return opsb + size_t(cc) * a.chunk_bytes; };
    auto Xof = [&](int cc) { return reinterpret_cast<const E *>(chunk_ops(cc) + chunk_f3_x_off(sizeof(E))); };
    auto Sof = [&](int cc) { return reinterpret_cast<const float *>(chunk_ops(cc) + chunk_f3_scal_off(DK, sizeof(E))); };

    FT xa[NKD], ta[NKC], qb[NKD], pb[NKC];
    uint4 xr[NXV];
    float s1[4], y1[4], s2[NXV], s3 = 0.f, s4;
    auto load1 = [&](int cc) {   // phase 1: X rows 16 w .., scal[i], y_i
        const E *X = Xof(cc);
        const float *scal = Sof(cc);
#pragma unroll
        for (int k = 0; k < NKD; ++k) xa[k] = F::load(X + size_t(16 * wave) * DK, DK, k * F::KS);
        const int j = lane & 15;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * wave + 4 * (lane >> 4) + r;
            const int p = rm.pair(cc, i);
            float y = 0.f;
            if (rm.token(i) >= 0) {
                if (p >= 0) {
                    if (p < T) y = ld(V, size_t(p) * dv + j0 + j);
                } else if (p >= -a.n_tail_in) {
                    y = a.taily_in[(size_t(bh) * halo + halo + p) * dv + j0 + j];
                }
            }
            y1[r] = y;
            s1[r] = scal[i];
        }
    };
    auto load2 = [&](int cc) {   // phase 2: Tp rows 16 w .., X pieces and their scales
        const E *Tp = reinterpret_cast<const E *>(chunk_ops(cc) + chunk_f1_tp_off());
        const E *X = Xof(cc);
        const float *scal = Sof(cc);
#pragma unroll
        for (int k = 0; k < NKC; ++k)
            if (k < kend2) ta[k] = F::load(Tp + size_t(16 * wave) * C, C, k * F::KS);
#pragma unroll
        for (int u = 0; u < NXV; ++u) {
            const int idx = (tid + 256 * u) * VEC;
            xr[u] = *reinterpret_cast<const uint4 *>(X + idx);
            s2[u] = scal[C + idx / DK];
        }
    };
    auto load3 = [&](int cc) {   // phase 3: Qh and Pg rows 16 w .., the scalars
        const float *scal = Sof(cc);
        if (outw) {
            const E *Pg = reinterpret_cast<const E *>(chunk_ops(cc) + chunk_f1_p_off(sizeof(E)));
            const E *Qh = Qall + size_t(cc) * ct * DK;   // 64 rows stay inside the padded buffer
#pragma unroll
            for (int k = 0; k < NKD; ++k) qb[k] = F::load(Qh + size_t(16 * wave) * DK, DK, k * F::KS);
#pragma unroll
            for (int k = 0; k < NKC; ++k) pb[k] = F::load(Pg + size_t(16 * wave) * C, C, k * F::KS);
            s3 = scal[2 * C + 16 * wave + (lane & 15)];
        }
        s4 = scal[3 * C];
    };
    load1(0);
    load2(0);
    load3(0);

    for (int c = 0; c < a.nchunks; ++c) {
        const int cn = c + 1 < a.nchunks ? c + 1 : c;   // the next chunk (the last reloads itself)

        // phase 1: R0 = Y - diag(Gamma_{t-1}) X S_0 for stacked rows 16w..16w+15
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NKD; ++k) acc = F::mma(xa[k], F::load(St[cur], LS, k * F::KS), acc);
            const int j = lane & 15;
            f32x4 r0;
#pragma unroll
            for (int r = 0; r < 4; ++r) r0[r] = y1[r] - s1[r] * acc[r];
            st4(R0t + j * LT + 16 * wave + 4 * (lane >> 4), r0);
        }
        load1(cn);
        __syncthreads();

        // phase 2: U = Tp R0; (diag(e^{b_C - b_t}) X)^T
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NKC; ++k)
                if (k < kend2) acc = F::mma(ta[k], F::load(R0t, LT, k * F::KS), acc);
            st4(Ut + (lane & 15) * LT + 16 * wave + 4 * (lane >> 4), acc);
#pragma unroll
            for (int u = 0; u < NXV; ++u) {
                const int idx = (tid + 256 * u) * VEC, i = idx / DK, d = idx % DK;
                const uint32_t w[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float f;
                    if constexpr (sizeof(E) == 2) f = __uint_as_float(e & 1 ? w[e >> 1] & 0xffff0000u : w[e >> 1] << 16);
                    else f = __uint_as_float(w[e]);
                    st(Xht, size_t(d + e) * LT + i, s2[u] * f);
                }
            }
        }
        load2(cn);
        __syncthreads();

        // phase 3a: outputs of the chunk's tokens (rows 16w..16w+15 < Ct)
        if (outw) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NKD; ++k) acc = F::mma(F::load(St[cur], LS, k * F::KS), qb[k], acc);
            const int i = 16 * wave + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= s3;
#pragma unroll
            for (int k = 0; k < NKC; ++k) acc = F::mma(F::load(Ut, LT, k * F::KS), pb[k], acc);
            const int t = c * ct + i;
            if (i < ct && t < T) st4(O + size_t(t) * dv + j0 + 4 * (lane >> 4), acc);
        }
        // phase 3b: S = Gamma_C S + (diag(e^{b_C - b_t}) X)^T U
        {
            const float gC = s4;
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
        load3(cn);
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
void launch_t(const ChunkF3Args &a, hipStream_t s, Marks *m) {
    f3_prep<E, DK><<<dim3(a.nchunks, a.BH), 256, 0, s>>>(a);
    m->mark(s);
    const int nslice = a.dv / 16;
    const int blocks = ((a.BH + 7) / 8) * 8 * nslice;
    f3_scan<E, DK><<<blocks, 256, 0, s>>>(a, nslice);
    m->mark(s);
}

}  // namespace

void launch_chunk_f3(const ChunkF3Args &a, bool bf16, hipStream_t s, Marks *m) {
    if (bf16) {
        if (a.dk == 32) launch_t<bf16_t, 32>(a, s, m);
        else if (a.dk == 64) launch_t<bf16_t, 64>(a, s, m);
        else launch_t<bf16_t, 128>(a, s, m);
    } else {
        if (a.dk == 32) launch_t<float, 32>(a, s, m);
        else if (a.dk == 64) launch_t<float, 64>(a, s, m);
        else launch_t<float, 128>(a, s, m);
    }
}

}  // namespace falcon
