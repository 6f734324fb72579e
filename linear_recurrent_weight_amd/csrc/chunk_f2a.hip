// Chunk-parallel Falcon-2A: the inner-product write with one gain, step and
// decay per value column (summary "B. Falcon-2A: per-channel inner-product
// write", §4.3, §4.5; Figures 6-8: per-column decay-weighted masks; §D.1:
// chunk-local log-prefix restarted in every chunk).
//
// Per value column j the recurrence S[:, j] <- gamma_{t,j} S[:, j] +
// eta_{t,j} x_t y_{t,j} is linear with scalar decay, so inside a chunk, with
// Gamma_{t,j} = prod_{s<=t} gamma_{s,j} (restarted at 1),
//     O_{t,j}  = Gamma_{t,j} ( (Qh S_0)_{t,j} + sum_{s<=t} (qh_t . x_s) yt_{s,j} ),
//     S_C[:,j] = Gamma_{C,j} ( S_0[:,j] + X^T yt[:,j] ),
//     yt_{s,j} = eta_{s,j} y_{s,j} / Gamma_{s,j},
// i.e. one shared decay-free score matrix L = lower(Qh X^T) and two products
// (L yt, X^T yt) for all columns, with the per-column decays applied
// elementwise.  The rewrite needs 1/Gamma in range: a chunk in which some
// column decays below 2^-64 is run token by token instead (exact, slower).
//
// One workgroup (4 waves) per (batch*head, slice of up to 64 value columns)
// walks its chunks in order; the fp32 state slice stays in LDS.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;
constexpr int NT = 256;
constexpr float kMinLog2Decay = -64.f;

template <class E, int DK, int DS>
struct F2aShared {
    static constexpr int PE = Pad<E>::v;
    E Qh[C][DK + PE];       // phi(q_t) rows
    E Xr[C][DK + PE];       // x_t rows (x_t = phi(k_{t-1}))
    E XT[DK][C + PE];       // x^T
    E YT[DS][C + PE];       // yt^T [j][s]
    E Lb[C][C + PE];        // lower(Qh X^T)
    E ST[DS][DK + PE];      // bf16/fp32 copy of S^T [j][d]
    float Sf[DK][DS];       // the state slice, fp32
    float Yf[C][DS];        // raw values of the chunk
    float Bf[C][DS];        // beta, then the log-prefix b (base 2)
    float n2[C], lam[C], ok[C];
    int fast;
};

template <class E, int DK, int DS>
__global__ __launch_bounds__(NT) void chunk_f2a_kernel(ChunkF2Args a, int nslice) {
    using Sh = F2aShared<E, DK, DS>;
    __shared__ __align__(16) Sh sh;
    const int bh = blockIdx.x / nslice, j0 = (blockIdx.x % nslice) * DS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T, DV = a.dv;
    const E *qg = static_cast<const E *>(a.q) + size_t(bh) * T * DK;
    const E *kg = static_cast<const E *>(a.k) + size_t(bh) * T * DK;
    const E *vg = static_cast<const E *>(a.v) + size_t(bh) * T * DV;
    E *og = static_cast<E *>(a.o) + size_t(bh) * T * DV;

    for (int i = tid; i < DK * DS; i += NT) {
        const int d = i / DS, j = i % DS;
        const float s0 = a.S_in ? a.S_in[(size_t(bh) * DK + d) * DV + j0 + j] : 0.f;
        sh.Sf[d][j] = s0;
        st(&sh.ST[j][0], d, s0);
    }

    // rows: thread (row = tid / 4, part = tid % 4) holds DK / 4 features and
    // DS / 4 values of one token
    const int row = tid >> 2, part = tid & 3;
    constexpr int EK = DK / 4, EV = DS / 4;
    for (int c = 0; c < a.nchunks; ++c) {
        __syncthreads();   // the previous chunk's readers are done
        {
            const int t = c * C + row;
            const bool qok = t < T;
            const int tq = qok ? t : T - 1;
            float q[EK], x[EK];
            float sq = 0.f, sx = 0.f;
#pragma unroll
            for (int e = 0; e < EK; ++e) {
                const int d = part * EK + e;
                q[e] = ld(qg, size_t(tq) * DK + d);
                if (t == 0) x[e] = a.xnext_in ? a.xnext_in[size_t(bh) * DK + d] : 0.f;
                else x[e] = ld(kg, size_t(t - 1 < T ? t - 1 : T - 1) * DK + d);
                sq += q[e] * q[e];
                sx += x[e] * x[e];
            }
            sq += dpp<kDppQuadXor1>(sq);
            sq += dpp<kDppQuadXor2>(sq);
            sx += dpp<kDppQuadXor1>(sx);
            sx += dpp<kDppQuadXor2>(sx);
            const float scq = qok ? phi_scale(sq, DK, a.eps_rms, a.phi) : 0.f;
            // x_0 of a continued sequence is already a feature; 0 when fresh
            const float scx = (t == 0) ? 1.f : (t <= T ? phi_scale(sx, DK, a.eps_rms, a.phi) : 0.f);
            float n2 = 0.f;
#pragma unroll
            for (int e = 0; e < EK; ++e) {
                const int d = part * EK + e;
                const float xs = x[e] * scx;
                n2 += xs * xs;
                st(&sh.Qh[row][0], d, q[e] * scq);
                st(&sh.Xr[row][0], d, xs);
                st(&sh.XT[d][0], row, xs);
            }
            n2 += dpp<kDppQuadXor1>(n2);
            n2 += dpp<kDppQuadXor2>(n2);
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const int j = part * EV + e;
                sh.Yf[row][j] = qok ? ld(vg, size_t(tq) * DV + j0 + j) : 0.f;
                sh.Bf[row][j] = a.beta[(size_t(bh) * T + tq) * DV + j0 + j];
            }
            if (part == 0) {
                sh.n2[row] = n2;
                sh.lam[row] = a.lambda[size_t(bh) * T + tq];
                sh.ok[row] = (qok && !(t == 0 && a.fresh)) ? 1.f : 0.f;   // the fresh first step writes nothing
            }
        }
        __syncthreads();

        // per-column steps and log-prefix (thread j walks the chunk's tokens)
        if (tid < DS) {
            const int j = tid;
            float b = 0.f;
            for (int t = 0; t < C; ++t) {
                const float den = sh.n2[t] + sh.lam[t] + a.eps;
                const float eta = sh.ok[t] != 0.f ? step_eta(sh.Bf[t][j], den) : 0.f;
                b += log2_1m(step_alpha(eta, sh.lam[t], a.eps_gamma));
                sh.Bf[t][j] = b;
                st(&sh.YT[j][0], t, eta * sh.Yf[t][j] * exp2f(-b));
            }
            const bool in_range = __ballot(j < DS && b >= kMinLog2Decay) == __ballot(j < DS);
            if (tid == 0) sh.fast = in_range ? 1 : 0;
        }
        __syncthreads();

        if (sh.fast) {
            // L = lower(Qh X^T), 16 x 16 tiles
            for (int tile = wave; tile < 16; tile += 4) {
                const int m = tile >> 2, n = tile & 3;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (n <= m) acc = Mma<E>::run(acc, &sh.Qh[16 * m][0], DK + Sh::PE, &sh.Xr[16 * n][0], DK + Sh::PE, 0, DK);
                const int colj = 16 * n + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ti = 16 * m + 4 * (lane >> 4) + r;
                    st(&sh.Lb[ti][0], colj, colj <= ti ? acc[r] : 0.f);
                }
            }
            __syncthreads();
            // outputs: O = Gamma (Qh S_0 + L yt)
            for (int tile = wave; tile < 4 * (DS / 16); tile += 4) {
                const int m = tile / (DS / 16), n = tile % (DS / 16);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = Mma<E>::run(acc, &sh.Qh[16 * m][0], DK + Sh::PE, &sh.ST[16 * n][0], DK + Sh::PE, 0, DK);
                acc = Mma<E>::run(acc, &sh.Lb[16 * m][0], C + Sh::PE, &sh.YT[16 * n][0], C + Sh::PE, 0, 16 * (m + 1));
                const int jj = 16 * n + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ti = 16 * m + 4 * (lane >> 4) + r, t = c * C + ti;
                    if (t < T) st(og, size_t(t) * DV + j0 + jj, acc[r] * exp2f(sh.Bf[ti][jj]));
                }
            }
            __syncthreads();
            // state: S_C = Gamma_C (S_0 + X^T yt)
            for (int tile = wave; tile < (DK / 16) * (DS / 16); tile += 4) {
                const int m = tile / (DS / 16), n = tile % (DS / 16);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = Mma<E>::run(acc, &sh.XT[16 * m][0], C + Sh::PE, &sh.YT[16 * n][0], C + Sh::PE, 0, C);
                const int jj = 16 * n + (lane & 15);
                const float gC = exp2f(sh.Bf[C - 1][jj]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 16 * m + 4 * (lane >> 4) + r;
                    const float s = gC * (sh.Sf[d][jj] + acc[r]);
                    sh.Sf[d][jj] = s;
                    st(&sh.ST[jj][0], d, s);
                }
            }
        } else {
            // token by token (a column decays below 2^-64 in this chunk):
            // thread (j = tid / 4, part) holds rows part * DK/4 .. of column
            // j; the gains are read again (their buffer holds the prefix now)
            const int j = tid >> 2;
            if (j < DS) {
                float s[EK];
#pragma unroll
                for (int e = 0; e < EK; ++e) s[e] = sh.Sf[part * EK + e][j];
                for (int t = 0; t < C; ++t) {
                    const int tg = c * C + t;
                    const int tq = tg < T ? tg : T - 1;
                    float eta = 0.f, gam = 1.f;
                    if (sh.ok[t] != 0.f) {
                        eta = step_eta(a.beta[(size_t(bh) * T + tq) * DV + j0 + j], sh.n2[t] + sh.lam[t] + a.eps);
                        gam = 1.f - step_alpha(eta, sh.lam[t], a.eps_gamma);
                    }
                    const float w = eta * sh.Yf[t][j];
                    float o = 0.f;
#pragma unroll
                    for (int e = 0; e < EK; ++e) {
                        const int d = part * EK + e;
                        s[e] = gam * s[e] + w * ld(&sh.Xr[t][0], d);
                        o += ld(&sh.Qh[t][0], d) * s[e];
                    }
                    o += dpp<kDppQuadXor1>(o);
                    o += dpp<kDppQuadXor2>(o);
                    if (part == 0 && tg < T) st(og, size_t(tg) * DV + j0 + j, o);
                }
#pragma unroll
                for (int e = 0; e < EK; ++e) {
                    const int d = part * EK + e;
                    sh.Sf[d][j] = s[e];
                    st(&sh.ST[j][0], d, s[e]);
                }
            }
        }
    }
    __syncthreads();
    if (a.S_out)
        for (int i = tid; i < DK * DS; i += NT) {
            const int d = i / DS, j = i % DS;
            a.S_out[(size_t(bh) * DK + d) * DV + j0 + j] = sh.Sf[d][j];
        }
    if (blockIdx.x % nslice == 0 && wave == 0 && a.xnext_out) {   // phi(k_{T-1})
        const float xv = lane < DK ? ld(kg, size_t(T - 1) * DK + lane) : 0.f;
        const float sc = phi_scale(wave_sum(xv * xv), DK, a.eps_rms, a.phi);
        if (lane < DK) a.xnext_out[size_t(bh) * DK + lane] = xv * sc;
    }
}

template <class E, int DK>
void launch_f2a_dk(const ChunkF2Args &a, hipStream_t s) {
    const int ds = a.dv < 64 ? a.dv : 64, nslice = a.dv / ds;
    const dim3 grid(a.BH * nslice);
    if (ds == 16) chunk_f2a_kernel<E, DK, 16><<<grid, NT, 0, s>>>(a, nslice);
    else if (ds == 32) chunk_f2a_kernel<E, DK, 32><<<grid, NT, 0, s>>>(a, nslice);
    else chunk_f2a_kernel<E, DK, 64><<<grid, NT, 0, s>>>(a, nslice);
}

}  // namespace

void launch_chunk_f2a(const ChunkF2Args &a, bool bf16, hipStream_t s, Marks *m) {
    if (bf16) {
        if (a.dk == 32) launch_f2a_dk<bf16_t, 32>(a, s);
        else launch_f2a_dk<bf16_t, 64>(a, s);
    } else {
        if (a.dk == 32) launch_f2a_dk<float, 32>(a, s);
        else launch_f2a_dk<float, 64>(a, s);
    }
    m->mark(s);
}

}  // namespace falcon
