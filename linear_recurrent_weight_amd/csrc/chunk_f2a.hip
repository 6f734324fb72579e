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
// One workgroup (8 waves) per (batch*head, slice of up to 32 value columns)
// walks its chunks in order; the fp32 state slice stays in LDS, and the next
// chunk's rows load into registers (first four waves) while a chunk is
// processed; all eight share the per-column scans, score, output and state
// tiles.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;
constexpr int NT = 512;   // 8 waves: the row phase takes the first 4 (NR threads)
constexpr int NR = 256;
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
    float Yf[C][DS + 1];    // raw values of the chunk (odd pitch: a token per lane reads distinct banks)
    float Bf[C][DS + 1];    // beta, then the log-prefix b (base 2)
    float n2[C], lam[C], ok[C];
    int fastw[NT / 64];
};

// 8-byte pieces <-> floats for the io type
template <class E> struct Io8;
template <> struct Io8<bf16_t> {
    static constexpr int n = 4;   // elements per 8 bytes
    __device__ static void unpack(const uint2 &u, float *f) {
        f[0] = __uint_as_float(u.x << 16);
        f[1] = __uint_as_float(u.x & 0xffff0000u);
        f[2] = __uint_as_float(u.y << 16);
        f[3] = __uint_as_float(u.y & 0xffff0000u);
    }
};
template <> struct Io8<float> {
    static constexpr int n = 2;
    __device__ static void unpack(const uint2 &u, float *f) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
    }
};

// n consecutive row elements (n a multiple of 4) from floats, as 8-byte
// (bf16) or 16-byte (fp32) stores
template <class E, int n>
__device__ __forceinline__ void put_row(E *dst, const float *v) {
#pragma unroll
    for (int i = 0; i < n; i += 4) {
        if constexpr (sizeof(E) == 2) {
            const uint32_t lo = uint32_t(f32_to_bf16(v[i])) | (uint32_t(f32_to_bf16(v[i + 1])) << 16);
            const uint32_t hi = uint32_t(f32_to_bf16(v[i + 2])) | (uint32_t(f32_to_bf16(v[i + 3])) << 16);
            *reinterpret_cast<uint2 *>(dst + i) = make_uint2(lo, hi);
        } else {
            *reinterpret_cast<float4 *>(dst + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
        }
    }
}

template <class E, int DK, int DS>
__global__ __launch_bounds__(NT, 4) void chunk_f2a_kernel(ChunkF2Args a, int nslice) {
    using Sh = F2aShared<E, DK, DS>;
    __shared__ __align__(16) Sh sh;
    // workgroup -> (head, slice): the slices of a head share an XCD (block
    // ids 8 apart), so they read the head's rows through one L2
    const int id = blockIdx.x, u8 = id & 7, rest = id >> 3;
    const int sl = rest % nslice, bh = (rest / nslice) * 8 + u8;
    if (bh >= a.BH) return;   // the whole workgroup leaves together
    const int j0 = sl * DS;
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

    // rows: thread (row = tid / 4, part = tid % 4) of the first NR holds
    // DK / 4 features and DS / 4 values and gains of one token, loaded as
    // 8-byte pieces one chunk ahead (unconditional loads from rows clamped
    // into [0, T)); the other waves take part in the later phases only
    const bool rower = tid < NR;
    const int row = (tid & (NR - 1)) >> 2, part = tid & 3;
    constexpr int EK = DK / 4, EV = DS / 4;
    constexpr int NQ = EK / Io8<E>::n, NVv = EV / Io8<E>::n;
    static_assert(NQ >= 1 && NVv >= 1 && EV % 4 == 0, "whole 8-byte pieces per thread");
    uint2 rq[NQ], rk[NQ], rv[NVv];
    float4 rb[EV / 4];
    float rlam;
    auto prefetch = [&](int c) {
        const int t = c * C + row;
        const int tq = t < T ? t : T - 1;
        const int tk = t < 1 ? 0 : (t - 1 < T ? t - 1 : T - 1);
        const uint2 *q2 = reinterpret_cast<const uint2 *>(qg + size_t(tq) * DK + part * EK);
        const uint2 *k2 = reinterpret_cast<const uint2 *>(kg + size_t(tk) * DK + part * EK);
        const uint2 *v2 = reinterpret_cast<const uint2 *>(vg + size_t(tq) * DV + j0 + part * EV);
        const float4 *b4 = reinterpret_cast<const float4 *>(a.beta + (size_t(bh) * T + tq) * DV + j0 + part * EV);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            rq[i] = q2[i];
            rk[i] = k2[i];
        }
#pragma unroll
        for (int i = 0; i < NVv; ++i) rv[i] = v2[i];
#pragma unroll
        for (int i = 0; i < EV / 4; ++i) rb[i] = b4[i];
        rlam = a.lambda[size_t(bh) * T + tq];
    };
    if (rower) prefetch(0);

    for (int c = 0; c < a.nchunks; ++c) {
        __syncthreads();   // the previous chunk's readers are done
        if (rower) {
            const int t = c * C + row;
            const bool qok = t < T;
            float q[EK], x[EK], y[EV];
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                Io8<E>::unpack(rq[i], q + i * Io8<E>::n);
                Io8<E>::unpack(rk[i], x + i * Io8<E>::n);
            }
#pragma unroll
            for (int i = 0; i < NVv; ++i) Io8<E>::unpack(rv[i], y + i * Io8<E>::n);
            if (t == 0) {   // x_0: the carried feature of a continued sequence, 0 when fresh
#pragma unroll
                for (int e = 0; e < EK; ++e) x[e] = a.xnext_in ? a.xnext_in[size_t(bh) * DK + part * EK + e] : 0.f;
            }
            float sq = 0.f, sx = 0.f;
#pragma unroll
            for (int e = 0; e < EK; ++e) {
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
                q[e] *= scq;
                x[e] *= scx;
                n2 += x[e] * x[e];
                st(&sh.XT[part * EK + e][0], row, x[e]);
            }
            put_row<E, EK>(&sh.Qh[row][part * EK], q);
            put_row<E, EK>(&sh.Xr[row][part * EK], x);
            n2 += dpp<kDppQuadXor1>(n2);
            n2 += dpp<kDppQuadXor2>(n2);
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const int j = part * EV + e;
                sh.Yf[row][j] = qok ? y[e] : 0.f;
                sh.Bf[row][j] = rb[e >> 2][e & 3];
            }
            if (part == 0) {
                sh.n2[row] = n2;
                sh.lam[row] = rlam;
                sh.ok[row] = (qok && !(t == 0 && a.fresh)) ? 1.f : 0.f;   // the fresh first step writes nothing
            }
            if (c + 1 < a.nchunks) prefetch(c + 1);   // (rower: inside the row phase)
        }
        __syncthreads();

        // per-column steps and log-prefix: wave w takes columns w, w + 4, ..,
        // lane = token; the prefix is a wave scan
        {
            const float den = sh.n2[lane] + sh.lam[lane] + a.eps;
            const bool live = sh.ok[lane] != 0.f;
            const float lam = sh.lam[lane];
            bool in_range = true;
            for (int j = wave; j < DS; j += NT / 64) {
                const float eta = live ? step_eta(sh.Bf[lane][j], den) : 0.f;
                const float b = wave_inclusive_scan(log2_1m(step_alpha(eta, lam, a.eps_gamma)));
                sh.Bf[lane][j] = b;
                st(&sh.YT[j][0], lane, eta * sh.Yf[lane][j] * exp2f(-b));
                in_range = in_range && __shfl(b, 63, 64) >= kMinLog2Decay;
            }
            if (lane == 0) sh.fastw[wave] = in_range ? 1 : 0;
        }
        __syncthreads();
        bool fast = true;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) fast = fast && sh.fastw[w] != 0;

        if (fast) {
            // L = lower(Qh X^T), 16 x 16 tiles
            for (int tile = wave; tile < 16; tile += NT / 64) {
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
            for (int tile = wave; tile < 4 * (DS / 16); tile += NT / 64) {
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
            for (int tile = wave; tile < (DK / 16) * (DS / 16); tile += NT / 64) {
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
    if (sl == 0 && wave == 0 && a.xnext_out) {   // phi(k_{T-1})
        const float xv = lane < DK ? ld(kg, size_t(T - 1) * DK + lane) : 0.f;
        const float sc = phi_scale(wave_sum(xv * xv), DK, a.eps_rms, a.phi);
        if (lane < DK) a.xnext_out[size_t(bh) * DK + lane] = xv * sc;
    }
}

template <class E, int DK>
void launch_f2a_dk(const ChunkF2Args &a, hipStream_t s) {
    // slices of 32 value columns (two workgroups per CU by LDS), or of 16
    // when 32-column slices would leave compute units idle; every slice forms
    // the head's shared features and scores again (its rows come from L2)
    const int ds = (a.dv < 32 || static_cast<long long>(a.BH) * (a.dv / 32) < 256) ? 16 : 32;
    const int nslice = a.dv / ds;
    const dim3 grid(((a.BH + 7) / 8) * 8 * nslice);
    if (ds == 16) chunk_f2a_kernel<E, DK, 16><<<grid, NT, 0, s>>>(a, nslice);
    else chunk_f2a_kernel<E, DK, 32><<<grid, NT, 0, s>>>(a, nslice);
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
