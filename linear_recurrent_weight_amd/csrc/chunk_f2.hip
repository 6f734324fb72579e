// Chunk-parallel Falcon-2 forward (per-column plasticity; summary §B.2 "per-
// channel plasticity", App. F "Falcon-2 Parallel Implementation", §F.2 and
// Figure 5: shared Gram per chunk, one triangular residual system per value
// column, merged into one solve per chunk).
//
// Column j of the state follows the Falcon-1 recurrence with its own step
// eta_{t,j} and carry gamma_{t,j} (lambda_t is shared).  In a chunk of 64
// tokens, with the per-column log-prefix b_{t,j} restarted at 0, the writes
// u_{t,j} = eta_{t,j} (y_{t,j} - S_{t-1}[:, j] . x_t) satisfy
//     u_t = eta_t (R0_t - sum_{l<t} e^{b_{t-1}-b_l} G_tl u_l),
//     R0_t = y_t - e^{b_{t-1}} (X S_0)_t,  G = X X^T (shared by the columns),
//     o_t = e^{b_t} (Qh S_0)_t + sum_{l<=t} e^{b_t-b_l} P0_tl u_l,  P0 = Qh X^T,
//     S_C = e^{b_C} S_0 + X^T (e^{b_C - b_l} u_l)_l        (all per column).
//
// The solve runs in four blocks of 16 tokens; s is the last token before a
// block and E_t = e^{b_t - b_s} <= 1 the block-local decay.  The writes of
// earlier blocks are kept rescaled to s, W_l = e^{b_s - b_l} u_l, so their
// contribution to a block is one MFMA, H = G[block, :] W, times E_{t-1}.
// Inside the block the decay factorises, e^{b_{t-1} - b_l} = E_{t-1} / E_l,
// so with w_l = u_l / E_l
//     u_t = eta_t (R0_t - E_{t-1} (H_t + sum_{l in block, l<t} G_tl w_l)),
// one multiply per step instead of rescaling every stored write; the block's
// outputs are then one MFMA, o_t = e^{b_t} (Qh S_0)_t + E_t (P0 [W; w])_t.
// When a block decays below 2^-100 (1 / E_l could overflow) it takes the
// exact form instead: v_l = e^{b_{t-1} - b_l} u_l multiplied by gamma_t at
// every step, outputs inside the step.  Both leave W rescaled to the block end.
// While every column of the slice keeps e^{b_C} >= 2^-100 (the usual case),
// the frame is the chunk start instead (s = -1 for every block: W_l =
// e^{-b_l} u_l, never rescaled), the outputs of all blocks are one MFMA pass
// after the solve, and the state update is S_C = e^{b_C} (S_0 + X^T W).
//
// Lanes of a solve wave: 4 per column (16 columns per wave), each owning the
// block positions l = q (mod 4); the in-block sums are quad sums (DPP).
// One workgroup owns one (head, DS value columns); the raw rows of the next
// chunk are prefetched while a chunk is processed.  It has four waves, or
// eight for bf16 with d_k = 128 and 32 columns (only one such workgroup fits
// a CU's LDS, and the second four waves share the features, step scalars,
// Gram, scores, X S and Qh S); the solve runs on the first DS / 16 waves.
// X^T is never stored: the state update reads its operand down the columns
// of the x rows.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;

// fp32 -> bf16, rounded to nearest even by the conversion instruction
// (two values packed in one word, the first in the low half)
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    typedef __bf16 h2v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2v{a, b}, h2v));
}
__device__ __forceinline__ void sth(bf16_t *p, size_t i, float v) { p[i].bits = __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ void sth(float *p, size_t i, float v) { p[i] = v; }

// One k step of an MFMA A operand A[m][k] = M[k][m] held down the columns
// of a row-major [k][m] tile (row stride ld): lane (m = lane % 16, k group)
// gathers its 8 (bf16) or 1 (fp32) values of k = k0 + ..
__device__ __forceinline__ bf16x8 col_frag(const bf16_t *M, int ld, int k0) {
    const int lane = threadIdx.x & 63;
    const bf16_t *p = M + (k0 + 8 * (lane >> 4)) * ld + (lane & 15);
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    u16x8 u;
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = p[e * ld].bits;
    return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ float col_frag(const float *M, int ld, int k0) {
    const int lane = threadIdx.x & 63;
    return M[(k0 + (lane >> 4)) * ld + (lane & 15)];
}

// 16-byte vectors <-> floats for the io type
template <class E> struct Io;
template <> struct Io<bf16_t> {
    static constexpr int per16 = 8;
    __device__ static void unpack(const uint4 &u, float *f) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = __uint_as_float(w[e] << 16);
            f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
    __device__ static uint32_t p2(float a, float b) { return bf16x2_rne(a, b); }
    __device__ static uint4 pack(const float *f) {
        return make_uint4(p2(f[0], f[1]), p2(f[2], f[3]), p2(f[4], f[5]), p2(f[6], f[7]));
    }
    // four consecutive outputs
    __device__ static void store4(bf16_t *p, const float *f) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(p2(f[0], f[1]), p2(f[2], f[3]));
    }
};
template <> struct Io<float> {
    static constexpr int per16 = 4;
    __device__ static void unpack(const uint4 &u, float *f) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
    __device__ static uint4 pack(const float *f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
    __device__ static void store4(float *p, const float *f) {
        *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
    }
};

// the value of lane h of each lane quad, in every lane of the quad (DPP
// quad_perm [h, h, h, h], CTRL = 0x55 h; every lane is written, so the
// destination needs no old value)
template <int CTRL>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// four consecutive elements of an LDS row (8- or 16-byte aligned) as fp32
__device__ __forceinline__ f32x4 ld4e(const bf16_t *p) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 ld4e(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4e(bf16_t *p, const f32x4 &v) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(Io<bf16_t>::p2(v[0], v[1]), Io<bf16_t>::p2(v[2], v[3]));
}
__device__ __forceinline__ void st4e(float *p, const f32x4 &v) { *reinterpret_cast<f32x4 *>(p) = v; }

__device__ __forceinline__ float quad_sum(float v) {
    v += dpp<kDppQuadXor1>(v);
    return v + dpp<kDppQuadXor2>(v);
}
// inclusive prefix inside each row of 16 lanes (= one 16-token block)
__device__ __forceinline__ float row_scan(float v) {
    v += dpp<kDppRowShr1>(v);
    v += dpp<kDppRowShr2>(v);
    v += dpp<kDppRowShr4>(v);
    return v + dpp<kDppRowShr8>(v);
}
template <class E>
__device__ __forceinline__ int kend_for(int n) {   // n rounded up to the MFMA k step
    return (n + Mma<E>::KS - 1) / Mma<E>::KS * Mma<E>::KS;
}

template <class E, int DK, int DS, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_f2(ChunkF2Args a, int nslice) {
    constexpr int NT = 64 * NW;     // threads; NW waves
    constexpr int TPR = NT / C;     // threads per token row
    constexpr int PD = Pad<E>::v;
    constexpr int LK = DK + PD;     // [t][d] rows
    constexpr int LC = C + PD;      // [.][token] rows
    constexpr int RS = DS + 1;      // fp32 [t][j] rows
    constexpr int SVS = C + 1;      // float4 [j][t] rows (odd pitch: no bank conflicts)
    constexpr int NCT = DS / 16;    // column tiles (= solve waves)
    constexpr int EPT = DK / TPR;   // features per thread
    constexpr int NV = EPT / Io<E>::per16;
    constexpr int YE = DS / TPR;    // value columns per thread
    constexpr int NB = YE / 4;      // 16-byte vectors of gains per thread
    constexpr int NDT = DK / (16 * NW);   // state d tiles per wave
    static_assert(NDT >= 1 && NB >= 1, "the thread mapping covers the tiles and gains");
    static_assert(YE * sizeof(E) == 16 || YE * sizeof(E) == 8, "values per thread fit one 16- or 8-byte load");

    __shared__ __align__(16) E XB[C * LK];     // x rows
    __shared__ __align__(16) E QB[C * LK];     // qh rows
    __shared__ __align__(16) E GB[C * LC];     // Gram, strictly lower tiles
    __shared__ __align__(16) E PB[C * LC];     // scores, lower incl. diagonal
    __shared__ float4 GDq[4 * 16 * 4];         // diagonal Gram blocks (fp32): [blk][i][q] = G_{i, 4m+q}, m = 0..3
    __shared__ float4 GDu[4 * 16 * 4];         // their strictly upper parts, same layout (G_{i, 4m+q} for 4m+q > i)
    __shared__ float PD4[4 * 16 * 17];         // diagonal score blocks (fp32)
    __shared__ __align__(16) E ST[DS * LK];    // S^T [j][d]
    __shared__ __align__(16) E WT[DS * LC];    // W^T [j][l]
    __shared__ float4 SV[DS * SVS];            // per (j, t): eta, y then R0, E_{t-1}, E_t
    __shared__ float GAM[C * RS];              // gamma
    __shared__ float EB[C * RS];               // log2 gamma, then e^{b_t}
    __shared__ float OA[C * RS];               // e^{b_t} (Qh S_0)_t
    __shared__ float Hs[NCT][2][16 * 17];      // per solve wave: cross sums

    const int id = blockIdx.x, u8 = id & 7, rest = id >> 3;
    const int s = rest % nslice;
    const int bh = (rest / nslice) * 8 + u8;
    if (bh >= a.BH) return;   // the whole workgroup leaves together
    const int j0 = DS * s;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.T, DV = a.dv;
    const int col = lane & 15, g4 = 4 * (lane >> 4);
    const E *qg = static_cast<const E *>(a.q) + size_t(bh) * T * DK;
    const E *kg = static_cast<const E *>(a.k) + size_t(bh) * T * DK;
    const E *vg = static_cast<const E *>(a.v) + size_t(bh) * T * DV;
    E *og = static_cast<E *>(a.o) + size_t(bh) * T * DV;
    const float *betag = a.beta + size_t(bh) * T * DV;
    const float *lamg = a.lambda + size_t(bh) * T;

    // ---- raw rows of the next chunk (thread: row, part), prefetched ----
    const int row = tid / TPR, part = tid % TPR;
    uint4 rq[NV], rk[NV], ry, rb[NB];
    float rlam;
    auto prefetch = [&](int c) {   // unconditional loads from rows clamped into [0, T)
        const int t = c * C + row;
        const int tq = t < T ? t : T - 1;
        const int tk = t < 1 ? 0 : (t - 1 < T ? t - 1 : T - 1);
        const uint4 *q4 = reinterpret_cast<const uint4 *>(qg + size_t(tq) * DK + part * EPT);
        const uint4 *k4 = reinterpret_cast<const uint4 *>(kg + size_t(tk) * DK + part * EPT);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            rq[v] = q4[v];
            rk[v] = k4[v];
        }
        if constexpr (YE * sizeof(E) == 16) {
            ry = *reinterpret_cast<const uint4 *>(vg + size_t(tq) * DV + j0 + part * YE);
        } else {
            const uint2 h = *reinterpret_cast<const uint2 *>(vg + size_t(tq) * DV + j0 + part * YE);
            ry = make_uint4(h.x, h.y, 0u, 0u);
        }
        const uint4 *b4 = reinterpret_cast<const uint4 *>(betag + size_t(tq) * DV + j0 + part * YE);
#pragma unroll
        for (int v = 0; v < NB; ++v) rb[v] = b4[v];
        rlam = lamg[tq];
    };

    // the tiles above the diagonal are never written but are read (times
    // zero) by the bf16 MFMA k steps of 32: they must hold zeros, not NaNs
    for (int idx = tid; idx < C * LC; idx += NT) {
        sth(GB, idx, 0.f);
        sth(PB, idx, 0.f);
    }

    // ---- state: d tiles {wave, wave + NW, ..} x all column tiles ----
    f32x4 S[NDT][NCT];
#pragma unroll
    for (int m = 0; m < NDT; ++m)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int dbase = 16 * (wave + NW * m);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = dbase + g4 + r;
                S[m][ct][r] = a.S_in ? a.S_in[(size_t(bh) * DK + d) * DV + j0 + 16 * ct + col] : 0.f;
            }
            st4e(ST + (16 * ct + col) * LK + dbase + g4, S[m][ct]);
        }
    prefetch(0);

    for (int c = 0; c < a.nchunks; ++c) {
        const int c0 = c * C;
        // ---- P1: features, values, step scalars; zero W; prefetch ----
        {
            const int t = c0 + row;
            float qv[EPT], xv[EPT];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                Io<E>::unpack(rq[v], qv + v * Io<E>::per16);
                Io<E>::unpack(rk[v], xv + v * Io<E>::per16);
            }
            const bool qok = t < T, kok = t >= 1 && t - 1 < T;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                qv[e] = qok ? qv[e] : 0.f;
                xv[e] = kok ? xv[e] : 0.f;
            }
            const bool first = t == 0;   // x_0 comes from the boundary state
            if (first && a.xnext_in) {
#pragma unroll
                for (int e = 0; e < EPT; ++e) xv[e] = a.xnext_in[size_t(bh) * DK + part * EPT + e];
            }
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                sq += qv[e] * qv[e];
                sk += xv[e] * xv[e];
            }
            const float scq = phi_scale(group_sum<TPR>(sq), DK, a.eps_rms, a.phi);
            const float sck = first ? 1.f : phi_scale(group_sum<TPR>(sk), DK, a.eps_rms, a.phi);
            float n2 = 0.f;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                xv[e] *= sck;
                qv[e] *= scq;
                n2 += xv[e] * xv[e];
            }
            n2 = group_sum<TPR>(n2);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                *reinterpret_cast<uint4 *>(XB + row * LK + part * EPT + v * Io<E>::per16) =
                    Io<E>::pack(xv + v * Io<E>::per16);
                *reinterpret_cast<uint4 *>(QB + row * LK + part * EPT + v * Io<E>::per16) =
                    Io<E>::pack(qv + v * Io<E>::per16);
            }
            float yv[Io<E>::per16], bv[YE];
            Io<E>::unpack(ry, yv);   // the first YE are this thread's values
#pragma unroll
            for (int v = 0; v < NB; ++v) {
                bv[4 * v] = __uint_as_float(rb[v].x);
                bv[4 * v + 1] = __uint_as_float(rb[v].y);
                bv[4 * v + 2] = __uint_as_float(rb[v].z);
                bv[4 * v + 3] = __uint_as_float(rb[v].w);
            }
            const bool noop = t >= T || (t == 0 && a.fresh);
            const float den = n2 + rlam + a.eps;
            const float rden = (noop || den == 0.f) ? 0.f : 1.f / den;   // eta = 0 when den == 0
#pragma unroll
            for (int e = 0; e < YE; ++e) {
                const int q = row * RS + part * YE + e;
                const float eta = bv[e] * rden;
                const float alpha = step_alpha(eta, rlam, a.eps_gamma);
                float4 *sv = SV + (part * YE + e) * SVS + row;
                sv->x = eta;
                sv->y = qok ? yv[e] : 0.f;
                GAM[q] = 1.f - alpha;
                EB[q] = log2_1m(alpha);   // log2 gamma
            }
            for (int idx = tid; idx < DS * LC; idx += NT) sth(WT, idx, 0.f);
            if (c + 1 < a.nchunks) prefetch(c + 1);
        }
        __syncthreads();

        // ---- P2a: per-column prefixes; Gram, scores, XS, Qh S on MFMA ----
        // Gram G = X X^T (strictly lower) and scores P0 = Qh X^T (lower with
        // the diagonal), one tile pair (I, J), J <= I, per job: the two share
        // the x rows of block J as their B operand
        for (int job = wave; job < 10; job += NW) {
            const int I = (0xffa94 >> (2 * job)) & 3, J = (0xe4910 >> (2 * job)) & 3;
            f32x4 g = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += MmaFrag<E>::KS) {
                const auto xj = MmaFrag<E>::load(XB + 16 * J * LK, LK, k0);
                g = MmaFrag<E>::mma(MmaFrag<E>::load(XB + 16 * I * LK, LK, k0), xj, g);
                p = MmaFrag<E>::mma(MmaFrag<E>::load(QB + 16 * I * LK, LK, k0), xj, p);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + g4 + r, jn = 16 * J + col;
                const float gv = jn < i ? g[r] : 0.f, pv = jn <= i ? p[r] : 0.f;
                sth(GB, size_t(i) * LC + jn, gv);
                sth(PB, size_t(i) * LC + jn, pv);
                if (I == J) {
                    const int e = ((I * 16 + g4 + r) * 4 + (col & 3)) * 4 + (col >> 2);
                    reinterpret_cast<float *>(GDq)[e] = gv;
                    reinterpret_cast<float *>(GDu)[e] = jn > i ? g[r] : 0.f;   // the block is symmetric
                    PD4[I * 272 + (g4 + r) * 17 + col] = pv;
                }
            }
        }
        // per-column prefixes (lane = token); with eight waves the six that
        // take one tile pair form them
        {
            constexpr int PW0 = NW == 8 ? 10 - NW : 0, NPW = NW - PW0;
            if (wave >= PW0) {
#pragma unroll
                for (int n = 0; n < (DS + NPW - 1) / NPW; ++n) {
                    const int j = wave - PW0 + NPW * n;
                    if (j >= DS) break;
                    const float lg = EB[lane * RS + j];
                    EB[lane * RS + j] = __builtin_amdgcn_exp2f(wave_inclusive_scan(lg));
                    const float el = __builtin_amdgcn_exp2f(row_scan(lg));   // block-local E_t
                    SV[j * SVS + lane].w = el;
                    if ((lane & 15) == 0) SV[j * SVS + lane].z = 1.f;
                    if ((lane & 15) != 15) SV[j * SVS + lane + 1].z = el;
                }
            }
        }
        // X S and Qh S for token rows 16 tw .. + 15: with eight waves, waves
        // 0-3 take X S and waves 4-7 Qh S
        const int tw = wave & 3;
        const bool doX = NW == 4 || wave < 4, doQ = NW == 4 || wave >= 4;
        // (the token rows are read once per k step for every column tile)
        f32x4 xs[NCT], qs[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            xs[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            qs[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += MmaFrag<E>::KS) {
            typename MmaFrag<E>::T ax{}, aq{};
            if (doX) ax = MmaFrag<E>::load(XB + 16 * tw * LK, LK, k0);
            if (doQ) aq = MmaFrag<E>::load(QB + 16 * tw * LK, LK, k0);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const auto sb = MmaFrag<E>::load(ST + 16 * ct * LK, LK, k0);
                if (doX) xs[ct] = MmaFrag<E>::mma(ax, sb, xs[ct]);
                if (doQ) qs[ct] = MmaFrag<E>::mma(aq, sb, qs[ct]);
            }
        }
        __syncthreads();

        // Chunk frame: while every column of the slice keeps e^{b_C} >=
        // 2^-100, the writes are kept as e^{-b_l} u_l (chunk-start frame), so
        // no block rescales the earlier ones and the state update scales once
        // by e^{b_C}; otherwise each block works in its own frame and rescales
        // (and a block that decays too far takes the exact form).  Every wave
        // forms the same flag from the chunk prefix.
        const bool cframe = __all(lane >= DS || EB[63 * RS + (lane < DS ? lane : 0)] >= 0x1p-100f);

        // ---- P2b: residuals and the state part of the outputs; in the chunk
        //      frame also the solve's step coefficients (P3) ----
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tw + g4 + r, j = 16 * ct + col;
                if (doX) {
                    const float ebp = t > 0 ? EB[(t - 1) * RS + j] : 1.f;
                    float4 *sv = SV + j * SVS + t;
                    const float4 v = *sv;
                    const float r0 = v.y - ebp * xs[ct][r];
                    if (cframe) {
                        // a_t = eta_t R0_t e^{-b_s} / E_t, c_t = eta_t E_{t-1} / E_t
                        // (s: the token before t's block)
                        const int s16 = 16 * (t >> 4) - 1;
                        const float iebs = s16 >= 0 ? __builtin_amdgcn_rcpf(EB[s16 * RS + j]) : 1.f;
                        const float re = __builtin_amdgcn_rcpf(v.w);
                        *reinterpret_cast<float2 *>(sv) = make_float2(v.x * r0 * iebs * re, v.x * v.z * re);
                    } else {
                        sv->y = r0;
                    }
                }
                if (doQ) OA[t * RS + j] = EB[t * RS + j] * qs[ct][r];
            }
        __syncthreads();

        // ---- P3: blocked per-column solve (wave sw: columns 16 sw ..) ----
        if (wave < NCT) {
            const int sw = wave, jj = lane >> 2, q = lane & 3, j = 16 * sw + jj;
            float *H0 = Hs[sw][0], *H1 = Hs[sw][1];
            const float own[4] = {q == 0 ? 1.f : 0.f, q == 1 ? 1.f : 0.f, q == 2 ? 1.f : 0.f,
                                  q == 3 ? 1.f : 0.f};
            // operands of steps i .. i + 3 in flight (a rotating buffer): the
            // two solving waves run alone on their SIMDs, so nothing else
            // hides an LDS round trip per step
            constexpr int PF = 4;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                // Running in-block sums: acc[m] of lane q holds sum_{l < t}
                // G_tl w_l for its position t = 4 m + q over the writes known
                // so far; once w_i is known, every later position adds G_ti w_i
                // (G_ti = G_it, row i of the upper part).  With a_i = eta_i
                // (R0_i e^{-b_s} - E_{i-1} h_i) / E_i and c_i = eta_i E_{i-1} /
                // E_i (neither depends on the writes of the block)
                //     w_i = a_i - c_i acc_i,
                // so a step's dependent chain is the broadcast of acc_i from its
                // owner lane and two multiply-adds.
                float w[4] = {0.f, 0.f, 0.f, 0.f};   // w_l = u_l / E_l, l = 4 m + q
                float acc[4] = {0.f, 0.f, 0.f, 0.f};
                auto step = [&](int i, float ai, float ci, const float4 &gu) {
                    const float x = acc[i >> 2];
                    const float s_i = (i & 3) == 0 ? quad_bcast<0x00>(x) : (i & 3) == 1 ? quad_bcast<0x55>(x)
                                    : (i & 3) == 2 ? quad_bcast<0xAA>(x) : quad_bcast<0xFF>(x);
                    const float wi = fmaf(-ci, s_i, ai);
                    // the owner lane of position i keeps w_i (its entry is
                    // still zero: a multiply-add by a 0/1 lane mask)
                    w[i >> 2] = fmaf(own[i & 3], wi, w[i >> 2]);
                    acc[0] = fmaf(gu.x, wi, acc[0]);
                    acc[1] = fmaf(gu.y, wi, acc[1]);
                    acc[2] = fmaf(gu.z, wi, acc[2]);
                    acc[3] = fmaf(gu.w, wi, acc[3]);
                };
                if (cframe) {
                    // chunk frame (s: the token before the block): P2b stored
                    // (a_i, c_i) without the cross-block term h = G[block, :] W
                    // of the earlier blocks, which folds in here once per block
                    if (I > 0) {
                        const f32x4 h = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, GB + 16 * I * LC, LC,
                                                    WT + 16 * sw * LC, LC, 0, kend_for<E>(16 * I));
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float2 *p = reinterpret_cast<float2 *>(SV + (16 * sw + col) * SVS + 16 * I + g4 + r);
                            const float2 ac = *p;
                            p->x = fmaf(-ac.y, h[r], ac.x);
                        }
                    }
                    wave_lds_sync();
                    float2 acb[PF];
                    float4 gub[PF];
#pragma unroll
                    for (int u = 0; u < PF; ++u) {
                        acb[u] = *reinterpret_cast<const float2 *>(SV + j * SVS + 16 * I + u);
                        gub[u] = GDu[(I * 16 + u) * 4 + q];
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float2 ac = acb[i % PF];
                        const float4 gu = gub[i % PF];
                        if (i + PF < 16) {
                            acb[i % PF] = *reinterpret_cast<const float2 *>(SV + j * SVS + 16 * I + i + PF);
                            gub[i % PF] = GDu[(I * 16 + i + PF) * 4 + q];
                        }
                        step(i, ac.x, ac.y, gu);
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) sth(WT, size_t(j) * LC + 16 * I + 4 * m + q, w[m]);
                    wave_lds_sync();
                    continue;
                }
                // block frame (s = 16 I - 1): SV holds (eta, R0, E_{t-1}, E_t)
                if (I > 0) {
                    const f32x4 h = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, GB + 16 * I * LC, LC,
                                                WT + 16 * sw * LC, LC, 0, kend_for<E>(16 * I));
#pragma unroll
                    for (int r = 0; r < 4; ++r) H0[(g4 + r) * 17 + col] = h[r];
                }
                const float fblk = SV[j * SVS + 16 * I + 15].w;   // e^{b_end - b_s}
                wave_lds_sync();
                if (__all(fblk >= 0x1p-100f)) {
                    float4 svb[PF], gub[PF];
                    float hb[PF];
#pragma unroll
                    for (int u = 0; u < PF; ++u) {
                        svb[u] = SV[j * SVS + 16 * I + u];
                        gub[u] = GDu[(I * 16 + u) * 4 + q];
                        hb[u] = I > 0 ? H0[u * 17 + jj] : 0.f;
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float4 sv = svb[i % PF], gu = gub[i % PF];
                        const float h = hb[i % PF];
                        if (i + PF < 16) {
                            svb[i % PF] = SV[j * SVS + 16 * I + i + PF];
                            gub[i % PF] = GDu[(I * 16 + i + PF) * 4 + q];
                            if (I > 0) hb[i % PF] = H0[(i + PF) * 17 + jj];
                        }
                        const float re = __builtin_amdgcn_rcpf(sv.w);
                        step(i, sv.x * (sv.y - sv.z * h) * re, sv.x * sv.z * re, gu);
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) sth(WT, size_t(j) * LC + 16 * I + 4 * m + q, w[m]);
                    wave_lds_sync();
                    // outputs of the block: o_t = OA_t + E_t (P0 [W; w])_t, as O^T tiles
                    {
                        const f32x4 o = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, WT + 16 * sw * LC, LC,
                                                    PB + 16 * I * LC, LC, 0, kend_for<E>(16 * I + 16));
                        const int t = 16 * I + col;
                        float ov[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int jr = 16 * sw + g4 + r;
                            ov[r] = OA[t * RS + jr] + SV[jr * SVS + t].w * o[r];
                        }
                        if (c0 + t < T) Io<E>::store4(og + size_t(c0 + t) * DV + j0 + 16 * sw + g4, ov);
                    }
                    // rescale W to the block end: the quad of column j takes the
                    // row's 4-element pieces, lane q pieces q, q + 4, .. (every
                    // load before the first store)
                    {
                        E *wrow = WT + size_t(j) * LC;
                        f32x4 pc[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (u <= I) pc[u] = ld4e(wrow + 4 * (q + 4 * u));
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (u <= I) st4e(wrow + 4 * (q + 4 * u), pc[u] * fblk);
                    }
                    wave_lds_sync();
                } else {
                    if (I > 0) {
                        const f32x4 h = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, PB + 16 * I * LC, LC,
                                                    WT + 16 * sw * LC, LC, 0, kend_for<E>(16 * I));
#pragma unroll
                        for (int r = 0; r < 4; ++r) H1[(g4 + r) * 17 + col] = h[r];
                        wave_lds_sync();
                    }
                    // exact form: v_l = e^{b_{t-1} - b_l} u_l, advanced by gamma_t
                    float v[4] = {0.f, 0.f, 0.f, 0.f};
                    float pb = 1.f;   // e^{b_{t-1} - b_s}
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int t = 16 * I + i;
                        const float gm = GAM[t * RS + j];
                        const float4 gq = GDq[(I * 16 + i) * 4 + q];
                        const float4 sv = SV[j * SVS + t];
                        float part_s = 0.f;   // v_l = 0 for l >= i
                        if (i > 0) part_s += gq.x * v[0];
                        if (i > 4) part_s += gq.y * v[1];
                        if (i > 8) part_s += gq.z * v[2];
                        if (i > 12) part_s += gq.w * v[3];
                        const float acc = quad_sum(part_s);
                        const float cross = I > 0 ? pb * H0[i * 17 + jj] : 0.f;
                        const float u = sv.x * (sv.y - cross - acc);
#pragma unroll
                        for (int m = 0; m < 4; ++m)
                            if (4 * m < i) v[m] *= gm;   // zero entries stay zero
                        v[i >> 2] = q == (i & 3) ? u : v[i >> 2];
                        pb *= gm;
                        float part_o = 0.f;   // P0's diagonal block is zero above its diagonal
#pragma unroll
                        for (int m = 0; m < 4; ++m)
                            if (4 * m <= i) part_o += PD4[I * 272 + i * 17 + 4 * m + q] * v[m];
                        const float oin = quad_sum(part_o);
                        if (q == 0 && c0 + t < T) {
                            float o = OA[t * RS + j] + oin;
                            if (I > 0) o += pb * H1[i * 17 + jj];
                            sth(og, size_t(c0 + t) * DV + j0 + j, o);
                        }
                    }
                    for (int l = q; l < 16 * I; l += 4) {
                        const size_t p = size_t(j) * LC + l;
                        sth(WT, p, pb * ld(WT, p));
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) sth(WT, size_t(j) * LC + 16 * I + 4 * m + q, v[m]);
                    wave_lds_sync();
                }
            }
        }
        __syncthreads();

        // ---- P4: S = e^{b_C} S + X^T W (W = writes rescaled to the chunk end),
        //      or in the chunk frame S = e^{b_C} (S + X^T W); the X^T operand
        //      is read down the columns of the x rows, once per k step for
        //      all column tiles ----
#pragma unroll
        for (int m = 0; m < NDT; ++m) {
            const int dbase = 16 * (wave + NW * m);
            f32x4 acc[NCT];
            float gC[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                gC[ct] = EB[63 * RS + 16 * ct + col];
                acc[ct] = cframe ? S[m][ct] : S[m][ct] * gC[ct];
            }
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += MmaFrag<E>::KS) {
                const auto xa = col_frag(XB + dbase, LK, k0);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    acc[ct] = MmaFrag<E>::mma(xa, MmaFrag<E>::load(WT + 16 * ct * LC, LC, k0), acc[ct]);
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                S[m][ct] = cframe ? acc[ct] * gC[ct] : acc[ct];
                st4e(ST + (16 * ct + col) * LK + dbase + g4, S[m][ct]);
            }
        }
        // ---- P3b (chunk frame): the outputs of every block at once,
        //      o_t = OA_t + e^{b_t} (P0 W)_t with W = e^{-b_l} u_l, one O^T tile
        //      (columns 16 ct .., tokens 16 I ..) per wave ----
        if (cframe) {
            for (int tile = wave; tile < 4 * NCT; tile += NW) {
                const int ct = tile % NCT, I = tile / NCT;
                const f32x4 o = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, WT + 16 * ct * LC, LC,
                                            PB + 16 * I * LC, LC, 0, kend_for<E>(16 * I + 16));
                const int t = 16 * I + col;
                float ov[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jr = 16 * ct + g4 + r;
                    ov[r] = OA[t * RS + jr] + EB[t * RS + jr] * o[r];
                }
                if (c0 + t < T) Io<E>::store4(og + size_t(c0 + t) * DV + j0 + 16 * ct + g4, ov);
            }
        }
        __syncthreads();
    }

    // ---- boundary state ----
    if (a.S_out) {
#pragma unroll
        for (int m = 0; m < NDT; ++m)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 16 * (wave + NW * m) + g4 + r;
                    a.S_out[(size_t(bh) * DK + d) * DV + j0 + 16 * ct + col] = S[m][ct][r];
                }
    }
    if (s == 0 && wave == 0 && a.xnext_out) {
        float x[2] = {0.f, 0.f};
        for (int m = 0; m < 2; ++m)
            if (lane + 64 * m < DK) x[m] = ld(kg, size_t(T - 1) * DK + lane + 64 * m);
        const float sc = phi_scale(wave_sum(x[0] * x[0] + x[1] * x[1]), DK, a.eps_rms, a.phi);
        for (int m = 0; m < 2; ++m)
            if (lane + 64 * m < DK) a.xnext_out[size_t(bh) * DK + lane + 64 * m] = x[m] * sc;
    }
}

template <class E, int DK, int DS, int NW = 4>
void launch_t(const ChunkF2Args &a, hipStream_t s, Marks *m) {
    const int nslice = a.dv / DS;
    const int blocks = ((a.BH + 7) / 8) * 8 * nslice;
    chunk_f2<E, DK, DS, NW><<<blocks, 64 * NW, 0, s>>>(a, nslice);
    m->mark(s);
}

}  // namespace

void launch_chunk_f2(const ChunkF2Args &a, bool bf16, hipStream_t s, Marks *m) {
    if (bf16) {
        // 32 value columns per workgroup when d_v allows it
        if (a.dv % 32 == 0) {
            if (a.dk == 64) launch_t<bf16_t, 64, 32>(a, s, m);
            else launch_t<bf16_t, 128, 32, 8>(a, s, m);   // eight waves, 8 threads per row
        } else {
            if (a.dk == 64) launch_t<bf16_t, 64, 16>(a, s, m);
            else launch_t<bf16_t, 128, 16>(a, s, m);
        }
    } else {
        launch_t<float, 64, 16>(a, s, m);   // the planner admits d_k = 64 only
    }
}

}  // namespace falcon
