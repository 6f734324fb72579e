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
// The solve runs in four blocks of 16 tokens.  Contributions of earlier blocks
// go through MFMA with the writes rescaled to the last token s of the
// previous block, U~_l = e^{b_s - b_l} u_l, and are multiplied by
// e^{b_{t-1} - b_s} <= 1 (e^{b_t - b_s} for the output).  Inside a block one
// lane per column runs the forward substitution, keeping v_l = e^{b_{t-1}-b_l}
// u_l and multiplying it by gamma_t at every step.  No factor exceeds 1.
//
// One workgroup owns one (batch*head, 16 value columns); all slices of a head
// share an XCD.  The state slice lives in MFMA accumulators.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;
constexpr int DS = 16;   // value columns per workgroup

template <class E, int DK>
__global__ __launch_bounds__(256) void chunk_f2(ChunkF2Args a, int nslice) {
    constexpr int PD = Pad<E>::v;
    constexpr int LK = DK + PD;     // [.][d] rows
    constexpr int LC = C + PD;      // [.][token] rows
    constexpr int NT = DK / 64;     // state row tiles per wave (DK = 64 or 128)
    __shared__ __align__(16) E XB[C * LK];      // x_t rows
    __shared__ __align__(16) E QB[C * LK];      // qh_t rows
    __shared__ __align__(16) E XT[DK * LC];     // x^T [d][t]
    __shared__ __align__(16) E GB[C * LC];      // Gram (strictly lower), MFMA operand
    __shared__ __align__(16) E PBm[C * LC];     // scores (lower incl. diagonal), MFMA operand
    __shared__ float GD[4 * 16 * 17];           // diagonal 16x16 blocks of the Gram, fp32
    __shared__ float PD4[4 * 16 * 17];          // diagonal 16x16 blocks of the scores, fp32
    __shared__ __align__(16) E ST[DS * LK];     // S^T copy [j][d]
    __shared__ __align__(16) E UTb[DS * LC];    // U~^T [j][l] (writes rescaled to a block edge)
    __shared__ __align__(16) E WT[DS * LC];     // (e^{b_C-b_l} u_l)^T [j][l]
    __shared__ float R0[C * 17];                // residual R0 [t][j]
    __shared__ float OA[C * 17];                // output accumulator [t][j]
    __shared__ float H[2][16 * 17];             // cross-block sums for the solve / output
    // per (token, column) step scalars; decay ratios are formed from short
    // sums (block-local prefixes, suffixes), never as differences of long
    // chunk prefixes, so they stay accurate when the carries are small
    __shared__ float ETA[C * 17];   // eta_t
    __shared__ float GAM[C * 17];   // gamma_t
    __shared__ float EB[C * 17];    // e^{b_t}, b restarted at the chunk start
    __shared__ float EBP[C * 17];   // e^{b_{t-1}}
    __shared__ float EBL[C * 17];   // e^{b_t - b_s}, s = last token before t's 16-block
    __shared__ float EBLP[C * 17];  // e^{b_{t-1} - b_s}
    __shared__ float ESF[C * 17];   // e^{b_C - b_t}
    __shared__ float nrm[C];

    const int id = blockIdx.x, u8 = id & 7, rest = id >> 3;
    const int s = rest % nslice;
    const int bh = (rest / nslice) * 8 + u8;
    if (bh >= a.BH) return;
    const int j0 = DS * s;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.T, DV = a.dv;
    const E *qg = static_cast<const E *>(a.q) + size_t(bh) * T * DK;
    const E *kg = static_cast<const E *>(a.k) + size_t(bh) * T * DK;
    const E *vg = static_cast<const E *>(a.v) + size_t(bh) * T * DV;
    E *og = static_cast<E *>(a.o) + size_t(bh) * T * DV;
    const float *betag = a.beta + size_t(bh) * T * DV;
    const float *lamg = a.lambda + size_t(bh) * T;

    // zero the never-written upper parts of the MFMA operands
    for (int idx = tid; idx < C * LC; idx += 256) {
        st(GB, idx, 0.f);
        st(PBm, idx, 0.f);
    }
    // state tiles: wave w owns rows 16 * (w * NT + m), columns j0 .. j0 + 15
    f32x4 S[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
        const int dbase = 16 * (wave * NT + m);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = dbase + 4 * (lane >> 4) + r;
            S[m][r] = a.S_in ? a.S_in[(size_t(bh) * DK + d) * DV + j0 + (lane & 15)] : 0.f;
        }
        st4(ST + (lane & 15) * LK + dbase + 4 * (lane >> 4), S[m]);
    }
    __syncthreads();

    for (int c = 0; c < a.nchunks; ++c) {
        const int c0 = c * C;
        // 1. features: one wave per row, lanes over d
        for (int t = wave; t < C; t += 4) {
            const int tt = c0 + t;
            float xv[2] = {0.f, 0.f}, qv[2] = {0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int e = lane + 64 * m;
                if (e < DK) {
                    if (tt < T) qv[m] = ld(qg, size_t(tt) * DK + e);
                    if (tt >= 1 && tt < T) xv[m] = ld(kg, size_t(tt - 1) * DK + e);
                    else if (tt == 0 && a.xnext_in) xv[m] = a.xnext_in[size_t(bh) * DK + e];
                }
            }
            const bool from_k = tt >= 1 && tt < T;
            const float sq = phi_scale(wave_sum(qv[0] * qv[0] + qv[1] * qv[1]), DK, a.eps_rms, a.phi);
            const float sk = from_k ? phi_scale(wave_sum(xv[0] * xv[0] + xv[1] * xv[1]), DK, a.eps_rms, a.phi)
                                    : 1.f;
            float n2 = 0.f;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int e = lane + 64 * m;
                xv[m] *= sk;
                n2 += xv[m] * xv[m];
                if (e < DK) {
                    st(XB, size_t(t) * LK + e, xv[m]);
                    st(QB, size_t(t) * LK + e, qv[m] * sq);
                    st(XT, size_t(e) * LC + t, xv[m]);
                }
            }
            n2 = wave_sum(n2);
            if (lane == 0) nrm[t] = n2;
        }
        // values of this slice; the rescaled writes start at zero (the
        // cross-block products read the not-yet-written columns too)
        for (int idx = tid; idx < C * DS; idx += 256) {
            const int t = idx / DS, j = idx % DS;
            R0[t * 17 + j] = (c0 + t < T) ? ld(vg, size_t(c0 + t) * DV + j0 + j) : 0.f;
            st(UTb, size_t(j) * LC + t, 0.f);
        }
        __syncthreads();

        // 2. per-column steps and log-prefixes (wave w: columns 4w..4w+3,
        //    lanes = tokens); Gram and score tiles; X S and Qh S
        {
            const int t = c0 + lane;
            const bool noop = t >= T || (t == 0 && a.fresh);
            const float lam = t < T ? lamg[t] : 0.f;
            const float den = nrm[lane] + lam + a.eps;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = 4 * wave + jj;
                float eta = 0.f, alpha = 0.f;
                if (!noop) {
                    eta = step_eta(betag[size_t(t) * DV + j0 + j], den);
                    alpha = step_alpha(eta, lam, a.eps_gamma);
                }
                const float lg = log1pf(-alpha);
                const float b = wave_inclusive_scan(lg);
                float bp = __shfl_up(b, 1, 64);
                if (lane == 0) bp = 0.f;
                float bl = lg;   // inclusive prefix inside the 16-token block
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    const float y = __shfl_up(bl, o, 16);
                    if ((lane & 15) >= o) bl += y;
                }
                float blp = __shfl_up(bl, 1, 16);
                if ((lane & 15) == 0) blp = 0.f;
                float sf = lg;   // inclusive suffix to the chunk end
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const float y = __shfl_down(sf, o, 64);
                    if (lane + o < 64) sf += y;
                }
                float sfx = __shfl_down(sf, 1, 64);
                if (lane == 63) sfx = 0.f;
                const int q = lane * 17 + j;
                ETA[q] = eta;
                GAM[q] = 1.f - alpha;
                EB[q] = expf(b);
                EBP[q] = expf(bp);
                EBL[q] = expf(bl);
                EBLP[q] = expf(blp);
                ESF[q] = expf(sfx);
            }
        }
        for (int job = wave; job < 20; job += 4) {
            const bool isG = job < 10;
            int t = isG ? job : job - 10, I = 0;
            while (t > I) {
                t -= I + 1;
                ++I;
            }
            const int J = t;
            const f32x4 g = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, (isG ? XB : QB) + 16 * I * LK, LK,
                                        XB + 16 * J * LK, LK, 0, DK);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * (lane >> 4) + r, jn = 16 * J + (lane & 15);
                const float v = isG ? (jn < i ? g[r] : 0.f) : (jn <= i ? g[r] : 0.f);
                st(isG ? GB : PBm, size_t(i) * LC + jn, v);
                if (I == J) (isG ? GD : PD4)[I * 272 + (i - 16 * I) * 17 + (jn - 16 * J)] = v;
            }
        }
        f32x4 xs = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, XB + 16 * wave * LK, LK, ST, LK, 0, DK);
        f32x4 o1 = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, QB + 16 * wave * LK, LK, ST, LK, 0, DK);
        __syncthreads();

        // 3. residuals and the state part of the outputs
        {
            const int j = lane & 15;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * wave + 4 * (lane >> 4) + r;
                R0[t * 17 + j] -= EBP[t * 17 + j] * xs[r];
                OA[t * 17 + j] = EB[t * 17 + j] * o1[r];
            }
        }
        __syncthreads();

        // 4. blocked per-column solve and outputs (wave 0)
        if (wave == 0) {
            const int j = lane & 15;
            for (int I = 0; I < 4; ++I) {
                // cross-block sums H = G[I, :16I] U~ and Hp = P0[I, :16I] U~
                if (I > 0) {
                    const int kend = (16 * I + Mma<E>::KS - 1) / Mma<E>::KS * Mma<E>::KS;
                    const f32x4 h = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, GB + 16 * I * LC, LC, UTb, LC, 0, kend);
                    const f32x4 hp = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, PBm + 16 * I * LC, LC, UTb, LC, 0, kend);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        H[0][(4 * (lane >> 4) + r) * 17 + j] = h[r];
                        H[1][(4 * (lane >> 4) + r) * 17 + j] = hp[r];
                    }
                    wave_lds_sync();
                }
                // forward substitution inside the block, lane j < 16 = column
                float v[16];   // v_l = e^{b_t - b_l} u_l for the block's l <= t
                float ucol[16];
                if (lane < 16) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int t = 16 * I + i;
                        // entering step t: v_l = e^{b_{t-1} - b_l} u_l
                        float acc = 0.f;
#pragma unroll
                        for (int l = 0; l < 16; ++l)
                            if (l < i) acc += GD[I * 272 + i * 17 + l] * v[l];
                        float cross = 0.f;
                        if (I > 0) cross = EBLP[t * 17 + j] * H[0][i * 17 + j];
                        const float u = ETA[t * 17 + j] * (R0[t * 17 + j] - cross - acc);
                        ucol[i] = u;
                        // advance to e^{b_t - b_l} u_l and append u_t
                        const float g = GAM[t * 17 + j];
#pragma unroll
                        for (int l = 0; l < 16; ++l)
                            if (l < i) v[l] *= g;
                        v[i] = u;
                        float oin = 0.f;
#pragma unroll
                        for (int l = 0; l < 16; ++l)
                            if (l <= i) oin += PD4[I * 272 + i * 17 + l] * v[l];
                        float ocross = 0.f;
                        if (I > 0) ocross = EBL[t * 17 + j] * H[1][i * 17 + j];
                        OA[t * 17 + j] += oin + ocross;
                    }
                    // U~ for the next block: rescale to its edge s' = 16 I + 15
                    const float f = EBL[(16 * I + 15) * 17 + j];
                    for (int l = 0; l < 16 * I; ++l) st(UTb, size_t(j) * LC + l, f * ld(UTb, size_t(j) * LC + l));
#pragma unroll
                    for (int l = 0; l < 16; ++l) {
                        st(UTb, size_t(j) * LC + 16 * I + l, v[l]);
                        R0[(16 * I + l) * 17 + j] = ucol[l];   // keep u for the state update
                    }
                }
                wave_lds_sync();
            }
        }
        __syncthreads();

        // 5. outputs to HBM; state update S = e^{b_C} S + X^T (e^{b_C-b_l} u_l)
        for (int idx = tid; idx < C * DS; idx += 256) {
            const int t = idx / DS, j = idx % DS;
            if (c0 + t < T) st(og, size_t(c0 + t) * DV + j0 + j, OA[t * 17 + j]);
            const float w = ESF[t * 17 + j] * R0[t * 17 + j];
            st(WT, size_t(j) * LC + t, w);
        }
        __syncthreads();
        {
            const int j = lane & 15;
            const float gC = EB[63 * 17 + j];
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                const int dbase = 16 * (wave * NT + m);
#pragma unroll
                for (int r = 0; r < 4; ++r) S[m][r] *= gC;
                S[m] = Mma<E>::run(S[m], XT + dbase * LC, LC, WT, LC, 0, C);
                st4(ST + j * LK + dbase + 4 * (lane >> 4), S[m]);
            }
        }
        __syncthreads();
    }

    // boundary state
    if (a.S_out) {
#pragma unroll
        for (int m = 0; m < NT; ++m) {
            const int dbase = 16 * (wave * NT + m);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = dbase + 4 * (lane >> 4) + r;
                a.S_out[(size_t(bh) * DK + d) * DV + j0 + (lane & 15)] = S[m][r];
            }
        }
    }
    if (s == 0 && wave == 0 && a.xnext_out && T > 0) {
        float x[2] = {0.f, 0.f};
        for (int m = 0; m < 2; ++m)
            if (lane + 64 * m < DK) x[m] = ld(kg, size_t(T - 1) * DK + lane + 64 * m);
        const float sc = phi_scale(wave_sum(x[0] * x[0] + x[1] * x[1]), DK, a.eps_rms, a.phi);
        for (int m = 0; m < 2; ++m)
            if (lane + 64 * m < DK) a.xnext_out[size_t(bh) * DK + lane + 64 * m] = x[m] * sc;
    }
}

template <class E, int DK>
void launch_t(const ChunkF2Args &a, hipStream_t s, Marks *m) {
    const int nslice = a.dv / DS;
    const int blocks = ((a.BH + 7) / 8) * 8 * nslice;
    chunk_f2<E, DK><<<blocks, 256, 0, s>>>(a, nslice);
    m->mark(s);
}

}  // namespace

void launch_chunk_f2(const ChunkF2Args &a, bool bf16, hipStream_t s, Marks *m) {
    if (bf16) {
        if (a.dk == 64) launch_t<bf16_t, 64>(a, s, m);
        else launch_t<bf16_t, 128>(a, s, m);
    } else {
        launch_t<float, 64>(a, s, m);   // the planner admits d_k = 64 only
    }
}

}  // namespace falcon
