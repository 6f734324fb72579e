// Fused chunk-parallel Falcon-1 forward for bf16 inputs (one kernel, no
// workspace).  Same chunk algebra as chunk_f1.hip (summary Figure 4, §D.1,
// §E.2, §G, §G.1): with the chunk-local log-prefix b (restarted at 0),
//     U   = Tp (Y - diag(e^{b_{i-1}}) X S_0),   Tp = (I + N)^{-1} diag(eta),
//     N_ij = eta_i e^{b_{i-1}-b_j} x_i.x_j (j < i),
//     O   = diag(e^{b_i}) Qh S_0 + P U,          P_ij = e^{b_i-b_j} qh_i.x_j (j <= i),
//     S_C = e^{b_C} S_0 + (diag(e^{b_C-b_i}) X)^T U.
//
// One workgroup owns one (batch*head, DS value columns) and walks the chunks
// in order; nothing but q, k, v, beta, lambda, o and the state touches HBM.
// Its 8 wavefronts form two groups that run one chunk apart:
//   chain waves 0-3 (state-dependent, chunk i):
//     S1  X S and Qh S (MFMA), residual R0 = Y - Gamma_{i-1} X S, (w X)^T
//     S2  U = Tp R0
//     S3  O = Gamma Qh S + P U -> HBM;  S = Gamma_C S + (w X)^T U
//   prep waves 4-7 (state-independent, chunk i+1 and the inverse of chunk i):
//     D   column block J of (I + N)^{-1} (wave J; blocked, MFMA off-diagonal
//         products), scaled into Tp                                  [chunk i]
//     A   QK-RMSNorm of the prefetched rows, the key shift, eta and log gamma,
//         and the prefetch of the following chunk's rows             [chunk i+1]
//     B   log-prefix scan; Gram X X^T and scores Qh X^T tiles (MFMA)  [chunk i+1]
//     C   decay scaling into N (fp32) and P (bf16); diagonal 16x16
//         inverses by forward substitution                          [chunk i+1]
// Phases are separated by three workgroup barriers per chunk:
//     [S1 | D, A]  #1  [S2 | B]  #2  [S3 | C]  #3
// Operators that one group writes while the other reads are double-buffered.
#include "chunk_layout.h"
#include "common.h"
#include "kernels.h"

namespace falcon {
namespace {

constexpr int C = kChunk;   // 64 tokens per chunk
constexpr int PC = C + 8;   // bf16 row stride of [.][token] buffers (16-byte rows)

__device__ __forceinline__ bf16x8 ld8(const bf16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}
// 4 floats -> 4 bf16 stored as one 8-byte word
__device__ __forceinline__ void st4bf(bf16_t *p, float a, float b, float c, float d) {
    uint2 u;
    u.x = pack2(a, b);
    u.y = pack2(c, d);
    *reinterpret_cast<uint2 *>(p) = u;
}
__device__ __forceinline__ bf16x8 zero8() {
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = __bf16(0.f);
    return z;
}
// acc += A[16 x K] * Bt[16 x K]^T with both operands bf16 in LDS, k contiguous
__device__ __forceinline__ f32x4 tile_mm(f32x4 acc, const bf16_t *A, int lda, const bf16_t *Bt, int ldb,
                                         int K) {
    const int lane = threadIdx.x & 63;
    const int row = lane & 15, kq = 8 * (lane >> 4);
    for (int k0 = 0; k0 < K; k0 += 32) acc = mfma(ld8(A + row * lda + k0 + kq), ld8(Bt + row * ldb + k0 + kq), acc);
    return acc;
}

template <int DK, int DS>
struct Layout {
    static constexpr int PK = DK + 8;   // bf16 row stride of [.][d] buffers
};
// SC rows: 0 Gamma_{i-1}, 1 Gamma_i, 2 e^{b_C-b_i}, 3 eta, 4 b, 5 b_{i-1}, 6 [Gamma_C]

template <int DK, int DS>
__global__ __launch_bounds__(512) void chunk_f1_fused(F1FusedArgs a, int nslice) {
    using L = Layout<DK, DS>;
    constexpr int PK = L::PK;
    constexpr int NCT = DS / 16;          // column tiles of the slice
    constexpr int TPR = 4;                // prep threads per row
    constexpr int EPT = DK / TPR;         // elements per prep thread (16 or 32)
    constexpr int NV = EPT / 8;           // 16-byte vectors per prep thread
    static_assert(DK == 64 && DS % 16 == 0, "four chain waves own the 16-row state tiles of d_k = 64");

    // every buffer is its own LDS object, so loads from one are never held
    // back behind stores to another
    __shared__ __align__(16) bf16_t XB[2 * C * PK];       // normalised keys (shifted), 2 chunks
    __shared__ __align__(16) bf16_t QB[2 * C * PK];       // normalised queries, 2 chunks
    __shared__ __align__(16) bf16_t TPB[C * PC];          // Tp = (I + N)^{-1} diag(eta)
    __shared__ __align__(16) bf16_t PB[2 * C * PC];       // decayed scores, 2 chunks
    __shared__ __align__(16) bf16_t XHT[DK * PC];         // (diag(w) X)^T
    __shared__ __align__(16) bf16_t ST[DS * PK];          // S^T (bf16 copy of the state slice)
    __shared__ __align__(16) bf16_t R0T[DS * PC];         // residual^T
    __shared__ __align__(16) bf16_t UT[DS * PC];          // U^T
    __shared__ __align__(16) bf16_t TDR[4 * 16 * 24];     // diagonal inverses T_JJ, row-major
    __shared__ __align__(16) bf16_t TCB[4 * 16 * PC];     // per prep wave: T[:, block J]^T
    __shared__ __align__(16) bf16_t MTB[4 * 16 * 24];     // per prep wave: M^T scratch
    __shared__ __align__(16) bf16_t NB[C * PC];           // system N (strictly lower)
    __shared__ __align__(16) float SC[2 * 7 * C];         // per-token scalars, 2 chunks
    __shared__ __align__(16) float LG[C];                 // log gamma of the chunk being prepared
    __shared__ __align__(16) bf16_t YB[2 * C * (DS + 8)]; // values of this slice, 2 chunks
    constexpr int PY = DS + 8;
    constexpr int YV = DS / 32;           // 16-byte vectors of Y per prep thread (8 bf16 each)

    // workgroup -> (head, slice); all slices of a head share an XCD
    int bh, s;
    if (nslice == 1) {
        bh = blockIdx.x;
        s = 0;
    } else {
        const int id = blockIdx.x, u = id & 7, rest = id >> 3;
        s = rest % nslice;
        bh = (rest / nslice) * 8 + u;
    }
    if (bh >= a.BH) return;  // whole workgroup leaves together
    const int j0 = s * DS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const bool chain = wave < 4;
    const int T = a.T, DV = a.dv, nch = a.nchunks;
    const bf16_t *qg = static_cast<const bf16_t *>(a.q) + size_t(bh) * T * DK;
    const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * DK;
    const bf16_t *vg = static_cast<const bf16_t *>(a.v) + size_t(bh) * T * DV;
    bf16_t *og = static_cast<bf16_t *>(a.o) + size_t(bh) * T * DV;
    const float *betag = a.beta + size_t(bh) * T;
    const float *lamg = a.lambda + size_t(bh) * T;

    // zero the operators whose upper blocks are never written
    for (int idx = tid; idx < C * PC; idx += 512) {
        TPB[idx].bits = 0;
        PB[idx].bits = 0;
        PB[C * PC + idx].bits = 0;
    }

    // ---------------- per-thread state ----------------
    // chain: state tiles S[d-tile = wave][col-tile ct], fp32 accumulators
    f32x4 Sacc[NCT];
    // prep: prefetched raw rows
    const int pt = tid - 256;           // prep thread index
    const int prow = pt / TPR, ppart = pt % TPR;
    uint4 rq[NV], rk[NV], ry[YV];
    float rbeta = 0.f, rlam = 0.f;

    auto prefetch_rows = [&](int c) {   // prep threads: raw rows of chunk c
        const int t = c * C + prow;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            rq[v] = t < T ? *reinterpret_cast<const uint4 *>(qg + size_t(t) * DK + ppart * EPT + 8 * v)
                          : make_uint4(0, 0, 0, 0);
            rk[v] = (t >= 1 && t - 1 < T)
                        ? *reinterpret_cast<const uint4 *>(kg + size_t(t - 1) * DK + ppart * EPT + 8 * v)
                        : make_uint4(0, 0, 0, 0);
        }
        if (ppart == 0) {
            rbeta = t < T ? betag[t] : 0.f;
            rlam = t < T ? lamg[t] : 0.f;
        }
        // this slice of Y: row t, columns j0 + (ppart * YV + v) * 8 ...
#pragma unroll
        for (int v = 0; v < YV; ++v)
            ry[v] = t < T ? *reinterpret_cast<const uint4 *>(vg + size_t(t) * DV + j0 + (ppart * YV + v) * 8)
                          : make_uint4(0, 0, 0, 0);
    };

    // A: features and step scalars of chunk c into buffer c & 1
    auto prep_A = [&](int c) {
        const int buf = c & 1;
        const int t = c * C + prow;
        float xv[EPT], qv[EPT];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const uint32_t wq[4] = {rq[v].x, rq[v].y, rq[v].z, rq[v].w};
            const uint32_t wk[4] = {rk[v].x, rk[v].y, rk[v].z, rk[v].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qv[8 * v + 2 * e] = __uint_as_float(wq[e] << 16);
                qv[8 * v + 2 * e + 1] = __uint_as_float(wq[e] & 0xffff0000u);
                xv[8 * v + 2 * e] = __uint_as_float(wk[e] << 16);
                xv[8 * v + 2 * e + 1] = __uint_as_float(wk[e] & 0xffff0000u);
            }
        }
        const bool first = (t == 0);     // x_0 comes from the boundary state
        if (first && a.xnext_in) {
#pragma unroll
            for (int e = 0; e < EPT; ++e) xv[e] = a.xnext_in[size_t(bh) * DK + ppart * EPT + e];
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            sq += qv[e] * qv[e];
            sk += xv[e] * xv[e];
        }
        sq = group_sum<TPR>(sq);
        sk = group_sum<TPR>(sk);
        const float scq = phi_scale(sq, DK, a.eps_rms, a.phi);
        const float sck = first ? 1.f : phi_scale(sk, DK, a.eps_rms, a.phi);
        float n2 = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            xv[e] *= sck;
            qv[e] *= scq;
            n2 += xv[e] * xv[e];
        }
        n2 = group_sum<TPR>(n2);
        bf16_t *xr = XB + (size_t(buf) * C + prow) * PK + ppart * EPT;
        bf16_t *qr = QB + (size_t(buf) * C + prow) * PK + ppart * EPT;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const float *x8 = xv + 8 * v;
            const float *q8 = qv + 8 * v;
            *reinterpret_cast<uint4 *>(xr + 8 * v) =
                make_uint4(pack2(x8[0], x8[1]), pack2(x8[2], x8[3]), pack2(x8[4], x8[5]), pack2(x8[6], x8[7]));
            *reinterpret_cast<uint4 *>(qr + 8 * v) =
                make_uint4(pack2(q8[0], q8[1]), pack2(q8[2], q8[3]), pack2(q8[4], q8[5]), pack2(q8[6], q8[7]));
        }
#pragma unroll
        for (int v = 0; v < YV; ++v)
            *reinterpret_cast<uint4 *>(YB + (size_t(buf) * C + prow) * PY + (ppart * YV + v) * 8) = ry[v];
        if (ppart == 0) {
            float eta = 0.f, alpha = 0.f;
            const bool noop = t >= T || (t == 0 && a.fresh);
            if (!noop) {
                eta = step_eta(rbeta, n2 + rlam + a.eps);
                alpha = step_alpha(eta, rlam, a.eps_gamma);
            }
            SC[(buf * 7 + 3) * C + prow] = eta;
            LG[prow] = log1pf(-alpha);
        }
    };

    // B: log-prefix scan (wave 4) and raw Gram / score tiles
    // job list: wave J owns G(J,J) and jobs J, J+4, J+8, J+12 of this list
    //   0-5: G (1,0) (2,0) (2,1) (3,0) (3,1) (3,2);  6-15: P (I,J), I >= J
    f32x4 jt[5];
    auto job_tile = [&](int jid, int &I, int &J, bool &isG) {
        // arithmetic enumeration (a lookup table would live in global memory)
        isG = jid < 6;
        int t = isG ? jid : jid - 6;
        int ii = isG ? 1 : 0;
        const int step0 = isG ? 0 : 1;   // strictly lower vs lower incl. diagonal
        while (t >= ii + step0) {
            t -= ii + step0;
            ++ii;
        }
        I = ii;
        J = t;
    };
    auto prep_B = [&](int c) {
        const int buf = c & 1;
        const int pw = wave - 4;
        const bf16_t *Xc = XB + size_t(buf) * C * PK;
        const bf16_t *Qc = QB + size_t(buf) * C * PK;
        if (pw == 0) {
            // log-prefix in base 2 (b2 = b / ln 2), so every decay factor is
            // one native exp2 of a non-positive difference
            const float lg2 = LG[lane] * 1.4426950408889634f;
            const float b = wave_inclusive_scan(lg2);
            float bp = __shfl_up(b, 1, 64);
            if (lane == 0) bp = 0.f;
            const float bC = __shfl(b, 63, 64);
            float *sc = SC + buf * 7 * C;
            sc[0 * C + lane] = __builtin_amdgcn_exp2f(bp);
            sc[1 * C + lane] = __builtin_amdgcn_exp2f(b);
            sc[2 * C + lane] = __builtin_amdgcn_exp2f(bC - b);
            sc[4 * C + lane] = b;
            sc[5 * C + lane] = bp;
            if (lane == 0) sc[6 * C] = __builtin_amdgcn_exp2f(bC);
        }
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        jt[0] = tile_mm(z, Xc + 16 * pw * PK, PK, Xc + 16 * pw * PK, PK, DK);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            int I, J;
            bool isG;
            job_tile(pw + 4 * m, I, J, isG);
            jt[1 + m] = tile_mm(z, (isG ? Xc : Qc) + 16 * I * PK, PK, Xc + 16 * J * PK, PK, DK);
        }
    };

    // C: decay scaling into N and P (bf16); diagonal inverse of block J
    auto prep_C = [&](int c) {
        const int buf = c & 1;
        const int pw = wave - 4;
        const float *sc = SC + buf * 7 * C;
        bf16_t *Pc = PB + size_t(buf) * C * PC;
        const int jj = lane & 15, g4 = 4 * (lane >> 4);
        int Im[5], Jm[5];
        bool Gm[5];
        Im[0] = Jm[0] = pw;
        Gm[0] = true;
#pragma unroll
        for (int m = 1; m < 5; ++m) job_tile(pw + 4 * (m - 1), Im[m], Jm[m], Gm[m]);
        // all scalar loads first (unconditional), then arithmetic, then stores
        float bcol[5], brow[5][4], erow[5][4];
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            bcol[m] = sc[4 * C + 16 * Jm[m] + jj];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * Im[m] + g4 + r;
                brow[m][r] = sc[(Gm[m] ? 5 : 4) * C + i];   // b_{i-1} for N, b_i for P
                erow[m][r] = sc[3 * C + i];
            }
        }
        float nd[4];   // this lane's entries of the diagonal block N_JJ (fp32)
        float vals[5][4];
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            const int j = 16 * Jm[m] + jj;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * Im[m] + g4 + r;
                const float e = __builtin_amdgcn_exp2f(fminf(brow[m][r] - bcol[m], 0.f));
                const float v = (Gm[m] ? erow[m][r] * e : e) * jt[m][r];
                const bool keep = Gm[m] ? (j < i) : (j <= i);
                vals[m][r] = keep ? v : 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) nd[r] = vals[0][r];
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            bf16_t *dst = (Gm[m] ? NB : Pc) + (16 * Im[m] + g4) * PC + 16 * Jm[m] + jj;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[r * PC].bits = f32_to_bf16(vals[m][r]);
        }
        // forward substitution for (I + N_JJ)^{-1}: every lane keeps column
        // `lane % 16`; the entries N[r][k] are broadcast from the lane that
        // holds them (row r = 4 g + rr sits in lane 16 g + k, register rr)
        float tcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = (r == jj) ? 1.f : 0.f;
#pragma unroll
            for (int k = 0; k < r; ++k)
                v -= __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, nd[r & 3]),
                                                                          16 * (r >> 2) + k)) * tcol[k];
            tcol[r] = v;
        }
        if (lane < 16) {
            const int base = 16 * pw;
            bf16_t *tdr = TDR + pw * 16 * 24;               // row-major T_JJ
            bf16_t *tc = TCB + pw * 16 * PC;                // this wave's T[:, J]^T
#pragma unroll
            for (int r = 0; r < 16; ++r) tdr[r * 24 + lane].bits = f32_to_bf16(tcol[r]);
#pragma unroll
            for (int r = 0; r < 16; r += 4) st4bf(tc + lane * PC + base + r, tcol[r], tcol[r + 1], tcol[r + 2], tcol[r + 3]);
        }
    };

    // D: column block J of (I + N)^{-1}, scaled by eta into Tp
    auto prep_D = [&](int c) {
        const int buf = c & 1;
        const int J = wave - 4;
        const float *eta = SC + (buf * 7 + 3) * C;
        bf16_t *tc = TCB + J * 16 * PC;     // [n][k] = T[k][16J + n]
        bf16_t *mt = MTB + J * 16 * 24;
        const int row = lane & 15, kq = 8 * (lane >> 4);
        // diagonal block: Tp_JJ = T_JJ diag(eta)
        {
            const int n = lane & 15;
            for (int r = 4 * (lane >> 4); r < 4 * (lane >> 4) + 4; ++r) {
                const float tv = bf16_to_f32(TDR[J * 16 * 24 + r * 24 + n].bits);
                TPB[(16 * J + r) * PC + 16 * J + n].bits = f32_to_bf16(tv * eta[16 * J + n]);
            }
        }
        for (int I = J + 1; I < 4; ++I) {
            // M = sum_{K=J}^{I-1} N_IK T_KJ over k in [16J, 16I)
            f32x4 M = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 16 * J; k0 < 16 * I; k0 += 32) {
                const int k = k0 + kq;
                const bool live = k < 16 * I;   // k < 64 always: the loads stay in bounds
                const bf16x8 al = ld8(NB + (16 * I + row) * PC + k);
                const bf16x8 bl = ld8(tc + row * PC + k);
                M = mfma(live ? al : zero8(), live ? bl : zero8(), M);
            }
            // M^T into scratch (B operand of the next product)
            st4bf(mt + (lane & 15) * 24 + 4 * (lane >> 4), M[0], M[1], M[2], M[3]);
            // T_IJ = -T_II M  (k = 16: lanes with kq >= 16 feed zeros)
            f32x4 Tij = {0.f, 0.f, 0.f, 0.f};
            {
                const bool live = kq < 16;
                const int kk = live ? kq : 0;   // dead lanes read a valid slot, then feed zeros
                const bf16x8 al = ld8(TDR + I * 16 * 24 + row * 24 + kk);
                const bf16x8 bl = ld8(mt + row * 24 + kk);
                Tij = mfma(live ? al : zero8(), live ? bl : zero8(), Tij);
            }
            // T_IJ^T into this wave's column buffer, Tp_IJ = T_IJ diag(eta)
            const int n = lane & 15;
            const int r0 = 16 * I + 4 * (lane >> 4);
            st4bf(tc + n * PC + r0, -Tij[0], -Tij[1], -Tij[2], -Tij[3]);
            const float en = eta[16 * J + n];
#pragma unroll
            for (int r = 0; r < 4; ++r) TPB[(r0 + r) * PC + 16 * J + n].bits = f32_to_bf16(-Tij[r] * en);
        }
    };

    // ---------------- prologue ----------------
    if (chain) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * wave + 4 * (lane >> 4) + r;
                Sacc[ct][r] = a.S_in ? a.S_in[(size_t(bh) * DK + d) * DV + j0 + 16 * ct + (lane & 15)] : 0.f;
            }
        }
    } else {
        prefetch_rows(0);
        prep_A(0);
        if (nch > 1) prefetch_rows(1);
    }
    __syncthreads();
    if (!chain) prep_B(0);
    __syncthreads();
    if (!chain) prep_C(0);
    if (chain) {
        // S^T copy for the MFMA operands: ST[j][d]
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            st4bf(ST + (16 * ct + (lane & 15)) * PK + 16 * wave + 4 * (lane >> 4), Sacc[ct][0], Sacc[ct][1],
                  Sacc[ct][2], Sacc[ct][3]);
    }
    __syncthreads();

    // ---------------- main loop ----------------
    f32x4 o1[NCT];
    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        const int t0 = c * C;
        const float *sc = SC + buf * 7 * C;
        const bf16_t *Xc = XB + size_t(buf) * C * PK;
        const bf16_t *Qc = QB + size_t(buf) * C * PK;
        if (chain) {
            // S1: X S and Qh S, residual, (w X)^T
            const int t = 16 * wave + (lane & 15);
            const float gp = sc[0 * C + t];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4 xs = tile_mm(z, ST + 16 * ct * PK, PK, Xc + 16 * wave * PK, PK, DK);
                o1[ct] = tile_mm(z, ST + 16 * ct * PK, PK, Qc + 16 * wave * PK, PK, DK);
                const int jb = 16 * ct + 4 * (lane >> 4);
                const uint2 y = *reinterpret_cast<const uint2 *>(YB + (size_t(buf) * C + t) * PY + jb);
                const float yv[4] = {__uint_as_float(y.x << 16), __uint_as_float(y.x & 0xffff0000u),
                                     __uint_as_float(y.y << 16), __uint_as_float(y.y & 0xffff0000u)};
#pragma unroll
                for (int r = 0; r < 4; ++r) R0T[(jb + r) * PC + t].bits = f32_to_bf16(yv[r] - gp * xs[r]);
            }
            // (w X)^T: thread -> token tt, 16 features
            {
                const int tt = tid >> 2, d0 = (tid & 3) * (DK / 4);
                const float wt = sc[2 * C + tt];
                for (int e = 0; e < DK / 4; ++e)
                    XHT[(d0 + e) * PC + tt].bits = f32_to_bf16(wt * bf16_to_f32(Xc[tt * PK + d0 + e].bits));
            }
        } else {
            prep_D(c);
            if (c + 1 < nch) {
                prep_A(c + 1);
                if (c + 2 < nch) prefetch_rows(c + 2);
            }
        }
        __syncthreads();  // #1
        if (chain) {
            // S2: U = Tp R0 (tokens 16w..16w+15)
            const int kend = wave < 2 ? 32 : 64;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4 u = tile_mm(z, TPB + 16 * wave * PC, PC, R0T + 16 * ct * PC, PC, kend);
                st4bf(UT + (16 * ct + (lane & 15)) * PC + 16 * wave + 4 * (lane >> 4), u[0], u[1], u[2], u[3]);
            }
        } else if (c + 1 < nch) {
            prep_B(c + 1);
        }
        __syncthreads();  // #2
        if (chain) {
            // S3a: O^T = diag(Gamma) (Qh S)^T + U^T P^T, tokens 16w..16w+15
            const int t = 16 * wave + (lane & 15);
            const float g = sc[1 * C + t];
            const int kend = wave < 2 ? 32 : 64;
            const bf16_t *Pc = PB + size_t(buf) * C * PC;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 acc = o1[ct];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= g;
                acc = tile_mm(acc, UT + 16 * ct * PC, PC, Pc + 16 * wave * PC, PC, kend);
                if (t0 + t < T) {
                    uint2 u;
                    u.x = pack2(acc[0], acc[1]);
                    u.y = pack2(acc[2], acc[3]);
                    *reinterpret_cast<uint2 *>(og + size_t(t0 + t) * DV + j0 + 16 * ct + 4 * (lane >> 4)) = u;
                }
            }
            // S3b: S = Gamma_C S + (w X)^T U, state rows 16w..16w+15
            const float gC = sc[6 * C];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Sacc[ct][r] *= gC;
                Sacc[ct] = tile_mm(Sacc[ct], XHT + 16 * wave * PC, PC, UT + 16 * ct * PC, PC, C);
                st4bf(ST + (16 * ct + (lane & 15)) * PK + 16 * wave + 4 * (lane >> 4), Sacc[ct][0], Sacc[ct][1],
                      Sacc[ct][2], Sacc[ct][3]);
            }
        } else if (c + 1 < nch) {
            prep_C(c + 1);
        }
        __syncthreads();  // #3
    }

    // ---------------- epilogue: boundary state ----------------
    if (chain && a.S_out) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * wave + 4 * (lane >> 4) + r;
                a.S_out[(size_t(bh) * DK + d) * DV + j0 + 16 * ct + (lane & 15)] = Sacc[ct][r];
            }
    }
    if (wave == 4 && s == 0 && a.xnext_out && T > 0) {
        float xv[DK / 64 > 0 ? DK / 64 : 1];
        float ss = 0.f;
#pragma unroll
        for (int m = 0; m < DK / 64; ++m) {
            xv[m] = bf16_to_f32(kg[size_t(T - 1) * DK + lane + 64 * m].bits);
            ss += xv[m] * xv[m];
        }
        ss = wave_sum(ss);
        const float scl = phi_scale(ss, DK, a.eps_rms, a.phi);
#pragma unroll
        for (int m = 0; m < DK / 64; ++m) a.xnext_out[size_t(bh) * DK + lane + 64 * m] = xv[m] * scl;
    }
}

template <int DK, int DS>
void launch_fused_t(const F1FusedArgs &a, hipStream_t s, Marks *m) {
    const int nslice = a.dv / DS;
    const int blocks = nslice == 1 ? a.BH : ((a.BH + 7) / 8) * 8 * nslice;
    chunk_f1_fused<DK, DS><<<blocks, 512, 0, s>>>(a, nslice);
    m->mark(s);
}

}  // namespace

void launch_chunk_f1_fused(const F1FusedArgs &a, int ds, hipStream_t s, Marks *m) {
    if (ds == 64) launch_fused_t<64, 64>(a, s, m);
    else launch_fused_t<64, 32>(a, s, m);
}

}  // namespace falcon
