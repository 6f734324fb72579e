// Chunk-parallel Falcon-1 forward for bf16 inputs, d_k = 64, in two kernels
// (summary Figure 4, §D.1, App. E.2: parallel per-chunk operators, a short
// sequential carry, parallel output).  With the chunk-local log-prefix b
// (restarted at 0 in every chunk) and the chunk-entry state S_0:
//     U   = Tp (Y - diag(e^{b_{i-1}}) X S_0),   Tp = (I + N)^{-1} diag(eta),
//     N_ij = eta_i e^{b_{i-1}-b_j} x_i.x_j (j < i),
//     O   = diag(e^{b_i}) Qh S_0 + P U,          P_ij = e^{b_i-b_j} qh_i.x_j (j <= i),
//     S_C = e^{b_C} S_0 + (diag(e^{b_C-b_i}) X)^T U.
//
// f1_ops: one workgroup per chunk, every chunk of every head in parallel.
//   QK-RMSNorm and the key shift, eta and log gamma, the chunk-local prefix
//   (and its suffix, so e^{b_C - b_i} is formed from a short sum), Gram and
//   scores on MFMA, the fp32 inverse of the unit-lower system (diagonal
//   blocks by substitution, the others on fp32 MFMA), and the operators Tp,
//   P and (diag(e^{b_C-b_t}) X)^T (bf16) plus the decay rows into the
//   workspace.
// f1_walk: one workgroup per (head, slice of DS value columns) walks the
//   chunks in order.  Chain wave w owns state columns 16w..16w+15 (all d_k
//   rows in MFMA accumulators) and needs no other chain wave inside a chunk:
//     XS -> R0 -> U = Tp R0 -> S' = Gamma_C S + (w X)^T U   (MFMA);
//   output wave w writes the previous chunk's O = Gamma Qh S + P U from the
//   state and writes that chunk started with.
//   Four loader waves stage the next chunk meanwhile: raw q, k, v rows and
//   the chunk operators prefetched a chunk ahead, QK-RMSNorm, all into the
//   other LDS buffer.  One workgroup barrier per chunk.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;
constexpr int kLs = C + 1;    // fp32 LDS row stride
constexpr int PC = C + 8;     // bf16 stride of [.][token] rows

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack2(a, b), pack2(c, d));
}
__device__ __forceinline__ void unpack8(const uint4 &u, float *f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint4 pack8(const float *f) {
    return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}
__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const bf16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// features of one row part: TPR threads per row, EPT elements each
template <int DK, int TPR = 4>
struct RowPart {
    static constexpr int EPT = DK / TPR, NV = EPT / 8;
    uint4 q[NV], k[NV];
    // Loads are unconditional, from rows clamped into [0, T) (T >= 1 here):
    // a load under a branch would be waited for where the branch joins.
    // Rows outside the sequence are zeroed when the features are formed.
    __device__ void load(const bf16_t *qg, const bf16_t *kg, int t, int T, int part) {
        const int tq = t < T ? t : T - 1;
        const int tk = t < 1 ? 0 : (t - 1 < T ? t - 1 : T - 1);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            q[v] = *reinterpret_cast<const uint4 *>(qg + size_t(tq) * DK + part * EPT + 8 * v);
            k[v] = *reinterpret_cast<const uint4 *>(kg + size_t(tk) * DK + part * EPT + 8 * v);
        }
    }
    // normalised features; returns ||x||^2 of the whole row
    __device__ float features(float *xv, float *qv, int t, int part, const F1SplitArgs &a, int bh) const {
        const bool qok = t < a.T, kok = t >= 1 && t - 1 < a.T;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            unpack8(q[v], qv + 8 * v);
            unpack8(k[v], xv + 8 * v);
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            qv[e] = qok ? qv[e] : 0.f;
            xv[e] = kok ? xv[e] : 0.f;
        }
        const bool first = (t == 0);   // x_0 comes from the boundary state
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
        return group_sum<TPR>(n2);
    }
};

// ---------------------------------------------------------------------------
// f1_ops: per-chunk operators
// ---------------------------------------------------------------------------
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DK>
__global__ __launch_bounds__(256) void f1_ops(F1SplitArgs a) {
    constexpr int PK = DK + 8;
    using RP = RowPart<DK>;
    // LDS: the system N stays; the feature / score staging area is reused
    // for the inverse once the features are no longer needed
    __shared__ float Nm[C * kLs];
    __shared__ __align__(16) unsigned char pool[3 * C * PK * 2 > C * kLs * 4 ? 3 * C * PK * 2 : C * kLs * 4];
    __shared__ float Mw[4][16 * 17];          // per wave: M blocks of the inverse
    __shared__ float eta_s[C], lg_s[C], b_s[C], bp_s[C], ew_s[C];
    bf16_t *XB = reinterpret_cast<bf16_t *>(pool);
    bf16_t *QB = XB + C * PK;
    bf16_t *PS = QB + C * PK;                 // stride PC <= PK
    float *Tm = reinterpret_cast<float *>(pool);

    const int c = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.T;
    const int row = tid >> 2, part = tid & 3;
    const int t = c * C + row;
    const int col = lane & 15, g4 = 4 * (lane >> 4), kq = lane >> 4;
    const bf16_t *qg = static_cast<const bf16_t *>(a.q) + size_t(bh) * T * DK;
    const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * DK;
    char *ops = static_cast<char *>(a.ops) + (size_t(bh) * a.nchunks + c) * kF1SplitChunkBytes;
    bf16_t *Tp = reinterpret_cast<bf16_t *>(ops);
    bf16_t *Pg = reinterpret_cast<bf16_t *>(ops + kF1SplitPOff);
    bf16_t *Xw = reinterpret_cast<bf16_t *>(ops + kF1SplitXwOff);
    float *scal = reinterpret_cast<float *>(ops + kF1SplitScalOff);

    // 1. features and step scalars (log gamma in base 2)
    {
        RP rp;
        rp.load(qg, kg, t, T, part);
        const int tc = t < T ? t : T - 1;
        const float beta = a.beta[size_t(bh) * T + tc];   // unused when t >= T
        const float lam = a.lambda[size_t(bh) * T + tc];
        float xv[RP::EPT], qv[RP::EPT];
        const float n2 = rp.features(xv, qv, t, part, a, bh);
#pragma unroll
        for (int v = 0; v < RP::NV; ++v) {
            *reinterpret_cast<uint4 *>(XB + row * PK + part * RP::EPT + 8 * v) = pack8(xv + 8 * v);
            *reinterpret_cast<uint4 *>(QB + row * PK + part * RP::EPT + 8 * v) = pack8(qv + 8 * v);
        }
        if (part == 0) {
            float eta = 0.f, alpha = 0.f;
            const bool noop = t >= T || (t == 0 && a.fresh);
            if (!noop) {
                eta = step_eta(beta, n2 + lam + a.eps);
                alpha = step_alpha(eta, lam, a.eps_gamma);
            }
            eta_s[row] = eta;
            lg_s[row] = log1pf(-alpha) * kLog2e;
        }
    }
    __syncthreads();

    // 2. chunk-local prefix (base 2) and its suffix, so that e^{b_C - b_i}
    //    comes from a short sum (wave 0, lane = token)
    if (wave == 0) {
        const float lg = lg_s[lane];
        const float b = wave_inclusive_scan(lg);
        float bp = __shfl_up(b, 1, 64);
        if (lane == 0) bp = 0.f;
        float sf = lg;   // inclusive suffix
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_down(sf, o, 64);
            if (lane + o < 64) sf += y;
        }
        float sfx = __shfl_down(sf, 1, 64);
        if (lane == 63) sfx = 0.f;
        const float bC = __shfl(b, 63, 64);
        b_s[lane] = b;
        bp_s[lane] = bp;
        const float ew = exp2_(sfx);
        ew_s[lane] = ew;
        scal[0 * C + lane] = exp2_(bp);
        scal[1 * C + lane] = exp2_(b);
        scal[2 * C + lane] = ew;
        scal[3 * C + lane] = lane == 0 ? exp2_(bC) : 0.f;
    }
    __syncthreads();

    // 3. Gram and score tiles (lower 16x16 tiles) with decays and masks;
    //    wave w takes jobs w, w+4, ..., tiles 0-9 Gram, 10-19 scores, tile
    //    index -> (I, J) from two packed 2-bit tables
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        const int job = wave + 4 * m;
        const bool isG = job < 10;
        const int tt = isG ? job : job - 10;
        const int I = (0xffa94 >> (2 * tt)) & 3, J = (0xe4910 >> (2 * tt)) & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32)
            acc = mfma(ld8((isG ? XB : QB) + (16 * I + col) * PK + k0 + 2 * g4), ld8(XB + (16 * J + col) * PK + k0 + 2 * g4), acc);
        const int j = 16 * J + col;
        const float bj = b_s[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + g4 + r;
            if (isG) Nm[i * kLs + j] = j < i ? eta_s[i] * exp2_(bp_s[i] - bj) * acc[r] : 0.f;
            else st(PS, size_t(i) * PC + j, j <= i ? exp2_(b_s[i] - bj) * acc[r] : 0.f);
        }
    }
    __syncthreads();

    // 4. scores and the scaled transposed keys to the workspace; diagonal
    //    blocks of the inverse by forward substitution (wave J: block J,
    //    lane k < 16: column k), kept in registers until the staging area
    //    is free
    {
        // P row part (columns 16 part ..): zero above the diagonal tiles
        const uint4 *sp = reinterpret_cast<const uint4 *>(PS + row * PC + part * 16);
        uint4 *dp = reinterpret_cast<uint4 *>(Pg + row * C + part * 16);
        const bool live = part <= (row >> 4);
        dp[0] = live ? sp[0] : make_uint4(0, 0, 0, 0);
        dp[1] = live ? sp[1] : make_uint4(0, 0, 0, 0);
        // Xw[d][t] for d = row, t = 16 part .. + 15
        float xw[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int tt = part * 16 + e;
            xw[e] = ew_s[tt] * bf16_to_f32(XB[tt * PK + row].bits);
        }
        uint4 *dx = reinterpret_cast<uint4 *>(Xw + row * C + part * 16);
        dx[0] = pack8(xw);
        dx[1] = pack8(xw + 8);
    }
    float tcol[16];
    {
        const int base = 16 * wave;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = (r == col) ? 1.f : 0.f;
#pragma unroll
            for (int k = 0; k < r; ++k) v -= Nm[(base + r) * kLs + base + k] * tcol[k];
            tcol[r] = v;
        }
    }
    __syncthreads();
    if (lane < 16) {
        const int base = 16 * wave;
#pragma unroll
        for (int r = 0; r < 16; ++r) Tm[(base + r) * kLs + base + col] = tcol[r];
    }
    __syncthreads();

    // 5. off-diagonal blocks by recursive doubling on the 2 x 2 split into
    //    32-blocks, [[A, 0], [C, D]]^{-1} = [[A^-1, 0], [-D^-1 C A^-1, D^-1]]
    //    (fp32 MFMA on 16x16 blocks; B(I, J) is block row I, column J):
    //    level 1: T10 = -T11 N10 T00, T32 = -T33 N32 T22 (waves 0, 1);
    //    level 2: X = C A^-1 (one block per wave), then -D^-1 X.
    {
        auto blk = [&](const float *A, const float *B, f32x4 acc) {   // acc += A B (16x16 each)
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 4)
                acc = mfma_f32(A[col * kLs + k0 + kq], B[(k0 + kq) * kLs + col], acc);
            return acc;
        };
        auto at = [&](float *M, int I, int J) { return M + 16 * I * kLs + 16 * J; };
        float *mw = Mw[wave];
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        if (wave < 2) {
            const int a0 = 2 * wave;   // blocks (a0 + 1, a0)
            const f32x4 M = blk(at(Nm, a0 + 1, a0), at(Tm, a0, a0), z);
#pragma unroll
            for (int r = 0; r < 4; ++r) mw[(g4 + r) * 17 + col] = M[r];
            wave_lds_sync();
            f32x4 Tb = z;
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 4)
                Tb = mfma_f32(at(Tm, a0 + 1, a0 + 1)[col * kLs + k0 + kq], mw[(k0 + kq) * 17 + col], Tb);
#pragma unroll
            for (int r = 0; r < 4; ++r) at(Tm, a0 + 1, a0)[(g4 + r) * kLs + col] = -Tb[r];
        }
        __syncthreads();
        // X(I, J) for I in {2, 3}, J in {0, 1}: N_I0 T_0J + N_I1 T_1J (T_01 = 0)
        {
            const int I = 2 + (wave >> 1), J = wave & 1;
            f32x4 X = blk(at(Nm, I, 1), at(Tm, 1, J), z);
            if (J == 0) X = blk(at(Nm, I, 0), at(Tm, 0, 0), X);
#pragma unroll
            for (int r = 0; r < 4; ++r) mw[(g4 + r) * 17 + col] = X[r];
        }
        __syncthreads();
        // T(I, J) = -(sum_{K=2}^{I} T_IK X(K, J)) for I in {2, 3}, J in {0, 1}
        {
            const int I = 2 + (wave >> 1), J = wave & 1;
            f32x4 Tb = z;
#pragma unroll
            for (int K = 2; K <= 3; ++K) {
                if (K > I) break;
                const float *Xk = Mw[2 * (K - 2) + J];
                const float *Tk = at(Tm, I, K);
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4)
                    Tb = mfma_f32(Tk[col * kLs + k0 + kq], Xk[(k0 + kq) * 17 + col], Tb);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) at(Tm, I, J)[(g4 + r) * kLs + col] = -Tb[r];
        }
    }
    __syncthreads();

    // 6. Tp = L^{-1} diag(eta) to the workspace (row part of 16)
    {
        float tv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = part * 16 + e;
            tv[e] = j <= row ? Tm[row * kLs + j] * eta_s[j] : 0.f;
        }
        uint4 *dt = reinterpret_cast<uint4 *>(Tp + row * C + part * 16);
        dt[0] = pack8(tv);
        dt[1] = pack8(tv + 8);
    }
}

// ---------------------------------------------------------------------------
// f1_walk: sequential walk over the chunks of one (head, DS-column slice)
// ---------------------------------------------------------------------------
template <int DK, int DS, int NLW>
__global__ __launch_bounds__((2 * (DS / 16) + NLW) * 64) void f1_walk(F1SplitArgs a, int nslice) {
    constexpr int NCW = DS / 16;          // chain waves (= output waves)
    constexpr int NLT = 64 * NLW;         // loader threads
    constexpr int PK = DK + 8;
    constexpr int YP = DS / 8;            // 16-byte pieces of a value row
    using RP = RowPart<DK, NLW>;          // NLW threads per feature row
    static_assert(DK == 64 && (NLW == 4 || NLW == 8), "loaders: 64 rows x NLW parts of the features");
    static_assert(DS == 32, "slice of 32 value columns");
    static_assert(64 * YP <= NLT && 512 % NLT == 0, "one value piece per thread; whole tiles");
    constexpr int TPT = 512 / NLT;        // 16-byte tile pieces per loader thread

    // chunk c uses buffers c % 2 (chain operands) and c % 3 (operands the
    // output waves read one chunk later)
    __shared__ __align__(16) bf16_t XB[2][C * PK];     // x rows [t][d]
    __shared__ __align__(16) bf16_t XWT[2][DK * PC];   // (e^{b_C-b_t} x_t)^T [d][t]
    __shared__ __align__(16) bf16_t YT[2][DS * PC];    // values^T [j][t]
    __shared__ __align__(16) bf16_t TPB[2][C * PC];    // Tp [t][s]
    __shared__ __align__(16) bf16_t QB[3][C * PK];     // qh rows [t][d]
    __shared__ __align__(16) bf16_t PB[3][C * PC];     // P [t][s]
    __shared__ float SC[3][4 * C];                     // decay rows
    __shared__ __align__(16) bf16_t STw[NCW][3][16 * PK];  // per column tile: S^T [j][d] at chunk start
    __shared__ __align__(16) bf16_t RTw[NCW][16 * PC];     // per column tile: R0^T [j][t]
    __shared__ __align__(16) bf16_t UTw[NCW][2][16 * PC];  // per column tile: U^T [j][t]

    int bh, s;
    if (nslice == 1) {
        bh = blockIdx.x;
        s = 0;
    } else {
        const int id = blockIdx.x, u = id & 7, rest = id >> 3;
        s = rest % nslice;
        bh = (rest / nslice) * 8 + u;
    }
    if (bh >= a.BH) return;   // the whole workgroup leaves together
    const int j0 = s * DS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = wave < NCW;
    const bool outw = wave >= NCW && wave < 2 * NCW;
    const bool loader = wave >= 2 * NCW;
    const int T = a.T, DV = a.dv, nch = a.nchunks;
    const bf16_t *qg = static_cast<const bf16_t *>(a.q) + size_t(bh) * T * DK;
    const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * DK;
    const bf16_t *vg = static_cast<const bf16_t *>(a.v) + size_t(bh) * T * DV;
    bf16_t *og = static_cast<bf16_t *>(a.o) + size_t(bh) * T * DV;
    const char *opsb = static_cast<const char *>(a.ops) + size_t(bh) * nch * kF1SplitChunkBytes;

    // ---- loaders: rows and operators of the next chunk, prefetched ----
    const int lt = tid - 2 * NCW * 64;    // loader thread index (valid for loaders)
    const int lrow = lt / NLW, lpart = lt % NLW;
    const int yrow = (lt / YP) % C, ypc = lt % YP;   // value piece of this thread (stored if lt < 64 YP)
    // two sets of prefetch registers: the rows of a chunk are loaded two
    // iterations before they are staged (the walk is short per chunk, a
    // global load round trip is not)
    struct Regs {
        RP rp;
        uint4 ry;
        uint4 rtp[TPT], rpp[TPT], rxw[TPT];
        float rsc;
    };
    Regs ra, rb;
    auto prefetch = [&](int c, Regs &R) {
        const int t = c * C + lrow;
        R.rp.load(qg, kg, t, T, lpart);
        const int ty = c * C + yrow;   // clamped row; zeroed at staging when ty >= T
        // every loader thread loads (a load under a branch would be waited for
        // at the join); threads past the value pieces re-read a valid piece
        R.ry = *reinterpret_cast<const uint4 *>(vg + size_t(ty < T ? ty : T - 1) * DV + j0 + 8 * ypc);
        const char *ops = opsb + size_t(c) * kF1SplitChunkBytes;
        const uint4 *tp = reinterpret_cast<const uint4 *>(ops);
        const uint4 *pp = reinterpret_cast<const uint4 *>(ops + kF1SplitPOff);
        const uint4 *xp = reinterpret_cast<const uint4 *>(ops + kF1SplitXwOff);
#pragma unroll
        for (int h = 0; h < TPT; ++h) {
            R.rtp[h] = tp[lt + NLT * h];
            R.rpp[h] = pp[lt + NLT * h];
            R.rxw[h] = xp[lt + NLT * h];
        }
        R.rsc = reinterpret_cast<const float *>(ops + kF1SplitScalOff)[lt % (4 * C)];
    };
    auto stage = [&](int c, const Regs &R) {   // prefetched rows of chunk c -> LDS buffers
        const int b2 = c & 1, b3 = c % 3;
        const int t = c * C + lrow;
        float xv[RP::EPT], qv[RP::EPT];
        (void)R.rp.features(xv, qv, t, lpart, a, bh);
#pragma unroll
        for (int v = 0; v < RP::NV; ++v) {
            *reinterpret_cast<uint4 *>(XB[b2] + lrow * PK + lpart * RP::EPT + 8 * v) = pack8(xv + 8 * v);
            *reinterpret_cast<uint4 *>(QB[b3] + lrow * PK + lpart * RP::EPT + 8 * v) = pack8(qv + 8 * v);
        }
        if (lt < 64 * YP) {   // values transposed: 8 columns of row yrow
            float yv[8];
            unpack8(R.ry, yv);
            const bool ok = c * C + yrow < T;
#pragma unroll
            for (int e = 0; e < 8; ++e) st(YT[b2], size_t(8 * ypc + e) * PC + yrow, ok ? yv[e] : 0.f);
        }
#pragma unroll
        for (int h = 0; h < TPT; ++h) {
            // 16-byte piece u of a 64 x 64 tile: row u / 8, columns 8 (u % 8) ..
            const int u = lt + NLT * h, r = u >> 3, c8 = 8 * (u & 7);
            *reinterpret_cast<uint4 *>(TPB[b2] + r * PC + c8) = R.rtp[h];
            *reinterpret_cast<uint4 *>(PB[b3] + r * PC + c8) = R.rpp[h];
            *reinterpret_cast<uint4 *>(XWT[b2] + r * PC + c8) = R.rxw[h];
        }
        if (lt < 4 * C) SC[b3][lt] = R.rsc;
    };

    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4);
    const int ct = chain ? wave : (outw ? wave - NCW : 0);   // column tile of a chain / output wave
    // ---- chain state: S[:, j0 + 16 ct ..] in accumulators (d tiles m) ----
    f32x4 S[DK / 16];
    if (chain) {
#pragma unroll
        for (int m = 0; m < DK / 16; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * m + g4 + r;
                S[m][r] = a.S_in ? a.S_in[(size_t(bh) * DK + d) * DV + j0 + 16 * ct + col] : 0.f;
            }
            *reinterpret_cast<uint2 *>(STw[ct][0] + col * PK + 16 * m + g4) = pack4(S[m][0], S[m][1], S[m][2], S[m][3]);
        }
    } else if (loader) {
        prefetch(0, ra);
        stage(0, ra);
        if (nch > 1) prefetch(1, rb);
        if (nch > 2) prefetch(2, ra);
    }
    __syncthreads();

    // iteration c: chain waves advance the state through chunk c, output
    // waves write the outputs of chunk c - 1, loaders stage chunk c + 1 (its
    // rows are in the register set (c + 1) % 2) and refill that set with
    // chunk c + 3
    auto iteration = [&](int c, Regs &R) {
        if (chain && c < nch) {
            const int b2 = c & 1, b3 = c % 3;
            const bf16_t *X = XB[b2], *Tp = TPB[b2];
            const bf16_t *Y = YT[b2] + (16 * ct + col) * PC;
            const float *sc = SC[b3];
            const bf16_t *st_w = STw[ct][b3];
            bf16_t *rt_w = RTw[ct];
            bf16_t *ut_w = UTw[ct][b2];
            bf16x8 sb[DK / 32];   // S^T operand (rows j, k = d)
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) sb[kk] = ld8(st_w + col * PK + 32 * kk + k8);
            // R0 = Y - Gamma_{t-1} XS (token tile m)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 xs = {0.f, 0.f, 0.f, 0.f};
                const int row = 16 * m + col;
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) xs = mfma(ld8(X + row * PK + 32 * kk + k8), sb[kk], xs);
                const uint2 yy = *reinterpret_cast<const uint2 *>(Y + 16 * m + g4);   // 4 tokens
                const float y[4] = {__uint_as_float(yy.x << 16), __uint_as_float(yy.x & 0xffff0000u),
                                    __uint_as_float(yy.y << 16), __uint_as_float(yy.y & 0xffff0000u)};
                float r0[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) r0[r] = y[r] - sc[16 * m + g4 + r] * xs[r];
                *reinterpret_cast<uint2 *>(rt_w + col * PC + 16 * m + g4) = pack4(r0[0], r0[1], r0[2], r0[3]);
            }
            wave_lds_sync();
            // U = Tp R0 (lower triangular: token tile m needs s < 16m + 16)
            {
                const bf16x8 rb0 = ld8(rt_w + col * PC + k8), rb1 = ld8(rt_w + col * PC + 32 + k8);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int row = 16 * m + col;
                    f32x4 u = {0.f, 0.f, 0.f, 0.f};
                    u = mfma(ld8(Tp + row * PC + k8), rb0, u);
                    if (m >= 2) u = mfma(ld8(Tp + row * PC + 32 + k8), rb1, u);
                    *reinterpret_cast<uint2 *>(ut_w + col * PC + 16 * m + g4) = pack4(u[0], u[1], u[2], u[3]);
                }
            }
            wave_lds_sync();
            // S = Gamma_C S + (diag(e^{b_C-b_t}) X)^T U  -> S^T copy of chunk c + 1
            const bf16x8 ub0 = ld8(ut_w + col * PC + k8), ub1 = ld8(ut_w + col * PC + 32 + k8);
            const float gC = sc[3 * C];
            const bf16_t *XW = XWT[b2];
            bf16_t *st_n = STw[ct][(c + 1) % 3];
#pragma unroll
            for (int m = 0; m < DK / 16; ++m) {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[m][r] *= gC;
                S[m] = mfma(ld8(XW + (16 * m + col) * PC + k8), ub0, S[m]);
                S[m] = mfma(ld8(XW + (16 * m + col) * PC + 32 + k8), ub1, S[m]);
                *reinterpret_cast<uint2 *>(st_n + col * PK + 16 * m + g4) = pack4(S[m][0], S[m][1], S[m][2], S[m][3]);
            }
        } else if (outw && c >= 1) {
            // outputs of chunk k = c - 1: O^T = diag(Gamma_t) (Qh S_k)^T + U^T P^T
            const int k = c - 1, b2 = k & 1, b3 = k % 3;
            const bf16_t *Q = QB[b3], *P = PB[b3];
            const float *sc = SC[b3];
            const bf16_t *st_w = STw[ct][b3];
            const bf16_t *ut_w = UTw[ct][b2];
            bf16x8 sb[DK / 32];
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) sb[kk] = ld8(st_w + col * PK + 32 * kk + k8);
            const bf16x8 ub0 = ld8(ut_w + col * PC + k8), ub1 = ld8(ut_w + col * PC + 32 + k8);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int t = 16 * m + col;
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) o = mfma(sb[kk], ld8(Q + t * PK + 32 * kk + k8), o);
                const float gt = sc[C + t];
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] *= gt;
                o = mfma(ub0, ld8(P + t * PC + k8), o);
                if (m >= 2) o = mfma(ub1, ld8(P + t * PC + 32 + k8), o);
                const int tg = k * C + t;
                if (tg < T)
                    *reinterpret_cast<uint2 *>(og + size_t(tg) * DV + j0 + 16 * ct + g4) = pack4(o[0], o[1], o[2], o[3]);
            }
        } else if (loader && c + 1 < nch) {
            stage(c + 1, R);
            if (c + 3 < nch) prefetch(c + 3, R);
        }
        __syncthreads();
    };
    for (int c = 0; c <= nch; c += 2) {   // unrolled by two: register sets by name
        iteration(c, rb);
        if (c + 1 <= nch) iteration(c + 1, ra);
    }

    // ---- boundary state ----
    if (chain && a.S_out) {
#pragma unroll
        for (int m = 0; m < DK / 16; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a.S_out[(size_t(bh) * DK + 16 * m + g4 + r) * DV + j0 + 16 * ct + col] = S[m][r];
    }
    if (wave == 2 * NCW && s == 0 && a.xnext_out && T > 0) {
        const float xv = bf16_to_f32(kg[size_t(T - 1) * DK + lane].bits);
        const float sc = phi_scale(wave_sum(xv * xv), DK, a.eps_rms, a.phi);
        a.xnext_out[size_t(bh) * DK + lane] = xv * sc;
    }
}

template <int DS>
void launch_walk(const F1SplitArgs &a, hipStream_t s, Marks *m) {
    constexpr int NLW = 8;   // loader waves
    const int nslice = a.dv / DS;
    const int blocks = nslice == 1 ? a.BH : ((a.BH + 7) / 8) * 8 * nslice;
    f1_walk<64, DS, NLW><<<blocks, (2 * (DS / 16) + NLW) * 64, 0, s>>>(a, nslice);
    m->mark(s);
}

}  // namespace

void launch_chunk_f1_split(const F1SplitArgs &a, int ds, hipStream_t s, Marks *m) {
    f1_ops<64><<<dim3(a.nchunks, a.BH), 256, 0, s>>>(a);
    m->mark(s);
    (void)ds;   // always 32 value columns per walk workgroup
    launch_walk<32>(a, s, m);
}

}  // namespace falcon
