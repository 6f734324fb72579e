// Chunk-parallel Falcon-1 forward for bf16 inputs, d_k = 64, through per-chunk
// transfer operators (summary Figure 4, §D.1, App. E.2: parallel per-chunk
// work, then a short sequential carry of the state between chunks).
//
// With the chunk-local log-prefix b (restarted at 0 in every chunk), the
// unit-lower system N_ij = eta_i e^{b_{i-1}-b_j} x_i.x_j (j < i),
// Tp = (I + N)^{-1} diag(eta), W = Tp diag(e^{b_{i-1}}) X, Ut = Tp Y and
// Xw = diag(e^{b_C-b_i}) X, the chunk update from the entry state S_0,
//     U = Ut - W S_0,  O = diag(e^{b_i}) Qh S_0 + P U,  S_C = e^{b_C} S_0 + Xw^T U,
// regroups into four operators that do not depend on S_0:
//     A = -Xw^T W  [d_k x d_k],   G = diag(e^{b_i}) Qh - P W  [C x d_k],
//     B =  Xw^T Ut [d_k x d_v],   H = P Ut                    [C x d_v],
// so that  S_C = e^{b_C} S_0 + A S_0 + B  and  O = G S_0 + H.
//
// f1_xfer: one chunk per workgroup at a time, all chunks of all heads in
//   parallel (persistent workgroups; the next chunk's rows load meanwhile):
//   QK-RMSNorm and the key shift, eta and log2 gamma, the prefix scan, Gram
//   and scores on MFMA, then Z = (I + N)^{-1} [-diag(eta e^{b_{i-1}}) X |
//   diag(eta) Y] = [-W | Ut] by forward substitution over 16-row blocks
//   (diagonal blocks inverted in fp32, the block steps on bf16 MFMA, kept in
//   registers), and the four operator products on MFMA; A, G, B^T and H go
//   to the workspace in bf16 with e^{b_C}.
// f1_carry: one workgroup per (head, slice of value columns) walks the
//   chunks: per chunk each compute wave owns 16 state columns (fp32 MFMA
//   accumulators) and issues 8 MFMAs for the carry and 8 for the outputs,
//   all from one bf16 copy of the entry state.  Loader waves copy the
//   operators of later chunks straight from memory into a ring of LDS slots
//   (global_load_lds), so no register staging sits between memory and the
//   matrix cores.  One workgroup barrier per chunk.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;
constexpr int DK = 64;
constexpr int PK = 72;          // bf16 pitch of LDS rows of 64 elements (144 bytes)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats -> bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint2 pk4(const f32x4 &v) { return make_uint2(pk2(v[0], v[1]), pk2(v[2], v[3])); }
__device__ __forceinline__ uint16_t bf(float v) { return uint16_t(pk2(v, 0.f)); }
__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ f32x4 unpk4(const uint2 &u) { return f32x4{lo16(u.x), hi16(u.x), lo16(u.y), hi16(u.y)}; }
__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <class P>
__device__ __forceinline__ bf16x8 ld8(const P *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ void put2(void *p, const uint2 &v) { *reinterpret_cast<uint2 *>(p) = v; }
// memory -> LDS copies (global_load_lds): lane i's 16 (4) bytes from `src`
// land at dst + 16 i (4 i); dst is the same for the whole wave.  Plain
// functions: inside a kernel template the builtin keeps the host pass from
// emitting the launch stub.
__device__ __forceinline__ void lds_copy16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// phi's RMS scale 1 / sqrt(mean(z^2) + eps_rms) (0 when that is 0) from the
// sum of squares over d_k = 64 elements, by the hardware reciprocal square
// root: the features are rounded to bf16 next
__device__ __forceinline__ float rms_scale(float ss, float eps_rms, int phi_kind) {
    if (phi_kind == FALCON_PHI_IDENTITY) return 1.f;
    const float ms = ss * (1.f / DK) + eps_rms;
    return ms > 0.f ? __builtin_amdgcn_rsqf(ms) : 0.f;
}

// per-token scalars of a chunk in LDS
enum { kEta = 0, kB, kBp, kEw, kRs, kQs, kCs, kLg, kNsv };

// ---------------------------------------------------------------------------
// f1_xfer: the transfer operators of one chunk
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(const s16x4 &a, const s16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 as_s4(const uint2 &u) { return __builtin_bit_cast(s16x4, u); }

constexpr int NBP = 20;         // bf16 pitch of the 16 x 16 solve blocks

// The raw rows of one chunk (16 q and 16 k elements and d_v / 4 values of
// row `row`, part `part`, and the row's beta and lambda), loaded into
// registers one chunk ahead.  Loads are unconditional from rows clamped into
// [0, T): a load under a branch would be waited for where the branch joins.
template <int DV>
struct XferRows {
    uint4 q0, q1, k0, k1, v[DV / 32];
    float beta, lam;
    __device__ __forceinline__ void load(const F1SplitArgs &a, int id, int row, int part) {
        const int c = id / a.BH, bh = id % a.BH, T = a.T, t = c * kChunk + row;
        const int tq = t < T ? t : T - 1;
        const int tk = t < 1 ? 0 : (t - 1 < T ? t - 1 : T - 1);
        const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.q) +
                                                          (size_t(bh) * T + tq) * DK + 16 * part);
        const uint4 *kp = reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.k) +
                                                          (size_t(bh) * T + tk) * DK + 16 * part);
        const uint4 *vp = reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.v) +
                                                          (size_t(bh) * T + tq) * DV + (DV / 4) * part);
        q0 = qp[0];
        q1 = qp[1];
        k0 = kp[0];
        k1 = kp[1];
#pragma unroll
        for (int i = 0; i < DV / 32; ++i) v[i] = vp[i];
        beta = a.beta[size_t(bh) * T + tq];
        lam = a.lambda[size_t(bh) * T + tq];
    }
};

template <int DV>
__global__ __launch_bounds__(256) void f1_xfer(F1SplitArgs a) {
    constexpr int VPT = DV / 4;               // value elements per thread (row part)
    constexpr int NJ = DV / 16;               // value column tiles
    constexpr int NT = 4 + NJ;                // column tiles of R = [x part | value part]
    constexpr int U1 = (DK + DV) * PK > C * PK ? (DK + DV) * PK : C * PK;
    __shared__ __align__(16) bf16_t QB[C * PK];     // qh rows [t][d]
    __shared__ __align__(16) bf16_t XT[DK * PK];    // x^T [d][t]
    __shared__ __align__(16) bf16_t XW[DK * PK];    // (diag(e^{b_C-b_t}) x)^T [d][t]
    __shared__ __align__(16) bf16_t YT[DV * PK];    // values^T [j][t]
    __shared__ __align__(16) bf16_t PB[C * PK];     // P [t][s]
    __shared__ __align__(16) bf16_t U1B[U1];        // x rows [t][d], then Z^T [n][t]
    __shared__ __align__(16) bf16_t NB[6][16 * NBP];   // -N below the diagonal blocks
    __shared__ __align__(16) bf16_t DB[4][16 * NBP];   // inverses of the diagonal blocks of I + N
    __shared__ float Nd[4][16 * 17];                   // diagonal blocks of N (fp32)
    __shared__ __align__(16) float sv[kNsv][C];

    const int nch = a.nchunks, total = nch * a.BH;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4), kq = lane >> 4;
    const int T = a.T;
    const int row = tid >> 2, part = tid & 3;
    bf16_t *XB = U1B;
    bf16_t *ZT = U1B;
    uint16_t *XT16 = reinterpret_cast<uint16_t *>(XT);
    uint16_t *YT16 = reinterpret_cast<uint16_t *>(YT);

    // persistent: chunk ids blockIdx.x, + gridDim.x, ...; the rows of the
    // next chunk are loaded while this one is worked on
    XferRows<DV> rows;
    rows.load(a, blockIdx.x, row, part);
    for (int id = blockIdx.x; id < total; id += gridDim.x) {
    const int c = id / a.BH, bh = id % a.BH;   // chunk-major: with 8 | BH a head stays on one XCD
    const int t = c * C + row;
    char *rec = static_cast<char *>(a.ops) + (size_t(bh) * nch + c) * f1_xfer_bytes(DV);

    // 1. rows: qh, x = phi(k_{t-1}) (x_0 from the boundary), values; eta and
    //    log2 gamma.  Rows past the end are zeroed here.
    {
        const uint4 qr0 = rows.q0, qr1 = rows.q1, kr0 = rows.k0, kr1 = rows.k1;
        uint4 vr[VPT / 8];
#pragma unroll
        for (int i = 0; i < VPT / 8; ++i) vr[i] = rows.v[i];
        const float beta = rows.beta, lam = rows.lam;
        {   // the next chunk's rows (the last chunk reloads its own)
            const int nid = id + int(gridDim.x);
            rows.load(a, nid < total ? nid : id, row, part);
        }
        // zero the tiles of P above the diagonal that k-steps of 32 read: (0,1), (2,3)
        if (tid < 64) {
            const int tile = tid >> 5, rr = (tid >> 1) & 15, h = tid & 1;
            *reinterpret_cast<uint4 *>(PB + (32 * tile + rr) * PK + 32 * tile + 16 + 8 * h) = make_uint4(0, 0, 0, 0);
        }
        const bool qok = t < T, kok = t >= 1 && t <= T, first = t == 0;
        const uint32_t qw[8] = {qr0.x, qr0.y, qr0.z, qr0.w, qr1.x, qr1.y, qr1.z, qr1.w};
        const uint32_t kw[8] = {kr0.x, kr0.y, kr0.z, kr0.w, kr1.x, kr1.y, kr1.z, kr1.w};
        float qv[16], xv[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qv[2 * e] = lo16(qw[e]);
            qv[2 * e + 1] = hi16(qw[e]);
            xv[2 * e] = lo16(kw[e]);
            xv[2 * e + 1] = hi16(kw[e]);
        }
        const bool carry_x = first && a.xnext_in;
        if (carry_x) {   // x_0 continues the previous segment (features already formed)
#pragma unroll
            for (int e = 0; e < 16; ++e) xv[e] = a.xnext_in[size_t(bh) * DK + 16 * part + e];
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            sq += qv[e] * qv[e];
            sk += xv[e] * xv[e];
        }
        sq = group_sum<4>(sq);
        sk = group_sum<4>(sk);
        // rows outside the sequence (clamped loads) get a zero scale
        const float scq = qok ? rms_scale(sq, a.eps_rms, a.phi) : 0.f;
        const float sck = carry_x ? 1.f : (kok ? rms_scale(sk, a.eps_rms, a.phi) : 0.f);
        float n2 = 0.f;
        uint32_t xo[8], qo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x0 = xv[2 * e] * sck, x1 = xv[2 * e + 1] * sck;
            n2 += x0 * x0 + x1 * x1;
            xo[e] = pk2(x0, x1);
            qo[e] = pk2(qv[2 * e] * scq, qv[2 * e + 1] * scq);
        }
        n2 = group_sum<4>(n2);
        uint4 *xr = reinterpret_cast<uint4 *>(XB + row * PK + 16 * part);
        uint4 *qrw = reinterpret_cast<uint4 *>(QB + row * PK + 16 * part);
        xr[0] = make_uint4(xo[0], xo[1], xo[2], xo[3]);
        xr[1] = make_uint4(xo[4], xo[5], xo[6], xo[7]);
        qrw[0] = make_uint4(qo[0], qo[1], qo[2], qo[3]);
        qrw[1] = make_uint4(qo[4], qo[5], qo[6], qo[7]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            XT16[(16 * part + 2 * e) * PK + row] = uint16_t(xo[e]);
            XT16[(16 * part + 2 * e + 1) * PK + row] = uint16_t(xo[e] >> 16);
        }
#pragma unroll
        for (int i = 0; i < VPT / 8; ++i) {
            const uint32_t vw[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = qok ? vw[e] : 0u;
                YT16[(VPT * part + 8 * i + 2 * e) * PK + row] = uint16_t(w);
                YT16[(VPT * part + 8 * i + 2 * e + 1) * PK + row] = uint16_t(w >> 16);
            }
        }
        if (part == 0) {
            float eta = 0.f, alpha = 0.f;
            if (!(t >= T || (first && a.fresh))) {   // the fresh first step writes nothing
                const float den = n2 + lam + a.eps;
                eta = den != 0.f ? beta * __builtin_amdgcn_rcpf(den) : 0.f;
                alpha = step_alpha(eta, lam, a.eps_gamma);
            }
            sv[kEta][row] = eta;
            sv[kLg][row] = log2_1m(alpha);
        }
    }
    __syncthreads();

    // 2. chunk-local prefix b (base 2), lane = token; every wave forms the
    //    same values (identical LDS writes), so no barrier is needed.  The
    //    decays are separable (2^{b_i} 2^{-b_j}) while 2^{-b} stays in range.
    bool sep;
    {
        const float lg = sv[kLg][lane];
        const float b = wave_inclusive_scan(lg);
        const float bp = b - lg;
        const float bC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b), 63));
        sep = bC >= -100.f;
        const float eta = sv[kEta][lane];
        const float gp = ex2(bp);
        sv[kB][lane] = b;
        sv[kBp][lane] = bp;
        sv[kEw][lane] = ex2(bC - b);
        sv[kRs][lane] = eta * gp;
        sv[kQs][lane] = ex2(b);
        sv[kCs][lane] = sep ? ex2(-b) : 0.f;
        if (wave == 0 && lane == 0) *reinterpret_cast<float *>(rec + f1_xfer_scal_off(DV)) = ex2(bC);
    }
    wave_lds_sync();

    // decayed Gram (isG: eta_i e^{b_{i-1}-b_j} x_i.x_j) or score (e^{b_i-b_j} qh_i.x_j)
    // tile (I, J): rows i = 16 I + g4 + r, column j = 16 J + col
    auto tile = [&](bool isG, int I, int J) {
        const bf16_t *ar = (isG ? XB : QB) + (16 * I + col) * PK + k8;
        const bf16_t *br = XB + (16 * J + col) * PK + k8;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma(ld8(ar), ld8(br), acc);
        acc = mfma(ld8(ar + 32), ld8(br + 32), acc);
        const int j = 16 * J + col, i0 = 16 * I + g4;
        f32x4 v;
        if (sep) {
            const float cj = sv[kCs][j];
            const f32x4 ri = *reinterpret_cast<const f32x4 *>(&sv[isG ? kRs : kQs][i0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[r] * (ri[r] * cj);
        } else {
            const float bj = sv[kB][j];
            const f32x4 bi = *reinterpret_cast<const f32x4 *>(&sv[isG ? kBp : kB][i0]);
            const f32x4 ei = *reinterpret_cast<const f32x4 *>(&sv[kEta][i0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[r] * ex2(bi[r] - bj) * (isG ? ei[r] : 1.f);
        }
        return v;
    };

    // 3. wave 0: diagonal Gram blocks, then the inverses of the diagonal
    //    blocks of I + N by forward substitution (lane = 16 J + column);
    //    waves 1-3: the Gram blocks below them (-> -N, bf16), the score tiles
    //    (-> P) and the decayed keys (diag(e^{b_C-b_t}) x)^T.
    if (wave == 0) {
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const f32x4 v = tile(true, I, I);
#pragma unroll
            for (int r = 0; r < 4; ++r) Nd[I][(g4 + r) * 17 + col] = col < g4 + r ? v[r] : 0.f;
        }
        wave_lds_sync();
        const int J = lane >> 4;
        const float *nd = Nd[J];
        float tcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = (r == col) ? 1.f : 0.f;
#pragma unroll
            for (int k = 0; k < r; ++k) v -= nd[r * 17 + k] * tcol[k];
            tcol[r] = v;
        }
        uint16_t *db = reinterpret_cast<uint16_t *>(DB[J]);
#pragma unroll
        for (int r = 0; r < 16; ++r) db[r * NBP + col] = bf(tcol[r]);
    } else {
        const int w1 = wave - 1;
        for (int job = w1; job < 16; job += 3) {
            if (job < 6) {   // Gram blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
                const int I = (0xFE9 >> (2 * job)) & 3, J = (0x910 >> (2 * job)) & 3;
                const f32x4 v = tile(true, I, J);
                uint16_t *nb = reinterpret_cast<uint16_t *>(NB[job]);
#pragma unroll
                for (int r = 0; r < 4; ++r) nb[(g4 + r) * NBP + col] = bf(-v[r]);
            } else {         // score tiles on and below the diagonal
                const int tt = job - 6;
                const int I = (0xffa94 >> (2 * tt)) & 3, J = (0xe4910 >> (2 * tt)) & 3;
                const f32x4 v = tile(false, I, J);
                const int j = 16 * J + col, i0 = 16 * I + g4;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    reinterpret_cast<uint16_t *>(PB)[(i0 + r) * PK + j] = bf((I != J || j <= i0 + r) ? v[r] : 0.f);
            }
        }
        for (int p = tid - 64; p < DK * 8; p += 192) {   // 16-byte pieces of XW
            const int d = p >> 3, t8 = 8 * (p & 7);
            const uint4 xx = *reinterpret_cast<const uint4 *>(XT + d * PK + t8);
            const f32x4 e0 = *reinterpret_cast<const f32x4 *>(&sv[kEw][t8]);
            const f32x4 e1 = *reinterpret_cast<const f32x4 *>(&sv[kEw][t8 + 4]);
            *reinterpret_cast<uint4 *>(XW + d * PK + t8) =
                make_uint4(pk2(lo16(xx.x) * e0[0], hi16(xx.x) * e0[1]), pk2(lo16(xx.y) * e0[2], hi16(xx.y) * e0[3]),
                           pk2(lo16(xx.z) * e1[0], hi16(xx.z) * e1[1]), pk2(lo16(xx.w) * e1[2], hi16(xx.w) * e1[3]));
        }
    }
    __syncthreads();

    // 4. Z = (I + N)^{-1} R, R = [-diag(eta e^{b_{t-1}}) X | diag(eta) Y], by
    //    forward substitution over 16-row blocks, one column tile per pass,
    //    in registers: the accumulator layout of a 16 x 16 tile (lane
    //    holds rows 4 (lane / 16) .. + 3 of column lane % 16) is the
    //    B-operand layout of the 16x16x16 MFMA.  Z^T -> LDS (rows n).
    //    Z[:, x part] = -W, Z[:, value part] = Ut.
    for (int n = wave; n < NT; n += 4) {
        const bool xp = n < 4;
        const int nr = 16 * n + col;                   // row of Z^T
        const bf16_t *src = xp ? XT + nr * PK : YT + (nr - DK) * PK;
        s16x4 zb[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const f32x4 sc = *reinterpret_cast<const f32x4 *>(&sv[xp ? kRs : kEta][16 * I + g4]);
            f32x4 acc = unpk4(*reinterpret_cast<const uint2 *>(src + 16 * I + g4)) * (xp ? -sc : sc);
#pragma unroll
            for (int J = 0; J < I; ++J) {
                const int blk = (I * (I - 1)) / 2 + J;   // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
                acc = mfma16(as_s4(*reinterpret_cast<const uint2 *>(NB[blk] + col * NBP + 4 * kq)), zb[J], acc);
            }
            const f32x4 z0 = {0.f, 0.f, 0.f, 0.f};
            const f32x4 z = mfma16(as_s4(*reinterpret_cast<const uint2 *>(DB[I] + col * NBP + 4 * kq)), as_s4(pk4(acc)), z0);
            const uint2 zp = pk4(z);
            zb[I] = as_s4(zp);
            put2(ZT + nr * PK + 16 * I + g4, zp);
        }
    }
    __syncthreads();

    // 5. the operators (token-k products on MFMA), bf16 to the workspace
    {
        const int m = wave;
        const bf16x8 z0 = ld8(ZT + (16 * m + col) * PK + k8), z1 = ld8(ZT + (16 * m + col) * PK + 32 + k8);
        const bf16x8 x0 = ld8(XW + (16 * m + col) * PK + k8), x1 = ld8(XW + (16 * m + col) * PK + 32 + k8);
#pragma unroll
        for (int n = 0; n < 4; ++n) {   // A^T [d][d'] = Z_W^T diag(e^{b_C-b_t}) X
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma(z0, ld8(XW + (16 * n + col) * PK + k8), acc);
            acc = mfma(z1, ld8(XW + (16 * n + col) * PK + 32 + k8), acc);
            put2(rec + ((16 * n + col) * DK + 16 * m + g4) * 2, pk4(acc));
        }
#pragma unroll
        for (int n = 0; n < 4; ++n) {   // G^T [d][t] = diag-scaled Qh^T + Z_W^T P^T
            const int tt = 16 * n + col;
            f32x4 acc = unpk4(*reinterpret_cast<const uint2 *>(QB + tt * PK + 16 * m + g4)) * sv[kQs][tt];
            acc = mfma(z0, ld8(PB + tt * PK + k8), acc);
            if (n >= 2) acc = mfma(z1, ld8(PB + tt * PK + 32 + k8), acc);
            put2(rec + kF1XferGOff + (tt * DK + 16 * m + g4) * 2, pk4(acc));
        }
#pragma unroll
        for (int n = 0; n < NJ; ++n) {   // B [d'][j] = (diag(e^{b_C-b_t}) X)^T Ut, stored as B^T [j][d']
            const bf16_t *zu = ZT + (DK + 16 * n + col) * PK;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma(x0, ld8(zu + k8), acc);
            acc = mfma(x1, ld8(zu + 32 + k8), acc);
            put2(rec + kF1XferBOff + ((16 * n + col) * DK + 16 * m + g4) * 2, pk4(acc));
        }
    }
    for (int m = wave; m < NJ; m += 4) {   // H^T [j][t] = Ut^T P^T, stored as H [t][j]
        const bf16_t *zu = ZT + (DK + 16 * m + col) * PK;
        const bf16x8 u0 = ld8(zu + k8), u1 = ld8(zu + 32 + k8);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int tt = 16 * n + col;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma(u0, ld8(PB + tt * PK + k8), acc);
            if (n >= 2) acc = mfma(u1, ld8(PB + tt * PK + 32 + k8), acc);
            put2(rec + f1_xfer_h_off(DV) + (size_t(tt) * DV + 16 * m + g4) * 2, pk4(acc));
        }
    }
    __syncthreads();   // the next chunk overwrites the LDS buffers
    }
}

// ---------------------------------------------------------------------------
// f1_carry: the sequential walk of one (head, slice of DS value columns)
// ---------------------------------------------------------------------------
// wait until at most N vector memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the loader waves, without the release fence of
// __syncthreads: their only LDS writes are the copies, whose completion they
// wait for explicitly (counted), and the fence would wait for every copy in
// flight.  The empty asm statements keep the compiler from moving memory
// operations across it.
__device__ __forceinline__ void loader_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int DS>
__global__ __launch_bounds__((DS / 16 + 4) * 64) void f1_carry(F1SplitArgs a, int nslice) {
    constexpr int NCW = DS / 16;                 // compute waves, 16 state columns each
    constexpr int NLW = 4;                       // loader waves
    constexpr int NB = 4;                        // ring slots (chunks in flight)
    constexpr int kA = 0, kG = 8192, kB = 16384, kH = 16384 + 128 * DS, kS = 16384 + 256 * DS;
    constexpr int SB = kS + 256;                 // slot bytes
    constexpr int NI = kS / 1024;                // 1 KB copies per chunk
    constexpr int IPW = NI / NLW;                // per loader wave (+ one scalar copy)
    constexpr int PPR = DS / 8;                  // 16-byte pieces per H row
    static_assert(NI % NLW == 0, "whole copies per loader wave");
    static_assert(2 * (IPW + 1) < 64, "vmcnt range");
    __shared__ __align__(16) unsigned char ring[NB * SB];
    __shared__ __align__(16) bf16_t STw[NCW][16 * PK];   // per compute wave: S^T [j][d] (bf16)

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
    const int T = a.T, DV = a.dv, nch = a.nchunks;
    const size_t rb = f1_xfer_bytes(DV);
    const char *recs = static_cast<const char *>(a.ops) + size_t(bh) * nch * rb;

    if (wave >= NCW) {
        // ---- loader waves: chunk cc's operators into slot cc % NB ----
        const int lw = wave - NCW;
        // source offset of this lane's 16-byte piece in each copy; the LDS
        // rows are stored with their 16-byte pieces permuted (piece q of row
        // r at q ^ (r & 7)) so that the column reads of the compute waves
        // spread over the banks
        int goff[IPW];
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int off = 1024 * (lw + NLW * i) + 16 * lane;
            if (off < kB) {
                const int base = off < kG ? 0 : kG, o = off - base, r = o >> 7, q = (o >> 4) & 7;
                goff[i] = (base == 0 ? 0 : int(kF1XferGOff)) + r * 128 + 16 * (q ^ (r & 7));
            } else if (off < kH) {
                const int o = off - kB, r = o >> 7, q = (o >> 4) & 7;
                goff[i] = int(kF1XferBOff) + (j0 + r) * 128 + 16 * (q ^ (r & 7));
            } else {
                const int o = off - kH, r = o / (2 * DS), q = (o % (2 * DS)) >> 4;
                goff[i] = int(f1_xfer_h_off(DV)) + r * 2 * DV + 2 * j0 + 16 * (q ^ (r & (PPR - 1)));
            }
        }
        const int soff = int(f1_xfer_scal_off(DV));
        auto issue = [&](int cc) {
            const char *rec = recs + size_t(cc) * rb;
            unsigned char *slot = ring + (cc % NB) * SB;
#pragma unroll
            for (int i = 0; i < IPW; ++i)
                lds_copy16(rec + goff[i], slot + 1024 * (lw + NLW * i));
            // e^{b_C}: every lane copies the same word (64 copies, one per lane)
            lds_copy4(rec + soff, slot + kS);
        };
        // wait until the chunk followed by `ahead` issued chunks has landed
        auto wait_chunk = [&](int ahead) {
            if (ahead <= 0) wait_vm<0>();
            else if (ahead == 1) wait_vm<IPW + 1>();
            else wait_vm<2 * (IPW + 1)>();
        };
        const int npro = nch < NB - 1 ? nch : NB - 1;
        for (int cc = 0; cc < npro; ++cc) issue(cc);
        wait_chunk(npro - 1);
        loader_barrier();
        for (int c = 0; c < nch; ++c) {
            // slot (c - 1) % NB was released by the barrier that ended step c - 1
            if (c + NB - 1 < nch) issue(c + NB - 1);
            const int last = c + NB - 1 < nch ? c + NB - 1 : nch - 1;
            wait_chunk(last - (c + 1));   // chunk c + 1 complete before the barrier
            loader_barrier();
        }
        if (lw == 0 && s == 0 && a.xnext_out) {   // x for the next segment: phi(k_{T-1})
            const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * DK;
            const float xv = bf16_to_f32(kg[size_t(T - 1) * DK + lane].bits);
            const float sc = phi_scale(wave_sum(xv * xv), DK, a.eps_rms, a.phi);
            a.xnext_out[size_t(bh) * DK + lane] = xv * sc;
        }
        return;
    }

    // ---- compute wave ct: state columns j0 + 16 ct .. + 15 ----
    const int ct = wave;
    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4), kq = lane >> 4;
    const int sw = col & 7;
    // byte offsets inside a slot (row 16 m + col of A and G; pieces 4 kk + kq)
    const int ao0 = col * 128 + 16 * (kq ^ sw), ao1 = col * 128 + 16 * ((4 + kq) ^ sw);
    // B^T row 16 ct + col, d = 16 m + g4 (piece 2 m + g4 / 8, half g4 & 4)
    const int bo = (16 * ct + col) * 128 + ((g4 & 4) << 1);
    // H row 16 m + col, j = 16 ct + g4 (piece 2 ct + g4 / 8)
    const int ho = col * (2 * DS) + 16 * ((2 * ct + (g4 >> 3)) ^ (col & (PPR - 1))) + ((g4 & 4) << 1);
    bf16_t *stw = STw[ct];
    bf16_t *og = static_cast<bf16_t *>(a.o) + size_t(bh) * T * DV + j0 + 16 * ct + g4;

    f32x4 S[DK / 16];
#pragma unroll
    for (int m = 0; m < DK / 16; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[m][r] = a.S_in ? a.S_in[(size_t(bh) * DK + 16 * m + g4 + r) * DV + j0 + 16 * ct + col] : 0.f;
        put2(stw + col * PK + 16 * m + g4, pk4(S[m]));
    }
    wave_lds_sync();
    bf16x8 sb0 = ld8(stw + col * PK + k8), sb1 = ld8(stw + col * PK + 32 + k8);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const unsigned char *sl = ring + (c % NB) * SB;
        const float gC = *reinterpret_cast<const float *>(sl + kS);
        f32x4 O[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // carry: S' = e^{b_C} S + B + A S
            const uint2 bq = *reinterpret_cast<const uint2 *>(sl + kB + bo + 16 * ((2 * m + (g4 >> 3)) ^ sw));
            f32x4 sn = unpk4(bq);
#pragma unroll
            for (int r = 0; r < 4; ++r) sn[r] += gC * S[m][r];
            sn = mfma(ld8(sl + kA + m * 2048 + ao0), sb0, sn);
            S[m] = mfma(ld8(sl + kA + m * 2048 + ao1), sb1, sn);
            // outputs: O^T = S^T G^T + H^T (token tile m)
            f32x4 o = unpk4(*reinterpret_cast<const uint2 *>(sl + kH + m * 16 * (2 * DS) + ho));
            o = mfma(sb0, ld8(sl + kG + m * 2048 + ao0), o);
            O[m] = mfma(sb1, ld8(sl + kG + m * 2048 + ao1), o);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int tg = c * C + 16 * m + col;
            if (tg < T) put2(og + size_t(tg) * DV, pk4(O[m]));
            put2(stw + col * PK + 16 * m + g4, pk4(S[m]));
        }
        wave_lds_sync();
        sb0 = ld8(stw + col * PK + k8);
        sb1 = ld8(stw + col * PK + 32 + k8);
        __syncthreads();
    }
    if (a.S_out) {
#pragma unroll
        for (int m = 0; m < DK / 16; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a.S_out[(size_t(bh) * DK + 16 * m + g4 + r) * DV + j0 + 16 * ct + col] = S[m][r];
    }
}

// compute units of the current device (read once per device)
int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int DV>
void launch_xfer(const F1SplitArgs &a, hipStream_t s, Marks *m) {
    // as many workgroups as fit at once (LDS: two per CU, one at d_v = 128),
    // each walking chunk ids with the grid as stride
    const int total = a.nchunks * a.BH;
    const int slots = cu_count() * (DV == 128 ? 1 : 2);
    f1_xfer<DV><<<total < slots ? total : slots, 256, 0, s>>>(a);
    m->mark(s);
}

template <int DS>
void launch_carry(const F1SplitArgs &a, hipStream_t s, Marks *m) {
    const int nslice = a.dv / DS;
    const int blocks = nslice == 1 ? a.BH : ((a.BH + 7) / 8) * 8 * nslice;
    f1_carry<DS><<<blocks, (DS / 16 + 4) * 64, 0, s>>>(a, nslice);
    m->mark(s);
}

}  // namespace

void launch_chunk_f1_xfer(const F1SplitArgs &a, hipStream_t s, Marks *m) {
    switch (a.dv) {
        case 32: launch_xfer<32>(a, s, m); break;
        case 64: launch_xfer<64>(a, s, m); break;
        default: launch_xfer<128>(a, s, m); break;
    }
    if (f1_xfer_slice(a.dv) == 32) launch_carry<32>(a, s, m);
    else launch_carry<64>(a, s, m);
}

}  // namespace falcon
