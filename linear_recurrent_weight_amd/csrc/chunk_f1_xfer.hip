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
//   chunks: per chunk each compute wave owns 16 (or 32) state rows of every
//   column tile of the slice (fp32 MFMA accumulators) and issues the MFMAs of
//   its rows of the carry and of the outputs of its 16 (or 32) tokens, all
//   from one bf16 copy of the entry state (double-buffered in LDS); a row
//   tile's operators are read once per step for all column tiles.  Loader waves copy the
//   operators of later chunks straight from memory into a ring of LDS slots
//   (global_load_lds), so no register staging sits between memory and the
//   matrix cores; the records hold their tiles in operand lane order, so
//   each operand is one contiguous 16- or 8-byte read per lane.  One
//   workgroup barrier per chunk.
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
enum { kEta = 0, kB, kBp, kEw, kRs, kQs, kCs, kLg, kSx, kSq, kNsv };

// ---------------------------------------------------------------------------
// f1_xfer: the transfer operators of one chunk
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(const s16x4 &a, const s16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 as_s4(const uint2 &u) { return __builtin_bit_cast(s16x4, u); }

constexpr int NBP = 20;         // bf16 pitch of the 16 x 16 solve blocks
constexpr int LFB = 16 * 16 + 4;   // fp32 stride of the blocks L_J (the four blocks' rows fall in different banks)

// the value of lane h of each lane quad, in every lane of the quad (DPP
// quad_perm [h, h, h, h], CTRL = 0x55 h)
template <int CTRL>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int XW_THREADS = 512; // 8 waves per chunk

// The raw rows of one chunk (8 q and 8 k elements and d_v / 8 values of row
// `row`, part `part`, and the row's beta and lambda), loaded into registers
// one chunk ahead.  Loads are unconditional from rows clamped into [0, T).
// The one conditional load, the 8 incoming features x_0 of the first token of
// a continued sequence, comes last: the counted wait for the other rows then
// does not depend on it.
template <int DV>
struct XferRows {
    static constexpr int VPT = DV / 8;                 // value elements per thread
    static constexpr int NV = VPT >= 8 ? VPT / 8 : 1;  // 16-byte pieces (8 bytes at d_v = 32)
    uint4 q, k, v[NV];
    float beta, lam;
    f32x4 xn[2];                                       // x_0 (row 0 of chunk 0 only)
    __device__ __forceinline__ void load(const F1XferArgs &a, int id, int row, int part) {
        const int c = id / a.BH, bh = id % a.BH, T = a.T, t = c * kChunk + row;
        const int tq = t < T ? t : T - 1;
        const int tk = t < 1 ? 0 : (t - 1 < T ? t - 1 : T - 1);
        q = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.q) + (size_t(bh) * T + tq) * DK + 8 * part);
        k = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.k) + (size_t(bh) * T + tk) * DK + 8 * part);
        const bf16_t *vp = static_cast<const bf16_t *>(a.v) + (size_t(bh) * T + tq) * DV + VPT * part;
        if constexpr (VPT >= 8) {
#pragma unroll
            for (int i = 0; i < NV; ++i) v[i] = reinterpret_cast<const uint4 *>(vp)[i];
        } else {
            const uint2 h = *reinterpret_cast<const uint2 *>(vp);
            v[0] = make_uint4(h.x, h.y, 0u, 0u);
        }
        beta = a.beta[size_t(bh) * T + tq];
        lam = a.lambda[size_t(bh) * T + tq];
        if (t == 0 && a.xnext_in) {
            const f32x4 *xp = reinterpret_cast<const f32x4 *>(a.xnext_in + size_t(bh) * DK + 8 * part);
            xn[0] = xp[0];
            xn[1] = xp[1];
        }
    }
};

template <int DV>
__global__ __launch_bounds__(XW_THREADS, DV == 128 ? 2 : 4) void f1_xfer(F1XferArgs a) {
    using Rows = XferRows<DV>;
    constexpr int VPT = Rows::VPT;
    constexpr int YP = DV + 8;                // bf16 pitch of the value rows
    constexpr int NJ = DV / 16;               // value column tiles
    constexpr int NT = 4 + NJ;                // column tiles of R = [x part | value part]
    __shared__ __align__(16) bf16_t QB[C * PK];     // q rows [t][d] (qh = s_q q)
    __shared__ __align__(16) bf16_t XW[DK * PK];    // (diag(e^{b_C-b_t}) x)^T [d][t], t in pair order
    __shared__ __align__(16) bf16_t YB[C * YP];     // value rows [t][j]
    __shared__ __align__(16) bf16_t PB[C * PK];     // P [t][s], s in pair order
    __shared__ __align__(16) bf16_t XB[C * PK];     // k_{t-1} rows [t][d] (x = s_x k_{t-1})
    __shared__ __align__(16) bf16_t NB[6][16 * NBP];   // -N below the diagonal blocks
    __shared__ __align__(16) bf16_t DB[4][16 * NBP];   // inverses of the diagonal blocks of I + N
    __shared__ __align__(16) float LF[4 * LFB];         // the strictly lower diagonal blocks L_J, fp32 row-major
    __shared__ __align__(16) float sv[kNsv][C];

    const int nch = a.nchunks, total = nch * a.BH;
    const int T = a.T;
    bf16x8 pick0, pick1;   // column pickers (see below), in registers
    {
    const int tid = threadIdx.x, lane = tid & 63;
    const int col = lane & 15, k8 = 8 * (lane >> 4);
    // B operands that pick 16 columns (half h) of a 32-wide A block: the MFMA
    // then hands back the block transposed into the accumulator layout (lane
    // holds 4 consecutive rows of one column).  Kept in registers (8 VGPRs):
    // read from LDS by every transpose they cost as many LDS reads as the rows.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
        u16x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = (k8 + e == 16 * h + col) ? 0x3F80 : 0;   // bf16 1.0
        (h ? pick1 : pick0) = __builtin_bit_cast(bf16x8, u);
    }
    // the score tiles above the diagonal that the paired products read,
    // (0, 1) and (2, 3), stay zero (no chunk writes them)
    for (int e = tid; e < C * PK / 8; e += XW_THREADS) reinterpret_cast<uint4 *>(PB)[e] = make_uint4(0, 0, 0, 0);
    }

    // persistent: chunk ids blockIdx.x, + gridDim.x, ...; the rows of the
    // next chunk are loaded while this one is worked on
    Rows rows;
    rows.load(a, blockIdx.x, threadIdx.x >> 3, threadIdx.x & 7);
    // The first chunk's rows are waited for here: the loop is then entered
    // with no load in flight, and the counted wait inside it for the rows of
    // the next chunk need not cover that chunk's record stores.
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
    for (int id = blockIdx.x; id < total; id += gridDim.x) {
    // lane quantities are formed afresh in every pass (an opaque copy of the
    // thread index), so that the compiler does not keep dozens of derived
    // addresses live across the loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4), kq = lane >> 4;
    const int row = tid >> 3, part = tid & 7;
    const int c = id / a.BH, bh = id % a.BH;   // chunk-major: with 8 | BH a head stays on one XCD
    const int t = c * C + row;
    char *rec = static_cast<char *>(a.ops) + (size_t(bh) * nch + c) * f1_xfer_bytes(DV);

    // 1. rows: q, k_{t-1} (x_0 from the boundary) and the values go to LDS as
    //    loaded; the RMS scales of phi (s_x for x = phi(k_{t-1}), s_q for qh)
    //    go to the scalars and are folded into the per-token factors that
    //    every later product applies anyway.  eta and log2 gamma.  Rows
    //    outside the sequence get a zero scale.
    {
        const uint4 qr = rows.q;
        uint4 xr = rows.k;
        uint4 vr[Rows::NV];
#pragma unroll
        for (int i = 0; i < Rows::NV; ++i) vr[i] = rows.v[i];
        const float beta = rows.beta, lam = rows.lam;
        const bool qok = t < T, kok = t >= 1 && t <= T, first = t == 0;
        const uint32_t qw[4] = {qr.x, qr.y, qr.z, qr.w};
        const uint32_t kw[4] = {xr.x, xr.y, xr.z, xr.w};
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16x2_t qe = __builtin_bit_cast(bf16x2_t, qw[e]), ke = __builtin_bit_cast(bf16x2_t, kw[e]);
            sq = __builtin_amdgcn_fdot2_f32_bf16(qe, qe, sq, false);
            sk = __builtin_amdgcn_fdot2_f32_bf16(ke, ke, sk, false);
        }
        const bool carry_x = first && a.xnext_in;
        if (carry_x) {   // x_0 continues the previous segment (features already formed, scale 1)
            sk = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) sk += rows.xn[0][e] * rows.xn[0][e] + rows.xn[1][e] * rows.xn[1][e];
            xr = make_uint4(pk2(rows.xn[0][0], rows.xn[0][1]), pk2(rows.xn[0][2], rows.xn[0][3]),
                            pk2(rows.xn[1][0], rows.xn[1][1]), pk2(rows.xn[1][2], rows.xn[1][3]));
        }
        sq = group_sum<8>(sq);
        sk = group_sum<8>(sk);
        const float scq = qok ? rms_scale(sq, a.eps_rms, a.phi) : 0.f;
        const float sck = carry_x ? 1.f : (kok ? rms_scale(sk, a.eps_rms, a.phi) : 0.f);
        const float n2 = sck * sck * sk;   // |x_t|^2
        *reinterpret_cast<uint4 *>(XB + row * PK + 8 * part) = xr;
        *reinterpret_cast<uint4 *>(QB + row * PK + 8 * part) = qr;
        if constexpr (VPT >= 8) {
#pragma unroll
            for (int i = 0; i < Rows::NV; ++i)
                *reinterpret_cast<uint4 *>(YB + row * YP + VPT * part + 8 * i) = qok ? vr[i] : make_uint4(0, 0, 0, 0);
        } else {
            *reinterpret_cast<uint2 *>(YB + row * YP + VPT * part) = qok ? make_uint2(vr[0].x, vr[0].y) : make_uint2(0, 0);
        }
        if (part == 0) {   // the step inputs; wave 0 forms eta and log2 gamma
            // beta = 0 past the sequence and at a fresh first step (no write)
            sv[kEta][row] = (t >= T || (first && a.fresh)) ? 0.f : beta;
            sv[kLg][row] = lam;
            sv[kB][row] = n2;
            sv[kSx][row] = sck;
            sv[kSq][row] = scq;
        }
        // the next chunk's rows (the last chunk reloads its own), issued once
        // this chunk's are consumed, so that they land in the same registers
        const int nid = id + int(gridDim.x);
        rows.load(a, nid < total ? nid : id, row, part);
    }
    __syncthreads();

    // 2. chunk-local prefix b (base 2), lane = token, and the per-token
    //    factors, formed by wave 0 and published by a barrier.  The decays
    //    are separable (2^{b_i} 2^{-b_j}) while 2^{-b} stays in range.
    if (wave == 0) {
        // eta and log2 gamma of token `lane` (a zero beta gives eta = 0 and
        // gamma = 1: no write)
        float eta;
        {
            const float beta = sv[kEta][lane], lam = sv[kLg][lane], n2 = sv[kB][lane];
            const float den = n2 + lam + a.eps;
            eta = den != 0.f ? beta * __builtin_amdgcn_rcpf(den) : 0.f;
        }
        const float lg = log2_1m(step_alpha(eta, sv[kLg][lane], a.eps_gamma));
        sv[kEta][lane] = eta;
        const float b = wave_inclusive_scan(lg);
        const float bp = b - lg;
        const float bC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b), 63));
        const bool sep = bC >= -100.f;
        const float sx = sv[kSx][lane], sq = sv[kSq][lane];
        sv[kB][lane] = b;
        sv[kBp][lane] = bp;
        // with the RMS scales of the rows folded in: x = s_x k_{t-1}, qh = s_q q
        sv[kEw][lane] = ex2(bC - b) * sx;
        sv[kRs][lane] = eta * ex2(bp) * sx;
        sv[kQs][lane] = ex2(b) * sq;
        sv[kCs][lane] = sep ? ex2(-b) * sx : 0.f;
        if (lane == 0) *reinterpret_cast<float *>(rec + f1_xfer_scal_off(DV)) = ex2(bC);
    }
    __syncthreads();
    const bool sep = sv[kB][C - 1] >= -100.f;

    // rows (pitch ld) of a 16 x 32 block, 16 of whose columns (block n of
    // 16) come back transposed into the accumulator layout: lane holds
    // rows 16 m + 4 (lane / 16) .. + 3 of column 16 n + lane % 16
    auto transposed = [&](const bf16_t *rows, int ld, int m, int n) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        return mfma(ld8(rows + (16 * m + col) * ld + 32 * (n >> 1) + k8), (n & 1) ? pick1 : pick0, z);
    };
    // (diag(e^{b_C-b_t}) x)^T, tile (token block m, feature block n)
    auto transpose_x = [&](int m, int n) {
        const f32x4 ew = *reinterpret_cast<const f32x4 *>(&sv[kEw][16 * m + g4]);
        put2(XW + (16 * n + col) * PK + pair_slot(16 * m + g4), pk4(transposed(XB, PK, m, n) * ew));
    };

    // 3. waves 0-3: diagonal block J = wave of I + N, inverted in fp32 on
    //    the vector ALUs (the matrix cores stay free for the other waves),
    //    then one score tile each; waves 4-7: the Gram blocks below the
    //    diagonal (-> -N, bf16) and the other score tiles (-> P); every
    //    wave: two transposes of x.
    auto job = [&](int jb) {
        // job 0-5: Gram block (1,0) (2,0) (2,1) (3,0) (3,1) (3,2) of
        // eta_i e^{b_{i-1}-b_j} x_i.x_j; job 6-15: score tile on or below the
        // diagonal, e^{b_i-b_j} qh_i.x_j.  The choices are uniform selects
        // (no branches), so that unrolled jobs overlap their reads.  The tile
        // is formed transposed (x rows as the A operand): lane (col, g4)
        // gets row i = 16 I + col at columns j = 16 J + g4 .. + 3, one
        // 8-byte write.
        const int tt = jb - 6;
        const bool isG = jb < 6;
        const int I = isG ? (0xFE9 >> (2 * jb)) & 3 : (0xffa94 >> (2 * tt)) & 3;
        const int J = isG ? (0x910 >> (2 * jb)) & 3 : (0xe4910 >> (2 * tt)) & 3;
        const bf16_t *ar = (isG ? XB : QB) + (16 * I + col) * PK + k8;
        const bf16_t *br = XB + (16 * J + col) * PK + k8;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 acc = mfma(ld8(br), ld8(ar), z);
        acc = mfma(ld8(br + 32), ld8(ar + 32), acc);
        const int i = 16 * I + col, j0 = 16 * J + g4;
        f32x4 v;
        if (sep) {
            const float ri = sv[isG ? kRs : kQs][i];
            const f32x4 cj = *reinterpret_cast<const f32x4 *>(&sv[kCs][j0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[r] * (ri * cj[r]);
        } else {
            const float bi = sv[isG ? kBp : kB][i], ei = (isG ? sv[kEta][i] : 1.f) * sv[isG ? kSx : kSq][i];
            const f32x4 bj = *reinterpret_cast<const f32x4 *>(&sv[kB][j0]);
            const f32x4 sj = *reinterpret_cast<const f32x4 *>(&sv[kSx][j0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[r] * ex2(bi - bj[r]) * (ei * sj[r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = isG ? -v[r] : ((I != J || j0 + r <= i) ? v[r] : 0.f);
        put2(isG ? NB[jb < 6 ? jb : 0] + col * NBP + g4 : PB + i * PK + pair_slot(j0), pk4(v));
    };
    if (wave < 4) {
        const int J = wave;
        {   // L_J row-major in fp32 (LF): the raw Gram block X_J X_J^T is
            // symmetric, so the accumulator tile also holds row col of L_J at
            // columns g4 .. + 3, scaled eta_i e^{b_{i-1}-b_j} (strictly lower)
            const bf16_t *xr = XB + (16 * J + col) * PK + k8;
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
            g = mfma(ld8(xr), ld8(xr), g);
            g = mfma(ld8(xr + 32), ld8(xr + 32), g);
            const int i = 16 * J + col, j0 = 16 * J + g4;
            f32x4 l;
            if (sep) {
                const float ri = sv[kRs][i];
                const f32x4 cj = *reinterpret_cast<const f32x4 *>(&sv[kCs][j0]);
#pragma unroll
                for (int r = 0; r < 4; ++r) l[r] = g4 + r < col ? g[r] * (ri * cj[r]) : 0.f;
            } else {
                const float bpi = sv[kBp][i], ei = sv[kEta][i] * sv[kSx][i];
                const f32x4 bj = *reinterpret_cast<const f32x4 *>(&sv[kB][j0]);
                const f32x4 sj = *reinterpret_cast<const f32x4 *>(&sv[kSx][j0]);
#pragma unroll
                for (int r = 0; r < 4; ++r) l[r] = g4 + r < col ? g[r] * ex2(bpi - bj[r]) * (ei * sj[r]) : 0.f;
            }
            *reinterpret_cast<f32x4 *>(&LF[J * LFB + col * 16 + g4]) = l;
        }
        wave_lds_sync();
        // lane (r = lane / 4, h = lane % 4): elements 4 h .. + 3 of row r of
        // D_J = (I + L_J)^{-1}, from d (I + L_J) = e_r, right-looking over the
        // columns from the last: once d_k is final (in lane (r, k / 4)) it is
        // broadcast over the lane quad and d_j -= d_k L_kj for the lane's four
        // j (L_kj = 0 for j >= k)
        const int r = lane >> 2, h = lane & 3;
        const float *lf = LF + J * LFB + 4 * h;
        f32x4 dq;
#pragma unroll
        for (int e = 0; e < 4; ++e) dq[e] = 4 * h + e == r ? 1.f : 0.f;
        f32x4 lr[3];   // rows of L_J read two steps ahead
        lr[15 % 3] = *reinterpret_cast<const f32x4 *>(lf + 15 * 16);
        lr[14 % 3] = *reinterpret_cast<const f32x4 *>(lf + 14 * 16);
#pragma unroll
        for (int k = 15; k > 0; --k) {
            if (k > 2) lr[(k - 2) % 3] = *reinterpret_cast<const f32x4 *>(lf + (k - 2) * 16);
            const float x = dq[k & 3];
            const int hk = k >> 2;
            const float dk = hk == 0 ? quad_bcast<0x00>(x) : hk == 1 ? quad_bcast<0x55>(x)
                           : hk == 2 ? quad_bcast<0xAA>(x) : quad_bcast<0xFF>(x);
            dq -= dk * lr[k % 3];
        }
        put2(DB[J] + r * NBP + 4 * h, pk4(dq));
        job(12 + J);
    } else {
#pragma unroll
        for (int u = 0; u < 3; ++u) job(wave - 4 + 4 * u);
    }
    transpose_x(wave >> 1, 2 * (wave & 1));
    transpose_x(wave >> 1, 2 * (wave & 1) + 1);
    __syncthreads();

    // 4. Z = (I + N)^{-1} R, R = [-diag(eta e^{b_{t-1}}) X | diag(eta) Y], by
    //    forward substitution over 16-row blocks, one column tile per wave,
    //    in registers: the accumulator layout of a 16 x 16 tile (lane holds
    //    rows 4 (lane / 16) .. + 3 of column lane % 16) is the B-operand
    //    layout of the 16x16x16 MFMA, and read as the A operand it is the
    //    tile transposed.  Z[:, x part] = -W, Z[:, value part] = Ut.
    // 5. With its column tile of Z still in registers, the same wave forms
    //    the operators that tile feeds (token-k products on 16x16x32 MFMA,
    //    32 tokens per step in pair order):
    //      x tile n (d rows):      A^T [d][d'] = Z_W^T diag(e^{b_C-b_t}) X,
    //                              G^T [d][t]  = diag-scaled Qh^T + Z_W^T P^T;
    //      value tile (j columns): B [d'][j]   = (diag(e^{b_C-b_t}) X)^T Ut,
    //                              H^T [j][t]  = Ut^T P^T;
    //    bf16 to the workspace (A and G row-major, B as B^T [j][d'], H [t][j]).
    // A fixed, unrolled count of tiles per wave: each wave then issues a
    // known number of stores per chunk, and the wait for the next chunk's
    // rows (loaded before those stores) leaves the stores in flight.
    __builtin_assume(wave >= 0 && wave < XW_THREADS / 64);
#pragma unroll
    for (int it = 0; it < (NT + 7) / 8; ++it) {
        const int n = wave + 8 * it;
        if (NT % 8 != 0 && n >= NT) break;
        const bool xp = n < 4;
        f32x4 r0[4];   // R, block by block, from the rows transposed on MFMA
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const f32x4 sc = *reinterpret_cast<const f32x4 *>(&sv[xp ? kRs : kEta][16 * I + g4]);
            r0[I] = xp ? transposed(XB, PK, I, n) * -sc : transposed(YB, YP, I, n - 4) * sc;
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
            const f32x4 z = mfma16(as_s4(*reinterpret_cast<const uint2 *>(DB[I] + col * NBP + 4 * kq)), as_s4(pk4(acc)), z0);
            zb[I] = as_s4(pk4(z));
            if (I == 1) zp01 = cat8(zb[0], zb[1]);
        }
        // The products contract over tokens 32 at a time: lane (col, q) of
        // the 16x16x32 MFMA takes the 8 tokens 32 p + 4 q .. + 3 (block 2 p)
        // and 32 p + 16 + 4 q .. + 3 (block 2 p + 1), so its Z operand is its
        // two register pieces side by side, and XW and P hold their token
        // index in that order (pair_slot), one 16-byte read per operand.
        const bf16x8 zp[2] = {cat8(zb[0], zb[1]), cat8(zb[2], zb[3])};
        auto tok8 = [&](const bf16_t *base, int r, int p) { return ld8(base + r * PK + 32 * p + k8); };
        // results first, stores after the branch: every wave then issues
        // the same 8 stores on one path
        uint2 o1[4], o2[4];
        const int jt = n - 4;
        if (xp) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {   // A^T tile (d rows of tile n, d' columns of tile m)
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p) acc = mfma(zp[p], tok8(XW, 16 * m + col, p), acc);
                o1[m] = pk4(acc);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {   // G^T tile (d rows of tile n, tokens of tile m; P lower)
                const int tt = 16 * m + col;
                f32x4 acc = unpk4(*reinterpret_cast<const uint2 *>(QB + tt * PK + 16 * n + g4)) * sv[kQs][tt];
#pragma unroll
                for (int p = 0; p <= m / 2; ++p) acc = mfma(zp[p], tok8(PB, tt, p), acc);
                o2[m] = pk4(acc);
            }
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) {   // B tile (d' rows of tile m, j columns of tile jt)
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p) acc = mfma(tok8(XW, 16 * m + col, p), zp[p], acc);
                o1[m] = pk4(acc);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {   // H^T tile (j rows of tile jt, tokens of tile m; P lower)
                const int tt = 16 * m + col;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p <= m / 2; ++p) acc = mfma(zp[p], tok8(PB, tt, p), acc);
                o2[m] = pk4(acc);
            }
        }
        // byte offsets in the record, whose tiles are in operand lane order:
        // this lane's 4 elements of A (row 16 m + col, d = 16 n + g4 ..) and
        // of G (token 16 m + col) go to lane 16 (2 (n % 2) + kq / 2) + col of
        // the k half n / 2, bytes 8 (kq % 2) ..; B and H tiles are stored as
        // the accumulators hold them.  Each store covers 512 contiguous bytes.
        const int xo = ((n >> 1) * 64 + 16 * (2 * (n & 1) + (kq >> 1)) + col) * 16 + 8 * (kq & 1);
        const int off1 = xp ? xo : int(kF1XferBOff) + (jt * 256 + lane) * 8;
        const int off2 = xp ? int(kF1XferGOff) + xo : int(f1_xfer_h_off(DV)) + (jt * 256 + lane) * 8;
        const int st1 = xp ? 2048 : 512, st2 = st1;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            put2(rec + off1 + m * st1, o1[m]);
            put2(rec + off2 + m * st2, o2[m]);
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

// row tiles of the state split over compute waves: each column tile has
// RS waves (RS = 4 while the workgroup stays within 16 waves)
template <int DS> constexpr int carry_rs() { return DS == 64 ? 2 : 4; }
template <int DS> constexpr int carry_threads() { return (carry_rs<DS>() + 4) * 64; }

template <int DS>
__global__ __launch_bounds__(carry_threads<DS>()) void f1_carry(F1XferArgs a, int nslice, int nbase) {
    constexpr int NCT = DS / 16;                 // column tiles of the slice
    constexpr int RS = carry_rs<DS>();           // row groups per column tile
    constexpr int MT = 4 / RS;                   // row tiles (of 16) per compute wave
    constexpr int NCW = RS;                      // compute waves (each takes every column tile)
    constexpr int NLW = 4;                       // loader waves
    constexpr int kA = 0, kG = 8192, kB = 16384, kH = 16384 + 128 * DS, kS = 16384 + 256 * DS;
    constexpr int SB = kS + 256;                 // slot bytes
    constexpr int NB = (150 * 1024 - 2 * NCT * 16 * PK * 2) / SB;   // ring slots: as many as fit
    static_assert(NB >= 3, "ring depth");
    constexpr int NI = kS / 1024;                // 1 KB copies per chunk
    constexpr int IPW = NI / NLW;                // per loader wave (+ one scalar copy)
    static_assert(NI % NLW == 0, "whole copies per loader wave");
    static_assert((NB - 2) * (IPW + 1) < 64, "vmcnt range");
    __shared__ __align__(16) unsigned char ring[NB * SB];
    __shared__ __align__(16) bf16_t STw[2][NCT][16 * PK];   // bf16 S^T [j][d] per column tile, by chunk parity

    // workgroup -> (segment, head, slice); the slices of a head share an XCD
    int bh, s;
    const int g = blockIdx.x / nbase, id = blockIdx.x % nbase;
    if (nslice == 1) {
        bh = id;
        s = 0;
    } else {
        const int u = id & 7, rest = id >> 3;
        s = rest % nslice;
        bh = (rest / nslice) * 8 + u;
    }
    if (bh >= a.BH) return;   // the whole workgroup leaves together
    const int j0 = s * DS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.T, DV = a.dv;
    // this workgroup's chunks: [c_lo, c_lo + nch) of segment g
    const int c_lo = g * a.seg_chunks;
    const int nch = (a.nchunks - c_lo) < a.seg_chunks ? a.nchunks - c_lo : a.seg_chunks;
    const bool last_seg = g == a.nseg - 1;
    const size_t rb = f1_xfer_bytes(DV);
    const char *recs = static_cast<const char *>(a.ops) + (size_t(bh) * a.nchunks + c_lo) * rb;
    // entry state: the incoming state (row-major), or the segment's from the
    // scan (accumulator tiles [row tile][value tile][lane])
    const float *S0 = g == 0 ? a.S_in : a.Sseg + (size_t(bh) * a.nseg + g) * DK * DV;

    if (wave >= NCW) {
        // ---- loader waves: chunk cc's operators into slot cc % NB ----
        const int lw = wave - NCW;
        // source offset of this lane's 16-byte piece in each copy: the slot
        // is A and G whole, then the slice's value tiles of B^T and of H, each
        // a contiguous range of the record (its tiles are in lane order)
        int goff[IPW];
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int off = 1024 * (lw + NLW * i) + 16 * lane;
            goff[i] = off < kB ? off
                    : off < kH ? int(kF1XferBOff) + 128 * j0 + (off - kB)
                               : int(f1_xfer_h_off(DV)) + 128 * j0 + (off - kH);
        }
        const int soff = int(f1_xfer_scal_off(DV));
        auto issue = [&](int cc) {
            const char *rec = recs + size_t(cc) * rb;
            unsigned char *slot = ring + (cc % NB) * SB;
#pragma unroll
            for (int i = 0; i < IPW; ++i) lds_copy16(rec + goff[i], slot + 1024 * (lw + NLW * i));
            // e^{b_C}: every lane copies the same word (64 copies, one per lane)
            lds_copy4(rec + soff, slot + kS);
        };
        // wait until the chunk followed by `ahead` issued chunks has landed
        // (ahead <= NB - 2)
        auto wait_chunk = [&](int ahead) {
            if (ahead <= 0) wait_vm<0>();
            else if (ahead == 1) wait_vm<IPW + 1>();
            else if (ahead == 2 || NB < 5) wait_vm<2 * (IPW + 1)>();
            else if (ahead == 3 || NB < 6) wait_vm<(NB >= 5 ? 3 : 2) * (IPW + 1)>();
            else if (ahead == 4 || NB < 7) wait_vm<(NB >= 6 ? 4 : 2) * (IPW + 1)>();
            else wait_vm<(NB >= 7 ? 5 : 2) * (IPW + 1)>();
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
        if (lw == 0 && s == 0 && last_seg && a.xnext_out) {   // x for the next call: phi(k_{T-1})
            const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * DK;
            const float xv = bf16_to_f32(kg[size_t(T - 1) * DK + lane].bits);
            const float sc = phi_scale(wave_sum(xv * xv), DK, a.eps_rms, a.phi);
            a.xnext_out[size_t(bh) * DK + lane] = xv * sc;
        }
        return;
    }

    // ---- compute wave: row tiles m = MT mh .. MT mh + MT - 1 of every
    //      column tile ct of the slice, and the outputs of the same token
    //      tiles for those columns; a row tile's A and G operands are read
    //      once per step for all column tiles ----
    const int mh = wave;
    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4);
    // byte offsets inside a slot: the operand pieces of this lane (tiles in
    // lane order), A and G at k half 0 (+ 1024 for half 1), B^T and H tiles
    // of column tile ct at + ct * 2048
    const int ao = 16 * lane, bo = 8 * lane;
    bf16_t *og = static_cast<bf16_t *>(a.o) + size_t(bh) * T * DV + j0 + g4;

    f32x4 S[NCT][MT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = MT * mh + h;
            if (g > 0) {
                S[ct][h] = reinterpret_cast<const f32x4 *>(S0)[(m * (DV / 16) + j0 / 16 + ct) * 64 + lane];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[ct][h][r] = S0 ? S0[(size_t(bh) * DK + 16 * m + g4 + r) * DV + j0 + 16 * ct + col] : 0.f;
            }
            put2(STw[0][ct] + col * PK + 16 * m + g4, pk4(S[ct][h]));
        }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const unsigned char *sl = ring + (c % NB) * SB;
        // every LDS read of the step first, so that one latency covers them
        bf16x8 sb0[NCT], sb1[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const bf16_t *stw = STw[c & 1][ct];
            sb0[ct] = ld8(stw + col * PK + k8);
            sb1[ct] = ld8(stw + col * PK + 32 + k8);
        }
        const float gC = *reinterpret_cast<const float *>(sl + kS);
        uint2 bq[NCT][MT], hq[NCT][MT];
        bf16x8 a0[MT], a1[MT], q0[MT], q1[MT];
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = MT * mh + h;
            a0[h] = ld8(sl + kA + m * 2048 + ao);
            a1[h] = ld8(sl + kA + m * 2048 + 1024 + ao);
            q0[h] = ld8(sl + kG + m * 2048 + ao);
            q1[h] = ld8(sl + kG + m * 2048 + 1024 + ao);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                bq[ct][h] = *reinterpret_cast<const uint2 *>(sl + kB + ct * 2048 + bo + m * 512);
                hq[ct][h] = *reinterpret_cast<const uint2 *>(sl + kH + ct * 2048 + bo + m * 512);
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            bf16_t *stn = STw[(c + 1) & 1][ct];
#pragma unroll
            for (int h = 0; h < MT; ++h) {
                const int m = MT * mh + h;
                // carry: S' = e^{b_C} S + B + A S  (row tile m); the two k
                // halves accumulate separately (two MFMA chains of one)
                f32x4 sn = unpk4(bq[ct][h]);
#pragma unroll
                for (int r = 0; r < 4; ++r) sn[r] += gC * S[ct][h][r];
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                sn = mfma(a0[h], sb0[ct], sn);
                S[ct][h] = sn + mfma(a1[h], sb1[ct], z);
                put2(stn + col * PK + 16 * m + g4, pk4(S[ct][h]));
                // outputs: O^T = S^T G^T + H^T (token tile m)
                const f32x4 o = mfma(sb0[ct], q0[h], unpk4(hq[ct][h])) + mfma(sb1[ct], q1[h], z);
                const int tg = (c_lo + c) * C + 16 * m + col;
                if (tg < T) put2(og + size_t(tg) * DV + 16 * ct, pk4(o));
            }
        }
        __syncthreads();
    }
    if (a.S_out && last_seg) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int h = 0; h < MT; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a.S_out[(size_t(bh) * DK + 16 * (MT * mh + h) + g4 + r) * DV + j0 + 16 * ct + col] = S[ct][h][r];
    }
}

// ---------------------------------------------------------------------------
// Segments: the chunk maps S -> Gamma_c S + A_c S + B_c of a head compose
// associatively (summary §H.1 "Affine Chunk Map", §H.2), so the walk over a
// long sequence splits into segments of G chunks that run in parallel:
//   f1_segmap: each segment's composed map, kept as gamma I + A~ (the
//     identity part as an exact fp32 scalar) and the offset beta;
//   f1_segscan: per head, the segments' entry states in order,
//     S_{g+1} = gamma_g S_g + A~_g S_g + beta_g;
//   f1_carry: every segment walks its chunks from its entry state.
// ---------------------------------------------------------------------------
constexpr int SM_THREADS = 256;
constexpr int NPF = 3;          // operator buffers in flight per wave (2 steps ahead)

// workgroup barrier after this wave's LDS writes have completed, without
// the release fence of __syncthreads (which would also wait for the global
// loads of the next step, issued ahead on purpose)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// the parts of a chunk's record one segment-map wave uses: its row tile m of
// A_c as MFMA A operands (both k halves), its rows of B_c per value tile and
// the chunk's scalar Gamma_c = e^{b_C}
template <int DV>
struct MapRec {
    bf16x8 a0, a1;
    uint2 b[DV / 16];
    float gc;
    __device__ __forceinline__ void load(const char *rec, int m, int lane) {
        a0 = ld8(rec + m * 2048 + 16 * lane);
        a1 = ld8(rec + m * 2048 + 1024 + 16 * lane);
#pragma unroll
        for (int n = 0; n < DV / 16; ++n)
            b[n] = *reinterpret_cast<const uint2 *>(rec + kF1XferBOff + n * 2048 + 8 * lane + m * 512);
        gc = *reinterpret_cast<const float *>(rec + f1_xfer_scal_off(DV));
    }
};

// composed map of segment g of head bh: wave m owns row tile m (16 rows of
// d) of [A~ | beta] (d_k x (d_k + d_v)) in fp32 accumulators; a bf16 copy of
// its transpose in LDS is the B operand of A_c [A~ | beta].  The term
// gamma A_c takes A_c's entries in accumulator order from an MFMA with the
// identity (exact: one product by 1 per output).
template <int DV>
__global__ __launch_bounds__(SM_THREADS) void f1_segmap(F1XferArgs a) {
    constexpr int NCOL = (DK + DV) / 16;        // column tiles of [A~ | beta]
    __shared__ __align__(16) bf16_t XT[2][DK + DV][PK];   // bf16 [A~ | beta]^T [col][d]
    const int nsm = a.nseg - 1;                 // the last segment's map is never used
    const int bh = blockIdx.x / nsm, g = blockIdx.x % nsm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int m = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4);
    const int nc = a.seg_chunks;                // every segment but the last is whole
    const size_t rb = f1_xfer_bytes(DV);
    const char *recs = static_cast<const char *>(a.ops) + (size_t(bh) * a.nchunks + size_t(g) * nc) * rb;

    // identity B operands: column 16 (n % 2) + col of a k half, rows k8 .. + 7
    bf16x8 id[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) id[p][e] = __bf16(16 * p + col == k8 + e ? 1.f : 0.f);

    f32x4 X[NCOL];
#pragma unroll
    for (int n = 0; n < NCOL; ++n) {
        X[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        put2(&XT[0][16 * n + col][16 * m + g4], make_uint2(0u, 0u));
    }
    float gam = 1.f;
    auto step = [&](int c, const MapRec<DV> &cur) {
        const bf16_t *xt = &XT[c & 1][0][0];
        bf16_t *xn = &XT[(c + 1) & 1][0][0];
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < NCOL; ++n) {
            // A~' = Gamma_c A~ + gamma A_c + A_c A~;  beta' = Gamma_c beta + A_c beta + B_c
            f32x4 acc = X[n] * cur.gc;
            if (n < DK / 16) acc += gam * mfma(n < 2 ? cur.a0 : cur.a1, id[n & 1], z);
            else acc += unpk4(cur.b[n - DK / 16]);
            acc = mfma(cur.a0, ld8(xt + (16 * n + col) * PK + k8), acc);
            acc = mfma(cur.a1, ld8(xt + (16 * n + col) * PK + 32 + k8), acc);
            X[n] = acc;
            put2(xn + (16 * n + col) * PK + 16 * m + g4, pk4(acc));
        }
        gam *= cur.gc;
        lds_barrier();
    };
    // NPF record buffers in turn: chunk c + NPF - 1 loads during step c (a
    // clamped index re-reads the last record at the end)
    MapRec<DV> buf[NPF];
#pragma unroll
    for (int u = 0; u + 1 < NPF; ++u) buf[u].load(recs + size_t(u < nc ? u : nc - 1) * rb, m, lane);
    lds_barrier();
    for (int c = 0; c < nc; c += NPF) {
#pragma unroll
        for (int u = 0; u < NPF; ++u) {
            if (c + u >= nc) break;
            const int cl = c + u + NPF - 1 < nc ? c + u + NPF - 1 : nc - 1;
            buf[(u + NPF - 1) % NPF].load(recs + size_t(cl) * rb, m, lane);
            asm volatile("" ::: "memory");   // issue the loads before the step
            step(c + u, buf[u]);
        }
    }
    // the composed map in the scan's operand order: A~ in bf16 as MFMA A
    // operands (row 16 m + col, k half h, elements 8 (lane / 16) ..), from
    // the transpose the last step left in LDS; beta as fp32 accumulator tiles
    char *M = reinterpret_cast<char *>(a.Mseg) + (size_t(bh) * a.nseg + g) * f1_segmap_bytes(DV);
    const bf16_t *xt = &XT[nc & 1][0][0];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = uint32_t(xt[(32 * h + k8 + 2 * e) * PK + 16 * m + col].bits) |
                   uint32_t(xt[(32 * h + k8 + 2 * e + 1) * PK + 16 * m + col].bits) << 16;
        *reinterpret_cast<uint4 *>(M + m * 2048 + h * 1024 + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
    }
#pragma unroll
    for (int n = 0; n < DV / 16; ++n)
        *reinterpret_cast<f32x4 *>(M + kF1SegBetaOff + ((m * (DV / 16) + n) * 64 + lane) * 16) = X[DK / 16 + n];
    if (tid == 0) a.Gseg[size_t(bh) * a.nseg + g] = gam;
}

// the parts of a segment map one scan wave uses: rows 16 m + l % 16 of A~
// as MFMA A operands, its accumulator tiles of beta, and gamma
template <int DV>
struct ScanMap {
    bf16x8 a0, a1;
    f32x4 b[DV / 16];
    float gam;
    __device__ __forceinline__ void load(const char *M, const float *G, int m, int lane) {
        a0 = ld8(M + m * 2048 + 16 * lane);
        a1 = ld8(M + m * 2048 + 1024 + 16 * lane);
#pragma unroll
        for (int n = 0; n < DV / 16; ++n)
            b[n] = *reinterpret_cast<const f32x4 *>(M + kF1SegBetaOff + ((m * (DV / 16) + n) * 64 + lane) * 16);
        gam = *G;
    }
};

// entry states of the segments of head bh, in order: S_{g+1} = gamma_g S_g +
// A~_g S_g + beta_g; wave m owns row tile m of S (all value columns)
template <int DV>
__global__ __launch_bounds__(SM_THREADS) void f1_segscan(F1XferArgs a) {
    constexpr int NJ = DV / 16;
    __shared__ __align__(16) bf16_t ST[2][DV][PK];   // bf16 S^T [j][d]
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int m = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4);
    const size_t msz = f1_segmap_bytes(DV);
    const char *Mh = reinterpret_cast<const char *>(a.Mseg) + size_t(bh) * a.nseg * msz;
    const float *Gh = a.Gseg + size_t(bh) * a.nseg;
    f32x4 S[NJ];
#pragma unroll
    for (int n = 0; n < NJ; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[n][r] = a.S_in ? a.S_in[(size_t(bh) * DK + 16 * m + g4 + r) * DV + 16 * n + col] : 0.f;
        put2(&ST[0][16 * n + col][16 * m + g4], pk4(S[n]));
    }
    const int ns = a.nseg - 1;                  // maps to apply
    auto step = [&](int g, const ScanMap<DV> &cur) {
        const bf16_t *st = &ST[g & 1][0][0];
        bf16_t *sn = &ST[(g + 1) & 1][0][0];
        // entry state of segment g + 1 as accumulator tiles [row tile][value tile][lane]
        f32x4 *Sout = reinterpret_cast<f32x4 *>(a.Sseg + (size_t(bh) * a.nseg + g + 1) * DK * DV);
#pragma unroll
        for (int n = 0; n < NJ; ++n) {
            f32x4 acc = S[n] * cur.gam + cur.b[n];
            acc = mfma(cur.a0, ld8(st + (16 * n + col) * PK + k8), acc);
            acc = mfma(cur.a1, ld8(st + (16 * n + col) * PK + 32 + k8), acc);
            S[n] = acc;
            put2(sn + (16 * n + col) * PK + 16 * m + g4, pk4(acc));
            Sout[(m * NJ + n) * 64 + lane] = acc;
        }
        lds_barrier();
    };
    // NPF map buffers in turn: map g + NPF - 1 loads during step g
    ScanMap<DV> buf[NPF];
#pragma unroll
    for (int u = 0; u + 1 < NPF; ++u) {
        const int gl = u < ns ? u : ns - 1;
        buf[u].load(Mh + gl * msz, Gh + gl, m, lane);
    }
    lds_barrier();
    for (int g = 0; g < ns; g += NPF) {
#pragma unroll
        for (int u = 0; u < NPF; ++u) {
            if (g + u >= ns) break;
            const int gl = g + u + NPF - 1 < ns ? g + u + NPF - 1 : ns - 1;
            buf[(u + NPF - 1) % NPF].load(Mh + gl * msz, Gh + gl, m, lane);
            asm volatile("" ::: "memory");   // issue the loads before the step
            step(g + u, buf[u]);
        }
    }
}

template <int DV>
void launch_xfer(const F1XferArgs &a, hipStream_t s, Marks *m) {
    // as many workgroups as fit at once (LDS: two per CU, one at d_v = 128),
    // each walking chunk ids with the grid as stride
    const int total = a.nchunks * a.BH;
    const int slots = cu_count() * (DV == 128 ? 1 : 2);
    f1_xfer<DV><<<total < slots ? total : slots, XW_THREADS, 0, s>>>(a);
    m->mark(s);
}

template <int DS>
void launch_carry(const F1XferArgs &a, hipStream_t s, Marks *m) {
    const int nslice = a.dv / DS;
    const int nbase = nslice == 1 ? a.BH : ((a.BH + 7) / 8) * 8 * nslice;
    f1_carry<DS><<<nbase * a.nseg, carry_threads<DS>(), 0, s>>>(a, nslice, nbase);
    m->mark(s);
}

template <int DV>
void launch_segments(const F1XferArgs &a, hipStream_t s, Marks *m) {
    f1_segmap<DV><<<a.BH * (a.nseg - 1), SM_THREADS, 0, s>>>(a);
    m->mark(s);
    f1_segscan<DV><<<a.BH, SM_THREADS, 0, s>>>(a);
    m->mark(s);
}

}  // namespace

void launch_chunk_f1_xfer(const F1XferArgs &a, int slice, hipStream_t s, Marks *m) {
    switch (a.dv) {
        case 32: launch_xfer<32>(a, s, m); break;
        case 64: launch_xfer<64>(a, s, m); break;
        default: launch_xfer<128>(a, s, m); break;
    }
    (void)slice;   // f1_xfer_slice: 32 columns for every d_v this path takes
    launch_f1_walk(a, s, m);
}

void launch_f1_walk(const F1XferArgs &a, hipStream_t s, Marks *m) {
    if (a.nseg > 1) {
        switch (a.dv) {
            case 32: launch_segments<32>(a, s, m); break;
            case 64: launch_segments<64>(a, s, m); break;
            default: launch_segments<128>(a, s, m); break;
        }
    }
    launch_carry<32>(a, s, m);
}

}  // namespace falcon
