// Chunk-parallel Falcon-1A and Falcon-3A forward for bf16 inputs with
// d_k = d_v = 64 (summary §4.3, §4.5, §4.6 "Parallel (Attention) Form of
// Mini-batch Inner Product Update", §D.1 "Mask Identities and Chunk-Local
// Evaluation"; Falcon-1A is the window-1 case).
//
// Per token s the write is  S_s = gamma_s S_{s-1} + w_s sum_{j in I_s} x_j y_j^T,
// w_s = eta_s / B_s, I_s the last B_s = min(W, #pairs) pairs, and the read is
// o_t = S_t^T qh_t.  Within a chunk of 64 tokens, with the chunk-local
// log-prefix b (restarted at 0 in every chunk),
//     o_t = e^{b_t} S_0^T qh_t + sum_j M_tj (qh_t . x_j) y_j,
//     S_C = e^{b_C} S_0 + sum_j M_{63,j} x_j y_j^T,
//     M_tj = sum_{s = max(j,0)}^{min(t, j+W-1)} e^{b_t - b_s} w_s,
// where j runs over the W - 1 pairs before the chunk (the halo) and the
// chunk's own pairs.  With c'_j = M_{hi_j, j}, hi_j = min(j + W - 1, 63) (a
// sum of at most W terms, every factor <= 1):
//   - past the window, t >= j + W - 1:  M_tj = e^{b_t - b_{hi_j}} c'_j, which
//     separates into a token factor e^{b_t} and a pair factor e^{-b_{hi_j}} c'_j
//     while e^{-b} stays in range (chunk decay above 2^-100), and is formed
//     pairwise otherwise;
//   - in the band j <= t < j + W - 1 (at most W - 1 pairs per token): the sum
//     itself, at most W - 1 terms;
//   - the chunk write coefficient: M_{63,j} = e^{b_63 - b_{hi_j}} c'_j.
//
// A head's sequence is cut into segments of G chunks:
//   a3_window  (Falcon-3A only, one wave per chunk): the window statistic
//       mu_t = lambda_max(window Gram) / B_t from the banded pair Gram (MFMA)
//       and the step scalars w_t, log2 gamma_t of every token;
//   a1_segment (parallel over segments): the segment's aggregate write
//       D_g = sum over its chunks c of e^{b_end - b_end(c)} dS_c and its carry,
//       and the boundary state (x_next, the last W - 1 pairs);
//   a1_segscan (parallel over state entries, more than kFoldSegs segments):
//       S_{g+1} = Gamma_g S_g + D_g (with fewer, every output walk folds its
//       own entry state from the aggregates);
//   a1_output  (parallel over segments): walks the segment's chunks from its
//       entry state and writes o.
// Both walking kernels put the raw rows (q, k_{t-1}, v) into LDS as loaded and
// fold the RMS scales of phi into per-token and per-pair factors (x = s_x
// k_{t-1}, qh = s_q q).  Every operand that runs over tokens comes from a
// transposed copy: a 16 x 16 block of a row-major LDS tile, multiplied on
// MFMA by a 0/1 column picker, lands in the accumulator layout (lane holds 4
// consecutive rows of one column), which is written to LDS with one 8-byte
// store per lane, once per block.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;
constexpr int D = 64;           // d_k = d_v
constexpr int PK = 72;          // bf16 pitch of LDS rows of 64 elements (144 bytes)
constexpr int NTH = 512;        // 8 waves

// pair rows of a chunk: WIN adds a 16-row halo tile in front (pair row of
// the chunk's first token OFF = 16; the halo pairs sit in rows 16 - (W - 1)
// .. 15, rows below are zero)
template <bool WIN>
struct Geo {
    static constexpr int OFF = WIN ? 16 : 0;
    static constexpr int NP = OFF + C;      // pair rows
    static constexpr int NMT = NP / 16;     // pair tiles
    static constexpr int PX = NP + 8;       // bf16 pitch of the transposed rows [d or j][pair]
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// two floats -> bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint2 pk4(const f32x4 &v) { return make_uint2(pk2(v[0], v[1]), pk2(v[2], v[3])); }
__device__ __forceinline__ s16x4 pk4s(const f32x4 &v) { return __builtin_bit_cast(s16x4, pk4(v)); }
__device__ __forceinline__ uint4 pk8(const f32x4 &a, const f32x4 &b) {
    return make_uint4(pk2(a[0], a[1]), pk2(a[2], a[3]), pk2(b[0], b[1]), pk2(b[2], b[3]));
}
__device__ __forceinline__ f32x4 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const s16x4 &a, const s16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
template <class P>
__device__ __forceinline__ bf16x8 ld8(const P *p) { return *reinterpret_cast<const bf16x8 *>(p); }
template <class P>
__device__ __forceinline__ s16x4 ld4(const P *p) { return __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(p)); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// sum of squares of 8 bf16 values (one 16-byte piece of a row)
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

// phi's RMS scale 1 / sqrt(mean(z^2) + eps_rms) (0 when that is 0) from the
// sum of squares over 64 elements; the features are rounded to bf16 next
__device__ __forceinline__ float a1_rms_scale(float ss, float eps_rms, int phi_kind) {
    if (phi_kind == FALCON_PHI_IDENTITY) return 1.f;
    const float ms = ss * (1.f / D) + eps_rms;
    return ms > 0.f ? __builtin_amdgcn_rsqf(ms) : 0.f;
}

// 8 fp32 features of an incoming boundary row (x_next or a tail pair, phi
// already applied) -> bf16 piece and its sum of squares
__device__ __forceinline__ uint4 feat8(const float *src, float &ss) {
    const f32x4 x0 = reinterpret_cast<const f32x4 *>(src)[0], x1 = reinterpret_cast<const f32x4 *>(src)[1];
    ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += x0[e] * x0[e] + x1[e] * x1[e];
    return pk8(x0, x1);
}

// A halo pair (position tau < c0, a row of the halo tile) as 8 elements
// (part `part`) of x and of y, with x's RMS scale: x = phi(k_{tau-1}) of the
// sequence, the incoming x_next (tau = 0) or an incoming tail pair (tau < 0);
// pairs that do not exist (before the incoming tail, rows outside the
// window, the fresh sentinel's x) are zero.  `hk`, `hv` are the raw rows
// k_{tau-1}, v_tau (loaded clamped).  The 8 lanes of a row take the same
// branches.
__device__ __forceinline__ void halo_pair(const ChunkAArgs &a, int bh, int tau, bool in_window, int part,
                                          const uint4 &hk, const uint4 &hv, uint4 &xr, uint4 &yr, float &sc) {
    const int H = a.window - 1;
    const bool exists = in_window && tau >= -a.n_tail_in;
    float ss = 0.f;
    bool raw = false;
    xr = make_uint4(0, 0, 0, 0);
    yr = make_uint4(0, 0, 0, 0);
    if (exists && tau >= 1) {
        xr = hk;
        ss = sumsq8(hk);
        raw = true;
    } else if (exists && tau == 0 && a.xnext_in) {
        xr = feat8(a.xnext_in + size_t(bh) * D + 8 * part, ss);
    } else if (exists && tau < 0) {
        xr = feat8(a.tailx_in + (size_t(bh) * H + H + tau) * D + 8 * part, ss);
    }
    if (exists && tau >= 0) {
        yr = hv;
    } else if (exists && tau < 0) {
        float dummy;
        yr = feat8(a.taily_in + (size_t(bh) * H + H + tau) * D + 8 * part, dummy);
    }
    ss = group_sum<8>(ss);
    const bool xz = !exists || (tau == 0 && !a.xnext_in);
    sc = xz ? 0.f : (raw ? a1_rms_scale(ss, a.eps_rms, a.phi) : 1.f);
}

constexpr int kFoldSegs = chunk_a1_fold_segments;

// s_waitcnt immediate (gfx9 encoding) that waits for all vector memory
// operations: vmcnt 0 (bits 3:0 and 15:14), expcnt 7 and lgkmcnt 15 (no wait)
constexpr int kWaitVmcnt0 = 0x0F70;

// per-token scalars of a chunk (LDS, [kind][token]) and per-pair scalars
// ([kind][pair row])
enum { kW = 0, kLg, kSq, kQg, kB, kNtv };
enum { pSx = 0, pCoef, pCol, pBh, kNpv };

// The raw rows of one chunk: 8 threads per token row, each with 8 elements of
// q, of k_{t-1} and of v, and the row's two step inputs (beta and lambda;
// with a window, w_t and log2 gamma_t from the window pass).  Loaded into
// registers one chunk ahead, unconditionally from rows clamped into [0, T).
template <bool WQ, bool WIN>
struct A1Rows {
    uint4 q, k, v;
    float s0, s1;
    __device__ __forceinline__ void load(const ChunkAArgs &a, int c, int bh, int row, int part) {
        const int T = a.T, t = c * C + row;
        const int tq = t < T ? t : T - 1;
        const int tk = t < 1 ? 0 : (t - 1 < T ? t - 1 : T - 1);
        const size_t base = size_t(bh) * T;
        const bf16_t *kg = static_cast<const bf16_t *>(a.k), *vg = static_cast<const bf16_t *>(a.v);
        if constexpr (WQ) q = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.q) + (base + tq) * D + 8 * part);
        k = *reinterpret_cast<const uint4 *>(kg + (base + tk) * D + 8 * part);
        v = *reinterpret_cast<const uint4 *>(vg + (base + tq) * D + 8 * part);
        if constexpr (WIN) {
            s0 = a.etaw[size_t(bh) * a.Tpad + t];
            s1 = a.lg[size_t(bh) * a.Tpad + t];
        } else {
            s0 = a.beta[base + tq];
            s1 = a.lambda[base + tq];
        }
    }
};

// One walk over the chunks [c_begin, c_end) of head bh.  OUT = false: the
// aggregate write of the segment (a1_segment); OUT = true: the outputs, from
// the segment's entry state (a1_output).  WIN: a window of W > 1 pairs.
//
// Per chunk, after the rows and the step scalars:
//   - the pair coefficients: c'_j, the chunk write coefficient and the score
//     column factor of every pair (without a window every wave forms the same
//     values; with one, two waves form them and a barrier publishes them);
//   - waves 0-3 transpose the key blocks (scaled by the write coefficients),
//     XT[d][p], and waves 4-7 the value blocks, VT[j][p], NMT each, on MFMA
//     into LDS; each block once per chunk;
//   - wave w updates the state tiles (d tiles 2 (w / 4), + 1; value tile
//     w % 4), S[d][j] += XT V by pair-contracting MFMAs from LDS, and
//     (a1_output) the next chunk writes them to the bf16 copy S^T[j][d] that
//     its outputs read (after this chunk's closing barrier);
//   - (a1_output) wave w forms the outputs of token tile n = 0, 0, 1, 1, 3,
//     3, 2, 2 (w = 0..7) and value tiles 2 (w % 2), + 1:
//     O^T (jt, n) = diag-scaled S^T Qh^T + V^T P^T, each score tile P^T of
//     the pair tiles up to the diagonal formed once and fed as the B operand
//     to both value tiles.  Waves w and w + 4 share a SIMD and hold token
//     tiles n and 3 - n, which balances the score work.
template <bool OUT, bool WIN>
__device__ __forceinline__ void a1_walk(const ChunkAArgs &a, int seg, int bh, bf16_t *QB, bf16_t *XB, bf16_t *VB,
                                        bf16_t *XH, bf16_t *VH, float (*hsx)[16], bf16_t *XT, bf16_t *VT,
                                        bf16_t *STb, float (*tv)[C], float (*pv)[Geo<WIN>::NP], float (*bf)[C]) {
    using G = Geo<WIN>;
    constexpr int OFF = G::OFF, NP = G::NP, NMT = G::NMT, PX = G::PX;
    constexpr int NS = 2;             // state tiles per wave
    const int T = a.T;
    const int H = WIN ? a.window - 1 : 0;
    const int c_begin = seg * a.seg_chunks;
    const int c_end = min(a.nchunks, c_begin + a.seg_chunks);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4);
    const int row = tid >> 3, part = tid & 7;
    const int sj = wave & 3;                 // value tile of the state tiles
    const int sd0 = 2 * (wave >> 2);         // first d tile of the state tiles

    // B operands that pick 16 columns (half h) of a 32-wide A block: the MFMA
    // then hands back that half transposed into the accumulator layout.  Kept
    // in registers (8 VGPRs): read from LDS by every transpose they were a
    // third of the transposes' LDS traffic.
    bf16x8 pick0, pick1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
        u16x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = (k8 + e == 16 * h + col) ? 0x3F80 : 0;   // bf16 1.0
        (h ? pick1 : pick0) = __builtin_bit_cast(bf16x8, u);
    }
    // a 16-row tile of row-major LDS rows (pitch PK), columns 16 n .. + 15,
    // in the accumulator layout: lane holds rows g4 .. + 3 of column 16 n + col
    auto transposed = [&](const bf16_t *tile, int n) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        return mfma32(ld8(tile + col * PK + 32 * (n >> 1) + k8), (n & 1) ? pick1 : pick0, z);
    };

    // first row of pair tile m: the halo tile (WIN, m = 0) of this chunk's
    // parity, else the token rows
    auto ptile = [&](const bf16_t *rows, const bf16_t *halo, int m, int par) {
        if constexpr (WIN) return m == 0 ? halo + par * (16 * PK) : rows + (m - 1) * (16 * PK);
        return rows + m * (16 * PK);
    };

    f32x4 S[NS];
    if constexpr (OUT) {
        if (a.nseg <= kFoldSegs) {
            // entry state folded here from the incoming state and the
            // earlier segments' aggregates, S_{g+1} = Gamma_g S_g + D_g (all
            // loads first)
            constexpr int NBF = 4;   // aggregates loaded per batch
            const size_t e0 = size_t(16 * sd0 + g4) * D + 16 * sj + col;
            float Sv[NS][4];
#pragma unroll
            for (int h = 0; h < NS; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Sv[h][r] = a.S_in ? a.S_in[size_t(bh) * D * D + e0 + size_t(16 * h + r) * D] : 0.f;
            for (int g0 = 0; g0 < seg; g0 += NBF) {
                float Dv[NBF][NS][4], Gv[NBF];
#pragma unroll
                for (int u = 0; u < NBF; ++u) {
                    const int gc = g0 + u < seg ? g0 + u : g0;   // loads stay inside the segments present
                    const float *Dg = a.Dseg + (size_t(bh) * a.nseg + gc) * D * D + e0;
#pragma unroll
                    for (int h = 0; h < NS; ++h)
#pragma unroll
                        for (int r = 0; r < 4; ++r) Dv[u][h][r] = Dg[size_t(16 * h + r) * D];
                    Gv[u] = a.Gseg[size_t(bh) * a.nseg + gc];
                }
#pragma unroll
                for (int u = 0; u < NBF; ++u)
#pragma unroll
                    for (int h = 0; h < NS; ++h)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            Sv[h][r] = g0 + u < seg ? Gv[u] * Sv[h][r] + Dv[u][h][r] : Sv[h][r];
            }
#pragma unroll
            for (int h = 0; h < NS; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[h][r] = Sv[h][r];
        } else {
            const float *Se = a.Sseg + (size_t(bh) * a.nseg + seg) * D * D;
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                const int dt = sd0 + h;
#pragma unroll
                for (int r = 0; r < 4; ++r) S[h][r] = Se[(16 * dt + g4 + r) * D + 16 * sj + col];
            }
        }
    } else {
#pragma unroll
        for (int h = 0; h < NS; ++h) S[h] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float bsum = 0.f;   // log2 of the segment's carry

    if constexpr (WIN) {
        // the first chunk's halo tile from memory (later chunks take theirs
        // from the previous chunk's rows); ordered by the first barrier
        if (row < 16) {
            const int tau = c_begin * C - 16 + row;
            const size_t base = size_t(bh) * T;
            const int hkr = tau < 1 ? 0 : tau - 1, hvr = tau < 0 ? 0 : tau;
            const uint4 hk = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.k) + (base + hkr) * D + 8 * part);
            const uint4 hv = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.v) + (base + hvr) * D + 8 * part);
            uint4 hx, hy;
            float hs;
            halo_pair(a, bh, tau, row >= 16 - H, part, hk, hv, hx, hy, hs);
            *reinterpret_cast<uint4 *>(XH + row * PK + 8 * part) = hx;
            *reinterpret_cast<uint4 *>(VH + row * PK + 8 * part) = hy;
            if (part == 0) hsx[0][row] = hs;
        }
    }

    // the incoming x_0 (features, scale 1) of a continued sequence, loaded
    // once, outside the chunk loop (a conditional load inside it added a wait
    // for every outstanding memory operation to each chunk), and kept in LDS
    // (registers would hold it through every chunk)
    __shared__ __align__(16) uint4 x0r[8];
    __shared__ float x0s;
    if (c_begin == 0 && row == 0 && a.xnext_in) {
        float ss;
        x0r[part] = feat8(a.xnext_in + size_t(bh) * D + 8 * part, ss);
        ss = group_sum<8>(ss);   // over the row's 8 lanes, all active here
        if (part == 0) x0s = ss;
    }

    A1Rows<OUT, WIN> rows;
    rows.load(a, c_begin, bh, row, part);
    // Wait for the first rows here, once, so that the loop is entered with
    // no loads pending: the compiler then waits for each row of the next
    // chunk as it is needed instead of for all of them at the loop head.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int c = c_begin; c < c_end; ++c) {
        // lane quantities formed afresh in every chunk from an opaque copy of
        // the thread index (hoisted, their derived addresses would hold
        // registers through the loop)
        int tid_o = tid;
        asm volatile("" : "+v"(tid_o));
        const int lane = tid_o & 63, col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4);
        const int row = tid_o >> 3, part = tid_o & 7;
        const int c0 = c * C, t = c0 + row;
        if constexpr (OUT) {
            // bf16 copy S^T [j][d] of the chunk's entry state for the output
            // products; the previous chunk's last reads of the copy came
            // before its closing barrier
#pragma unroll
            for (int h = 0; h < NS; ++h)
                *reinterpret_cast<uint2 *>(STb + (16 * sj + col) * PK + 16 * (sd0 + h) + g4) = pk4(S[h]);
        }
        // 1. rows to LDS as loaded; RMS scales; the step scalars
        {
            uint4 xr = rows.k;
            float sk = sumsq8(xr);
            float sq = 0.f;
            if constexpr (OUT) sq = sumsq8(rows.q);
            const bool qok = t < T, kok = t >= 1 && t <= T, first = t == 0;
            const bool carry_x = first && a.xnext_in;
            sk = group_sum<8>(sk);
            if (carry_x) {   // x_0: features, scale 1 (row 0 of the first chunk, its 8 lanes together)
                xr = x0r[part];
                sk = x0s;
            }
            const float sck = carry_x ? 1.f : (kok ? a1_rms_scale(sk, a.eps_rms, a.phi) : 0.f);
            const uint4 yr = qok ? rows.v : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(XB + row * PK + 8 * part) = xr;
            *reinterpret_cast<uint4 *>(VB + row * PK + 8 * part) = yr;
            float scq = 0.f;
            if constexpr (OUT) {
                sq = group_sum<8>(sq);
                scq = qok ? a1_rms_scale(sq, a.eps_rms, a.phi) : 0.f;
                *reinterpret_cast<uint4 *>(QB + row * PK + 8 * part) = rows.q;
            }
            // the step scalars, formed on every lane of the row without
            // branches; part 0 stores them
            float w, lg;
            if constexpr (WIN) {
                w = rows.s0;     // eta_t / B_t and log2 gamma_t from the window pass
                lg = rows.s1;
            } else {
                const bool live = !(t >= T || (first && a.fresh));   // the fresh first step writes nothing
                const float den = sck * sck * sk + rows.s1 + a.eps;    // |x_t|^2 + lambda_t + eps
                const float eta = (live && den != 0.f) ? rows.s0 * __builtin_amdgcn_rcpf(den) : 0.f;
                const float alpha = live ? step_alpha(eta, rows.s1, a.eps_gamma) : 0.f;
                w = eta;
                lg = log2_1m(alpha);
            }
            if (part == 0) {
                tv[kW][row] = w;
                tv[kLg][row] = lg;
                tv[kSq][row] = scq;
                pv[pSx][OFF + row] = sck;
            }
            if constexpr (WIN) {
                // the last 16 pair rows are the next chunk's halo tile (rows
                // outside its window zero), in the other parity's buffer
                if (row >= C - 16) {
                    const int h = row - (C - 16), nxt = (c + 1 - c_begin) & 1;
                    const bool inw = h >= 16 - H;
                    *reinterpret_cast<uint4 *>(XH + (nxt * 16 + h) * PK + 8 * part) = inw ? xr : make_uint4(0, 0, 0, 0);
                    *reinterpret_cast<uint4 *>(VH + (nxt * 16 + h) * PK + 8 * part) = inw ? yr : make_uint4(0, 0, 0, 0);
                    if (part == 0) hsx[nxt][h] = inw ? sck : 0.f;
                }
            }
            if (c + 1 < c_end) rows.load(a, c + 1, bh, row, part);
        }
        __syncthreads();

        // 2. chunk-local prefix b (base 2), lane = token, and the pair
        //    coefficients.  Every wave forms b (identical LDS writes).  Without
        //    a window every wave also forms the pair coefficients, so no
        //    barrier is needed; with one (band of the mask, 80 pair rows of up
        //    to W terms each) wave 0 forms the band and waves 1 and 2 the pair
        //    rows, and a barrier publishes them
        bool sep;
        float bC;
        {
            const float lg = tv[kLg][lane];
            const float b = wave_inclusive_scan(lg);
            bC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b), 63));
            sep = bC >= -100.f;
            tv[kB][lane] = b;
            if constexpr (OUT) tv[kQg][lane] = ex2(b) * tv[kSq][lane];   // e^{b_t} s_q
            wave_lds_sync();
            if constexpr (OUT && WIN) {
                // band of the mask: bf[u][t] = M_{t, t-u} = sum_{s = max(t-u, 0)}^{t}
                // e^{b_t - b_s} w_s for u < W - 1 (pairs still in the window at t)
                if (wave == 0) {
                    float mc = 0.f;
                    for (int u = 0; u < H; ++u) {
                        const int s = lane - u, sc = s > 0 ? s : 0;
                        mc += s >= 0 ? ex2(b - tv[kB][sc]) * tv[kW][sc] : 0.f;
                        bf[u][lane] = mc;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < (NP + 63) / 64; ++u) {
                const int p = lane + 64 * u;
                if (p < NP && (!WIN || wave == 1 + u)) {
                    const int j = p - OFF;                     // pair's token (chunk-local)
                    const int lo = j > 0 ? j : 0, hi = j + H < C - 1 ? j + H : C - 1;
                    // c'_j: at most W terms (none for rows before the window)
                    const bool live = j >= -H;
                    const float bhi = live ? tv[kB][hi] : 0.f;
                    float cp = 0.f;
                    for (int u = 0; u <= H; ++u) {
                        const int s = lo + u, sc = s < hi ? s : hi;
                        cp += (live && s <= hi) ? ex2(bhi - tv[kB][sc]) * tv[kW][sc] : 0.f;
                    }
                    const float sx = p < OFF ? hsx[(c - c_begin) & 1][p] : pv[pSx][p];
                    if (p < OFF) pv[pSx][p] = sx;
                    pv[pCoef][p] = ex2(bC - bhi) * cp * sx;              // M_{63,j} s_x
                    pv[pCol][p] = (sep ? ex2(-bhi) : 1.f) * cp * sx;     // (e^{-b_hi}) c'_j s_x
                    pv[pBh][p] = bhi;
                }
            }
        }
        if constexpr (WIN) __syncthreads();
        else wave_lds_sync();
        bsum += bC;

        // 3. transposes, once per block: waves 0-3 the key blocks (scaled by
        //    the write coefficients), waves 4-7 the value blocks; NMT blocks
        //    each (pair tile m, d or value tile n)
        {
            const int par = (c - c_begin) & 1;
            if (wave < 4) {
#pragma unroll
                for (int e = 0; e < NMT; ++e) {
                    const int b = wave * NMT + e, m = b >> 2, n = b & 3;
                    const f32x4 cf = *reinterpret_cast<const f32x4 *>(&pv[pCoef][16 * m + g4]);
                    const f32x4 tb = transposed(ptile(XB, XH, m, par), n) * cf;
                    *reinterpret_cast<uint2 *>(XT + (16 * n + col) * PX + 16 * m + g4) = pk4(tb);
                }
            } else {
#pragma unroll
                for (int e = 0; e < NMT; ++e) {
                    const int b = (wave - 4) * NMT + e, m = b >> 2, n = b & 3;
                    const f32x4 tb = transposed(ptile(VB, VH, m, par), n);
                    *reinterpret_cast<uint2 *>(VT + (16 * n + col) * PX + 16 * m + g4) = pk4(tb);
                }
            }
        }
        __syncthreads();

        {
            // 4. state tiles: S = e^{b_C} S + X^T diag(coef) V over the pairs
            const float gC = ex2(bC);
            const bf16_t *vr = VT + (16 * sj + col) * PX;
            const bf16x8 v0 = ld8(vr + k8), v1 = ld8(vr + 32 + k8);
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                const bf16_t *xr = XT + (16 * (sd0 + h) + col) * PX;
                f32x4 s = S[h] * gC;
                s = mfma32(ld8(xr + k8), v0, s);
                s = mfma32(ld8(xr + 32 + k8), v1, s);
                // the halo pairs' 16-deep product in an accumulator of its
                // own, added on the vector ALU: an accumulator handed from a
                // 16x16x32 MFMA straight to a 16x16x16 one is not safe
                if constexpr (WIN) s += mfma16(ld4(xr + 64 + g4), ld4(vr + 64 + g4), f32x4{0.f, 0.f, 0.f, 0.f});
                S[h] = s;
            }
        }
        if constexpr (OUT) {
            // 5. outputs O^T (jt, n) = diag-scaled S^T Qh^T + V^T P^T, from the
            //    entry state's copy
            const bf16_t *stc = STb;
            bf16_t *og = static_cast<bf16_t *>(a.o) + size_t(bh) * T * D + g4;
            const int n = wave < 4 ? wave >> 1 : 3 - ((wave - 4) >> 1);
            const int tq = 16 * n + col;   // this lane's token
            const bf16_t *qr = QB + tq * PK + k8;
            const bf16x8 q0 = ld8(qr), q1 = ld8(qr + 32);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const float qg = tv[kQg][tq];
            const float bq = tv[kB][tq], sqq = tv[kSq][tq];
            // past the window: separable, (e^{b_t} s_q)(e^{-b_hi} c' s_x), or
            // e^{b_t - b_hi} s_q (c' s_x)
            const float qf = sep ? qg : sqq;
            // O^T for value tiles jt0 = 2 (w % 2) and jt0 + 1: the state term
            // first, then each score tile P^T (m, n) (lane holds x_p . q_t at
            // pair row p = 16 m + g4 + r, token t = tq) is formed once and fed
            // to both
            const int jt0 = 2 * (wave & 1);
            f32x4 o0, o1;
            {
                const bf16_t *sr0 = stc + (16 * jt0 + col) * PK + k8, *sr1 = sr0 + 16 * PK;
                o0 = mfma32(ld8(sr0), q0, z);
                o0 = mfma32(ld8(sr0 + 32), q1, o0) * qg;
                o1 = mfma32(ld8(sr1), q0, z);
                o1 = mfma32(ld8(sr1 + 32), q1, o1) * qg;
            }
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                if (m > n + OFF / 16) break;
                const bf16_t *xr = ptile(XB, XH, m, (c - c_begin) & 1) + col * PK + k8;
                f32x4 p = mfma32(ld8(xr), q0, z);
                p = mfma32(ld8(xr + 32), q1, p);
                const f32x4 cl = *reinterpret_cast<const f32x4 *>(&pv[pCol][16 * m + g4]);
                const f32x4 bh4 = *reinterpret_cast<const f32x4 *>(&pv[pBh][16 * m + g4]);
                // t - j >= 16 (n - m) + OFF - 15 over the tile: every pair of a
                // tile that far back is past the window (or, with no window,
                // at or before every token), so it takes the plain factor
                if (16 * (n - m) + OFF - 15 >= (WIN ? H : 0)) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) p[r] *= (sep ? 1.f : ex2(bq - bh4[r])) * cl[r] * qf;
                } else {
                    f32x4 sxb;
                    if constexpr (WIN) sxb = *reinterpret_cast<const f32x4 *>(&pv[pSx][16 * m + g4]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * m + g4 + r - OFF;   // pair's token (chunk-local)
                        // past the window, before the pair (0), or in the band
                        // (the pair still in the window at t)
                        float f = (sep ? 1.f : ex2(bq - bh4[r])) * cl[r] * qf;
                        if constexpr (WIN) {
                            const int u = tq - j, uc = u < 0 ? 0 : (u < FALCON_MAX_WINDOW - 1 ? u : FALCON_MAX_WINDOW - 2);
                            const float fb = bf[uc][tq] * sxb[r] * sqq;
                            f = u >= H ? f : (u < 0 ? 0.f : fb);
                        } else {
                            f = tq >= j ? f : 0.f;
                        }
                        p[r] *= f;
                    }
                }
                const s16x4 pt = pk4s(p);
                o0 = mfma16(ld4(VT + (16 * jt0 + col) * PX + 16 * m + g4), pt, o0);
                o1 = mfma16(ld4(VT + (16 * jt0 + 16 + col) * PX + 16 * m + g4), pt, o1);
            }
            if (c0 + tq < T) {
                *reinterpret_cast<uint2 *>(og + size_t(c0 + tq) * D + 16 * jt0) = pk4(o0);
                *reinterpret_cast<uint2 *>(og + size_t(c0 + tq) * D + 16 * jt0 + 16) = pk4(o1);
            }
        }
        // The next chunk overwrites the rows, scalars and halo tiles, and then
        // the transposes.  The outputs read the rows here, so a1_output
        // closes the chunk with a barrier.  The segment walk's last reads of
        // them come before the second barrier, and its state tiles (the last
        // reads of the transposes) finish before any wave passes the next
        // chunk's first barrier.
        if constexpr (OUT) __syncthreads();
    }

    if constexpr (OUT) {
        // with the entry states folded in the walks, the final state comes
        // from the last segment's walk
        if (a.nseg <= kFoldSegs && c_end == a.nchunks && a.S_out) {
#pragma unroll
            for (int h = 0; h < NS; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a.S_out[size_t(bh) * D * D + size_t(16 * (sd0 + h) + g4 + r) * D + 16 * sj + col] = S[h][r];
        }
    }
    if constexpr (!OUT) {
        // segment aggregate D_g (fp32, [d][j]) and its carry
        float *Dg = a.Dseg + (size_t(bh) * a.nseg + seg) * D * D;
#pragma unroll
        for (int h = 0; h < NS; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) Dg[(16 * (sd0 + h) + g4 + r) * D + 16 * sj + col] = S[h][r];
        if (tid == 0) a.Gseg[size_t(bh) * a.nseg + seg] = ex2(bsum);
        // the boundary state from the segment holding the last token
        if (c_end == a.nchunks && wave == 0) {
            const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * D;
            const bf16_t *vg = static_cast<const bf16_t *>(a.v) + size_t(bh) * T * D;
            if (a.xnext_out) {   // x for the next segment: phi(k_{T-1})
                const float xv = bf16_to_f32(kg[size_t(T - 1) * D + lane].bits);
                const float sc = phi_scale(wave_sum(xv * xv), D, a.eps_rms, a.phi);
                a.xnext_out[size_t(bh) * D + lane] = xv * sc;
            }
            if (WIN && a.tailx_out) {   // the last W - 1 pairs (features, values), right-aligned
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
}

template <bool WIN>
__global__ __launch_bounds__(NTH, 4) void a1_segment(ChunkAArgs a) {
    using G = Geo<WIN>;
    __shared__ __align__(16) bf16_t XB[C * PK];
    __shared__ __align__(16) bf16_t VB[C * PK];
    __shared__ __align__(16) bf16_t XH[WIN ? 2 * 16 * PK : 8];   // halo tiles by chunk parity
    __shared__ __align__(16) bf16_t VH[WIN ? 2 * 16 * PK : 8];
    __shared__ __align__(16) float hsx[2][16];
    __shared__ __align__(16) bf16_t XT[D * G::PX];
    __shared__ __align__(16) bf16_t VT[D * G::PX];
    __shared__ __align__(16) float tv[kNtv][C];
    __shared__ __align__(16) float pv[kNpv][G::NP];
    a1_walk<false, WIN>(a, blockIdx.x, blockIdx.y, nullptr, XB, VB, XH, VH, hsx, XT, VT, nullptr, tv, pv, nullptr);
}

template <bool WIN>
__global__ __launch_bounds__(NTH, 4) void a1_output(ChunkAArgs a) {
    using G = Geo<WIN>;
    __shared__ __align__(16) bf16_t QB[C * PK];
    __shared__ __align__(16) bf16_t XB[C * PK];
    __shared__ __align__(16) bf16_t VB[C * PK];
    __shared__ __align__(16) bf16_t XH[WIN ? 2 * 16 * PK : 8];   // halo tiles by chunk parity
    __shared__ __align__(16) bf16_t VH[WIN ? 2 * 16 * PK : 8];
    __shared__ __align__(16) float hsx[2][16];
    __shared__ __align__(16) bf16_t XT[D * G::PX];
    __shared__ __align__(16) bf16_t VT[D * G::PX];
    __shared__ __align__(16) bf16_t STb[D * PK];
    __shared__ __align__(16) float tv[kNtv][C];
    __shared__ __align__(16) float pv[kNpv][G::NP];
    __shared__ __align__(16) float bf[WIN ? FALCON_MAX_WINDOW - 1 : 1][C];
    // (the entry state's bf16 copy is written inside the walk; the first
    // barrier of the walk orders it before its first reads)
    a1_walk<true, WIN>(a, blockIdx.x, blockIdx.y, QB, XB, VB, XH, VH, hsx, XT, VT, STb, tv, pv, bf);
}

// Falcon-3A window statistic and step scalars of one chunk (one wave): the
// pair rows of the chunk and its halo, the band of the pair Gram
// (x_p . x_{p-d}, d < 8) on MFMA, then per token t the window Gram of its
// B_t pairs, mu_t = lambda_max / B_t, eta_t = beta_t / (mu_t + lambda_t + eps),
// w_t = eta_t / B_t and log2 gamma_t to the workspace (0 past T and at a
// fresh first token).
__global__ __launch_bounds__(64) void a3_window(ChunkAArgs a) {
    // pair rows without padding, the 16-byte pieces of row p at positions
    // piece ^ (p % 8) (conflict-free operand reads); the band rows padded to
    // 9 floats, so that the 64 lanes (consecutive rows p) of each gather
    // below fall in 64 different banks.  13.1 KB, so that every chunk of the
    // workload finds a slot at once (twelve per CU)
    __shared__ __align__(16) bf16_t XR[80 * D];
    __shared__ float sx[80];
    __shared__ float band[80][9];
    const int c = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
    const int W = a.window, H = W - 1, T = a.T, c0 = c * C;
    const int part = lane & 7, col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4);
    const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * D;
    // pair rows p = 0..79 at positions tau = c0 - 16 + p, eight rows a pass;
    // all ten passes' key rows, and this lane's token's beta and lambda, are
    // requested before any is used
    uint4 raws[10];
#pragma unroll
    for (int it = 0; it < 10; ++it) {
        const int tau = c0 - 16 + 8 * it + (lane >> 3);
        const int kr = tau < 1 ? 0 : (tau - 1 < T ? tau - 1 : T - 1);
        raws[it] = *reinterpret_cast<const uint4 *>(kg + size_t(kr) * D + 8 * part);
    }
    const int tl = c0 + lane < T ? c0 + lane : T - 1;
    const float beta = a.beta[size_t(bh) * T + tl], lam = a.lambda[size_t(bh) * T + tl];
#pragma unroll
    for (int it = 0; it < 10; ++it) {
        const int p = 8 * it + (lane >> 3);
        const int tau = c0 - 16 + p;
        const uint4 raw = raws[it];
        uint4 xr, yr;
        float sc;
        if (p < 16) {
            halo_pair(a, bh, tau, p >= 16 - H, part, raw, make_uint4(0, 0, 0, 0), xr, yr, sc);
        } else {   // the chunk's own pairs (x_0 from the boundary when continuing)
            float ss = sumsq8(raw);
            xr = raw;
            const bool carry_x = tau == 0 && a.xnext_in;
            if (carry_x) xr = feat8(a.xnext_in + size_t(bh) * D + 8 * part, ss);
            ss = group_sum<8>(ss);
            sc = carry_x ? 1.f : ((tau >= 1 && tau < T) ? a1_rms_scale(ss, a.eps_rms, a.phi) : 0.f);
        }
        *reinterpret_cast<uint4 *>(XR + p * D + 8 * (part ^ (p & 7))) = xr;
        if (part == 0) sx[p] = sc;
    }
    __syncthreads();
    // band of the pair Gram: tiles (m, m) for m = 0..4 and (m, m - 1) for m = 1..4
    for (int tile = 0; tile < 9; ++tile) {
        const int m = tile < 5 ? tile : tile - 4, mp = tile < 5 ? m : m - 1;
        // row r's elements 8 k .. + 7 (piece k), for this lane's k8 and the
        // two k halves
        auto piece = [&](int r, int k) { return ld8(XR + r * D + 8 * (k ^ (r & 7))); };
        const int ra = 16 * m + col, rb = 16 * mp + col, kq = k8 >> 3;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 g = mfma32(piece(ra, kq), piece(rb, kq), z);
        g = mfma32(piece(ra, kq + 4), piece(rb, kq + 4), g);
        // lane holds x_p . x_q for p = 16 m + g4 + r, q = 16 mp + col
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int p = 16 * m + g4 + r, q = 16 * mp + col, d = p - q;
            if (d >= 0 && d < 8) band[p][d] = g[r] * sx[p] * sx[q];
        }
    }
    __syncthreads();
    const int t = c0 + lane, p = 16 + lane;
    float w = 0.f, lg = 0.f;
    if (t < T && !(t == 0 && a.fresh)) {
        const long long pairs = (long long)a.n_tail_in + t + 1;
        const int bt = pairs < W ? int(pairs) : W;
        float g[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int lo = i < j ? i : j, df = i < j ? j - i : i - j;
                g[i][j] = (i < bt && j < bt) ? band[p - lo][df] : 0.f;
            }
        const float mu = psd_lambda_max(g, bt) / float(bt);
        const float eta = step_eta(beta, mu + lam + a.eps);
        w = eta / float(bt);
        lg = log2_1m(step_alpha(eta, lam, a.eps_gamma));
    }
    a.etaw[size_t(bh) * a.Tpad + t] = w;
    a.lg[size_t(bh) * a.Tpad + t] = lg;
}

// entry state of every segment: S_{g+1} = Gamma_g S_g + D_g (one thread per
// state entry; the segment writes are loaded 32 at a time, so that one
// memory latency covers a whole head at the usual segment counts)
template <int NB>   // segment writes loaded per batch
__global__ __launch_bounds__(256) void a1_segscan(ChunkAArgs a) {
    const int bh = blockIdx.x;
    const int e = blockIdx.y * 256 + threadIdx.x;   // d * 64 + j
    if (e >= D * D) return;
    float S = a.S_in ? a.S_in[size_t(bh) * D * D + e] : 0.f;
    const size_t stride = size_t(D) * D;
    const float *Dg = a.Dseg + size_t(bh) * a.nseg * stride + e;
    float *Se = a.Sseg + size_t(bh) * a.nseg * stride + e;
    const float *Gg = a.Gseg + size_t(bh) * a.nseg;
    const int nseg = a.nseg;
    for (int g0 = 0; g0 < nseg; g0 += NB) {
        float dv[NB], gv[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int g = g0 + u < nseg ? g0 + u : nseg - 1;
            dv[u] = Dg[g * stride];
            gv[u] = Gg[g];
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (g0 + u < nseg) {
                Se[(g0 + u) * stride] = S;
                S = gv[u] * S + dv[u];
            }
        }
    }
    if (a.S_out) a.S_out[size_t(bh) * D * D + e] = S;
}

template <bool WIN>
void launch_walks(const ChunkAArgs &a, hipStream_t s, Marks *m) {
    a1_segment<WIN><<<dim3(a.nseg, a.BH), NTH, 0, s>>>(a);
    m->mark(s);
    if (a.nseg > kFoldSegs) {
        a1_segscan<32><<<dim3(a.BH, D * D / 256), 256, 0, s>>>(a);
        m->mark(s);
    }
    a1_output<WIN><<<dim3(a.nseg, a.BH), NTH, 0, s>>>(a);
    m->mark(s);
}

}  // namespace

void launch_a3_window(const ChunkAArgs &a, hipStream_t s, Marks *m) {
    a3_window<<<dim3(a.nchunks, a.BH), 64, 0, s>>>(a);
    m->mark(s);
}

void launch_chunk_a1(const ChunkAArgs &a, hipStream_t s, Marks *m) {
    if (a.window > 1) {
        launch_a3_window(a, s, m);
        launch_walks<true>(a, s, m);
    } else {
        launch_walks<false>(a, s, m);
    }
}

}  // namespace falcon
