// Chunk-parallel Falcon-1A forward for bf16 inputs with d_k = d_v = 64
// (summary §4.3, §4.6 "Parallel (Attention) Form of Mini-batch Inner Product
// Update", §D.1 "Mask Identities and Chunk-Local Evaluation").
//
// Per token the write is  S_t = gamma_t S_{t-1} + eta_t x_t y_t^T  and the read
// o_t = S_t^T qh_t.  Within a chunk of 64 tokens, with the chunk-local
// log-prefix b (restarted at 0 in every chunk),
//     o_i = e^{b_i} S_0^T qh_i + sum_{j <= i} e^{b_i - b_j} eta_j (qh_i . x_j) y_j,
//     S_C = e^{b_C} S_0 + sum_j e^{b_C - b_j} eta_j x_j y_j^T.
// A head's sequence is cut into segments of G chunks:
//   a1_segment (parallel over segments): the segment's aggregate write
//       D_g = sum over its chunks c of e^{b_end - b_end(c)} dS_c and its carry;
//   a1_segscan (parallel over state entries): S_{g+1} = Gamma_g S_g + D_g;
//   a1_output  (parallel over segments): walks the segment's chunks from its
//       entry state and writes o.
// Both walking kernels put the raw rows (q, k_{t-1}, v) into LDS as loaded and
// fold the RMS scales of phi into per-token factors (x = s_x k_{t-1},
// qh = s_q q).  Every operand that runs over tokens comes from registers: a
// 16 x 16 block of a row-major LDS tile, multiplied on MFMA by a 0/1 column
// picker, lands in the accumulator layout (lane holds 4 consecutive rows of
// one column).  That is the B operand of the 16x16x16 MFMA as it stands, and
// the block transposed when read as its A operand.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;
constexpr int D = 64;           // d_k = d_v
constexpr int PK = 72;          // bf16 pitch of LDS rows of 64 elements (144 bytes)
constexpr int NTH = 512;        // 8 waves

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// two floats -> bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint2 pk4(const f32x4 &v) { return make_uint2(pk2(v[0], v[1]), pk2(v[2], v[3])); }
__device__ __forceinline__ s16x4 pk4s(const f32x4 &v) { return __builtin_bit_cast(s16x4, pk4(v)); }
__device__ __forceinline__ f32x4 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const s16x4 &a, const s16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
template <class P>
__device__ __forceinline__ bf16x8 ld8(const P *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// phi's RMS scale 1 / sqrt(mean(z^2) + eps_rms) (0 when that is 0) from the
// sum of squares over 64 elements; the features are rounded to bf16 next
__device__ __forceinline__ float a1_rms_scale(float ss, float eps_rms, int phi_kind) {
    if (phi_kind == FALCON_PHI_IDENTITY) return 1.f;
    const float ms = ss * (1.f / D) + eps_rms;
    return ms > 0.f ? __builtin_amdgcn_rsqf(ms) : 0.f;
}

// per-token scalars of a chunk in LDS
enum { kEta = 0, kLg, kSx, kSq, kCoef, kQg, kCs, kB, kNsv };

// The raw rows of one chunk: 8 threads per token row, each with 8 elements of
// q, of k_{t-1} and of v, and the row's beta and lambda; loaded into registers
// one chunk ahead, unconditionally from rows clamped into [0, T).
template <bool WQ>
struct A1Rows {
    uint4 q, k, v;
    float beta, lam;
    __device__ __forceinline__ void load(const ChunkAArgs &a, int c, int bh, int row, int part) {
        const int T = a.T, t = c * C + row;
        const int tq = t < T ? t : T - 1;
        const int tk = t < 1 ? 0 : (t - 1 < T ? t - 1 : T - 1);
        const size_t base = size_t(bh) * T;
        if constexpr (WQ) q = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.q) + (base + tq) * D + 8 * part);
        k = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.k) + (base + tk) * D + 8 * part);
        v = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(a.v) + (base + tq) * D + 8 * part);
        beta = a.beta[base + tq];
        lam = a.lambda[base + tq];
    }
};

// One walk over the chunks [c_begin, c_end) of head bh.  OUT = false: the
// aggregate write of the segment (a1_segment); OUT = true: the outputs, from
// the segment's entry state (a1_output).
//
// Per chunk, after the rows and the step scalars:
//   - every wave transposes four 16 x 16 blocks on MFMA into LDS: key blocks
//     scaled by the write coefficients, XT[d][s] = coef_s x_s[d] / s_x, and
//     value blocks VT[j][s]; each block once per chunk;
//   - wave w updates the state tiles (d tiles 2 (w / 4), + 1; value tile
//     w % 4), S[d][j] += XT V by token-contracting 16x16x32 MFMAs from LDS,
//     and (a1_output) writes them to the bf16 copy S^T[j][d] that the next
//     chunk's outputs read (double-buffered by chunk parity);
//   - (a1_output) wave w forms the outputs of token tile n = 0, 0, 1, 1, 3,
//     3, 2, 2 (w = 0..7) and value tiles 2 (w % 2), + 1: the causal score
//     tiles P^T (s tile m <= n) once, kept as B operands, then
//     O^T (jt, n) = diag-scaled S^T Qh^T + V^T P^T.  Waves w and w + 4 share
//     a SIMD and hold token tiles n and 3 - n: five score tiles per SIMD.
template <bool OUT>
__device__ __forceinline__ void a1_walk(const ChunkAArgs &a, int seg, int bh, bf16_t *QB, bf16_t *XB, bf16_t *VB,
                                        bf16_t *XT, bf16_t *VT, bf16_t *STb, float (*sv)[C],
                                        bf16x8 (*IDT)[64]) {
    constexpr int NS = 2;             // state tiles per wave
    const int T = a.T;
    const int c_begin = seg * a.seg_chunks;
    const int c_end = min(a.nchunks, c_begin + a.seg_chunks);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g4 = 4 * (lane >> 4), k8 = 8 * (lane >> 4);
    const int row = tid >> 3, part = tid & 7;
    const int sj = wave & 3;                 // value tile of the state tiles
    const int sd0 = 2 * (wave >> 2);         // first d tile of the state tiles

    // rows 16 m .. + 15 of a row-major LDS tile (pitch PK), columns
    // 16 n .. + 15, in the accumulator layout: lane holds rows 16 m + g4 .. + 3
    // of column 16 n + col
    auto transposed = [&](const bf16_t *rows, int m, int n) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        return mfma32(ld8(rows + (16 * m + col) * PK + 32 * (n >> 1) + k8), IDT[n & 1][lane], z);
    };

    f32x4 S[NS];
    {
        if constexpr (OUT) {
            const float *Se = a.Sseg + (size_t(bh) * a.nseg + seg) * D * D;
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                const int dt = sd0 + h;
#pragma unroll
                for (int r = 0; r < 4; ++r) S[h][r] = Se[(16 * dt + g4 + r) * D + 16 * sj + col];
                // bf16 copy S^T [j][d] for the output products (buffer 0 of two)
                *reinterpret_cast<uint2 *>(STb + (16 * sj + col) * PK + 16 * dt + g4) = pk4(S[h]);
            }
        } else {
#pragma unroll
            for (int h = 0; h < NS; ++h) S[h] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    float bsum = 0.f;   // log2 of the segment's carry

    // one chunk step; the rows of chunk c + 1 go into `rows` once chunk c's
    // are consumed
    A1Rows<OUT> rows;
    rows.load(a, c_begin, bh, row, part);
    for (int c = c_begin; c < c_end; ++c) {
        const int c0 = c * C, t = c0 + row;
        // 1. rows to LDS as loaded; RMS scales, eta and log2 gamma
        {
            uint4 xr = rows.k;
            float sq = 0.f, sk = 0.f;
            const uint32_t kw[4] = {xr.x, xr.y, xr.z, xr.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2_t ke = __builtin_bit_cast(bf16x2_t, kw[e]);
                sk = __builtin_amdgcn_fdot2_f32_bf16(ke, ke, sk, false);
            }
            if constexpr (OUT) {
                const uint32_t qw[4] = {rows.q.x, rows.q.y, rows.q.z, rows.q.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bf16x2_t qe = __builtin_bit_cast(bf16x2_t, qw[e]);
                    sq = __builtin_amdgcn_fdot2_f32_bf16(qe, qe, sq, false);
                }
            }
            const bool qok = t < T, kok = t >= 1 && t <= T, first = t == 0;
            const bool carry_x = first && a.xnext_in;
            if (carry_x) {   // x_0 continues the previous segment (features formed, scale 1)
                const f32x4 *xp = reinterpret_cast<const f32x4 *>(a.xnext_in + size_t(bh) * D + 8 * part);
                const f32x4 x0 = xp[0], x1 = xp[1];
                sk = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) sk += x0[e] * x0[e] + x1[e] * x1[e];
                xr = make_uint4(pk2(x0[0], x0[1]), pk2(x0[2], x0[3]), pk2(x1[0], x1[1]), pk2(x1[2], x1[3]));
            }
            sk = group_sum<8>(sk);
            const float sck = carry_x ? 1.f : (kok ? a1_rms_scale(sk, a.eps_rms, a.phi) : 0.f);
            *reinterpret_cast<uint4 *>(XB + row * PK + 8 * part) = xr;
            *reinterpret_cast<uint4 *>(VB + row * PK + 8 * part) = qok ? rows.v : make_uint4(0, 0, 0, 0);
            float scq = 0.f;
            if constexpr (OUT) {
                sq = group_sum<8>(sq);
                scq = qok ? a1_rms_scale(sq, a.eps_rms, a.phi) : 0.f;
                *reinterpret_cast<uint4 *>(QB + row * PK + 8 * part) = rows.q;
            }
            if (part == 0) {
                float eta = 0.f, alpha = 0.f;
                if (!(t >= T || (first && a.fresh))) {   // the fresh first step writes nothing
                    const float den = sck * sck * sk + rows.lam + a.eps;   // |x_t|^2 + lambda_t + eps
                    eta = den != 0.f ? rows.beta * __builtin_amdgcn_rcpf(den) : 0.f;
                    alpha = step_alpha(eta, rows.lam, a.eps_gamma);
                }
                sv[kEta][row] = eta;
                sv[kLg][row] = log2_1m(alpha);
                sv[kSx][row] = sck;
                sv[kSq][row] = scq;
            }
            if (c + 1 < c_end) rows.load(a, c + 1, bh, row, part);
        }
        __syncthreads();

        // 2. chunk-local prefix b (base 2), lane = token; every wave forms the
        //    same values (identical LDS writes), so no barrier is needed
        bool sep;
        float bC;
        {
            const float lg = sv[kLg][lane];
            const float b = wave_inclusive_scan(lg);
            bC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b), 63));
            sep = bC >= -100.f;
            const float eta = sv[kEta][lane], sx = sv[kSx][lane];
            sv[kCoef][lane] = ex2(bC - b) * eta * sx;   // chunk write coefficient of token lane
            if constexpr (OUT) {
                const float sq = sv[kSq][lane];
                sv[kQg][lane] = ex2(b) * sq;                         // e^{b_i} s_q
                sv[kCs][lane] = (sep ? ex2(-b) : 1.f) * eta * sx;    // (e^{-b_j}) eta_j s_x
                sv[kB][lane] = b;
            }
        }
        wave_lds_sync();
        bsum += bC;

        // 3. transposes, once per block: wave w takes token block m = w / 2
        //    and the d / value tiles 2 (w % 2), + 1
        {
            const int m = wave >> 1;
            const f32x4 cf = *reinterpret_cast<const f32x4 *>(&sv[kCoef][16 * m + g4]);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int n = 2 * (wave & 1) + e;
                const f32x4 xb = transposed(XB, m, n) * cf;
                const f32x4 vb = transposed(VB, m, n);
                *reinterpret_cast<uint2 *>(XT + (16 * n + col) * PK + 16 * m + g4) = pk4(xb);
                *reinterpret_cast<uint2 *>(VT + (16 * n + col) * PK + 16 * m + g4) = pk4(vb);
            }
        }
        __syncthreads();

        {
            // 4. state tiles: S = e^{b_C} S + X^T diag(coef) V
            const float gC = ex2(bC);
            const bf16_t *vr = VT + (16 * sj + col) * PK + k8;
            const bf16x8 v0 = ld8(vr), v1 = ld8(vr + 32);
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                const bf16_t *xr = XT + (16 * (sd0 + h) + col) * PK + k8;
                f32x4 s = S[h] * gC;
                s = mfma32(ld8(xr), v0, s);
                S[h] = mfma32(ld8(xr + 32), v1, s);
            }
            if constexpr (OUT) {
                // the next chunk's S^T copy goes to the other buffer: its last
                // reads were before the previous chunk's closing barrier
                bf16_t *stn = STb + ((c + 1 - c_begin) & 1) * (D * PK);
#pragma unroll
                for (int h = 0; h < NS; ++h)
                    *reinterpret_cast<uint2 *>(stn + (16 * sj + col) * PK + 16 * (sd0 + h) + g4) = pk4(S[h]);
            }
        }
        if constexpr (OUT) {
            // 5. outputs O^T (jt, n) = diag-scaled S^T Qh^T + V^T P^T, from the
            //    entry state's copy
            const bf16_t *stc = STb + ((c - c_begin) & 1) * (D * PK);
            bf16_t *og = static_cast<bf16_t *>(a.o) + size_t(bh) * T * D + g4;
            const int n = wave < 4 ? wave >> 1 : 3 - ((wave - 4) >> 1);
            const int tq = 16 * n + col;   // this lane's token
            const bf16_t *qr = QB + tq * PK + k8;
            const bf16x8 q0 = ld8(qr), q1 = ld8(qr + 32);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const float qg = sv[kQg][tq];
            // separable decays: e^{-b_s} eta_s s_x times e^{b_t} s_q; else
            // e^{b_t - b_s} times eta_s s_x times s_q
            const float bq = sep ? 0.f : sv[kB][tq], qf = sep ? qg : sv[kSq][tq];
            // score tiles P^T (m, n): lane holds x_s . q_t at s = 16 m + g4 + r, t = tq
            s16x4 pt[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m > n) break;
                const bf16_t *xr = XB + (16 * m + col) * PK + k8;
                f32x4 p = mfma32(ld8(xr), q0, z);
                p = mfma32(ld8(xr + 32), q1, p);
                const f32x4 cs = *reinterpret_cast<const f32x4 *>(&sv[kCs][16 * m + g4]);
                const f32x4 bs = *reinterpret_cast<const f32x4 *>(&sv[kB][16 * m + g4]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float f = (sep ? 1.f : ex2(bq - bs[r])) * cs[r] * qf;
                    p[r] = (m < n || g4 + r <= col) ? p[r] * f : 0.f;
                }
                pt[m] = pk4s(p);
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int jt = 2 * (wave & 1) + e;
                const bf16_t *sr = stc + (16 * jt + col) * PK + k8;
                f32x4 o = mfma32(ld8(sr), q0, z);
                o = mfma32(ld8(sr + 32), q1, o);
                o *= qg;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (m > n) break;
                    const s16x4 va = __builtin_bit_cast(
                        s16x4, *reinterpret_cast<const uint2 *>(VT + (16 * jt + col) * PK + 16 * m + g4));
                    o = mfma16(va, pt[m], o);
                }
                if (c0 + tq < T) *reinterpret_cast<uint2 *>(og + size_t(c0 + tq) * D + 16 * jt) = pk4(o);
            }
        }
        __syncthreads();   // the next chunk overwrites the rows, transposes and scalars
    }

    if constexpr (!OUT) {
        // segment aggregate D_g (fp32, [d][j]) and its carry
        float *Dg = a.Dseg + (size_t(bh) * a.nseg + seg) * D * D;
#pragma unroll
        for (int h = 0; h < NS; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) Dg[(16 * (sd0 + h) + g4 + r) * D + 16 * sj + col] = S[h][r];
        if (tid == 0) a.Gseg[size_t(bh) * a.nseg + seg] = ex2(bsum);
        // x for the next segment, phi(k_{T-1}), from the segment holding the last token
        if (c_end == a.nchunks && wave == 0 && a.xnext_out) {
            const bf16_t *kg = static_cast<const bf16_t *>(a.k) + size_t(bh) * T * D;
            const float xv = bf16_to_f32(kg[size_t(T - 1) * D + lane].bits);
            const float sc = phi_scale(wave_sum(xv * xv), D, a.eps_rms, a.phi);
            a.xnext_out[size_t(bh) * D + lane] = xv * sc;
        }
    }
}

// B operands that pick 16 columns (half h) of a 32-wide A block
__device__ __forceinline__ void init_pickers(bf16x8 (*IDT)[64]) {
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 128) {
        typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
        const int h = tid >> 6, col = lane & 15, k8 = 8 * (lane >> 4);
        u16x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = (k8 + e == 16 * h + col) ? 0x3F80 : 0;   // bf16 1.0
        IDT[h][lane] = __builtin_bit_cast(bf16x8, u);
    }
}

__global__ __launch_bounds__(NTH, 4) void a1_segment(ChunkAArgs a) {
    __shared__ __align__(16) bf16_t XB[C * PK];
    __shared__ __align__(16) bf16_t VB[C * PK];
    __shared__ __align__(16) bf16_t XT[D * PK];
    __shared__ __align__(16) bf16_t VT[D * PK];
    __shared__ __align__(16) float sv[kNsv][C];
    __shared__ __align__(16) bf16x8 IDT[2][64];
    init_pickers(IDT);
    __syncthreads();
    a1_walk<false>(a, blockIdx.x, blockIdx.y, nullptr, XB, VB, XT, VT, nullptr, sv, IDT);
}

__global__ __launch_bounds__(NTH, 4) void a1_output(ChunkAArgs a) {
    __shared__ __align__(16) bf16_t QB[C * PK];
    __shared__ __align__(16) bf16_t XB[C * PK];
    __shared__ __align__(16) bf16_t VB[C * PK];
    __shared__ __align__(16) bf16_t XT[D * PK];
    __shared__ __align__(16) bf16_t VT[D * PK];
    __shared__ __align__(16) bf16_t STb[2 * D * PK];
    __shared__ __align__(16) float sv[kNsv][C];
    __shared__ __align__(16) bf16x8 IDT[2][64];
    init_pickers(IDT);
    // (the entry state's bf16 copy is written inside the walk; the first
    // barrier of the walk orders it and the pickers before their first reads)
    a1_walk<true>(a, blockIdx.x, blockIdx.y, QB, XB, VB, XT, VT, STb, sv, IDT);
}

// entry state of every segment: S_{g+1} = Gamma_g S_g + D_g (one thread per
// state entry; the segment writes are loaded 32 at a time, so that one
// memory latency covers a whole head at the usual segment counts)
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
    constexpr int NB = 32;
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

}  // namespace

void launch_chunk_a1(const ChunkAArgs &a, hipStream_t s, Marks *m) {
    a1_segment<<<dim3(a.nseg, a.BH), NTH, 0, s>>>(a);
    m->mark(s);
    a1_segscan<<<dim3(a.BH, D * D / 256), 256, 0, s>>>(a);
    m->mark(s);
    a1_output<<<dim3(a.nseg, a.BH), NTH, 0, s>>>(a);
    m->mark(s);
}

}  // namespace falcon
