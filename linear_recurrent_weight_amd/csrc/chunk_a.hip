// Chunk-parallel Falcon-1A / Falcon-3A forward (inner-product writes with a
// scalar ridge carry; summary §4.3, §4.5, §4.6 "Parallel (Attention) Form of
// Mini-batch Inner Product Update", §D.1 "Mask Identities and Chunk-Local
// Evaluation"; Falcon-1A is the window-1 case).
//
// Per token s the write is  S_s = gamma_s S_{s-1} + w_s sum_{j in I_s} x_j y_j^T,
// w_s = eta_s / B_s, I_s the last min(W, #pairs) pairs.  Within a chunk of 64
// tokens (chunk-local log-prefix b, restarted at 0) this unrolls to
//     o_t = e^{b_t} S_0^T qh_t + sum_j M_tj (qh_t . x_j) y_j,
//     S_C = e^{b_C} S_0 + sum_j M_{C,j} x_j y_j^T,
//     M_tj = sum_{s = max(j,0)}^{min(t, j+W-1)} e^{b_t - b_s} w_s,
// where j runs over the W-1 halo pairs before the chunk and the chunk's own
// pairs.  Each column of M obeys the first-order recurrence
//     M_tj = gamma_t M_{t-1,j} + [max(j,0) <= t <= j+W-1] w_t,
// so every decay factor is a product of carries in (0, 1] and nothing can
// overflow however strong the ridge.
//
// The sequence of a head is cut into segments of G chunks:
//   a_segment  (parallel over segments): features (QK-RMSNorm, key shift),
//              step scalars (window statistic lambda_max for Falcon-3A), and
//              the segment's aggregate write D_g = sum over its chunks of the
//              decayed chunk writes (MFMA), with its carry Gamma_g;
//   a_segscan  (parallel over state entries): S_{g+1} = Gamma_g S_g + D_g;
//   a_output   (parallel over segments): walks the segment's chunks from its
//              entry state, with S^T held in MFMA accumulators, and writes o.
#include "chunk_layout.h"
#include "kernels.h"
#include "mma.h"

namespace falcon {
namespace {

constexpr int C = kChunk;
constexpr int HMAX = FALCON_MAX_WINDOW - 1;  // halo pairs
constexpr int KP = 96;                       // pair slots per chunk (64 + halo, padded)
constexpr int kOutThreads = 512;             // a_output: 8 waves (its LDS allows one workgroup per CU)
constexpr int kSegThreads = 256;             // a_segment: 4 waves (the window solver's registers)

// N consecutive elements of a row held as raw words (16- or 8-byte loads)
template <class E, int N>
struct RowPart {
    static constexpr int BYTES = N * int(sizeof(E));
    static constexpr int W4 = BYTES / 16;
    static constexpr int W2 = (BYTES % 16) / 8;
    static_assert(BYTES % 8 == 0, "row parts are whole 8-byte words");
    uint4 a[W4 > 0 ? W4 : 1];
    uint2 b[W2 > 0 ? W2 : 1];
    __device__ void clear() {
#pragma unroll
        for (int i = 0; i < (W4 > 0 ? W4 : 1); ++i) a[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < (W2 > 0 ? W2 : 1); ++i) b[i] = make_uint2(0, 0);
    }
    __device__ void load(const E *p) {
#pragma unroll
        for (int i = 0; i < W4; ++i) a[i] = reinterpret_cast<const uint4 *>(p)[i];
#pragma unroll
        for (int i = 0; i < W2; ++i) b[i] = reinterpret_cast<const uint2 *>(p + W4 * 16 / int(sizeof(E)))[i];
    }
    __device__ uint32_t word(int w) const {   // 32-bit word w of the part
        if (w < 4 * W4) {
            const uint4 &u = a[w >> 2];
            const int c = w & 3;
            return c == 0 ? u.x : c == 1 ? u.y : c == 2 ? u.z : u.w;
        }
        const uint2 &u = b[(w - 4 * W4) >> 1];
        return ((w - 4 * W4) & 1) ? u.y : u.x;
    }
    __device__ float get(int i) const {
        if constexpr (sizeof(E) == 2) {
            const uint32_t w = word(i >> 1);
            return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
        } else {
            return __uint_as_float(word(i));
        }
    }
};

// N consecutive values (N a multiple of 8 for bf16, of 4 for fp32) to a
// 16-byte aligned destination with vector stores
template <class E, int N>
__device__ __forceinline__ void store_vec(E *dst, const float *v) {
    if constexpr (sizeof(E) == 2) {
        static_assert(N % 8 == 0, "bf16 rows in 16-byte pieces");
        auto p2 = [](float x, float y) { return uint32_t(f32_to_bf16(x)) | (uint32_t(f32_to_bf16(y)) << 16); };
#pragma unroll
        for (int i = 0; i < N / 8; ++i)
            reinterpret_cast<uint4 *>(dst)[i] = make_uint4(p2(v[8 * i], v[8 * i + 1]), p2(v[8 * i + 2], v[8 * i + 3]),
                                                           p2(v[8 * i + 4], v[8 * i + 5]), p2(v[8 * i + 6], v[8 * i + 7]));
    } else {
        static_assert(N % 4 == 0, "fp32 rows in 16-byte pieces");
#pragma unroll
        for (int i = 0; i < N / 4; ++i)
            reinterpret_cast<float4 *>(dst)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
}

// Raw rows of one chunk, prefetched into registers: 4 threads per row, pair
// rows p = row and 64 + row (the halo makes at most 71 pairs), and the
// chunk's query rows.  tau = c0 - halo + p is the pair's token.
template <class E, int DK, int DV, bool WITH_Q>
struct ChunkRows {
    RowPart<E, DK / 4> kr[2];
    RowPart<E, DV / 4> vr[2];
    RowPart<E, DK / 4> qr;

    __device__ void prefetch(const ChunkAArgs &a, int bh, int c0, int halo) {
        const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
        const int np = C + halo;
        const E *k = static_cast<const E *>(a.k) + size_t(bh) * a.T * DK;
        const E *v = static_cast<const E *>(a.v) + size_t(bh) * a.T * a.dv;
        // unconditional loads from rows clamped into [0, T) (a load under a
        // branch is waited for where the branch joins); rows outside the
        // sequence are zeroed when the pairs are staged
        auto clampT = [&](int r) { return r < 0 ? 0 : (r < a.T ? r : a.T - 1); };
        (void)np;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int p = 64 * pass + row;
            const int tau = c0 - halo + p;
            kr[pass].load(k + size_t(clampT(tau - 1)) * DK + part * (DK / 4));
            vr[pass].load(v + size_t(clampT(tau)) * a.dv + part * (DV / 4));
        }
        if constexpr (WITH_Q) {
            const E *q = static_cast<const E *>(a.q) + size_t(bh) * a.T * DK;
            qr.load(q + size_t(clampT(c0 + row)) * DK + part * (DK / 4));
        }
    }

    // normalised pair features into xf[p][ldx] (fp32) and / or xe[p][lde]
    // (storage type, 16-byte vector stores), their squared norms into nrm[p]
    // and values into yt[j][p]
    __device__ void store_pairs(const ChunkAArgs &a, int bh, int c0, int halo, float *xf, int ldx, E *xe,
                                int lde, E *yt, int ldy, float *nrm) const {
        const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
        const int np = C + halo;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int p = 64 * pass + row;
            const int tau = c0 - halo + p;
            float x[DK / 4];
            bool from_k = p < np && tau >= 1 && tau < a.T;
#pragma unroll
            for (int e = 0; e < DK / 4; ++e) x[e] = from_k ? kr[pass].get(e) : 0.f;
            if (p < np && tau == 0 && a.xnext_in) {
#pragma unroll
                for (int e = 0; e < DK / 4; ++e) x[e] = a.xnext_in[size_t(bh) * DK + part * (DK / 4) + e];
            } else if (p < np && tau < 0 && tau >= -a.n_tail_in) {
                const float *src = a.tailx_in + (size_t(bh) * halo + tau + halo) * DK + part * (DK / 4);
#pragma unroll
                for (int e = 0; e < DK / 4; ++e) x[e] = src[e];
            }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < DK / 4; ++e) ss += x[e] * x[e];
            ss = group_sum<4>(ss);
            const float sc = from_k ? phi_scale(ss, DK, a.eps_rms, a.phi) : 1.f;
#pragma unroll
            for (int e = 0; e < DK / 4; ++e) x[e] *= sc;
            if (p < 64 + HMAX) {
                if (xf) {
#pragma unroll
                    for (int e = 0; e < DK / 4; ++e) xf[p * ldx + part * (DK / 4) + e] = x[e];
                }
                if (nrm && part == 0) nrm[p] = sc * sc * ss;
            }
            if (xe && p < KP) store_vec<E, DK / 4>(xe + size_t(p) * lde + part * (DK / 4), x);
            const bool y_ok = p < np && tau >= 0 && tau < a.T;
            float y[DV / 4];
#pragma unroll
            for (int e = 0; e < DV / 4; ++e) y[e] = y_ok ? vr[pass].get(e) : 0.f;
            if (p < np && tau < 0 && tau >= -a.n_tail_in) {
                const float *src = a.taily_in + (size_t(bh) * halo + tau + halo) * a.dv + part * (DV / 4);
#pragma unroll
                for (int e = 0; e < DV / 4; ++e) y[e] = src[e];
            }
            if (p < KP) {
#pragma unroll
                for (int e = 0; e < DV / 4; ++e) st(yt, size_t(part * (DV / 4) + e) * ldy + p, y[e]);
            }
        }
        // padding pair slots [128, KP) never exist (KP <= 128); slots [np, KP)
        // were written with zeros above (their rows were cleared)
    }

    // normalised query features into qe[t][ldq] (16-byte vector stores)
    __device__ void store_queries(const ChunkAArgs &a, int c0, E *qe, int ldq) const {
        const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
        const bool ok = c0 + row < a.T;
        float y[DK / 4];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < DK / 4; ++e) {
            y[e] = ok ? qr.get(e) : 0.f;
            ss += y[e] * y[e];
        }
        ss = group_sum<4>(ss);
        const float sc = phi_scale(ss, DK, a.eps_rms, a.phi);
#pragma unroll
        for (int e = 0; e < DK / 4; ++e) y[e] *= sc;
        store_vec<E, DK / 4>(qe + size_t(row) * ldq + part * (DK / 4), y);
    }
};

// ---------------------------------------------------------------------------
// a_segment
// ---------------------------------------------------------------------------
template <class E, int DK, int DV>
__global__ __launch_bounds__(kSegThreads) void a_segment(ChunkAArgs a) {
    constexpr int PD = Pad<E>::v;
    constexpr int LDX = DK + 1;         // fp32 feature rows
    constexpr int LDT = KP + PD;        // [.][pair] rows
    constexpr int NPM = C + HMAX;       // max pairs per chunk
    __shared__ float XF[NPM * LDX];
    __shared__ __align__(16) E XT[DK * LDT];     // (diag(coef) X)^T  [d][p]
    __shared__ __align__(16) E YT[DV * LDT];     // Y^T               [j][p]
    __shared__ float band[NPM * 8];
    __shared__ float mu_s[C], ew_s[C], gam_s[C], coef[KP], nrm[NPM];
    __shared__ float bC_s;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.T, dv = a.dv, W = a.window, halo = W - 1;
    const int np = C + halo;
    ChunkRows<E, DK, DV, false> rows;

    // aggregate write of the segment, transposed: D^T[j][d] in accumulators.
    // tile (jt, dt) with jt < dv/16, dt < DK/16, spread over the waves
    constexpr int NW = kSegThreads / 64;
    constexpr int MAXT = (DV / 16 * DK / 16 + NW - 1) / NW;   // state tiles per wave
    constexpr int njt = DV / 16, ntiles = njt * (DK / 16);
    f32x4 acc[MAXT];
#pragma unroll
    for (int m = 0; m < MAXT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float bsum = 0.f;

    const int c_begin = seg * a.seg_chunks;
    const int c_end = min(a.nchunks, c_begin + a.seg_chunks);
    // the row loads and the feature pass run on waves 0-3 (4 threads per row)
    const bool rw = wave < 4;
    if (rw) rows.prefetch(a, bh, c_begin * C, halo);
    for (int c = c_begin; c < c_end; ++c) {
        const int c0 = c * C;
        if (rw) rows.store_pairs(a, bh, c0, halo, XF, LDX, static_cast<E *>(nullptr), 0, YT, LDT, nrm);
        // unconditional (clamped) loads; unused past the sequence end
        const int tcl = c0 + (tid & 63) < T ? c0 + (tid & 63) : T - 1;
        const float beta_t = a.beta[size_t(bh) * T + tcl];
        const float lam_t = a.lambda[size_t(bh) * T + tcl];
        if (rw && c + 1 < c_end) rows.prefetch(a, bh, c0 + C, halo);
        __syncthreads();
        // window statistic / feature energy of the chunk's own tokens
        if (W > 1) {
            for (int idx = tid; idx < np * W; idx += kSegThreads) {
                const int r = idx / W, d = idx % W;
                float s = 0.f;
                if (r - d >= 0) {
                    for (int e = 0; e < DK; ++e) s += XF[r * LDX + e] * XF[(r - d) * LDX + e];
                }
                band[r * 8 + d] = s;
            }
            __syncthreads();
            if (tid < C) {
                const int r = tid + halo;
                float g[8][8];
#pragma unroll
                for (int aa = 0; aa < 8; ++aa)
#pragma unroll
                    for (int bb = 0; bb < 8; ++bb) {
                        float v = 0.f;
                        if (aa < W && bb < W) {
                            const int lo = aa < bb ? aa : bb, df = aa < bb ? bb - aa : aa - bb;
                            v = band[(r - lo) * 8 + df];
                        }
                        g[aa][bb] = v;
                    }
                const long long pairs = (long long)a.n_tail_in + c0 + tid + 1;
                const int bt = pairs < W ? int(pairs) : W;
                mu_s[tid] = psd_lambda_max(g, W) / float(bt);
                ew_s[tid] = 1.f / float(bt);
            }
        } else if (tid < C) {
            mu_s[tid] = nrm[tid + halo];   // ||x_t||^2 from the feature pass
            ew_s[tid] = 1.f;
        }
        __syncthreads();
        // step scalars; log-prefix of the chunk
        if (wave == 0) {
            const int t = c0 + lane;
            float eta = 0.f, alpha = 0.f;
            const bool noop = t >= T || (t == 0 && a.fresh);
            if (!noop) {
                eta = step_eta(beta_t, mu_s[lane] + lam_t + a.eps);
                alpha = step_alpha(eta, lam_t, a.eps_gamma);
            }
            const float lg = log1pf(-alpha);
            const float ew = eta * ew_s[lane];
            ew_s[lane] = ew;
            gam_s[lane] = 1.f - alpha;
            a.etaw[size_t(bh) * a.Tpad + t] = ew;
            a.lg[size_t(bh) * a.Tpad + t] = lg;
            const float b = wave_inclusive_scan(lg);
            if (lane == 63) bC_s = b;
        }
        __syncthreads();
        // coefficients of the chunk write: coef_p = M_{63, p}
        if (tid < KP) {
            const int p = tid, j = p - halo, t_lo = j > 0 ? j : 0, t_hi = j + halo;
            float m = 0.f;
            for (int t0 = 0; t0 < C; t0 += 8) {
                float gm[8], ew[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    gm[u] = gam_s[t0 + u];
                    ew[u] = ew_s[t0 + u];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int t = t0 + u;
                    m = gm[u] * m + ((t >= t_lo && t <= t_hi) ? ew[u] : 0.f);
                }
            }
            coef[p] = p < np ? m : 0.f;
        }
        __syncthreads();
        for (int idx = tid; idx < KP * DK; idx += kSegThreads) {
            const int p = idx / DK, d = idx % DK;
            st(XT, size_t(d) * LDT + p, p < np ? coef[p] * XF[p * LDX + d] : 0.f);
        }
        __syncthreads();
        // D^T = e^{b_C} D^T + Y^T diag(coef) X
        const float gC = expf(bC_s);
        bsum += bC_s;
#pragma unroll
        for (int m = 0; m < MAXT; ++m) {
            const int tile = wave + NW * m;
            if (tile < ntiles) {
                const int jt = tile % njt, dt = tile / njt;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[m][r] *= gC;
                acc[m] = Mma<E>::run(acc[m], YT + 16 * jt * LDT, LDT, XT + 16 * dt * LDT, LDT, 0, KP);
            }
        }
        // boundary state out from the last chunk of the sequence
        if (c == a.nchunks - 1 && halo > 0 && a.tailx_out) {
            const int n_out = a.n_tail_out;
            for (int idx = tid; idx < halo * DK; idx += kSegThreads) {
                const int sl = idx / DK, e = idx % DK;
                const int tau = T - halo + sl;
                const int p = tau - (c0 - halo);
                a.tailx_out[(size_t(bh) * halo + sl) * DK + e] = sl >= halo - n_out ? XF[p * LDX + e] : 0.f;
            }
            for (int idx = tid; idx < halo * dv; idx += kSegThreads) {
                const int sl = idx / dv, e = idx % dv;
                const int tau = T - halo + sl;
                const int p = tau - (c0 - halo);
                a.taily_out[(size_t(bh) * halo + sl) * dv + e] =
                    sl >= halo - n_out ? ld(YT, size_t(e) * LDT + p) : 0.f;
            }
        }
        __syncthreads();
    }
    // segment aggregate (fp32, [j][d]) and carry
    float *Dg = a.Dseg + (size_t(bh) * a.nseg + seg) * dv * DK;
#pragma unroll
    for (int m = 0; m < MAXT; ++m) {
        const int tile = wave + NW * m;
        if (tile < ntiles) {
            const int jt = tile % njt, dt = tile / njt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jt + 4 * (lane >> 4) + r, d = 16 * dt + (lane & 15);
                Dg[size_t(j) * DK + d] = acc[m][r];
            }
        }
    }
    if (tid == 0) a.Gseg[size_t(bh) * a.nseg + seg] = expf(bsum);
    // x_next = phi(k_{T-1}) from the segment holding the last token
    if (c_end == a.nchunks && wave == 0 && a.xnext_out) {
        const E *k = static_cast<const E *>(a.k) + size_t(bh) * T * DK;
        float x[2] = {0.f, 0.f};
        for (int m = 0; m < 2; ++m)
            if (lane + 64 * m < DK) x[m] = ld(k, size_t(T - 1) * DK + lane + 64 * m);
        const float sc = phi_scale(wave_sum(x[0] * x[0] + x[1] * x[1]), DK, a.eps_rms, a.phi);
        for (int m = 0; m < 2; ++m)
            if (lane + 64 * m < DK) a.xnext_out[size_t(bh) * DK + lane + 64 * m] = x[m] * sc;
    }
}

// ---------------------------------------------------------------------------
// a_segscan: entry state of every segment
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void a_segscan(ChunkAArgs a) {
    const int bh = blockIdx.x;
    const int e = blockIdx.y * 256 + threadIdx.x;
    const int dk = a.dk, dv = a.dv;
    if (e >= dk * dv) return;
    const int j = e / dk, d = e % dk;
    float S = a.S_in ? a.S_in[(size_t(bh) * dk + d) * dv + j] : 0.f;
    const size_t stride = size_t(dk) * dv;
    const float *Dg = a.Dseg + size_t(bh) * a.nseg * stride + e;
    float *Se = a.Sseg + size_t(bh) * a.nseg * stride + e;
    const float *Gg = a.Gseg + size_t(bh) * a.nseg;
    for (int g = 0; g < a.nseg; ++g) {
        Se[g * stride] = S;
        S = Gg[g] * S + Dg[g * stride];
    }
    if (a.S_out) a.S_out[(size_t(bh) * dk + d) * dv + j] = S;
}

// ---------------------------------------------------------------------------
// a_output
// ---------------------------------------------------------------------------
template <class E> struct PBuf;     // bf16: separate scores buffer; fp32: scores in place
template <> struct PBuf<bf16_t> { static constexpr bool separate = true; };
template <> struct PBuf<float> { static constexpr bool separate = false; };

template <class E, int DK, int DV>
__global__ __launch_bounds__(kOutThreads) void a_output(ChunkAArgs a) {
    constexpr int PD = Pad<E>::v;
    constexpr int LDK = DK + PD;        // [.][d] rows
    constexpr int LDT = KP + PD;        // [.][pair] rows
    constexpr int LDF = KP + 1;         // fp32 score rows
    constexpr int NPM = C + HMAX;
    __shared__ __align__(16) E XE[KP * LDK];             // pair features [p][d]
    __shared__ __align__(16) E XT[DK * LDT];             // (diag(coef) X)^T [d][p]
    __shared__ __align__(16) E QE[C * LDK];              // query features [t][d]
    __shared__ __align__(16) E YT[DV * LDT];             // Y^T [j][p]
    __shared__ __align__(16) E ST[DV * LDK];             // S^T copy [j][d]
    __shared__ __align__(16) float PF[C * LDF];          // scores, then decayed scores
    __shared__ __align__(16) E PE[PBuf<E>::separate ? C * LDT : 1];
    __shared__ float ew_s[C], gam_s[C], g_s[C], coef[KP], mend_s[KP];
    __shared__ float bC_s;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.T, dv = a.dv, W = a.window, halo = W - 1;
    const int np = C + halo;
    ChunkRows<E, DK, DV, true> rows;
    E *o = static_cast<E *>(a.o) + size_t(bh) * T * dv;

    // entry state S^T[j][d] of this segment in accumulators, tiles spread
    // over the 8 waves
    constexpr int NW = kOutThreads / 64;
    constexpr int MAXT = (DV / 16 * DK / 16 + NW - 1) / NW;
    constexpr int njt = DV / 16, ntiles = njt * (DK / 16);
    f32x4 acc[MAXT];
    const float *Se = a.Sseg + (size_t(bh) * a.nseg + seg) * dv * DK;
#pragma unroll
    for (int m = 0; m < MAXT; ++m) {
        const int tile = wave + NW * m;
        if (tile < ntiles) {
            const int jt = tile % njt, dt = tile / njt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jt + 4 * (lane >> 4) + r, d = 16 * dt + (lane & 15);
                acc[m][r] = Se[size_t(j) * DK + d];
                st(ST, size_t(j) * LDK + d, acc[m][r]);
            }
        }
    }

    const int c_begin = seg * a.seg_chunks;
    const int c_end = min(a.nchunks, c_begin + a.seg_chunks);
    // the row loads and the feature pass run on waves 0-3 (4 threads per row)
    const bool rw = wave < 4;
    if (rw) rows.prefetch(a, bh, c_begin * C, halo);
    for (int c = c_begin; c < c_end; ++c) {
        const int c0 = c * C;
        if (rw) {
            rows.store_pairs(a, bh, c0, halo, nullptr, 0, XE, LDK, YT, LDT, nullptr);
            rows.store_queries(a, c0, QE, LDK);
        }
        float ew = 0.f, lg = 0.f;
        if (wave == 0) {
            ew = a.etaw[size_t(bh) * a.Tpad + c0 + lane];
            lg = a.lg[size_t(bh) * a.Tpad + c0 + lane];
        }
        if (rw && c + 1 < c_end) rows.prefetch(a, bh, c0 + C, halo);
        if (wave == 0) {
            ew_s[lane] = ew;
            gam_s[lane] = expf(lg);
            const float b = wave_inclusive_scan(lg);
            g_s[lane] = expf(b);
            if (lane == 63) bC_s = b;
        }
        __syncthreads();
        // scores Qh X_ext^T (4 token tiles x 6 pair tiles)
        for (int tile = wave; tile < 4 * (KP / 16); tile += NW) {
            const int tt = tile % 4, pt = tile / 4;
            f32x4 s = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, QE + 16 * tt * LDK, LDK, XE + 16 * pt * LDK, LDK,
                                  0, DK);
#pragma unroll
            for (int r = 0; r < 4; ++r) PF[(16 * tt + 4 * (lane >> 4) + r) * LDF + 16 * pt + (lane & 15)] = s[r];
        }
        __syncthreads();
        // mask by the column recurrence; coefficients of the chunk write
        // Each column of the mask in two halves of 32 tokens (thread: column
        // p, half h): the recurrence from 0 inside the half and the running
        // product of carries, then the second half adds that product times
        // the first half's end value (an exact split of the linear recurrence).
        const int mp = tid % KP, mh = tid / KP;   // threads 0 .. 2 KP - 1
        float mloc[32], mpr[32];
        if (tid < 2 * KP) {
            const int j = mp - halo, t_lo = j > 0 ? j : 0, t_hi = mp < np ? j + halo : -1;
            float m = 0.f, pr = 1.f;
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const int t = 32 * mh + u;
                const float gm = gam_s[t];
                m = gm * m + ((t >= t_lo && t <= t_hi) ? ew_s[t] : 0.f);
                pr *= gm;
                mloc[u] = m;
                mpr[u] = pr;
            }
            if (mh == 0) mend_s[mp] = m;
        }
        __syncthreads();
        if (tid < 2 * KP) {
            const float m_in = mh == 1 ? mend_s[mp] : 0.f;
            float m = 0.f;
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const int t = 32 * mh + u;
                m = mloc[u] + mpr[u] * m_in;
                const float pv = PF[t * LDF + mp] * m;
                if constexpr (PBuf<E>::separate)
                    st(PE, size_t(t) * LDT + mp, pv);
                else
                    PF[t * LDF + mp] = pv;
            }
            if (mh == 1) coef[mp] = m;
        }
        __syncthreads();
        for (int idx = tid; idx < KP * DK; idx += kOutThreads) {
            const int p = idx / DK, d = idx % DK;
            st(XT, size_t(d) * LDT + p, p < np ? coef[p] * ld(XE, size_t(p) * LDK + d) : 0.f);
        }
        __syncthreads();
        // outputs: O^T = (S^T Qh^T) diag(Gamma) + Y^T P^T;  tiles (jt, token tile)
        const E *Pm;
        int ldp;
        if constexpr (PBuf<E>::separate) {
            Pm = PE;
            ldp = LDT;
        } else {
            Pm = reinterpret_cast<const E *>(PF);
            ldp = LDF;
        }
        for (int tile = wave; tile < njt * 4; tile += NW) {
            const int jt = tile % njt, tt = tile / njt;
            f32x4 r0 = Mma<E>::run(f32x4{0.f, 0.f, 0.f, 0.f}, ST + 16 * jt * LDK, LDK, QE + 16 * tt * LDK, LDK,
                                   0, DK);
            const int t = 16 * tt + (lane & 15);
            const float gt = g_s[t];
#pragma unroll
            for (int r = 0; r < 4; ++r) r0[r] *= gt;
            r0 = Mma<E>::run(r0, YT + 16 * jt * LDT, LDT, Pm + 16 * tt * ldp, ldp, 0, KP);
            if (c0 + t < T) {
                E *dst = o + size_t(c0 + t) * dv + 16 * jt + 4 * (lane >> 4);
                st4(dst, r0);
            }
        }
        // state: S^T = e^{b_C} S^T + Y^T diag(coef) X
        const float gC = expf(bC_s);
#pragma unroll
        for (int m = 0; m < MAXT; ++m) {
            const int tile = wave + NW * m;
            if (tile < ntiles) {
                const int jt = tile % njt, dt = tile / njt;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[m][r] *= gC;
                acc[m] = Mma<E>::run(acc[m], YT + 16 * jt * LDT, LDT, XT + 16 * dt * LDT, LDT, 0, KP);
            }
        }
        __syncthreads();   // every read of ST / YT / XT of this chunk is done
#pragma unroll
        for (int m = 0; m < MAXT; ++m) {
            const int tile = wave + NW * m;
            if (tile < ntiles) {
                const int jt = tile % njt, dt = tile / njt;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    st(ST, size_t(16 * jt + 4 * (lane >> 4) + r) * LDK + 16 * dt + (lane & 15), acc[m][r]);
            }
        }
        __syncthreads();
    }
}

template <class E, int DK, int DV>
void launch_t(const ChunkAArgs &a, hipStream_t s, Marks *m) {
    a_segment<E, DK, DV><<<dim3(a.nseg, a.BH), kSegThreads, 0, s>>>(a);
    m->mark(s);
    a_segscan<<<dim3(a.BH, (a.dk * a.dv + 255) / 256), 256, 0, s>>>(a);
    m->mark(s);
    a_output<E, DK, DV><<<dim3(a.nseg, a.BH), kOutThreads, 0, s>>>(a);
    m->mark(s);
}

template <class E, int DK>
void launch_dv(const ChunkAArgs &a, hipStream_t s, Marks *m) {
    if (a.dv == 16) launch_t<E, DK, 16>(a, s, m);
    else if (a.dv == 32) launch_t<E, DK, 32>(a, s, m);
    else launch_t<E, DK, 64>(a, s, m);
}

}  // namespace

void launch_chunk_a(const ChunkAArgs &a, bool bf16, hipStream_t s, Marks *m) {
    if (bf16) {
        if (a.dk == 32) launch_dv<bf16_t, 32>(a, s, m);
        else launch_dv<bf16_t, 64>(a, s, m);
    } else {
        if (a.dk == 32) launch_dv<float, 32>(a, s, m);
        else launch_dv<float, 64>(a, s, m);
    }
}

}  // namespace falcon
