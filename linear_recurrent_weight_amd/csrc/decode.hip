// Single-token decode step of every Falcon variant in one launch: the
// constant-cost-per-token recurrent inference of the summary (§1
// "Recurrent alternatives": O(1) state per step; Figure 2, recurrent view),
// continuing from a carried boundary state (summary §C.7, §4.4).
//
// For the one token of the call (t = 1 of this segment):
//   x   = x_next of the incoming state (already phi(k) of the previous
//         segment's last key), or the sentinel 0 on a fresh sequence;
//   y   = v_1, qh = phi(q_1);
//   mu  = ||x||^2 (Falcon-1, -2, -1A) or lambda_max of the window covariance
//         (Falcon-3, -3A) over the last min(W, n_tail + 1) pairs, the carried
//         tail followed by (x, y) (summary §C.6, §4.4);
//   eta = beta / (mu + lambda + eps) (0 if that is 0), alpha = min(eta
//         lambda, 1 - eps_gamma), gamma = 1 - alpha; the fresh first step is
//         a strict no-op (summary §3.1, §C.3; explainer "Method");
//   F1 : S = gamma S + eta x (y - S^T x)^T       F2: per value column
//   F3 : S = gamma S + (eta/B) sum_j x_j (y_j - S^T x_j)^T
//   F1A: S = gamma S + eta x y^T                  F2A: per value column
//   F3A: S = gamma S + (eta/B) sum_j x_j y_j^T
//   o   = S^T qh (read after write);
//   out: S, x_next = phi(k_1), the last W-1 pairs.
//
// One wavefront per (batch*head, 4 value columns): lane l holds row l (and
// l + 64 when d_k = 128) of those columns of S, so every contraction over
// d_k is a lane reduction; the window Gram is at most 8 x 8 reductions.
#include "common.h"
#include "kernels.h"
#include "lambda_max.h"

namespace falcon {
namespace {

constexpr int kCpw = 4;                  // value columns per wavefront
constexpr int kWm = FALCON_MAX_WINDOW;

template <class E, int RPL, int VK>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int groups = a.dv / kCpw;
    if (gw >= a.BH * groups) return;     // the whole wave leaves together
    const int bh = gw / groups;
    const int c0 = (gw % groups) * kCpw;
    const int dk = a.dk, dv = a.dv, W = a.window, halo = W - 1;
    constexpr bool kWin = (VK == FALCON_V3 || VK == FALCON_V3A);
    const E *qg = static_cast<const E *>(a.q) + size_t(bh) * dk;
    const E *kg = static_cast<const E *>(a.k) + size_t(bh) * dk;
    const E *vg = static_cast<const E *>(a.v) + size_t(bh) * dv;

    // Every input is requested here, before any arithmetic, so that the
    // step waits for one memory round trip: the state columns, the step's
    // beta (per column for the per-column variants) and lambda, then the
    // pair, the query and the next pair's feature.
    float S[RPL][kCpw];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int i = lane + 64 * r;
#pragma unroll
        for (int c = 0; c < kCpw; ++c)
            S[r][c] = (a.S_in && i < dk) ? a.S_in[(size_t(bh) * dk + i) * dv + c0 + c] : 0.f;
    }
    float beta_c[kCpw];
#pragma unroll
    for (int c = 0; c < kCpw; ++c)
        beta_c[c] = (VK == FALCON_V2 || VK == FALCON_V2A) ? a.beta[size_t(bh) * dv + c0 + c] : a.beta[bh];
    const float lam = a.lambda[bh];
    float y[kCpw];
#pragma unroll
    for (int c = 0; c < kCpw; ++c) y[c] = ld(vg, c0 + c);

    // this token's pair (x, y), query and the next pair's feature
    float x[RPL], q[RPL], kn[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int i = lane + 64 * r;
        x[r] = (a.xnext_in && i < dk) ? a.xnext_in[size_t(bh) * dk + i] : 0.f;
        q[r] = i < dk ? ld(qg, i) : 0.f;
        kn[r] = i < dk ? ld(kg, i) : 0.f;
    }
    {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            sq += q[r] * q[r];
            sk += kn[r] * kn[r];
        }
        const float scq = phi_scale(wave_sum(sq), dk, a.eps_rms, a.phi);
        const float sck = phi_scale(wave_sum(sk), dk, a.eps_rms, a.phi);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            q[r] *= scq;
            kn[r] *= sck;
        }
    }

    // the window: the carried pairs (slot s holds the pair W-1-s before this
    // one), then (x, y) in slot W-1
    const int n_in = a.n_tail_in;
    const int bt = n_in + 1 < W ? n_in + 1 : W;   // window size B
    float xw[kWin ? kWm : 1][RPL], yw[kWin ? kWm : 1][kCpw];
    if constexpr (kWin) {
#pragma unroll
        for (int s = 0; s < kWm; ++s) {
            const bool tail = s < W - 1 && s >= halo - n_in;
            const bool self = s == W - 1;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int i = lane + 64 * r;
                xw[s][r] = self ? x[r] : (tail && i < dk ? a.tailx_in[(size_t(bh) * halo + s) * dk + i] : 0.f);
            }
#pragma unroll
            for (int c = 0; c < kCpw; ++c)
                yw[s][c] = self ? y[c] : (tail ? a.taily_in[(size_t(bh) * halo + s) * dv + c0 + c] : 0.f);
        }
    }

    // step scalars
    float mu;
    if constexpr (kWin) {
        // Gram of the B window pairs (the last B slots before W), the
        // covariance's lambda_max / B
        float G[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) G[i][j] = 0.f;
#pragma unroll
        for (int i = 0; i < kWm; ++i) {
            const int si = W - bt + i;            // slot of window pair i
            if (i >= bt) break;
#pragma unroll
            for (int j = 0; j <= i; ++j) {
                const int sj = W - bt + j;
                float d = 0.f;
#pragma unroll
                for (int r = 0; r < RPL; ++r) d += xw[si][r] * xw[sj][r];
                d = wave_sum(d);
                G[i][j] = d;
                G[j][i] = d;
            }
        }
        mu = psd_lambda_max(G, bt) / float(bt);
    } else {
        float n2 = 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) n2 += x[r] * x[r];
        mu = wave_sum(n2);
    }
    const float den = mu + lam + a.eps;
    const bool noop = a.fresh != 0;              // the fresh first step writes nothing
    float eta[kCpw], gam[kCpw];
#pragma unroll
    for (int c = 0; c < kCpw; ++c) {
        const float e = noop ? 0.f : step_eta(beta_c[c], den);
        eta[c] = e;
        gam[c] = 1.f - (noop ? 0.f : step_alpha(e, lam, a.eps_gamma));
    }

    // the write (residuals at the pre-update state)
    if constexpr (VK == FALCON_V1 || VK == FALCON_V2) {
#pragma unroll
        for (int c = 0; c < kCpw; ++c) {
            float s = 0.f;
#pragma unroll
            for (int r = 0; r < RPL; ++r) s += S[r][c] * x[r];
            const float res = y[c] - wave_sum(s);
#pragma unroll
            for (int r = 0; r < RPL; ++r) S[r][c] = gam[c] * S[r][c] + eta[c] * x[r] * res;
        }
    } else if constexpr (VK == FALCON_V1A || VK == FALCON_V2A) {
#pragma unroll
        for (int c = 0; c < kCpw; ++c)
#pragma unroll
            for (int r = 0; r < RPL; ++r) S[r][c] = gam[c] * S[r][c] + eta[c] * x[r] * y[c];
    } else {
        float acc[RPL][kCpw];
#pragma unroll
        for (int r = 0; r < RPL; ++r)
#pragma unroll
            for (int c = 0; c < kCpw; ++c) acc[r][c] = 0.f;
#pragma unroll
        for (int s = 0; s < kWm; ++s) {
            if (s < W - bt || s >= W) continue;  // outside the window
            if constexpr (VK == FALCON_V3) {
#pragma unroll
                for (int c = 0; c < kCpw; ++c) {
                    float p = 0.f;
#pragma unroll
                    for (int r = 0; r < RPL; ++r) p += S[r][c] * xw[s][r];
                    const float res = yw[s][c] - wave_sum(p);
#pragma unroll
                    for (int r = 0; r < RPL; ++r) acc[r][c] += xw[s][r] * res;
                }
            } else {
#pragma unroll
                for (int c = 0; c < kCpw; ++c)
#pragma unroll
                    for (int r = 0; r < RPL; ++r) acc[r][c] += xw[s][r] * yw[s][c];
            }
        }
        const float scale = eta[0] / float(bt);
#pragma unroll
        for (int c = 0; c < kCpw; ++c)
#pragma unroll
            for (int r = 0; r < RPL; ++r) S[r][c] = gam[c] * S[r][c] + scale * acc[r][c];
    }

    // read after write
    float oc = 0.f;
#pragma unroll
    for (int c = 0; c < kCpw; ++c) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) s += S[r][c] * q[r];
        s = wave_sum(s);
        if (lane == c) oc = s;
    }
    if (lane < kCpw) st(static_cast<E *>(a.o), size_t(bh) * dv + c0 + lane, oc);

    // boundary state out
    if (a.S_out) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            if (i < dk)
#pragma unroll
                for (int c = 0; c < kCpw; ++c) a.S_out[(size_t(bh) * dk + i) * dv + c0 + c] = S[r][c];
        }
    }
    if (a.xnext_out && c0 == 0) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            if (i < dk) a.xnext_out[size_t(bh) * dk + i] = kn[r];
        }
    }
    if constexpr (kWin) {
        // last W-1 pairs: slot s of the output is slot s + 1 of the window
        // list (the oldest carried pair drops out); slots before the valid
        // ones are zero
        if (a.tailx_out) {
            const int n_out = a.n_tail_out;
#pragma unroll
            for (int s = 0; s < kWm - 1; ++s) {
                if (s >= halo) break;
                const bool valid = s >= halo - n_out;
                if (c0 == 0) {
#pragma unroll
                    for (int r = 0; r < RPL; ++r) {
                        const int i = lane + 64 * r;
                        if (i < dk) a.tailx_out[(size_t(bh) * halo + s) * dk + i] = valid ? xw[s + 1][r] : 0.f;
                    }
                }
                if (lane < kCpw) {
                    float yv = 0.f;
#pragma unroll
                    for (int c = 0; c < kCpw; ++c)
                        if (lane == c) yv = valid ? yw[s + 1][c] : 0.f;
                    a.taily_out[(size_t(bh) * halo + s) * dv + c0 + lane] = yv;
                }
            }
        }
    }
}

template <class E, int RPL>
void launch_dec_variant(const DecodeArgs &a, dim3 grid, hipStream_t s) {
    switch (a.variant) {
        case FALCON_V1: decode_kernel<E, RPL, FALCON_V1><<<grid, 256, 0, s>>>(a); break;
        case FALCON_V2: decode_kernel<E, RPL, FALCON_V2><<<grid, 256, 0, s>>>(a); break;
        case FALCON_V3: decode_kernel<E, RPL, FALCON_V3><<<grid, 256, 0, s>>>(a); break;
        case FALCON_V1A: decode_kernel<E, RPL, FALCON_V1A><<<grid, 256, 0, s>>>(a); break;
        case FALCON_V2A: decode_kernel<E, RPL, FALCON_V2A><<<grid, 256, 0, s>>>(a); break;
        default: decode_kernel<E, RPL, FALCON_V3A><<<grid, 256, 0, s>>>(a); break;
    }
}

}  // namespace

void launch_decode(const DecodeArgs &a, bool io_bf16, hipStream_t s, Marks *m) {
    const int waves = a.BH * (a.dv / kCpw);
    dim3 grid((waves + 3) / 4);
    const bool two_rows = a.dk > 64;
    if (io_bf16) {
        if (two_rows) launch_dec_variant<bf16_t, 2>(a, grid, s);
        else launch_dec_variant<bf16_t, 1>(a, grid, s);
    } else {
        if (two_rows) launch_dec_variant<float, 2>(a, grid, s);
        else launch_dec_variant<float, 1>(a, grid, s);
    }
    m->mark(s);
}

}  // namespace falcon
