// Token-recurrent form of every Falcon variant (summary Figure 2 and
// Figure 4 "recurrent view"; §A "Recurrent Form (per-channel rates)"), in
// fp32.  It is the generic GPU path (any variant, any length) and the
// single-token decode shape.
//
// One wavefront owns one (batch*head, group of 4 value columns).  Lane l
// holds rows l (and l+64 when d_k = 128) of those columns of S, so both
// contractions over d_k (the pre-update prediction S^T x and the read
// S^T qh) are lane reductions (over the first RW lanes, RW >= d_k) and no
// LDS or barrier is needed.  The inputs of kTb tokens are requested at once
// and then consumed from registers, so a token step does not wait for a
// memory round trip of its own.
//   F1 : S = gamma S + eta x (y - S^T x)^T           (residual at S_{t-1})
//   F2 : the same per column with eta_j, gamma_j
//   F3 : S = gamma S + (eta/B_t) sum_{j in I_t} x_j (y_j - S^T x_j)^T
//   F1A: S = gamma S + eta x y^T                 F2A: per column with eta_j, gamma_j
//   F3A: S = gamma S + (eta/B_t) sum_{j in I_t} x_j y_j^T
//   o_t = S_t^T qh_t (read after write)
// eta/alpha come from the feature pass, so the fresh first step (eta =
// alpha = 0) is already a no-op here.
#include "common.h"
#include "kernels.h"

namespace falcon {
namespace {

constexpr int kCpw = 4;                  // value columns per wavefront
constexpr int kWm = FALCON_MAX_WINDOW;   // pair ring length

template <class E, int RPL, int VK, int RW>
__global__ __launch_bounds__(256) void recurrent_kernel(RecurrentArgs a) {
    // sum over the lanes that hold rows of S (lanes >= d_k hold zeros)
    auto rsum = [](float v) { return group_sum<RW>(v); };
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int groups = a.dv / kCpw;
    if (gw >= a.BH * groups) return;
    const int bh = gw / groups;
    const int c0 = (gw % groups) * kCpw;
    const int dk = a.dk, dv = a.dv, T = a.T, W = a.window;
    const int halo = W - 1;
    constexpr bool kWin = (VK == FALCON_V3 || VK == FALCON_V3A);

    float S[RPL][kCpw];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int i = lane + 64 * r;
#pragma unroll
        for (int c = 0; c < kCpw; ++c)
            S[r][c] = (a.S_in && i < dk) ? a.S_in[(size_t(bh) * dk + i) * dv + c0 + c] : 0.f;
    }

    // ring of the last kWm pairs: slot kWm-1 is the newest
    float xw[kWin ? kWm : 1][RPL];
    float yw[kWin ? kWm : 1][kCpw];
    if constexpr (kWin) {
#pragma unroll
        for (int j = 0; j < kWm; ++j) {
            const int p = j - kWm;  // pair index relative to this segment's first pair
            const bool have = p >= -a.n_tail_in;
            const int slot = p + halo;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int i = lane + 64 * r;
                xw[j][r] = (have && i < dk) ? a.tailx_in[(size_t(bh) * halo + slot) * dk + i] : 0.f;
            }
#pragma unroll
            for (int c = 0; c < kCpw; ++c)
                yw[j][c] = have ? a.taily_in[(size_t(bh) * halo + slot) * dv + c0 + c] : 0.f;
        }
    }

    const E *v = static_cast<const E *>(a.v);
    E *o = static_cast<E *>(a.o);
    constexpr bool kPerCol = VK == FALCON_V2 || VK == FALCON_V2A;
    constexpr int NE = kPerCol ? kCpw : 1;           // step scalars per token
    constexpr int kTb = kPerCol ? 8 : 16;            // tokens whose inputs are loaded together
    for (int t0 = 0; t0 < T; t0 += kTb) {
        // the inputs of tokens t0 .. t0 + kTb - 1 (rows clamped into [0, T))
        float xb[kTb][RPL], qb[kTb][RPL], yb[kTb][kCpw], eb[kTb][NE], ab[kTb][NE];
#pragma unroll
        for (int u = 0; u < kTb; ++u) {
            const size_t row = size_t(bh) * T + (t0 + u < T ? t0 + u : T - 1);
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int i = lane + 64 * r;
                xb[u][r] = i < dk ? a.xn[row * dk + i] : 0.f;
                qb[u][r] = i < dk ? a.qn[row * dk + i] : 0.f;
            }
#pragma unroll
            for (int c = 0; c < kCpw; ++c) yb[u][c] = ld(v, row * dv + c0 + c);
#pragma unroll
            for (int c = 0; c < NE; ++c) {
                eb[u][c] = NE > 1 ? a.eta[row * dv + c0 + c] : a.eta[row];
                ab[u][c] = NE > 1 ? a.alpha[row * dv + c0 + c] : a.alpha[row];
            }
        }
#pragma unroll
        for (int u = 0; u < kTb; ++u) {
            const int t = t0 + u;
            if (t >= T) break;
            const size_t row = size_t(bh) * T + t;
            const float *x = xb[u], *q = qb[u], *y = yb[u];
            float eta[kCpw], gam[kCpw];
#pragma unroll
            for (int c = 0; c < kCpw; ++c) {
                eta[c] = eb[u][NE > 1 ? c : 0];
                gam[c] = 1.f - ab[u][NE > 1 ? c : 0];
            }

            if constexpr (VK == FALCON_V1 || VK == FALCON_V2) {
                float pred[kCpw];
#pragma unroll
                for (int c = 0; c < kCpw; ++c) {
                    float s = 0.f;
#pragma unroll
                    for (int r = 0; r < RPL; ++r) s += S[r][c] * x[r];
                    pred[c] = rsum(s);
                }
#pragma unroll
                for (int c = 0; c < kCpw; ++c) {
                    const float res = y[c] - pred[c];
#pragma unroll
                    for (int r = 0; r < RPL; ++r) S[r][c] = gam[c] * S[r][c] + eta[c] * x[r] * res;
                }
            } else if constexpr (VK == FALCON_V1A || VK == FALCON_V2A) {
#pragma unroll
                for (int c = 0; c < kCpw; ++c)
#pragma unroll
                    for (int r = 0; r < RPL; ++r) S[r][c] = gam[c] * S[r][c] + eta[c] * x[r] * y[c];
            } else {
                // shift the ring and append the pair (x_t, y_t)
#pragma unroll
                for (int j = 0; j < kWm - 1; ++j) {
#pragma unroll
                    for (int r = 0; r < RPL; ++r) xw[j][r] = xw[j + 1][r];
#pragma unroll
                    for (int c = 0; c < kCpw; ++c) yw[j][c] = yw[j + 1][c];
                }
#pragma unroll
                for (int r = 0; r < RPL; ++r) xw[kWm - 1][r] = x[r];
#pragma unroll
                for (int c = 0; c < kCpw; ++c) yw[kWm - 1][c] = y[c];
                const long long pairs = (long long)a.n_tail_in + t + 1;
                const int bt = pairs < W ? int(pairs) : W;
                const float scale = eta[0] / float(bt);
                float acc[RPL][kCpw];
#pragma unroll
                for (int r = 0; r < RPL; ++r)
#pragma unroll
                    for (int c = 0; c < kCpw; ++c) acc[r][c] = 0.f;
#pragma unroll
                for (int j = 0; j < kWm; ++j) {
                    if (j < kWm - W) continue;  // older than the window
                    if constexpr (VK == FALCON_V3) {
#pragma unroll
                        for (int c = 0; c < kCpw; ++c) {
                            float s = 0.f;
#pragma unroll
                            for (int r = 0; r < RPL; ++r) s += S[r][c] * xw[j][r];
                            const float res = yw[j][c] - rsum(s);
#pragma unroll
                            for (int r = 0; r < RPL; ++r) acc[r][c] += xw[j][r] * res;
                        }
                    } else {
#pragma unroll
                        for (int c = 0; c < kCpw; ++c)
#pragma unroll
                            for (int r = 0; r < RPL; ++r) acc[r][c] += xw[j][r] * yw[j][c];
                    }
                }
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
                s = rsum(s);
                if (lane == c) oc = s;
            }
            if (lane < kCpw) st(o, row * dv + c0 + lane, oc);
        }
    }

    if (a.S_out) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            if (i < dk)
#pragma unroll
                for (int c = 0; c < kCpw; ++c) a.S_out[(size_t(bh) * dk + i) * dv + c0 + c] = S[r][c];
        }
    }
}

template <class E, int RPL, int RW>
void launch_rec_width(const RecurrentArgs &a, dim3 grid, hipStream_t s) {
    switch (a.variant) {
        case FALCON_V1: recurrent_kernel<E, RPL, FALCON_V1, RW><<<grid, 256, 0, s>>>(a); break;
        case FALCON_V2: recurrent_kernel<E, RPL, FALCON_V2, RW><<<grid, 256, 0, s>>>(a); break;
        case FALCON_V3: recurrent_kernel<E, RPL, FALCON_V3, RW><<<grid, 256, 0, s>>>(a); break;
        case FALCON_V1A: recurrent_kernel<E, RPL, FALCON_V1A, RW><<<grid, 256, 0, s>>>(a); break;
        case FALCON_V2A: recurrent_kernel<E, RPL, FALCON_V2A, RW><<<grid, 256, 0, s>>>(a); break;
        default: recurrent_kernel<E, RPL, FALCON_V3A, RW><<<grid, 256, 0, s>>>(a); break;
    }
}

// lane reductions as wide as d_k needs (16, 32 or the whole wave)
template <class E, int RPL>
void launch_rec_variant(const RecurrentArgs &a, dim3 grid, hipStream_t s) {
    if (RPL == 1 && a.dk <= 16) launch_rec_width<E, RPL, 16>(a, grid, s);
    else if (RPL == 1 && a.dk <= 32) launch_rec_width<E, RPL, 32>(a, grid, s);
    else launch_rec_width<E, RPL, 64>(a, grid, s);
}

}  // namespace

void launch_recurrent(const RecurrentArgs &a, bool io_bf16, hipStream_t s, Marks *m) {
    const int waves = a.BH * (a.dv / kCpw);
    dim3 grid((waves + 3) / 4);
    const bool two_rows = a.dk > 64;
    if (io_bf16) {
        if (two_rows) launch_rec_variant<bf16_t, 2>(a, grid, s);
        else launch_rec_variant<bf16_t, 1>(a, grid, s);
    } else {
        if (two_rows) launch_rec_variant<float, 2>(a, grid, s);
        else launch_rec_variant<float, 1>(a, grid, s);
    }
    m->mark(s);
}

}  // namespace falcon
