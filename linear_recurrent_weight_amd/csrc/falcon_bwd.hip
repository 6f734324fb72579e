// Falcon-1 backward pass, token-recurrent (summary §D.2 "Backward Pass",
// §E.3 "Chunk-Parallel Backward Pass", §G.3 "Forward and Backward
// Algorithms"), in fp32, and the falcon_bwd entry point.
//
// The reverse recursion of the state adjoint G_t = dL/dS_t,
//   G_t += qh_t do_t^T;   w_t = G_t^T x_t;   G_{t-1} = gamma_t G_t - eta_t x_t w_t^T,
// acts on every value column on its own once eta_t and gamma_t are known
// (they are shared by the columns), so the kernels keep the forward's
// layout: one wavefront per (head, group of 4 value columns), lane l holding
// rows l (and l + 64) of those columns.  The gradients that sum over the
// columns (dgamma_t = <G_t, S_{t-1}>, deta_t = w_t . r_t, dx_t = eta_t (G_t
// r_t - S_{t-1} w_t), dqh_t = S_t do_t) are added up over the four waves of a
// workgroup in LDS, leave it as partial sums per 16 columns, and are added
// up per token afterwards; every sum runs in a fixed order.
//   feature     (the forward's feature pass) x_t, qh_t, eta_t, alpha_t;
//   bwd_states  the forward recurrence again, keeping the state before every
//               4th token and each token's residual r_t;
//   bwd_sweep   the reverse sweep: dv_t, the partial sums, and dS_0;
//   bwd_reduce  per token: the sums of the records, the decay and step chain
//               (clamp-gated, zero steps masked, the fresh first step a
//               boundary constant), phi's vector-Jacobian products for q_t
//               and k_{t-1}, and the carried feature's gradient.
#include <cstdio>

#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace falcon {
namespace {

constexpr int kCpw = 4;               // value columns per wavefront
constexpr int kTb = kBwdCheckpoint;   // tokens whose inputs are loaded together (a checkpoint block)

// rows of the checkpointed state before token kTb * k of (head bh, column
// group g), one float4 (the 4 columns) per row
__device__ __forceinline__ float4 *state_at(const BwdArgs &a, int bh, int k, int g) {
    const int groups = a.dv / kCpw;
    const size_t nck = size_t(bwd_checkpoints(a.T));
    return reinterpret_cast<float4 *>(a.states) + ((size_t(bh) * nck + k) * groups + g) * a.dk;
}

template <int RPL>
__device__ __forceinline__ float4 ld_row(const float4 *p, int lane, int r, int dk) {
    const int i = lane + 64 * r;
    return i < dk ? p[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

__device__ __forceinline__ float col(const float4 &v, int c) {
    return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// bwd_states: S_0 .. S_T and r_t of 4 value columns (the forward recurrence)
// ---------------------------------------------------------------------------
// the inputs of kTb consecutive tokens (rows clamped into [0, T)); two sets
// alternate so that one block's loads are in flight while the previous
// block computes
template <class E, int RPL>
struct FwdBlock {
    float x[kTb][RPL], y[kTb][kCpw], eta[kTb], gam[kTb];
    __device__ __forceinline__ void load(const BwdArgs &a, const E *v, int bh, int t0, int lane, int c0) {
        const int T = a.T, dk = a.dk, dv = a.dv;
#pragma unroll
        for (int u = 0; u < kTb; ++u) {
            const size_t row = size_t(bh) * T + (t0 + u < T ? t0 + u : T - 1);
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int i = lane + 64 * r;
                x[u][r] = i < dk ? a.xn[row * dk + i] : 0.f;
            }
#pragma unroll
            for (int c = 0; c < kCpw; ++c) y[u][c] = ld(v, row * dv + c0 + c);
            eta[u] = a.eta[row];
            gam[u] = 1.f - a.alpha[row];
        }
    }
};

template <class E, int RPL, int RW>
__global__ __launch_bounds__(256) void bwd_states(BwdArgs a) {
    auto rsum = [](float v) { return group_sum<RW>(v); };
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int groups = a.dv / kCpw;
    if (gw >= a.BH * groups) return;
    const int bh = gw / groups, g = gw % groups, c0 = g * kCpw;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const E *v = static_cast<const E *>(a.v);

    float S[RPL][kCpw];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int i = lane + 64 * r;
#pragma unroll
        for (int c = 0; c < kCpw; ++c)
            S[r][c] = (a.S_in && i < dk) ? a.S_in[(size_t(bh) * dk + i) * dv + c0 + c] : 0.f;
    }
    auto put = [&](int k) {   // the state before token kTb * k
        float4 *p = state_at(a, bh, k, g);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            if (i < dk) p[i] = make_float4(S[r][0], S[r][1], S[r][2], S[r][3]);
        }
    };
    auto step = [&](const FwdBlock<E, RPL> &b, int t0) {
        put(t0 / kTb);
#pragma unroll
        for (int u = 0; u < kTb; ++u) {
            const int t = t0 + u;
            if (t >= T) break;
            float res[kCpw];
#pragma unroll
            for (int c = 0; c < kCpw; ++c) {
                float s = 0.f;
#pragma unroll
                for (int r = 0; r < RPL; ++r) s += S[r][c] * b.x[u][r];
                res[c] = b.y[u][c] - rsum(s);
            }
            if (lane == 0)
                *reinterpret_cast<float4 *>(a.res + (size_t(bh) * T + t) * dv + c0) = make_float4(res[0], res[1], res[2], res[3]);
#pragma unroll
            for (int c = 0; c < kCpw; ++c)
#pragma unroll
                for (int r = 0; r < RPL; ++r) S[r][c] = b.gam[u] * S[r][c] + b.eta[u] * b.x[u][r] * res[c];
        }
    };
    FwdBlock<E, RPL> b0, b1;
    if (T > 0) b0.load(a, v, bh, 0, lane, c0);
    for (int t0 = 0; t0 < T; t0 += 2 * kTb) {
        if (t0 + kTb < T) b1.load(a, v, bh, t0 + kTb, lane, c0);
        asm volatile("" ::: "memory");   // the next block's loads issue before this block's steps
        step(b0, t0);
        if (t0 + kTb >= T) break;
        if (t0 + 2 * kTb < T) b0.load(a, v, bh, t0 + 2 * kTb, lane, c0);
        asm volatile("" ::: "memory");
        step(b1, t0 + kTb);
    }
}

// ---------------------------------------------------------------------------
// bwd_sweep: the reverse sweep over the tokens of 4 value columns
// ---------------------------------------------------------------------------
// the inputs of the tokens kTb k .. kTb k + kTb - 1 of checkpoint block k
// (rows clamped into [0, T)): features, step scalars, r_t, do_t, and the
// checkpointed state before the block; the states inside the block are
// rebuilt from it, S_t = gamma_t S_{t-1} + eta_t x_t r_t^T
template <class E, int RPL>
struct RevBlock {
    float x[kTb][RPL], q[kTb][RPL], res[kTb][kCpw], o[kTb][kCpw], eta[kTb], gam[kTb];
    float4 ck[RPL];
    __device__ __forceinline__ void load(const BwdArgs &a, const E *dO, int bh, int g, int k, int lane, int c0) {
        const int T = a.T, dk = a.dk, dv = a.dv;
#pragma unroll
        for (int r = 0; r < RPL; ++r) ck[r] = ld_row<RPL>(state_at(a, bh, k, g), lane, r, dk);
#pragma unroll
        for (int u = 0; u < kTb; ++u) {
            const int t = kTb * k + u < T ? kTb * k + u : T - 1;
            const size_t row = size_t(bh) * T + t;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int i = lane + 64 * r;
                x[u][r] = i < dk ? a.xn[row * dk + i] : 0.f;
                q[u][r] = i < dk ? a.qn[row * dk + i] : 0.f;
            }
            const float4 rr = *reinterpret_cast<const float4 *>(a.res + row * dv + c0);
            res[u][0] = rr.x;
            res[u][1] = rr.y;
            res[u][2] = rr.z;
            res[u][3] = rr.w;
#pragma unroll
            for (int c = 0; c < kCpw; ++c) o[u][c] = ld(dO, row * dv + c0 + c);
            eta[u] = a.eta[row];
            gam[u] = 1.f - a.alpha[row];
        }
    }
};

template <class E, int RPL, int RW>
__global__ __launch_bounds__(256) void bwd_sweep(BwdArgs a) {
    auto rsum = [](float v) { return group_sum<RW>(v); };
    constexpr int PFM = bwd_part_floats(64 * RPL);   // record size at the largest d_k of this shape
    // the four waves' partial sums of a block of tokens, by block parity
    __shared__ float red[2][4][kTb][PFM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gw = blockIdx.x * 4 + wave;
    const int groups = a.dv / kCpw;   // a multiple of 4: the grid's waves fill it exactly,
                                      // and the four waves of a workgroup share one head
    const int bh = gw / groups, g = gw % groups, c0 = g * kCpw;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const int PF = bwd_part_floats(dk);
    const int ngp = groups / 4, gp = g / 4;   // records per token; this workgroup's record
    const E *dO = static_cast<const E *>(a.d_o);
    E *dV = static_cast<E *>(a.d_v);

    float G[RPL][kCpw];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int i = lane + 64 * r;
#pragma unroll
        for (int c = 0; c < kCpw; ++c)
            G[r][c] = (a.d_S_out && i < dk) ? a.d_S_out[(size_t(bh) * dk + i) * dv + c0 + c] : 0.f;
    }
    auto step = [&](const RevBlock<E, RPL> &b, int k) {
        // the block's states: sb[u] = S before token kTb k + u, sb[kTb] after its last token
        float4 sb[kTb + 1][RPL];
#pragma unroll
        for (int r = 0; r < RPL; ++r) sb[0][r] = b.ck[r];
#pragma unroll
        for (int u = 0; u < kTb; ++u)
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const float ex = b.eta[u] * b.x[u][r], gm = b.gam[u];
                sb[u + 1][r] = make_float4(gm * sb[u][r].x + ex * b.res[u][0], gm * sb[u][r].y + ex * b.res[u][1],
                                           gm * sb[u][r].z + ex * b.res[u][2], gm * sb[u][r].w + ex * b.res[u][3]);
            }
#pragma unroll
        for (int u = kTb - 1; u >= 0; --u) {
            const int t = kTb * k + u;
            if (t >= T) continue;
            const size_t row = size_t(bh) * T + t;
            const float eta = b.eta[u], gam = b.gam[u];
            const float4 *sp = sb[u], *sn = sb[u + 1];   // S_{t-1}, S_t
            // read after write: G_t += qh_t do_t^T, dqh_t = S_t do_t
            float dq[RPL];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                dq[r] = 0.f;
#pragma unroll
                for (int c = 0; c < kCpw; ++c) {
                    G[r][c] += b.q[u][r] * b.o[u][c];
                    dq[r] += col(sn[r], c) * b.o[u][c];
                }
            }
            // w = G^T x, dgamma = <G, S_{t-1}>
            float w[kCpw], gs = 0.f;
#pragma unroll
            for (int c = 0; c < kCpw; ++c) {
                float sw = 0.f;
#pragma unroll
                for (int r = 0; r < RPL; ++r) {
                    sw += G[r][c] * b.x[u][r];
                    gs += G[r][c] * col(sp[r], c);
                }
                w[c] = rsum(sw);
            }
            const float dgam = rsum(gs);
            float deta = 0.f;
#pragma unroll
            for (int c = 0; c < kCpw; ++c) deta += w[c] * b.res[u][c];
            // dv_t = eta w (this group's columns, lanes 0..3)
            if (lane < kCpw) {
                const float wl = lane == 0 ? w[0] : lane == 1 ? w[1] : lane == 2 ? w[2] : w[3];
                st(dV, row * dv + c0 + lane, eta * wl);
            }
            // dx_t = eta (G r - S_{t-1} w), then G_{t-1} = gamma G - eta x w^T
            float dx[RPL];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                float s = 0.f;
#pragma unroll
                for (int c = 0; c < kCpw; ++c) s += G[r][c] * b.res[u][c] - col(sp[r], c) * w[c];
                dx[r] = eta * s;
#pragma unroll
                for (int c = 0; c < kCpw; ++c) G[r][c] = gam * G[r][c] - eta * b.x[u][r] * w[c];
            }
            float *P = red[k & 1][wave][u];
            if (lane == 0) {
                P[0] = dgam;
                P[1] = deta;
            }
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int i = lane + 64 * r;
                if (i < dk) {
                    P[4 + i] = dx[r];
                    P[4 + dk + i] = dq[r];
                }
            }
        }
        // the four waves' sums of the block, in wave order, to this
        // workgroup's record; the other parity's buffer is rewritten only
        // after the next block's barrier, which every wave passes after
        // finishing these sums
        __syncthreads();
        for (int idx = tid; idx < kTb * PF; idx += 256) {
            const int u = idx / PF, e = idx % PF, t = kTb * k + u;
            if (t >= T) continue;
            const float v = ((red[k & 1][0][u][e] + red[k & 1][1][u][e]) + red[k & 1][2][u][e]) + red[k & 1][3][u][e];
            a.part[((size_t(bh) * T + t) * ngp + gp) * PF + e] = v;
        }
    };
    // checkpoint blocks from the last; two input sets alternate so that the
    // next block's loads are in flight while a block computes
    RevBlock<E, RPL> b0, b1;
    const int nck = int(bwd_checkpoints(T));
    if (nck > 0) b0.load(a, dO, bh, g, nck - 1, lane, c0);
    for (int k = nck - 1; k >= 0; k -= 2) {
        if (k - 1 >= 0) b1.load(a, dO, bh, g, k - 1, lane, c0);
        asm volatile("" ::: "memory");   // the next block's loads issue before this block's steps
        step(b0, k);
        if (k - 1 < 0) break;
        if (k - 2 >= 0) b0.load(a, dO, bh, g, k - 2, lane, c0);
        asm volatile("" ::: "memory");
        step(b1, k - 1);
    }
    if (a.d_S_in) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            if (i < dk)
#pragma unroll
                for (int c = 0; c < kCpw; ++c) a.d_S_in[(size_t(bh) * dk + i) * dv + c0 + c] = G[r][c];
        }
    }
    // an empty segment passes the carried feature's gradient through
    if (T == 0 && g == 0 && a.d_x_next_in) {
        for (int i = lane; i < dk; i += 64)
            a.d_x_next_in[size_t(bh) * dk + i] = (!a.fresh && a.d_x_next_out) ? a.d_x_next_out[size_t(bh) * dk + i] : 0.f;
    }
}

// ---------------------------------------------------------------------------
// bwd_reduce: one wavefront per (head, token)
// ---------------------------------------------------------------------------
// phi's vector-Jacobian product: dz = s g - (s^3 / d)(z . g) z (RMSNorm), g
// (identity); z and g hold rows lane + 64 r, zero past d
template <int RPL, int RW>
__device__ __forceinline__ void phi_vjp(const float (&z)[RPL], const float (&gv)[RPL], float (&out)[RPL], int d,
                                        float eps_rms, int phi_kind) {
    if (phi_kind == FALCON_PHI_IDENTITY) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) out[r] = gv[r];
        return;
    }
    float ss = 0.f, zg = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        ss += z[r] * z[r];
        zg += z[r] * gv[r];
    }
    ss = group_sum<RW>(ss);
    zg = group_sum<RW>(zg);
    const float ms = ss / float(d) + eps_rms;
    const float s = ms > 0.f ? 1.f / sqrtf(ms) : 0.f;
    const float k3 = s * s * s / float(d) * zg;
#pragma unroll
    for (int r = 0; r < RPL; ++r) out[r] = s * gv[r] - k3 * z[r];
}

template <class E, int RPL, int RW>
__global__ __launch_bounds__(256) void bwd_reduce(BwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int id = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int T = a.T, dk = a.dk;
    if (id >= a.BH * T) return;
    const int bh = id / T, t = id % T;
    const int ngp = a.dv / (4 * kCpw), PF = bwd_part_floats(dk);   // records per token
    const size_t row = size_t(bh) * T + t;
    const float *P = a.part + row * ngp * PF;
    const E *q = static_cast<const E *>(a.q);
    const E *k = static_cast<const E *>(a.k);

    // sums over the records, in order
    float dx[RPL], dqh[RPL], x[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int i = lane + 64 * r;
        float sx = 0.f, sq = 0.f;
        if (i < dk)
            for (int gi = 0; gi < ngp; ++gi) {
                sx += P[gi * PF + 4 + i];
                sq += P[gi * PF + 4 + dk + i];
            }
        dx[r] = sx;
        dqh[r] = sq;
        x[r] = i < dk ? a.xn[row * dk + i] : 0.f;
    }
    float dgam = 0.f, deta = 0.f;
    for (int gi = 0; gi < ngp; ++gi) {
        dgam += P[gi * PF + 0];
        deta += P[gi * PF + 1];
    }

    // gamma = 1 - alpha, alpha = min(eta lambda, 1 - eps_gamma);
    // eta = beta / den, den = ||x||^2 + lambda + eps
    const bool noop = a.fresh && t == 0;
    float xx = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) xx += x[r] * x[r];
    xx = group_sum<RW>(xx);
    const float lam = a.lambda[row], eta = a.eta[row], alpha = a.alpha[row];
    const float den = xx + lam + a.eps;
    float dbeta = 0.f, dlam = 0.f;
    if (!noop) {
        const float dalpha = -dgam;
        if (alpha < 1.f - a.eps_gamma) {   // the clamp does not bind
            deta += dalpha * lam;
            dlam = dalpha * eta;
        }
        if (den != 0.f) {
            dbeta = deta / den;
            const float dden = -deta * eta / den;
            dlam += dden;
#pragma unroll
            for (int r = 0; r < RPL; ++r) dx[r] += 2.f * dden * x[r];
        }
    }
    if (lane == 0) {
        a.d_beta[row] = dbeta;
        a.d_lambda[row] = dlam;
    }

    // dq_t through phi
    float z[RPL], out[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int i = lane + 64 * r;
        z[r] = i < dk ? ld(q, row * dk + i) : 0.f;
    }
    phi_vjp<RPL, RW>(z, dqh, out, dk, a.eps_rms, a.phi);
    E *dQ = static_cast<E *>(a.d_q);
    E *dK = static_cast<E *>(a.d_k);
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int i = lane + 64 * r;
        if (i < dk) st(dQ, row * dk + i, out[r]);
    }
    // x_t = phi(k_{t-1}): dk_{t-1}; for t = 0 the carried feature's gradient
    if (t > 0) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            z[r] = i < dk ? ld(k, (row - 1) * dk + i) : 0.f;
        }
        phi_vjp<RPL, RW>(z, dx, out, dk, a.eps_rms, a.phi);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            if (i < dk) st(dK, (row - 1) * dk + i, out[r]);
        }
    } else if (a.d_x_next_in) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            if (i < dk) a.d_x_next_in[size_t(bh) * dk + i] = a.fresh ? 0.f : dx[r];
        }
    }
    // k_{T-1} feeds only the next segment's first pair
    if (t == T - 1) {
        float gx[RPL];
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            z[r] = i < dk ? ld(k, row * dk + i) : 0.f;
            gx[r] = (a.d_x_next_out && i < dk) ? a.d_x_next_out[size_t(bh) * dk + i] : 0.f;
        }
        phi_vjp<RPL, RW>(z, gx, out, dk, a.eps_rms, a.phi);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int i = lane + 64 * r;
            if (i < dk) st(dK, row * dk + i, out[r]);
        }
    }
}

template <class E, int RPL, int RW>
void launch_shape(const BwdArgs &a, hipStream_t s, Marks *m) {
    const int waves = a.BH * (a.dv / kCpw);
    const int blocks = (waves + 3) / 4;
    bwd_states<E, RPL, RW><<<blocks, 256, 0, s>>>(a);
    m->mark(s);
    bwd_sweep<E, RPL, RW><<<blocks, 256, 0, s>>>(a);
    m->mark(s);
    if (a.T > 0) {
        const long long rw = static_cast<long long>(a.BH) * a.T;
        bwd_reduce<E, RPL, RW><<<static_cast<unsigned>((rw + 3) / 4), 256, 0, s>>>(a);
        m->mark(s);
    }
}

template <class E>
void launch_io(const BwdArgs &a, hipStream_t s, Marks *m) {
    switch (a.dk) {
        case 16: launch_shape<E, 1, 16>(a, s, m); break;
        case 32: launch_shape<E, 1, 32>(a, s, m); break;
        case 64: launch_shape<E, 1, 64>(a, s, m); break;
        default: launch_shape<E, 2, 64>(a, s, m); break;
    }
}

}  // namespace

void launch_bwd(const BwdArgs &a, bool io_bf16, hipStream_t s, Marks *m) {
    if (io_bf16) launch_io<bf16_t>(a, s, m);
    else launch_io<float>(a, s, m);
}

}  // namespace falcon

namespace {

const char *const kNamesBwd[] = {"feature", "bwd_states", "bwd_sweep", "bwd_reduce"};
const char *const kNamesBwdChunk[] = {"bwd_ops", "bwd_carry_fwd", "bwd_carry_rev", "bwd_grads"};
const char *const kNamesBwdEmpty[] = {"bwd_states", "bwd_sweep"};

// returns the number of kernels launched, or a negative status
int run_bwd(const falcon_bwd_args *args, void *stream, falcon::Marks &m) {
    using namespace falcon;
    BwdPlan p;
    const int rc = build_bwd_plan(args, &p, true);
    if (rc != FALCON_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    m.sync_check = sync_check_enabled();
    m.mark(s);
    const bool bf16 = p.dtype == FALCON_BF16;
    if (p.T > 0 && !p.chunked) {
        FeatureArgs fa{};
        fa.variant = FALCON_V1;
        fa.phi = p.phi;
        fa.BH = p.BH;
        fa.T = p.T;
        fa.Tpad = p.T;
        fa.dk = p.dk;
        fa.dv = p.dv;
        fa.window = 1;
        fa.eps = p.eps;
        fa.eps_gamma = p.eps_gamma;
        fa.eps_rms = p.eps_rms;
        fa.fresh = p.fresh ? 1 : 0;
        fa.q = args->q;
        fa.k = args->k;
        fa.v = args->v;
        fa.beta = args->beta;
        fa.lambda = args->lambda;
        fa.xnext_in = p.xnext_in;
        fa.xn = p.ws_at<float>(p.off_xn);
        fa.qn = p.ws_at<float>(p.off_qn);
        fa.eta = p.ws_at<float>(p.off_eta);
        fa.alpha = p.ws_at<float>(p.off_alpha);
        launch_features(fa, bf16, false, s, &m);
    }
    BwdArgs ba{};
    ba.phi = p.phi;
    ba.BH = p.BH;
    ba.T = p.T;
    ba.dk = p.dk;
    ba.dv = p.dv;
    ba.fresh = p.fresh ? 1 : 0;
    ba.eps = p.eps;
    ba.eps_gamma = p.eps_gamma;
    ba.eps_rms = p.eps_rms;
    ba.q = args->q;
    ba.k = args->k;
    ba.v = args->v;
    ba.d_o = args->d_o;
    ba.beta = args->beta;
    ba.lambda = args->lambda;
    ba.S_in = p.S_in;
    ba.d_S_out = args->d_S_out;
    ba.d_x_next_out = args->d_x_next_out;
    ba.xn = p.ws_at<float>(p.off_xn);
    ba.qn = p.ws_at<float>(p.off_qn);
    ba.eta = p.ws_at<float>(p.off_eta);
    ba.alpha = p.ws_at<float>(p.off_alpha);
    ba.states = p.ws_at<float>(p.off_states);
    ba.res = p.ws_at<float>(p.off_res);
    ba.part = p.ws_at<float>(p.off_part);
    ba.d_q = args->d_q;
    ba.d_k = args->d_k;
    ba.d_v = args->d_v;
    ba.d_beta = args->d_beta;
    ba.d_lambda = args->d_lambda;
    ba.d_S_in = args->d_S_in;
    ba.d_x_next_in = args->d_x_next_in;
    if (p.chunked) {
        ba.nchunks = p.nchunks;
        ba.xnext_in = p.xnext_in;
        ba.ops = p.ws_at<float>(p.off_ops);
        ba.cst = p.ws_at<float>(p.off_cst);
        ba.hg = p.ws_at<float>(p.off_hg);
        ba.phip = p.ws_at<float>(p.off_phip);
        launch_bwd_chunk(ba, bf16, s, &m);
    } else {
        launch_bwd(ba, bf16, s, &m);
    }
    if (m.failed_at >= 0) {
        std::fprintf(stderr, "falcon_bwd: FALCON_SYNC_CHECK: kernel %d of the call failed\n", m.failed_at);
        return FALCON_ERR_HIP;
    }
    if (hipGetLastError() != hipSuccess) return FALCON_ERR_HIP;
    return m.count - 1;
}

}  // namespace

extern "C" int falcon_bwd(const falcon_bwd_args *args, void *stream) {
    falcon::Marks m;
    const int rc = run_bwd(args, stream, m);
    return rc < 0 ? rc : FALCON_OK;
}

extern "C" int falcon_bwd_profile(const falcon_bwd_args *args, void *stream, void *const *events,
                                  int n_events) {
    falcon::Marks m;
    m.ev = events;
    m.n = n_events < 0 ? 0 : n_events;
    return run_bwd(args, stream, m);
}

extern "C" const char *falcon_bwd_kernel_name(const falcon_bwd_args *args, int i) {
    falcon::BwdPlan p;
    if (falcon::build_bwd_plan(args, &p, false) != FALCON_OK || i < 0) return nullptr;
    if (p.T == 0) return i < 2 ? kNamesBwdEmpty[i] : nullptr;
    if (p.chunked) return i < 4 ? kNamesBwdChunk[i] : nullptr;
    return i < 4 ? kNamesBwd[i] : nullptr;
}
