// Feature pass: QK-RMSNorm, one-step key shift, step scalars, window
// statistic and boundary state (x_next, tail) for every variant.
//
// Per token t of one head (summary §3, Appendix, §3.1, §C.3, §4.6; explainer
// "Method"; sungsoo.github.io post):
//   qh_t = phi(q_t);  x_t = phi(k_{t-1}), x_0 = x_next (continuing) or 0;
//   mu_t = ||x_t||^2, or lambda_max of the window covariance for Falcon-3/3A
//          (summary §C.6: exact top eigenvalue of the small window Gram);
//   eta_t = beta_t / (mu_t + lambda_t + eps), 0 if that denominator is 0;
//   alpha_t = min(eta_t lambda_t, 1 - eps_gamma);
//   the first step of a fresh sequence is a strict no-op: eta = alpha = 0.
// Falcon-2 has one eta/alpha per value column (summary App. F; lambda is
// shared by the columns).
//
// Grid: (tiles of 64 tokens, B*H).  Rows past the sequence end (padding of a
// chunked layout) get zero features and zero eta/alpha, which makes them
// exact no-op tokens for the chunk kernels.
#include "common.h"
#include "kernels.h"
#include "lambda_max.h"

namespace falcon {
namespace {

constexpr int kTile = 64;
constexpr int kWmax = FALCON_MAX_WINDOW;
constexpr int kDmax = 128;
constexpr int kXStride = kDmax + 1;  // odd stride: row-parallel LDS reads hit distinct banks

template <class Ein, class Ef>
__global__ __launch_bounds__(256) void feature_kernel(FeatureArgs a) {
    __shared__ float xs[(kTile + kWmax - 1) * kXStride];  // pair features, fp32
    __shared__ float band[(kTile + kWmax - 1) * kWmax];   // x_r . x_{r-d}
    __shared__ float mu_s[kTile];
    __shared__ float den_s[kTile];

    const int t0 = blockIdx.x * kTile;
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int dk = a.dk, dv = a.dv, T = a.T, W = a.window;
    const int halo = W - 1;
    const int nrows = kTile + halo;
    const size_t head_k = size_t(bh) * T * dk;
    const Ein *q = static_cast<const Ein *>(a.q) + head_k;
    const Ein *k = static_cast<const Ein *>(a.k) + head_k;
    Ef *xn = static_cast<Ef *>(a.xn) + size_t(bh) * a.Tpad * dk;
    Ef *qn = static_cast<Ef *>(a.qn) + size_t(bh) * a.Tpad * dk;

    // lanes per row: 4 elements per lane
    const int lpr = dk / 4;           // 4, 8, 16 or 32
    const int rpw = 64 / lpr;         // rows per wave step
    const int sub = lane / lpr;       // row slot within the wave step
    const int e0 = (lane % lpr) * 4;  // first element of this lane

    auto grp_sum = [&](float v) {
        // sum over the lpr lanes of this row group
        for (int off = lpr / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        return v;
    };

    // 1. pair features x_p for p in [t0 - halo, t0 + 64): row r = p - t0 + halo
    for (int r0 = wave * rpw; r0 < nrows; r0 += 4 * rpw) {
        const int r = r0 + sub;
        const int p = t0 - halo + r;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        bool from_k = false;
        if (r < nrows) {
            if (p >= 1 && p < T) {
                from_k = true;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = ld(k, size_t(p - 1) * dk + e0 + e);
            } else if (p == 0) {
                if (a.xnext_in)
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = a.xnext_in[size_t(bh) * dk + e0 + e];
            } else if (p < 0 && p >= -a.n_tail_in) {
                const int slot = p + halo;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = a.tailx_in[(size_t(bh) * halo + slot) * dk + e0 + e];
            }
        }
        float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        ss = grp_sum(ss);
        const float sc = from_k ? phi_scale(ss, dk, a.eps_rms, a.phi) : 1.f;
        float n2 = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] *= sc;
            n2 += x[e] * x[e];
        }
        n2 = grp_sum(n2);
        if (r < nrows) {
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[r * kXStride + e0 + e] = x[e];
            const int i = r - halo;  // token index within the tile
            if (i >= 0) {
                const int t = t0 + i;
                if (t < a.Tpad)
#pragma unroll
                    for (int e = 0; e < 4; ++e) st(xn, size_t(t) * dk + e0 + e, x[e]);
                if ((lane % lpr) == 0) mu_s[i] = n2;
            }
        }
    }
    // query features
    for (int i0 = wave * rpw; i0 < kTile; i0 += 4 * rpw) {
        const int i = i0 + sub;
        const int t = t0 + i;
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        if (t < T)
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = ld(q, size_t(t) * dk + e0 + e);
        float ss = grp_sum(y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3]);
        const float sc = phi_scale(ss, dk, a.eps_rms, a.phi);
        if (t < a.Tpad)
#pragma unroll
            for (int e = 0; e < 4; ++e) st(qn, size_t(t) * dk + e0 + e, y[e] * sc);
    }
    __syncthreads();

    // 2. window statistic (Falcon-3 / 3A): lambda_max of the W x W window Gram
    if (W > 1) {
        for (int idx = tid; idx < nrows * W; idx += 256) {
            const int r = idx / W, d = idx % W;
            float s = 0.f;
            if (r - d >= 0) {
                const float *x1 = xs + r * kXStride;
                const float *x2 = xs + (r - d) * kXStride;
                for (int e = 0; e < dk; ++e) s += x1[e] * x2[e];
            }
            band[r * kWmax + d] = s;
        }
        __syncthreads();
        if (tid < kTile) {
            const int i = tid, r = i + halo;
            float m[8][8];
#pragma unroll
            for (int aa = 0; aa < 8; ++aa)
#pragma unroll
                for (int bb = 0; bb < 8; ++bb) {
                    float g = 0.f;
                    if (aa < W && bb < W) {
                        const int lo = aa < bb ? aa : bb;
                        const int df = aa < bb ? bb - aa : aa - bb;
                        g = band[(r - lo) * kWmax + df];
                    }
                    m[aa][bb] = g;
                }
            const int t = t0 + i;
            const long long pairs = (long long)a.n_tail_in + t + 1;
            const int bt = pairs < W ? int(pairs) : W;
            mu_s[i] = psd_lambda_max(m, W) / float(bt);
        }
        __syncthreads();
    }

    // 3. step scalars
    const bool per_col = (a.variant == FALCON_V2 || a.variant == FALCON_V2A);
    if (tid < kTile) {
        const int t = t0 + tid;
        float den = 0.f;
        if (t < T) den = mu_s[tid] + a.lambda[size_t(bh) * T + t] + a.eps;
        den_s[tid] = den;
        if (!per_col && t < a.Tpad) {
            float eta = 0.f, alpha = 0.f;
            const bool noop = (t == 0 && a.fresh) || t >= T;
            if (!noop) {
                eta = step_eta(a.beta[size_t(bh) * T + t], den);
                alpha = step_alpha(eta, a.lambda[size_t(bh) * T + t], a.eps_gamma);
            }
            a.eta[size_t(bh) * a.Tpad + t] = eta;
            a.alpha[size_t(bh) * a.Tpad + t] = alpha;
        }
    }
    if (per_col) {
        __syncthreads();
        for (int idx = tid; idx < kTile * dv; idx += 256) {
            const int i = idx / dv, j = idx % dv;
            const int t = t0 + i;
            if (t >= a.Tpad) continue;
            float eta = 0.f, alpha = 0.f;
            const bool noop = (t == 0 && a.fresh) || t >= T;
            if (!noop) {
                eta = step_eta(a.beta[(size_t(bh) * T + t) * dv + j], den_s[i]);
                alpha = step_alpha(eta, a.lambda[size_t(bh) * T + t], a.eps_gamma);
            }
            a.eta[(size_t(bh) * a.Tpad + t) * dv + j] = eta;
            a.alpha[(size_t(bh) * a.Tpad + t) * dv + j] = alpha;
        }
    }

    // 4. boundary state out, from the tile holding the last token
    if (T > 0 && t0 <= T - 1 && T - 1 < t0 + kTile) {
        if (a.xnext_out) {
            // x_next = phi(k_{T-1}) is the feature of pair row T - t0 + halo
            // (not stored in xs when it falls past the tile): recompute it
            if (wave == 0) {
                float x[2] = {0.f, 0.f};
                float ss = 0.f;
                for (int e = lane; e < dk; e += 64) {
                    const float z = ld(k, size_t(T - 1) * dk + e);
                    x[e >> 6] = z;
                    ss += z * z;
                }
                ss = wave_sum(ss);
                const float sc = phi_scale(ss, dk, a.eps_rms, a.phi);
                for (int e = lane; e < dk; e += 64) a.xnext_out[size_t(bh) * dk + e] = x[e >> 6] * sc;
            }
        }
        if (halo > 0 && a.tailx_out) {
            const int n_out = a.n_tail_out;
            for (int idx = tid; idx < halo * dk; idx += 256) {
                const int s = idx / dk, e = idx % dk;
                const int p = T - halo + s;
                const bool valid = s >= halo - n_out;
                const int r = p - t0 + halo;
                a.tailx_out[(size_t(bh) * halo + s) * dk + e] = valid ? xs[r * kXStride + e] : 0.f;
            }
            const Ein *v = static_cast<const Ein *>(a.v) + size_t(bh) * T * dv;
            for (int idx = tid; idx < halo * dv; idx += 256) {
                const int s = idx / dv, e = idx % dv;
                const int p = T - halo + s;
                float y = 0.f;
                if (s >= halo - n_out) {
                    if (p >= 0)
                        y = ld(v, size_t(p) * dv + e);
                    else
                        y = a.taily_in[(size_t(bh) * halo + (p + halo)) * dv + e];
                }
                a.taily_out[(size_t(bh) * halo + s) * dv + e] = y;
            }
        }
    }
}

// seqlen == 0: the boundary state passes through unchanged
__global__ void passthrough_kernel(PassArgs a) {
    const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t nS = size_t(a.BH) * a.dk * a.dv;
    const size_t nX = size_t(a.BH) * a.dk;
    const size_t nTx = size_t(a.BH) * a.halo * a.dk;
    const size_t nTy = size_t(a.BH) * a.halo * a.dv;
    if (i < nS && a.S_out) a.S_out[i] = a.S_in ? a.S_in[i] : 0.f;
    if (i < nX && a.xnext_out) a.xnext_out[i] = a.xnext_in ? a.xnext_in[i] : 0.f;
    // tail slots before the valid ones are zero-filled
    if (i < nTx && a.tailx_out) {
        const int slot = int((i / a.dk) % a.halo);
        a.tailx_out[i] = (a.tailx_in && slot >= a.halo - a.n_tail) ? a.tailx_in[i] : 0.f;
    }
    if (i < nTy && a.taily_out) {
        const int slot = int((i / a.dv) % a.halo);
        a.taily_out[i] = (a.taily_in && slot >= a.halo - a.n_tail) ? a.taily_in[i] : 0.f;
    }
}

}  // namespace

void launch_features(const FeatureArgs &a, bool in_bf16, bool feat_bf16, hipStream_t s, Marks *m) {
    dim3 grid((a.Tpad + kTile - 1) / kTile, a.BH);
    if (in_bf16 && feat_bf16)
        feature_kernel<bf16_t, bf16_t><<<grid, 256, 0, s>>>(a);
    else if (in_bf16)
        feature_kernel<bf16_t, float><<<grid, 256, 0, s>>>(a);
    else if (feat_bf16)
        feature_kernel<float, bf16_t><<<grid, 256, 0, s>>>(a);
    else
        feature_kernel<float, float><<<grid, 256, 0, s>>>(a);
    m->mark(s);
}

void launch_passthrough(const PassArgs &a, hipStream_t s, Marks *m) {
    size_t n = size_t(a.BH) * a.dk * a.dv;
    const size_t nt = size_t(a.BH) * (a.halo > 0 ? a.halo : 1) * (a.dk > a.dv ? a.dk : a.dv);
    if (nt > n) n = nt;
    passthrough_kernel<<<(n + 255) / 256, 256, 0, s>>>(a);
    m->mark(s);
}

}  // namespace falcon
