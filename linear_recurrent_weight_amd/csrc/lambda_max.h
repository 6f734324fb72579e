// Window statistic helper, shared by the HIP kernels and a host-side test
// build (it includes no HIP header).
#pragma once

#include <math.h>

#if defined(__HIPCC__)
#define FALCON_HD __host__ __device__
#else
#define FALCON_HD
#endif

namespace falcon {

// Largest eigenvalue of a symmetric positive semi-definite n x n matrix
// (n <= 8, entries beyond n ignored), fp32.  Lanczos with full
// re-orthogonalisation reduces G to a symmetric tridiagonal matrix with the
// same spectrum (whenever the Krylov space closes before n steps, the next
// vector is the unit vector with the largest component outside the space
// found so far, and the coupling is 0, so the reduction always covers the
// whole space).  Newton's method from an upper bound then converges
// monotonically to the largest root of det(T - x I).  Used for the window
// statistic mu_t = lambda_max(window covariance) (summary §C.6: the exact
// top eigenvalue of the small active-window Gram).
FALCON_HD inline float psd_lambda_max(const float (&G)[8][8], int n) {
    float tr = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) tr += i < n ? G[i][i] : 0.f;
    if (!(tr > 0.f)) return 0.f;
    const float inv = 1.f / tr;   // work on G / trace: eigenvalues in [0, 1]
    float Q[8][8];
    float al[8], be[8];
    float v[8];
    const float v0 = 1.f / sqrtf(float(n));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = i < n ? v0 : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        al[k] = 0.f;
        be[k] = 0.f;
        if (k < n) {
            if (k > 0) {
                if (be[k - 1] > 1e-5f) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] *= 1.f / be[k - 1];
                } else {
                    // the Krylov space closed: continue with a fresh direction
                    be[k - 1] = 0.f;
                    float best = -1.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if (j < n) {
                            float u[8];
#pragma unroll
                            for (int i = 0; i < 8; ++i) u[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
                            for (int q = 0; q < 8; ++q) {
                                if (q < k) {
                                    const float h = Q[q][j];
#pragma unroll
                                    for (int i = 0; i < 8; ++i) u[i] -= h * Q[q][i];
                                }
                            }
                            float nn = 0.f;
#pragma unroll
                            for (int i = 0; i < 8; ++i) nn += u[i] * u[i];
                            if (nn > best) {
                                best = nn;
#pragma unroll
                                for (int i = 0; i < 8; ++i) v[i] = u[i];
                            }
                        }
                    }
                    const float s = 1.f / sqrtf(best);
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] *= s;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) Q[k][i] = v[i];
            float w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) s += (i < n && j < n ? G[i][j] : 0.f) * v[j];
                w[i] = s * inv;
            }
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) a += v[i] * w[i];
            al[k] = a;
            // full re-orthogonalisation against every Lanczos vector, twice
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (j <= k) {
                        float h = 0.f;
#pragma unroll
                        for (int i = 0; i < 8; ++i) h += Q[j][i] * w[i];
#pragma unroll
                        for (int i = 0; i < 8; ++i) w[i] -= h * Q[j][i];
                    }
                }
            }
            float b2 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) b2 += w[i] * w[i];
            be[k] = sqrtf(b2);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = w[i];
        }
    }
    // Newton from above on det(T_n - x I) (three-term recurrence)
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i < n) {
            const float r = al[i] + (i > 0 ? fabsf(be[i - 1]) : 0.f) + (i + 1 < n ? fabsf(be[i]) : 0.f);
            x = fmaxf(x, r);
        }
    }
    x = x * 1.0000001f + 1e-12f;
    for (int it = 0; it < 80; ++it) {
        float p0 = 1.f, p1 = al[0] - x, d0 = 0.f, d1 = -1.f;
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            if (i < n) {
                const float b2 = be[i - 1] * be[i - 1];
                const float p2 = (al[i] - x) * p1 - b2 * p0;
                const float d2 = (al[i] - x) * d1 - p1 - b2 * d0;
                p0 = p1;
                p1 = p2;
                d0 = d1;
                d1 = d2;
            }
        }
        if (d1 == 0.f) break;
        const float step = p1 / d1;
        const float xn = x - step;
        if (!(xn < x)) break;   // monotone from above: stop when no progress
        x = xn;
        if (step <= 1e-7f * x) break;
    }
    return fmaxf(x, 0.f) * tr;
}

}  // namespace falcon
