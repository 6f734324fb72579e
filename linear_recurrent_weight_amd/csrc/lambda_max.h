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

// Reciprocal and square root: the hardware's approximations (about one ulp)
// in GPU code, where the exact sequences sit on the dependency chain of every
// step; the exact operations in the host build that the eigenvalue tests use.
FALCON_HD inline float lm_rcp(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_rcpf(x);
#else
    return 1.f / x;
#endif
}
FALCON_HD inline float lm_sqrt(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_sqrtf(x);
#else
    return sqrtf(x);
#endif
}

// Largest eigenvalue of a symmetric positive semi-definite n x n matrix
// (n <= 8, entries beyond n ignored), fp32.  The matrix, zero-padded to
// 8 x 8 (the padding only adds zero eigenvalues) and scaled by its trace,
// is reduced to a symmetric tridiagonal matrix with the same spectrum by six
// Householder reflections (A <- H A H, H = I - beta v v^T, applied as the
// rank-two update A - v w^T - w v^T); Laguerre's method from the Gershgorin
// bound then descends monotonically, with cubic convergence, to the largest
// root of det(x I - T) (a few iterations where Newton needs about ten).  Used
// for the window statistic mu_t = lambda_max(window covariance) (summary
// §C.6: the exact top eigenvalue of the small active-window Gram).
FALCON_HD inline float psd_lambda_max(const float (&G)[8][8], int n) {
    float tr = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) tr += i < n ? G[i][i] : 0.f;
    if (!(tr > 0.f)) return 0.f;
    const float inv = lm_rcp(tr);   // work on G / trace: eigenvalues in [0, 1]
    // A stays symmetric under the reflections: only its lower triangle
    // (j <= i) is read, kept and updated, and only G's lower triangle is read
    float A[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j) A[i][j] = (i < n && j < n) ? G[i][j] * inv : 0.f;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        // reflect x = A[k+1..7][k] onto (alpha, 0, ..., 0)
        float xx = 0.f;
#pragma unroll
        for (int i = k + 1; i < 8; ++i) xx += A[i][k] * A[i][k];
        const float x0 = A[k + 1][k];
        const float nx = lm_sqrt(xx);
        const float alpha = x0 > 0.f ? -nx : nx;
        float v[8];
#pragma unroll
        for (int i = k + 1; i < 8; ++i) v[i] = i == k + 1 ? x0 - alpha : A[i][k];
        const float vv = 2.f * (xx - alpha * x0);   // |v|^2
        const float beta = vv > 1e-30f ? 2.f * lm_rcp(vv) : 0.f;
        float p[8];
#pragma unroll
        for (int i = k + 1; i < 8; ++i) {
            float s = 0.f;
#pragma unroll
            for (int j = k + 1; j < 8; ++j) s += (j <= i ? A[i][j] : A[j][i]) * v[j];
            p[i] = beta * s;
        }
        float vp = 0.f;
#pragma unroll
        for (int i = k + 1; i < 8; ++i) vp += v[i] * p[i];
        const float K = 0.5f * beta * vp;
#pragma unroll
        for (int i = k + 1; i < 8; ++i) p[i] -= K * v[i];   // w
#pragma unroll
        for (int i = k + 1; i < 8; ++i)
#pragma unroll
            for (int j = k + 1; j <= i; ++j) A[i][j] -= v[i] * p[j] + p[i] * v[j];
        A[k + 1][k] = beta > 0.f ? alpha : x0;
    }
    float al[8], be[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        al[i] = A[i][i];
        be[i] = i < 7 ? A[i + 1][i] : 0.f;
    }
    // Laguerre's method from above on q(x) = det(x I - T) (degree 8, all
    // roots real): every iterate stays above the largest root and the
    // convergence is cubic.  g = q'/q, h = g^2 - q''/q from the three-term
    // recurrence of det(T_k - x I) and its first two derivatives.
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float r = al[i] + (i > 0 ? fabsf(be[i - 1]) : 0.f) + (i < 7 ? fabsf(be[i]) : 0.f);
        x = fmaxf(x, r);
    }
    x = x * 1.0000001f + 1e-12f;
    for (int it = 0; it < 32; ++it) {
        float p0 = 1.f, p1 = al[0] - x, d0 = 0.f, d1 = -1.f, e0 = 0.f, e1 = 0.f;
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            const float b2 = be[i - 1] * be[i - 1], ai = al[i] - x;
            const float p2 = ai * p1 - b2 * p0;
            const float d2 = ai * d1 - p1 - b2 * d0;
            const float e2 = ai * e1 - 2.f * d1 - b2 * e0;
            p0 = p1; p1 = p2;
            d0 = d1; d1 = d2;
            e0 = e1; e1 = e2;
        }
        // above every root q > 0 and q'/q > 0; a rounding step onto or past
        // the largest root ends the iteration there
        if (!(p1 > 0.f)) break;
        const float ip = lm_rcp(p1);
        const float g = d1 * ip, h = g * g - e1 * ip;
        if (!(g > 0.f)) break;
        const float den = g + lm_sqrt(fmaxf(7.f * (8.f * h - g * g), 0.f));
        const float step = 8.f * lm_rcp(den);
        const float xn = x - step;
        if (!(xn < x)) break;   // monotone from above: stop when no progress
        x = xn;
        if (step <= 1e-7f * x) break;
    }
    return fmaxf(x, 0.f) * tr;
}

}  // namespace falcon
