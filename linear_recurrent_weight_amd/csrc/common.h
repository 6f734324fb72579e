// Device helpers shared by the Falcon HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/falcon.h"

namespace falcon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 is carried as its 16-bit pattern.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// round to nearest even; inputs are finite
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

template <class E> struct elem;
template <> struct elem<float> {
    __device__ static float load(const float *p, size_t i) { return p[i]; }
    __device__ static void store(float *p, size_t i, float v) { p[i] = v; }
};
template <> struct elem<bf16_t> {
    __device__ static float load(const bf16_t *p, size_t i) { return bf16_to_f32(p[i].bits); }
    __device__ static void store(bf16_t *p, size_t i, float v) { p[i].bits = f32_to_bf16(v); }
};

template <class E> __device__ __forceinline__ float ld(const E *p, size_t i) { return elem<E>::load(p, i); }
template <class E> __device__ __forceinline__ void st(E *p, size_t i, float v) { elem<E>::store(p, i, v); }

// Cross-lane moves through DPP (no LDS round trip).  `src` moved by the
// DPP control `ctrl`; lanes whose source is outside the row, or whose row is
// masked off, read 0.
template <int ctrl, int row_mask = 0xf>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, row_mask,
                                                                 0xf, true));
}
// DPP controls (gfx9): quad permutations, row shifts, mirrors, broadcasts
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Sum over the lanes of a group of `width` consecutive lanes (width a power
// of two <= 64); every lane of the group receives the total.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(width >= 1 && width <= 64 && (width & (width - 1)) == 0, "power of two");
    if constexpr (width >= 2) v += dpp<kDppQuadXor1>(v);
    if constexpr (width >= 4) v += dpp<kDppQuadXor2>(v);
    if constexpr (width >= 8) v += dpp<kDppRowHalfMirror>(v);   // other quad of the half row
    if constexpr (width >= 16) v += dpp<kDppRowMirror>(v);      // other half of the row
    if constexpr (width >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (width >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// Inclusive prefix sum over the 64 lanes of a wave: scans inside each row of
// 16 lanes by shifted adds, then carries the row totals forward.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
    v += dpp<kDppRowShr1>(v);
    v += dpp<kDppRowShr2>(v);
    v += dpp<kDppRowShr4>(v);
    v += dpp<kDppRowShr8>(v);
    v += dpp<kDppRowBcast15, 0xa>(v);   // rows 1, 3 += last lane of rows 0, 2
    v += dpp<kDppRowBcast31, 0xc>(v);   // rows 2, 3 += last lane of row 1
    return v;
}

// Feature map phi (reading: z / sqrt(mean(z^2) + eps_rms), and 0 when that
// denominator is 0); `ss` is the sum of squares over d elements.
__device__ __forceinline__ float phi_scale(float ss, int d, float eps_rms, int phi_kind) {
    if (phi_kind == FALCON_PHI_IDENTITY) return 1.f;
    float ms = ss / float(d) + eps_rms;
    return ms > 0.f ? 1.f / sqrtf(ms) : 0.f;
}

// Orders LDS traffic between the lanes of one wave (no workgroup barrier):
// waits for this wave's outstanding LDS operations and keeps the compiler
// from moving memory accesses across the call.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

// log2(1 - alpha) for alpha in [0, 1), to about 1e-7 relative: for alpha
// < 1/4 the series log(1 - a) = -2 atanh(z) = -2 (z + z^3/3 + z^5/5 + ...),
// z = a / (2 - a) <= 1/7 (five terms); above, the native log2 of 1 - alpha
// (exact in fp32 there).
__device__ __forceinline__ float log2_1m(float alpha) {
    if (alpha < 0.25f) {
        const float z = alpha * __builtin_amdgcn_rcpf(2.f - alpha), z2 = z * z;
        const float p = z * (1.f + z2 * (1.f / 3.f + z2 * (1.f / 5.f + z2 * (1.f / 7.f + z2 * (1.f / 9.f)))));
        return -2.f * 1.4426950408889634f * p;
    }
    return __builtin_amdgcn_logf(1.f - alpha);
}

// eta = beta / den (0 if den == 0), alpha = min(eta * lambda, 1 - eps_gamma)
__device__ __forceinline__ float step_eta(float beta, float den) { return den != 0.f ? beta / den : 0.f; }
__device__ __forceinline__ float step_alpha(float eta, float lam, float eps_gamma) {
    return fminf(eta * lam, 1.f - eps_gamma);
}

}  // namespace falcon
