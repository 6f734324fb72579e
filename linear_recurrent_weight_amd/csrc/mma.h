// MFMA tile helpers for the chunk kernels (gfx950, wave64).
#pragma once

#include "common.h"
#include "lambda_max.h"

namespace falcon {

// One 16x16 output tile: acc += A[16 x K] * B[K x 16].  A is row-major with k
// contiguous (row stride lda); B is given transposed, Bt[16 x K] with k
// contiguous (row stride ldb).  Result lane layout: acc[r] holds row
// 4*(lane/16)+r, column lane%16.  bf16 uses v_mfma_f32_16x16x32_bf16 (k step
// 32), fp32 uses v_mfma_f32_16x16x4_f32 (k step 4).
template <class E> struct Mma;

template <> struct Mma<bf16_t> {
    static constexpr int KS = 32;
    __device__ static f32x4 run(f32x4 acc, const bf16_t *A, int lda, const bf16_t *Bt, int ldb, int kbeg,
                                int kend) {
        const int lane = threadIdx.x & 63;
        const int row = lane & 15, kq = 8 * (lane >> 4);
        for (int k0 = kbeg; k0 < kend; k0 += KS) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(A + row * lda + k0 + kq);
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(Bt + row * ldb + k0 + kq);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
        return acc;
    }
};

template <> struct Mma<float> {
    static constexpr int KS = 4;
    __device__ static f32x4 run(f32x4 acc, const float *A, int lda, const float *Bt, int ldb, int kbeg,
                                int kend) {
        const int lane = threadIdx.x & 63;
        const int row = lane & 15, kq = lane >> 4;
        for (int k0 = kbeg; k0 < kend; k0 += KS) {
            const float a = A[row * lda + k0 + kq];
            const float b = Bt[row * ldb + k0 + kq];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
        return acc;
    }
};

// One k step of an MFMA operand held in registers, for operands that are
// loaded ahead of their use: row lane % 16 of a row-major [16 x K] tile,
// k = k0 + (the lane's k group).  Same layouts as Mma<E>::run.
template <class E> struct MmaFrag;

template <> struct MmaFrag<bf16_t> {
    using T = bf16x8;
    static constexpr int KS = 32;
    __device__ static T load(const bf16_t *M, int ld, int k0) {
        const int lane = threadIdx.x & 63;
        return *reinterpret_cast<const bf16x8 *>(M + (lane & 15) * ld + k0 + 8 * (lane >> 4));
    }
    __device__ static f32x4 mma(const T &a, const T &b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
};

template <> struct MmaFrag<float> {
    using T = float;
    static constexpr int KS = 4;
    __device__ static T load(const float *M, int ld, int k0) {
        const int lane = threadIdx.x & 63;
        return M[(lane & 15) * ld + k0 + (lane >> 4)];
    }
    __device__ static f32x4 mma(const T &a, const T &b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
};

// 32-deep contractions from 16-deep register pieces.  A 16x16 accumulator
// tile read back as a 16x16x16 operand gives lane (col, q) the 4 k values
// 4 q .. + 3 of its 16-block.  Two such pieces of consecutive 16-blocks side
// by side (cat8) are the lane's 8 k values of a 16x16x32 operand whose k
// index runs in pair order: within each 32, the 4-groups of the two 16-blocks
// alternate (k, k + 16, k + 4, k + 20, ...).  The other operand is stored
// with its k index in that same order (pair_slot of the first k of each
// aligned 4-group), so one 16-byte read gives its lane piece.
typedef short bf16x4_bits __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 cat8(const bf16x4_bits &lo, const bf16x4_bits &hi) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ int pair_slot(int k) {
    return (k & ~31) | (((k & 15) >> 2) << 3) | (((k >> 4) & 1) << 2);
}

// LDS row padding (elements) that keeps bf16 rows 16-byte aligned
template <class E> struct Pad;
template <> struct Pad<bf16_t> { static constexpr int v = 8; };
template <> struct Pad<float> { static constexpr int v = 4; };

template <class E>
__device__ __forceinline__ void st4(E *p, const f32x4 &v) {
#pragma unroll
    for (int r = 0; r < 4; ++r) st(p, r, v[r]);
}

}  // namespace falcon
