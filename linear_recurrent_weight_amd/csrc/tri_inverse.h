// Inverse of a 64 x 64 unit-lower-triangular matrix I + L held in LDS (fp32),
// by 16 x 16 blocks, for one workgroup of 256 threads (4 waves).
//   diagonal blocks: forward substitution, one column per lane (wave J does
//     block J);
//   off-diagonal blocks, by distance d = I - J:
//     T_IJ = -T_II * sum_{K=J}^{I-1} L_IK T_KJ.
// Lm holds the strictly lower part of L (its upper blocks are never read),
// row stride ld.  Tm receives the inverse's lower blocks; its upper blocks are
// left as they were.  Mt is 3 * 16 * 17 floats of scratch.  Must be called by
// all 256 threads (it contains workgroup barriers); Lm must be complete and
// visible (barrier before the call).
#pragma once

#include <hip/hip_runtime.h>

namespace falcon {

__device__ __forceinline__ void unit_lower_inverse64(const float *Lm, float *Tm, float *Mt, int ld) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (lane < 16) {
        const int base = 16 * wave;
        float tcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == lane) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < r; ++kk) s -= Lm[(base + r) * ld + base + kk] * tcol[kk];
            tcol[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Tm[(base + r) * ld + base + lane] = tcol[r];
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        const int nblk = 4 - d;
        for (int idx = tid; idx < nblk * 256; idx += 256) {
            const int blk = idx >> 8, e = idx & 255;
            const int J = blk, I = blk + d;
            const int r = e >> 4, cc = e & 15;
            float s = 0.f;
            for (int K = J; K < I; ++K)
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    s += Lm[(16 * I + r) * ld + 16 * K + kk] * Tm[(16 * K + kk) * ld + 16 * J + cc];
            Mt[blk * 272 + r * 17 + cc] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < nblk * 256; idx += 256) {
            const int blk = idx >> 8, e = idx & 255;
            const int J = blk, I = blk + d;
            const int r = e >> 4, cc = e & 15;
            float s = 0.f;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) s += Tm[(16 * I + r) * ld + 16 * I + kk] * Mt[blk * 272 + kk * 17 + cc];
            Tm[(16 * I + r) * ld + 16 * J + cc] = -s;
        }
        __syncthreads();
    }
}

}  // namespace falcon
