// Chunk size and per-chunk operator layout of the chunk-parallel paths.
// Pure C++: used by the host planner and by the kernels.
#pragma once

#include <cstddef>

namespace falcon {

constexpr int kChunk = 64;

// Falcon-1: per chunk, in the storage type E of the features (bf16 or fp32):
//   Tp [64][64]  = Linv diag(eta), Linv the inverse of the unit-lower system
//   P  [64][64]  = decayed causal scores (diagonal included)
// followed by fp32 [4][64]: Gamma_{i-1}, Gamma_i, e^{b_C - b_i}, {Gamma_C, 0...}
constexpr bool chunk_f1_supported(int dk, int dv) {
    return (dk == 32 || dk == 64 || dk == 128) && dv % 16 == 0;
}
constexpr size_t chunk_f1_tp_off() { return 0; }
constexpr size_t chunk_f1_p_off(size_t esz) { return size_t(kChunk) * kChunk * esz; }
constexpr size_t chunk_f1_scal_off(size_t esz) { return 2 * size_t(kChunk) * kChunk * esz; }
constexpr size_t chunk_f1_bytes(int /*dk*/, int /*dv*/, int dtype_is_f32) {
    const size_t esz = dtype_is_f32 ? 4 : 2;
    return chunk_f1_scal_off(esz) + 4 * size_t(kChunk) * 4;
}

}  // namespace falcon
