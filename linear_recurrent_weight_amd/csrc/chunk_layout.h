// Chunk size and per-chunk operator layout of the chunk-parallel paths.
// Pure C++: used by the host planner and by the kernels.
#pragma once

#include <cstddef>

#include "../../include/falcon.h"

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

// Falcon-3 (window W): a chunk holds 64 / W tokens; each token contributes
// its W window rows, so the stacked system has at most 64 rows.  Per chunk,
// in the storage type E:  Tp [64][64], P [64][64] (token rows x stacked rows),
// the stacked write features X [64][dk]; then fp32 [4][64]: per stacked row
// Gamma_{t-1}, e^{b_C - b_t}; per token Gamma_t; {Gamma_C, 0...}.
constexpr int chunk_f3_tokens(int window) { return kChunk / window; }
constexpr bool chunk_f3_supported(int dk, int dv) { return chunk_f1_supported(dk, dv); }
constexpr size_t chunk_f3_x_off(size_t esz) { return 2 * size_t(kChunk) * kChunk * esz; }
constexpr size_t chunk_f3_scal_off(int dk, size_t esz) { return chunk_f3_x_off(esz) + size_t(kChunk) * dk * esz; }
constexpr size_t chunk_f3_bytes(int dk, int dtype_is_f32) {
    return chunk_f3_scal_off(dk, dtype_is_f32 ? 4 : 2) + 4 * size_t(kChunk) * 4;
}

// bf16 Falcon-3 at d_k = d_v = 64 with a window of 2, 4 or 8 pairs: per
// 64-token chunk the Falcon-1 transfer operators (chunk_f3_xfer.hip, W
// sub-chunks of 64 stacked rows), walked by the Falcon-1 carry.
constexpr bool chunk_f3_xfer_supported(bool bf16, int dk, int dv, int window) {
    return bf16 && dk == 64 && dv == 64 && (window == 2 || window == 4 || window == 8);
}

// Falcon-2 chunk path: one kernel, no workspace.  bf16: d_k in {64, 128};
// fp32: d_k = 64 (on-chip buffers); any d_v (a multiple of 16).
constexpr bool chunk_f2_supported(bool bf16, int dk, int dv) {
    return (bf16 ? (dk == 64 || dk == 128) : dk == 64) && dv % 16 == 0;
}

// Transfer-operator bf16 Falcon-1 path (d_k = 64): per chunk, bf16
//   A   [64 d'][64 d] = -(diag(e^{b_C-b_t}) X)^T W        (state transfer, less e^{b_C} I)
//   G   [64 t][64 d]  = diag(e^{b_t}) Qh - P W             (outputs from the entry state)
//   B^T [d_v j][64 d] = ((diag(e^{b_C-b_t}) X)^T Ut)^T      (state write)
//   H   [64 t][d_v j] = P Ut                               (outputs from the chunk's writes)
// with W = Tp diag(e^{b_{t-1}}) X and Ut = Tp Y; then fp32 e^{b_C} in a
// 256-byte block.  Each block is stored in the lane order of the MFMA
// operands that read it, 16 x 16 (or 16 x 32) tiles one after another:
//   A, G: [row tile m 4][k half h 2][lane l 64] x 16 bytes, lane l holding
//         row 16 m + l % 16, elements 32 h + 8 (l / 16) .. + 7;
//   B^T, H: [value tile jt][row tile m 4][lane l 64] x 8 bytes, lane l holding
//         B rows 16 m + 4 (l / 16) .. + 3 of column 16 jt + l % 16, and H
//         row 16 m + l % 16, columns 16 jt + 4 (l / 16) .. + 3.
constexpr bool chunk_f1_xfer_supported(bool bf16, int dk, int dv) {
    return bf16 && dk == 64 && (dv == 32 || dv == 64 || dv == 128);
}
constexpr size_t kF1XferGOff = 8192;
constexpr size_t kF1XferBOff = 16384;
constexpr size_t f1_xfer_h_off(int dv) { return 16384 + size_t(dv) * 128; }
constexpr size_t f1_xfer_scal_off(int dv) { return 16384 + size_t(dv) * 256; }
constexpr size_t f1_xfer_bytes(int dv) { return f1_xfer_scal_off(dv) + 256; }
// value columns per workgroup of the carry kernel: 32 (two workgroups per
// head share the operator traffic), never more than d_v
constexpr int f1_xfer_slice(int dv) { return dv < 32 ? dv : 32; }
// Composed map of a segment, S -> gamma S + A~ S + beta (gamma apart):
//   A~   [64 d][64 d'] bf16 in MFMA A-operand lane order, [row tile m 4][k half
//        h 2][lane l 64] x 16 bytes (row 16 m + l % 16, d' = 32 h + 8 (l / 16) ..);
//   beta [64 d][d_v j] fp32 in accumulator order, [row tile m 4][value tile
//        d_v / 16][lane l 64] x 16 bytes (rows 16 m + 4 (l / 16) .. + 3 of
//        column 16 jt + l % 16).
constexpr size_t kF1SegBetaOff = 8192;
constexpr size_t f1_segmap_bytes(int dv) { return kF1SegBetaOff + size_t(dv) * 256; }
// workgroups of the carry for bh heads walking in slices of ds columns
// (heads rounded up to 8 when a head has several slices)
constexpr long long f1_carry_groups(long long bh, int dv, int ds) {
    return dv / ds == 1 ? bh : (bh + 7) / 8 * 8 * (dv / ds);
}
// Chunks per segment of the carry.  The walk over a head's chunks is the
// sequential part; when few walks run (few heads) over many chunks, it
// splits into segments whose composed maps are scanned first.  A carry
// workgroup (one per compute unit) moves its operators at about a fixed
// rate, so the carry's time follows its chunk steps per compute unit, and
// the segment maps stream every record once more whatever their length.
// Segments are sized for about two passes of carry workgroups (512), and
// hold at least 16 chunks.  A walk of fewer than 48 chunks, or one whose
// heads alone exceed one pass (256 workgroups), is not split (returns
// nchunks).
constexpr int f1_xfer_segment_chunks(long long bh, int dv, int nchunks) {
    const long long groups = f1_carry_groups(bh, dv, f1_xfer_slice(dv));
    if (nchunks < 48 || groups > 256) return nchunks;
    const long long nseg = 512 / groups;
    const long long g = (nchunks + nseg - 1) / nseg;
    return static_cast<int>(g < 16 ? 16 : g);
}

// Falcon-2A chunk path (chunk_f2a.hip): d_k in {32, 64}, any d_v (slices of
// up to 64 columns), no workspace.
constexpr bool chunk_f2a_supported(int dk, int dv) { return (dk == 32 || dk == 64) && dv % 16 == 0; }

// Falcon-1A / Falcon-3A chunk path: d_k in {32, 64}, d_v in {16, 32, 64}.
constexpr bool chunk_a_supported(int dk, int dv) {
    return (dk == 32 || dk == 64) && (dv == 16 || dv == 32 || dv == 64);
}
// chunks per segment: enough segments for a few workgroups per compute unit
inline int chunk_a_segment_chunks(long long bh, int nchunks) {
    long long g = (bh * nchunks + 639) / 640;
    if (g < 1) g = 1;
    if (g > 32) g = 32;
    return int(g);
}

// The bf16 Falcon-1A / Falcon-3A path with every token-contracting operand
// transposed once per chunk (chunk_a1.hip): d_k = d_v = 64.
inline bool chunk_a1_supported(bool bf16, int variant, int window, int dk, int dv) {
    const bool var_ok = (variant == FALCON_V1A && window == 1) || (variant == FALCON_V3A && window >= 1);
    return bf16 && var_ok && dk == 64 && dv == 64;
}
// Up to this many segments per head, each output walk of that path folds its
// own entry state from the segment aggregates (no scan launch); more segments
// take the scan.
constexpr int chunk_a1_fold_segments = 8;
// chunks per segment of that path: the fewest that keep all segments of all
// heads resident at once (two 512-thread workgroups per compute unit, 256
// units), so that the walks run as one wave of workgroups
inline int chunk_a1_segment_chunks(long long bh, int nchunks) {
    constexpr long long kSlots = 512;
    for (int g = 1; g < nchunks; ++g)
        if (bh * ((nchunks + g - 1) / g) <= kSlots) return g;
    return nchunks > 0 ? nchunks : 1;
}

}  // namespace falcon
