// Internal constants and launch-shape helpers shared by the host plan and the
// kernels of the GPU library (not part of the public ABI).
#pragma once

#include <cstddef>
#include <cstdint>

namespace smla {

// The one problem shape the kernels implement.
constexpr int kHeads = 64;       // query heads sharing one latent row
constexpr int kDqk = 576;        // c_kv (512) + rope (64)
constexpr int kDv = 512;         // value width = c_kv part
constexpr int kDr = kDqk - kDv;  // rope width
constexpr int kBlock = 64;       // tokens per cache block

// Workgroup shape of the partial-attention kernel: 8 waves of 64 lanes, two
// per SIMD, in two roles that work on consecutive tiles at the same time.
//   QK waves 0-3: wave w computes the scores and softmax weights of heads
//     [16w, 16w + 16) over all 32 tokens of tile k;
//   PV waves 4-7: wave 4+p accumulates value dims [128p, 128p + 128) of all
//     64 heads over tile k-1, and issues the tile gathers.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;        // tokens gathered per pipeline stage

// Bytes of one latent row in HBM.
constexpr int kRowBytesBf16 = 2 * kDqk;                       // 1152 = 9 x 128
constexpr int kRowBytesFp8 = kDv + 2 * kDr + 4 * (kDv / 128); // 656 = 41 x 16

// LDS image of one stage (kTile tokens).  Rows are stored as 128-byte bands:
// band j of every token of the tile is contiguous ([band][token][128 B]), and
// the eight 16-byte chunks inside a band are XOR-swizzled by the token index.
//   bf16: 9 bands (576 bf16)                               -> 36864 B
//   fp8 : 4 bands of e4m3 c_kv + 1 band of bf16 rope, then
//         kTile x 16 B of fp32 scales                      -> 20992 B
constexpr int kBandsBf16 = 9;
constexpr int kBandsFp8 = 5;
constexpr int kStageBytesBf16 = kBandsBf16 * kTile * 128;
constexpr int kStageBytesFp8 = kBandsFp8 * kTile * 128 + kTile * 16;
constexpr int kStagesBf16 = 4;
constexpr int kStagesFp8 = 5;

// Exchange area after the stage ring, double-buffered by tile parity:
//   P      the softmax weights of a tile, bf16, in the order of the PV B
//          operand: [16-head block][4 lane groups][16 heads] x 16 bytes; for
//          fp8 rows one copy per 128-group with that group's per-token scale
//          folded in;
//   alpha  per-head factors [64] fp32 that rescale the output accumulators
//          when a head's reference maximum was raised at that tile;
//   flags  one int per QK wave: it raised a reference at that tile;
// then denom, the per-head softmax denominators [64] fp32.
constexpr int kPBytesPerCopy = kHeads * kTile * 2;
inline constexpr int aux_p_buffer_bytes(int kv_format) { return kv_format == 0 ? kPBytesPerCopy : 4 * kPBytesPerCopy; }
inline constexpr int aux_alpha_offset(int kv_format) { return 2 * aux_p_buffer_bytes(kv_format); }
inline constexpr int aux_flag_offset(int kv_format) { return aux_alpha_offset(kv_format) + 2 * kHeads * 4; }
inline constexpr int aux_denom_offset(int kv_format) { return aux_flag_offset(kv_format) + 2 * 16; }
inline constexpr int aux_bytes(int kv_format) { return aux_denom_offset(kv_format) + kHeads * 4; }

constexpr int kLdsLimit = 160 * 1024;  // bytes of LDS a gfx950 workgroup may use

inline int stage_bytes(int kv_format) { return kv_format == 0 ? kStageBytesBf16 : kStageBytesFp8; }
inline int num_stages(int kv_format) { return kv_format == 0 ? kStagesBf16 : kStagesFp8; }

// LDS of one workgroup: the stage ring, the exchange area, and one int32
// physical-row entry per token of its part of the top-k list.
inline size_t partial_lds_bytes(int kv_format, int tokens_per_split) {
    return (size_t)num_stages(kv_format) * stage_bytes(kv_format) + aux_bytes(kv_format) + 4 * (size_t)tokens_per_split;
}

// Largest part of the list (a multiple of kTile) whose row table still fits.
inline int max_tokens_per_split(int kv_format) {
    long room = (long)kLdsLimit - (long)num_stages(kv_format) * stage_bytes(kv_format) - aux_bytes(kv_format);
    return (int)((room / 4) / kTile * kTile);
}

}  // namespace smla
