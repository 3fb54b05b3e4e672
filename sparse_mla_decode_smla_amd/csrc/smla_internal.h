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

// kv_format 2, the pages' paged layout: d_qk = d_v = 512; a token row is 448
// e4m3 "nope" values then 64 bf16 rope values (576 bytes); a block holds its
// 64 rows, then its 64 scale records of 8 bytes (7 UE8M0 exponents, one per
// 64 nope values, and a pad byte).
constexpr int kDqkV4 = 512;
constexpr int kNopeV4 = 448;
constexpr int kRowBytesV4 = kNopeV4 + 2 * (kDqkV4 - kNopeV4);  // 576 = 36 x 16
constexpr int kScaleRecBytesV4 = 8;
constexpr int kSlotBytesV4 = kRowBytesV4 + kScaleRecBytesV4;   // 584 gathered per token
constexpr int kBlockBytesV4 = kBlock * kSlotBytesV4;           // 37376

// LDS image of one stage (kTile tokens).  Rows are stored as 128-byte bands:
// band j of every token of the tile is contiguous ([band][token][128 B]), and
// the eight 16-byte chunks inside a band are XOR-swizzled by the token index.
//   bf16: 9 bands (576 bf16)                               -> 36864 B
//   fp8 : 4 bands of e4m3 c_kv + 1 band of bf16 rope, then
//         kTile x 16 B of fp32 scales                      -> 20992 B
//   v4  : 4 bands (row bytes 0..511: the 448 e4m3 values and rope values
//         0..31), a half band [token][64 B] (rope values 32..63, its four
//         chunks XOR-swizzled by (token >> 2) & 3), then the kTile scale
//         records [token][8 B]                             -> 18688 B
constexpr int kBandsBf16 = 9;
constexpr int kBandsFp8 = 5;
constexpr int kBandsV4 = 4;
constexpr int kStageBytesBf16 = kBandsBf16 * kTile * 128;
constexpr int kStageBytesFp8 = kBandsFp8 * kTile * 128 + kTile * 16;
constexpr int kStageBytesV4 = kBandsV4 * kTile * 128 + kTile * 64 + kTile * kScaleRecBytesV4;
constexpr int kStagesBf16 = 4;
constexpr int kStagesFp8 = 5;
constexpr int kStagesV4 = 4;

// Exchange area after the stage ring, double-buffered by tile parity:
//   P      the softmax weights of a tile, bf16, in the order of the PV B
//          operand: [16-head block][4 lane groups][16 heads] x 16 bytes; for
//          fp8 rows one copy per 128-group with that group's per-token scale
//          folded in; for v4 rows one copy per 64-group of nope values with
//          that group's per-token scale folded in, and an unscaled copy for
//          the rope values (8 copies);
//   alpha  per-head factors [64] fp32 that rescale the output accumulators
//          when a head's reference maximum was raised at that tile;
//   flags  one int per 16-head block: its references were raised at that tile;
// then denom, the per-head softmax denominators [64] fp32, and (fp8 rows)
// the area in which the two QK waves that share 32 heads swap per-head
// values once a step: per QK wave, 16 records of 16 bytes (two heads' values
// and a step tag twice).
constexpr int kPBytesPerCopy = kHeads * kTile * 2;
inline constexpr int aux_p_copies(int kv_format) { return kv_format == 0 ? 1 : kv_format == 1 ? 4 : 8; }
inline constexpr int aux_p_buffer_bytes(int kv_format) { return aux_p_copies(kv_format) * kPBytesPerCopy; }
inline constexpr int aux_alpha_offset(int kv_format) { return 2 * aux_p_buffer_bytes(kv_format); }
inline constexpr int aux_flag_offset(int kv_format) { return aux_alpha_offset(kv_format) + 2 * kHeads * 4; }
inline constexpr int aux_denom_offset(int kv_format) { return aux_flag_offset(kv_format) + 2 * 16; }
inline constexpr int aux_swap_offset(int kv_format) { return aux_denom_offset(kv_format) + kHeads * 4; }
inline constexpr int aux_bytes(int kv_format) { return aux_swap_offset(kv_format) + (kv_format == 1 ? 4 * 16 * 16 : 0); }

constexpr int kLdsLimit = 160 * 1024;  // bytes of LDS a gfx950 workgroup may use

inline int stage_bytes(int kv_format) {
    return kv_format == 0 ? kStageBytesBf16 : kv_format == 1 ? kStageBytesFp8 : kStageBytesV4;
}
inline int num_stages(int kv_format) { return kv_format == 0 ? kStagesBf16 : kv_format == 1 ? kStagesFp8 : kStagesV4; }
// Bytes gathered from HBM per selected token.
inline int gathered_bytes_per_token(int kv_format) {
    return kv_format == 0 ? kRowBytesBf16 : kv_format == 1 ? kRowBytesFp8 : kSlotBytesV4;
}

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
