// Partial-attention kernel of head-batched sparse MLA decode, and the
// smla_decode_run entry point.
//
// One workgroup handles one query row (b, s), all 64 heads, and one part of
// that row's top-k list.  Every selected latent row is gathered from the
// paged cache into LDS once and read from there by all eight waves: QK
// waves 0..3 (wave w owns heads [16w, 16w + 16); for fp8 rows waves 2c and
// 2c + 1 share heads [32c, 32c + 32) and split each tile's tokens) and PV
// waves 4..7 (wave 4 + p owns value dims [128p, 128p + 128) and issues a
// quarter of the gathers).  This is the head batching of "The MMA Sparse-MLA
// Decode Kernel: A Deep Dive into AI Inference Optimization on Blackwell
// GPUs" (Agent Reasoning, "Design Decisions" 1 and "Memory Budgeting"), here
// with all 64 heads in one workgroup since a gfx950 CU has 160 KB of LDS.
// Cutting the list into parts is the split-K of "The Moment of Truth:
// Analyzing a Custom MMA Kernel's Performance on Blackwell GPUs" ("The
// Split-K Solution: Reasoning About the Fix"); each part writes a normalised
// partial output and its log-sum-exp, merged by the combine kernel.
//
// Per tile of 32 tokens:
//   gather  : 16-byte LDS-DMA loads (global_load_lds_dwordx4) of whole rows,
//             pipelined over a ring of LDS stages; masked tokens load zeros;
//   QK^T    : S^T[token, head] = K . Q^T with v_mfma_f32_16x16x32_bf16,
//             Q held in registers, K read from LDS (fp8 rows are widened to
//             bf16 in registers; the per-128 fp32 scale multiplies the
//             per-group partial scores; the power-of-two UE8M0 scales of the
//             pages' layout are applied exactly inside the widening);
//   softmax : online, base 2, running max and sum per head in registers,
//             masked tokens get -inf ("Edge Case Handling": invalid tokens
//             never enter the softmax);
//   PV      : O^T[dim, head] += V^T . P^T with the same MFMA; V^T comes from
//             the same LDS tile through transpose reads (ds_read_b64_tr_b16,
//             ds_read_b64_tr_b8); fp32 accumulation, bf16 only at the store
//             ("Design Decisions" 6).  A transposed fp8 operand holds eight
//             tokens per lane, so per-token scales are folded into the
//             weights P instead: one scaled copy of P per scale group.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "smla.h"
#include "smla_internal.h"

namespace smla {

smla_status_t launch_combine(const uint16_t* part_out, const float* part_lse, int num_splits, int64_t pairs,
                             void* out, float* lse, hipStream_t stream, bool stream_parts);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Source of the 16-byte loads of masked tokens: their LDS slots become zeros,
// so a masked token contributes 0 * 0 to the PV product.
__device__ __attribute__((aligned(16))) const unsigned char kZeroChunk[16] = {0};

struct PartialArgs {
    const uint16_t* q;
    const uint8_t* kv;
    const int32_t* block_table;
    const int32_t* indices;
    const int32_t* seq_lens;
    uint16_t* out;
    float* lse;
    uint16_t* part_out;  // bf16 partial outputs [S, rows, H, d_v]
    float* part_lse;
    int64_t num_kv_blocks;
    int32_t rows, q_len, topk, max_blocks, tokens_per_split, num_splits;
    int32_t num_workgroups;  // the grid size (read here rather than from the dispatch packet)
    int32_t stream_out;      // 1: the results are written with non-temporal stores
    float scale_log2;
};

// 16-byte LDS-DMA load: lane l's 16 bytes from `src` land at LDS byte
// lds_base + 16*l (lds_base is the same in every lane).  Issued from inline assembly so the compiler does not
// serialise the stage ring with conservative waits; the kernel waits on
// vmcnt itself.  M0 is written only here (the kernel has no other M0 use).
// NT: the load is marked non-temporal (streaming row gathers).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT = false>
__device__ __forceinline__ void lds_dma16(const void* src, unsigned lds_base) {
    if (NT)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src),
                     "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
                     "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory", "m0");
}
// 4-byte variant: lane l's 4 bytes land at lds_base + 4*l.
__device__ __forceinline__ void lds_dma4(const void* src, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Lane swaps between the halves of a wave (v_permlane32_swap: lanes 32..63
// of a with lanes 0..31 of b) and between odd and even rows of 16 lanes
// (v_permlane16_swap: rows 1, 3 of a with rows 0, 2 of b).  With a = b = x,
// max(a, b) or a + b afterwards reduces x over lanes l and l ^ 32 (l ^ 16).
// (The results are copied out of the returned pair before the bit cast: a
// bit cast of a vector element expression reads element 0.)
__device__ __forceinline__ void lane_swap32(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                    false, false);
    const unsigned r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void lane_swap16(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                    false, false);
    const unsigned r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// XOR swizzle of the eight 16-byte chunks of a band, by token (both cache
// formats).  Measured free of LDS bank conflicts on gfx950 for the three read
// shapes of the kernel: 16-byte QK reads of 16 consecutive tokens, 8-byte
// bf16 transpose reads of 4 tokens per 16-lane group, and 8-byte fp8
// transpose reads of tokens {4g..4g+3, 16+4g..16+4g+3} per 16-lane group g.
__device__ __forceinline__ int swz(int t) { return (t & 7) ^ ((t >> 4) & 1); }

// Swizzle of the four 16-byte chunks of a 64-byte half-band row (v4 rows):
// the 16-byte QK reads of 16 consecutive tokens then cover all banks.
__device__ __forceinline__ int swz4(int t) { return (t >> 2) & 3; }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T lds_load(const lds_u8* p) {
    return *(const __attribute__((address_space(3))) T*)p;
}

// Eight e4m3fn codes (two dwords) -> eight bf16 (exact).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(unsigned lo, unsigned hi) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// Eight e4m3fn codes times the power of two `scale` -> eight bf16 (exact
// while the products are normal bf16 numbers).
__device__ __forceinline__ bf16x8 e4m3x8_scaled_to_bf16(unsigned lo, unsigned hi, float scale) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// UE8M0 exponent byte `sel` (0..7) of an 8-byte scale record -> 2^(e-127)
// as fp32 (codes 1..254; code 0 gives +0).
__device__ __forceinline__ float ue8m0_scale(i32x2 rec, int sel) {
    const unsigned w = (unsigned)rec[sel >> 2];
    return __builtin_bit_cast(float, ((w >> (8 * (sel & 3))) & 0xffu) << 23);
}

template <int N>
__device__ __forceinline__ void wait_tiles(int after) {
    // wait until at most `after` tiles of N DMA instructions each are still in flight
    switch (after) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<N>(); break;
        case 2: wait_vmcnt<2 * N>(); break;
        case 3: wait_vmcnt<3 * N>(); break;
        default: wait_vmcnt<4 * N>(); break;
    }
}


// NTG: the row gathers are non-temporal loads.
template <int FMT, bool NTG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void partial_kernel(PartialArgs a_arg) {
    // Every argument is taken into scalar registers here, in one batch of
    // loads with one wait: left to itself, the compiler read the argument
    // block in pieces where each field was first used, each piece one more
    // dependent round trip before the first memory access of the list.
    PartialArgs a = a_arg;
    asm volatile("" : "+s"(a.q), "+s"(a.kv), "+s"(a.block_table), "+s"(a.indices), "+s"(a.seq_lens), "+s"(a.out),
                 "+s"(a.lse), "+s"(a.part_out), "+s"(a.part_lse), "+s"(a.num_kv_blocks), "+s"(a.rows),
                 "+s"(a.q_len), "+s"(a.topk), "+s"(a.max_blocks), "+s"(a.tokens_per_split), "+s"(a.num_splits),
                 "+s"(a.num_workgroups), "+s"(a.stream_out), "+s"(a.scale_log2));
    constexpr int STAGE = FMT == 0 ? kStageBytesBf16 : FMT == 1 ? kStageBytesFp8 : kStageBytesV4;
    constexpr int NST = FMT == 0 ? kStagesBf16 : FMT == 1 ? kStagesFp8 : kStagesV4;
    constexpr int ROWB = FMT == 0 ? kRowBytesBf16 : FMT == 1 ? kRowBytesFp8 : kRowBytesV4;
    constexpr int NBANDS = FMT == 0 ? kBandsBf16 : FMT == 1 ? kBandsFp8 : kBandsV4;
    constexpr int DQK = FMT == 2 ? kDqkV4 : kDqk;
    constexpr int PBUF = aux_p_buffer_bytes(FMT);
    constexpr int HALF_OFF = kBandsV4 * kTile * 128;  // v4: half band [token][64 B]
    constexpr int REC_OFF = HALF_OFF + kTile * 64;    // v4: scale records [token][8 B]
    static_assert(NST >= 2 && NST - 2 <= 4, "stage ring depth outside what the waits cover");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem_generic[];
    lds_u8* lds = (lds_u8*)smem_generic;
    const unsigned lds0 = (unsigned)(uintptr_t)lds;
    constexpr int AUX_ALPHA = aux_alpha_offset(FMT);
    constexpr int AUX_FLAG = aux_flag_offset(FMT);
    constexpr int AUX_DENOM = aux_denom_offset(FMT);
    constexpr int AUX_SWAP = aux_swap_offset(FMT);
    lds_u8* aux = lds + NST * STAGE;
    lds_u8* rowtab = aux + aux_bytes(FMT);  // int32 per token of this part: physical row or -1

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;    // 16-lane group
    const int i16 = lane & 15;  // lane within the group

    // (row, part) of this workgroup.  Consecutive workgroup ids are dispatched round-robin over the 8
    // XCDs, each with its own L2; the ids are renumbered so that the parts of a row, contiguous items,
    // share ids congruent mod 8 (one XCD), and the row's query block and block-table row come from HBM
    // once per XCD rather than once per part.  (A bijection of [0, grid); it only affects locality.)
    const int nwg = a.num_workgroups;
    const int xcd = blockIdx.x & 7, within = blockIdx.x >> 3;
    const int item = xcd * (nwg >> 3) + min(xcd, nwg & 7) + within;
    const int r = item / a.num_splits;
    const int sp = item - r * a.num_splits;
    const int b = r / a.q_len;
    const int k0 = sp * a.tokens_per_split;
    const int nk = max(0, min(a.tokens_per_split, a.topk - k0));
    const int ntiles = (nk + kTile - 1) / kTile;

    // ---- logical positions -> physical rows (masked entries -> -1), by the PV
    // waves (threads 256..511); the QK waves copy Q only once the copies below
    // have landed (T1): Q's first-touch loads issued next to them had held the
    // copies up by about half a microsecond.  The index list
    // goes into the row table, and (when the sequence's block-table row is
    // short) the block-table row into the still empty stage ring, by LDS-DMA:
    // every copy instruction is issued before the one wait, so the copy costs
    // one memory round trip, not one per 256 entries.  Each entry then costs
    // one LDS lookup.  Barriers T1 (copies done) and B0 (row table done) are
    // run by every wave.
    auto build_row_table = [&]() {
        const int pt = tid - 4 * 64;  // 0..255
        const int pw = pt >> 6;       // PV wave 0..3
        const int32_t* idx = a.indices + (int64_t)r * a.topk + k0;
        const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks;
        const int nent = ntiles * kTile;
        constexpr int kMaxBtInLds = 4096;
        static_assert(kMaxBtInLds * 4 <= NST * STAGE, "block-table copy exceeds the stage ring");
        const bool bt_in_lds = a.max_blocks <= kMaxBtInLds;
        // Whole 256-entry chunks of a 16-byte aligned row by 16-byte LDS-DMA (lane
        // l copies entries 4l .. 4l + 3), chunk c by PV wave c % 4; the rest in
        // 64-entry chunks, one entry per lane (lanes past the end copy nothing;
        // index-list entries past nk are -1).
        if (bt_in_lds) {
            const int full = ((uintptr_t)bt & 15) == 0 ? a.max_blocks / 256 : 0;
            for (int c = pw; c < full; c += 4) lds_dma16<false>(bt + 256 * c + 4 * lane, lds0 + 1024u * c);
            for (int c = pw; 256 * full + 64 * c < a.max_blocks; c += 4) {
                const int e = 256 * full + 64 * c + lane;
                if (e < a.max_blocks) lds_dma4(bt + e, lds0 + 4u * (256 * full + 64 * c));
            }
        }
        const unsigned rt0 = (unsigned)(uintptr_t)rowtab;
        const int full_i = ((uintptr_t)idx & 15) == 0 ? nk / 256 : 0;
        for (int c = pw; c < full_i; c += 4) lds_dma16<false>(idx + 256 * c + 4 * lane, rt0 + 1024u * c);
        for (int c = pw; 256 * full_i + 64 * c < nent; c += 4) {
            const int i = 256 * full_i + 64 * c + lane;
            if (i < nk)
                lds_dma4(idx + i, rt0 + 4u * (256 * full_i + 64 * c));
            else if (i < nent)
                *(__attribute__((address_space(3))) int*)(rowtab + 4 * i) = -1;
        }
        // (read after the copies are issued: the compiler waits for this load
        // where it is made, and it would otherwise delay them by a round trip)
        int64_t cap = (int64_t)kBlock * a.max_blocks;
        if (a.seq_lens) cap = min(cap, (int64_t)a.seq_lens[b]);
        wait_vmcnt<0>();
        __syncthreads();  // T1
        __attribute__((address_space(3))) int* const rt = (__attribute__((address_space(3))) int*)rowtab;
        if (bt_in_lds && nent > 256) {
            // 4 lookups in flight per lane, so a round of LDS reads costs one round
            // trip for up to 1024 entries (lanes past the end read entry i0 and
            // discard it)
            const __attribute__((address_space(3))) int* btl = (const __attribute__((address_space(3))) int*)lds;
            for (int i0 = pt; i0 < nent; i0 += 4 * 256) {
                int pos[4], blk[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + 256 * j;
                    pos[j] = rt[i < nent ? i : i0];
                    if (!(i < nent && pos[j] >= 0 && (int64_t)pos[j] < cap)) pos[j] = -1;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) blk[j] = btl[pos[j] >= 0 ? pos[j] / kBlock : 0];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + 256 * j;
                    if (i < nent)
                        rt[i] = pos[j] >= 0 && blk[j] >= 0 && (int64_t)blk[j] < a.num_kv_blocks
                                    ? blk[j] * kBlock + (pos[j] % kBlock)
                                    : -1;
                }
            }
        } else if (bt_in_lds) {
            const __attribute__((address_space(3))) int* btl = (const __attribute__((address_space(3))) int*)lds;
            for (int i = pt; i < nent; i += 256) {
                const int pos = rt[i];
                int row = -1;
                if (pos >= 0 && (int64_t)pos < cap) {
                    const int blk = btl[pos / kBlock];
                    if (blk >= 0 && (int64_t)blk < a.num_kv_blocks) row = blk * kBlock + (pos % kBlock);
                }
                rt[i] = row;
            }
        } else {
            // long block-table row: 8 lookups in flight per lane (an entry
            // out of range reads entry 0 and discards it)
            for (int i0 = pt; i0 < nent; i0 += 8 * 256) {
                int pos[8], blk[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = i0 + 256 * j;
                    pos[j] = i < nent ? rt[i] : -1;
                    if (!(pos[j] >= 0 && (int64_t)pos[j] < cap)) pos[j] = -1;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) blk[j] = bt[pos[j] >= 0 ? pos[j] / kBlock : 0];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = i0 + 256 * j;
                    if (i < nent)
                        rt[i] = pos[j] >= 0 && blk[j] >= 0 && (int64_t)blk[j] < a.num_kv_blocks
                                    ? blk[j] * kBlock + (pos[j] % kBlock)
                                    : -1;
                }
            }
        }
    };

    // ---- output staging: the normalised output, rounded to bf16, goes through
    // the (then idle) stage ring, so that every head's row is written to HBM
    // with contiguous 1 KB stores.  Rows are padded by 16 bytes: the staging
    // writes of a 16-lane group (16 heads, same dims) then fall on distinct
    // banks.  All 64 rows fit every layout's ring: the PV waves stage every
    // head, and after one barrier each wave stores 8 heads.
    constexpr int kRowPitch = 2 * kDv + 16;
    static_assert(64 * kRowPitch <= NST * STAGE, "staging area exceeds the stage ring");
    // Output rows of this workgroup: out[r] (one part) or part_out[sp][r].
    // Both pointers are taken into scalar registers before the choice.  Left
    // to itself, the compiler chose between the two argument fields' addresses
    // and read the chosen field with a vector load and a full wait, once per
    // head stored.
    // The same for the lse rows.
    uint64_t out_p = (uint64_t)(uintptr_t)a.out, part_p = (uint64_t)(uintptr_t)a.part_out;
    uint64_t lse_p = (uint64_t)(uintptr_t)a.lse, plse_p = (uint64_t)(uintptr_t)a.part_lse;
    asm volatile("" : "+s"(out_p), "+s"(part_p), "+s"(lse_p), "+s"(plse_p));
    typedef __attribute__((address_space(1))) uint16_t g_u16;
    typedef __attribute__((address_space(1))) float g_f32;
    const int64_t orow = a.num_splits == 1 ? (int64_t)r : (int64_t)sp * a.rows + r;
    g_u16* const obase = (g_u16*)(uintptr_t)(a.num_splits == 1 ? out_p : part_p) + orow * kHeads * kDv;
    g_f32* const lbase = (g_f32*)(uintptr_t)(a.num_splits == 1 ? lse_p : plse_p) + orow * kHeads;
    auto store_all = [&]() {
        // wave w stores heads 8w .. 8w + 7; lane l holds dims [8l, 8l + 8); all
        // eight LDS reads first
        i32x4 xs[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xs[j] = lds_load<i32x4>(lds + (8 * wave + j) * kRowPitch + 16 * lane);
        __builtin_amdgcn_sched_barrier(0);
        // (several parts: bf16 partials, rounded once more than the output; the
        // combine adds them in fp32)
        typedef __attribute__((address_space(1))) i32x4 g_i32x4;
        if (a.stream_out) {
            // (non-temporal stores written out: with the builtin, the compiler merged
            // the two branches' identical stores and dropped the hint)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                g_u16* o = obase + (8 * wave + j) * kDv + 8 * lane;
                asm volatile("global_store_dwordx4 %0, %1, off nt" ::"v"(o), "v"(xs[j]) : "memory");
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                g_u16* o = obase + (8 * wave + j) * kDv + 8 * lane;
                *(g_i32x4*)o = xs[j];
            }
        }
    };

    // ---- gather: the PV wave 4+o moves the tokens [8o, 8o + 8) of each tile,
    // all bands (and, for fp8 rows, the fp32 scales, lanes 0..7 fetching the
    // 16 bytes of their token), so it issues a fixed number of DMA
    // instructions per tile and counts them itself.  (The split between the
    // roles is a parameter: LPT_QK bands of each slice could go to the QK
    // waves instead; measured, that was not faster.)  A tile's DMAs are
    // prepared (row-table read, addresses) first and issued one at a time, so
    // they can be spread between MFMAs.
    //   v4 rows: 4 full bands, the half band (lanes 0..31: 8 tokens x 4
    //   chunks) and the scale records (lanes 0..15: 8 tokens x 2 dwords).
    constexpr int DMAS_PER_SLICE = FMT == 0 ? 9 : 6;
    constexpr int LPT_PV = DMAS_PER_SLICE;
    constexpr int LPT_QK = 0;
    const int oct = wave & 3;
    const int band0 = wave < 4 ? LPT_PV : 0;  // first band of this wave
    struct Gather {
        const unsigned char* src;   // this lane's 16 bytes of band 0 (or the zero chunk)
        const unsigned char* src2;  // fp8: this lane's scale bytes; v4: its half-band chunk
        const unsigned char* src3;  // v4: this lane's 4 bytes of a scale record
        int bstride;                // 128, or 0 for a masked token
        unsigned sbase;             // LDS byte address of the stage
    };
    // The cache pointer, held in scalar registers for the whole kernel (the
    // compiler otherwise reloaded it from the arguments after every step's
    // barrier, and the wait for that load also waited for the LDS reads).
    uint64_t kv_p = (uint64_t)(uintptr_t)a.kv;
    asm volatile("" : "+s"(kv_p));
    const uint8_t* const kvb = (const uint8_t*)(uintptr_t)kv_p;
    // start of the row of a physical token (v4: rows and scale records are
    // separate areas of a block)
    auto row_base = [&](int row) -> const unsigned char* {
        if (FMT == 2) return kvb + (int64_t)(row >> 6) * kBlockBytesV4 + (row & 63) * kRowBytesV4;
        return kvb + (int64_t)row * ROWB;
    };
    auto prepare = [&](int tile) {
        Gather gt;
        gt.sbase = lds0 + (unsigned)((tile % NST) * STAGE);
        const int t = 8 * oct + (lane >> 3);  // token of this lane within the tile
        const int row = *(const __attribute__((address_space(3))) int*)(rowtab + 4 * (tile * kTile + t));
        const int chunk = (lane & 7) ^ swz(t);
        gt.src = row >= 0 ? row_base(row) + chunk * 16 : kZeroChunk;
        gt.bstride = row >= 0 ? 128 : 0;
        gt.src2 = kZeroChunk;
        gt.src3 = kZeroChunk;
        if (FMT == 1) {
            const int t2 = 8 * oct + (lane & 7);
            const int row2 = *(const __attribute__((address_space(3))) int*)(rowtab + 4 * (tile * kTile + t2));
            gt.src2 = row2 >= 0 ? kvb + (int64_t)row2 * ROWB + NBANDS * 128 : kZeroChunk;
        }
        if (FMT == 2) {
            const int th = 8 * oct + ((lane >> 2) & 7);
            const int rowh = *(const __attribute__((address_space(3))) int*)(rowtab + 4 * (tile * kTile + th));
            gt.src2 = rowh >= 0 ? row_base(rowh) + 4 * 128 + (((lane & 3) ^ swz4(th)) << 4) : kZeroChunk;
            const int ts = 8 * oct + ((lane >> 1) & 7);
            const int rows = *(const __attribute__((address_space(3))) int*)(rowtab + 4 * (tile * kTile + ts));
            gt.src3 = rows >= 0 ? kvb + (int64_t)(rows >> 6) * kBlockBytesV4 + kBlock * kRowBytesV4 +
                                      (rows & 63) * kScaleRecBytesV4 + 4 * (lane & 1)
                                : kZeroChunk;
        }
        return gt;
    };
    auto issue_one = [&](const Gather& gt, int i) {  // DMA i of this wave's share of a tile
        const int bd = band0 + i;
        if (bd < NBANDS)
            lds_dma16<NTG>(gt.src + bd * gt.bstride, gt.sbase + (unsigned)((bd * kTile + 8 * oct) * 128));
        else if (FMT == 1) {
            if (lane < 8) lds_dma16<NTG>(gt.src2, gt.sbase + (unsigned)(NBANDS * kTile * 128 + 8 * oct * 16));
        } else if (bd == NBANDS) {
            if (lane < 32) lds_dma16<NTG>(gt.src2, gt.sbase + (unsigned)(HALF_OFF + 8 * oct * 64));
        } else {
            if (lane < 16) lds_dma4(gt.src3, gt.sbase + (unsigned)(REC_OFF + 8 * oct * kScaleRecBytesV4));
        }
    };
    static_assert(LPT_PV + LPT_QK == DMAS_PER_SLICE, "the two roles cover every DMA of a slice");

    // Every wave runs the same sequence of workgroup barriers: T1 and B0 (row
    // table ready), P0 (tile 0 in LDS), E_k at the end of each step k in
    // [0, ntiles] (the QK waves publish the denominators in the last one),
    // then one for the staged output.  In
    // step k the QK waves turn tile k into softmax weights P(k); the PV waves
    // add tile k-1 to the output with P(k-1) (from V held in registers) while
    // refilling the stage of tile k-1 with tile k + NST - 1, copy their V slice
    // of tile k into registers and wait for tile k+1 to land.  NST - 2 tiles
    // beyond the next one are in flight while a tile is computed.
    // ---- query staging: a QK wave's 16 query rows (HB bytes each, contiguous in
    // HBM) are copied into LDS by LDS-DMA, 1 KB per instruction, with the 16-byte
    // chunks of each row XOR-swizzled so that the operand reads (16 rows, the
    // same chunk) fall on distinct banks: bf16 rows (1152 bytes) keep groups of 8
    // chunks and swizzle by row / 2 (odd rows start 128 bytes further into the
    // banks), v4 rows (1024 bytes) swizzle groups of 16 chunks by row.
    constexpr int HB = DQK * 2;
    auto q_swz = [](int h, int c) {
        return FMT == 2 ? (c & ~15) | ((c ^ h) & 15) : (c & ~7) | ((c ^ (h >> 1)) & 7);
    };
    // copy 16 rows starting at row `row0` of this workgroup's query into LDS at `dst`
    auto q_copy = [&](int row0, unsigned dst) {
        const unsigned char* qsrc = (const unsigned char*)(a.q + ((int64_t)r * kHeads + row0) * DQK);
#pragma unroll
        for (int j = 0; j < 16 * HB / 1024; ++j) {
            const int o = j * 1024 + 16 * lane;
            const int h = o / HB;
            lds_dma16<false>(qsrc + h * HB + 16 * q_swz(h, (o - h * HB) / 16), dst + j * 1024);
        }
    };
    // operand of row i16, dims d .. d + 7, from a staged block at `src`
    auto q_read = [&](const lds_u8* src, int d) { return lds_load<bf16x8>(src + i16 * HB + 16 * q_swz(i16, d / 8)); };
    if (wave < 4) {
        if constexpr (FMT == 1) {
            // ====== QK waves: wave 2c + h, heads [32c, 32c + 32), tokens [16h, 16h + 16) of each tile ======
            // The two waves of pair c own the same 32 heads (16-head blocks 2c and
            // 2c + 1) and split each tile's tokens between them: every K operand
            // read from LDS then feeds two MFMAs, one per head block, and every
            // fp8 code is widened by two waves rather than four.  The pair agrees
            // on the reference maximum of each head by swapping per-head values
            // through LDS once a step (`swap_post`, `swap_wait`).  Head block A of
            // wave 2c + h is block 2c + h, its block B the partner's block A.
            const int hp = wave >> 1;    // head pair
            const int half = wave & 1;   // token half
            const int headA = 16 * (2 * hp + half) + i16, headB = 16 * (2 * hp + 1 - half) + i16;
            // Q of headA / headB as the B operand of S^T = K . Q^T (8 dims of
            // k-step kk per lane); for fp8 rows the c_kv dims of k-steps 2p and
            // 2p+1 inside a 128-group are the two halves of one 16-byte run, so
            // one LDS read feeds two k-steps.
            // Each wave loads block A from HBM between T1 and B0 (see the row
            // table), as every QK wave loads one block, and hands it to its
            // partner through the stages of tiles 2 .. (and the P buffers), which
            // are empty until P0: loading both blocks from HBM made the first-touch
            // loads of the second block (whose address translations miss) hold up
            // the first tiles' gathers.  (Staging the block by LDS-DMA, as the other
            // layouts do, measured 0.3-0.8 us slower here.)
            constexpr int NQ = 18;
            bf16x8 qa[NQ], qb[NQ];
            // this wave's slot in the swap area: 16-byte records {headA, headB, seq, seq}
            // per head of a block (read by the partner only after T1)
            typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
            volatile lds_f32x4* const swap_mine = (volatile lds_f32x4*)(aux + AUX_SWAP) + 16 * wave + i16;
            const volatile lds_f32x4* const swap_part = (const volatile lds_f32x4*)(aux + AUX_SWAP) + 16 * (wave ^ 1) + i16;
            if (g == 0) *swap_mine = f32x4{0.f, 0.f, 0.f, 0.f};
            // Per-head swap with the partner wave: this lane's values for headA and
            // headB go out (lanes of group 0) in one 16-byte record tagged with the
            // step count `seq` (written by one instruction, so a record whose tags
            // read `seq` holds this step's values), and the partner's record is
            // read until it carries `seq`.  The partner posts its record in the
            // same step without waiting on this wave, so the wait ends.  One record
            // suffices: the next one is written after the step's barrier, which the
            // partner passes only after reading this one.
            // (vector elements are copied to scalars before any bit cast: a bit
            // cast of an element expression read element 0)
            auto swap_post = [&](float va, float vb, int seq) {
                const float tag = __builtin_bit_cast(float, seq);
                if (g == 0) *swap_mine = f32x4{va, vb, tag, tag};
            };
            auto swap_wait = [&](int seq, float& pa, float& pb) {
                f32x4 o = *swap_part;
                while (true) {
                    const float t0 = o[2], t1 = o[3];
                    if (__all(__builtin_bit_cast(int, t0) == seq && __builtin_bit_cast(int, t1) == seq)) break;
                    __builtin_amdgcn_s_sleep(1);
                    o = *swap_part;
                }
                pa = o[1];  // the partner's block B is this wave's block A
                pb = o[0];
            };
            // sum or maximum over the four lanes of a head (lane groups g), by lane swaps
            auto head_max = [](float x) {
                float u = x, v = x;
                lane_swap32(u, v);
                x = fmaxf(u, v);
                u = x;
                v = x;
                lane_swap16(u, v);
                return fmaxf(u, v);
            };
            auto head_sum = [](float x) {
                float u = x, v = x;
                lane_swap32(u, v);
                x = u + v;
                u = x;
                v = x;
                lane_swap16(u, v);
                return u + v;
            };
            static_assert(2 * STAGE + 4 * NQ * 1024 <= NST * STAGE + 2 * PBUF && NST >= 3,
                          "the query hand-over area exceeds the stages of tiles 2.. and the P buffers");
            __syncthreads();  // T1
            {
                const uint16_t* const qh = a.q + ((int64_t)r * kHeads + headA) * DQK;
#pragma unroll
                for (int kk = 0; kk < NQ; ++kk) {
                    const int d = kk >= 16 ? 32 * kk + 8 * g : 128 * (kk >> 2) + 64 * ((kk >> 1) & 1) + 16 * g + 8 * (kk & 1);
                    qa[kk] = *(const bf16x8*)(qh + d);
                }
            }
            __syncthreads();  // B0
            wait_vmcnt<0>();
            {
                // ---- the query hand-over: this wave's block A is the partner's block
                // B.  (The hand-over and the swaps share the records: tag 1 here,
                // k + 2 for the maxima of tile k, ntiles + 2 for the denominators.)
                typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
                lds_bf16x8* const xq = (lds_bf16x8*)(lds + 2 * STAGE) + lane;
#pragma unroll
                for (int kk = 0; kk < NQ; ++kk) xq[(wave * NQ + kk) * 64] = qa[kk];
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // block A is in LDS before its tag
                float d0, d1;
                swap_post(0.f, 0.f, 1);
                swap_wait(1, d0, d1);
#pragma unroll
                for (int kk = 0; kk < NQ; ++kk) qb[kk] = xq[((wave ^ 1) * NQ + kk) * 64];
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before P0 (tile 2 is gathered there after it)
            }
#pragma unroll
            for (int kk = 0; kk < NQ; ++kk) asm volatile("" : "+v"(qa[kk]), "+v"(qb[kk]));  // no waits in the loop

            // K operand row of this lane: token tokA.  Accumulator entry e of a
            // lane: token tokC + e (the partner's: tokO + e).
            const int tokA = 16 * half + i16;
            const int tokC = 16 * half + 4 * g, tokO = 16 * (1 - half) + 4 * g;
            int qk[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) qk[e] = tokA * 128 + (((4 * e + g) ^ swz(tokA)) << 4);
            // P slots of this lane for headA (+ pb_off: headB): (block, group g, lane i16) holds the
            // k-slots 8g .. 8g + 7 of the PV B operand, i.e. tokens 4g .. 4g + 3 (bytes 0..7) and
            // 16 + 4g .. 16 + 4g + 3 (bytes 8..15); this wave writes its half.
            lds_u8* const p_mine = aux + ((((2 * hp + half) * 4 + g) * 16 + i16) * 16) + 8 * half;  // + buffer (+ group copy)
            const int pb_off = half ? -1024 : 1024;

            // Online softmax of headA and headB, base 2.  Weights are taken against
            // a reference maximum m_ref, set at the first tile with a valid token;
            // it is raised only when a tile's maximum exceeds it by more than
            // kMaxRise (weights up to 2^kMaxRise stay finite in fp32 and bf16), and
            // then the denominator here and the output accumulators of the PV waves
            // are rescaled by alpha = 2^(old - new).  Both waves of the pair take
            // the same decisions from the same maxima.
            constexpr float kMaxRise = 32.f;
            float mrA = -INFINITY, mrB = -INFINITY;  // the same in the four lanes of a head and in both waves
            float lA = 0.f, lB = 0.f;                // this lane's share of the denominators
            bool ref_set = false;                    // the same in every lane of both waves
            const int pro = min(NST - 1, ntiles);  // tiles issued before the loop
            if (LPT_QK > 0) {
                for (int t = 0; t < pro; ++t) {
                    const Gather gt = prepare(t);
#pragma unroll
                    for (int i = 0; i < LPT_QK; ++i) issue_one(gt, i);
                }
                if (ntiles > 0) wait_tiles<LPT_QK>(pro - 1);  // this wave's part of tile 0 has landed
            }
            __syncthreads();  // P0
            for (int k = 0; k <= ntiles; ++k) {
                int raised = 0;
                // tile k + NST - 1 goes into the stage of tile k - 1 (free since E_{k-1})
                if (LPT_QK > 0 && k + NST - 1 < ntiles) {
                    const Gather gt = prepare(k + NST - 1);
#pragma unroll
                    for (int i = 0; i < LPT_QK; ++i) issue_one(gt, i);
                }
                if (k < ntiles) {
                    const lds_u8* st = lds + (k % NST) * STAGE;
                    const lds_u8* rt = rowtab + 4 * k * kTile;
                    const i32x4 vc = lds_load<i32x4>(rt + 4 * tokC);  // row entries of this lane's tokens
                    const i32x4 vo = lds_load<i32x4>(rt + 4 * tokO);  // and of the partner's

                    // ---- S^T = K . Q^T for this half's 16 tokens and the two head blocks
                    f32x4 sA = f32x4{0.f, 0.f, 0.f, 0.f}, sB = sA;
                    f32x4 sc[4];  // fp8: sc[e][grp] = scale of group grp of accumulator token tokC + e
                    {
                    // 10 load units: rope k-steps 16, 17 (bf16), then c_kv pairs (group, pair)
                    constexpr int PF = 4;
                    u32x4 kr[PF];
                    auto unit_off = [&](int u) {
                        return u < 2 ? qk[u] + 4 * kTile * 128 : qk[(u - 2) & 1] + ((u - 2) >> 1) * kTile * 128;
                    };
                    const lds_u8* scl = st + NBANDS * kTile * 128;
#pragma unroll
                    for (int u = 0; u < PF; ++u) kr[u] = lds_load<u32x4>(st + unit_off(u));
#pragma unroll
                    for (int e = 0; e < 4; ++e) sc[e] = lds_load<f32x4>(scl + 16 * (tokC + e));
                    f32x4 pA = sA, pB = sA;
#pragma unroll
                    for (int u = 0; u < 10; ++u) {
                        const int sl = u % PF;
                        if (u < 2) {
                            const bf16x8 w = __builtin_bit_cast(bf16x8, kr[sl]);
                            sA = mfma16(w, qa[16 + u], sA);
                            sB = mfma16(w, qb[16 + u], sB);
                        } else {
                            const int grp = (u - 2) >> 1, pq = (u - 2) & 1;
                            if (pq == 0) { pA = f32x4{0.f, 0.f, 0.f, 0.f}; pB = pA; }
                            const bf16x8 w0 = e4m3x8_to_bf16(kr[sl][0], kr[sl][1]);
                            const bf16x8 w1 = e4m3x8_to_bf16(kr[sl][2], kr[sl][3]);
                            pA = mfma16(w0, qa[4 * grp + 2 * pq], pA);
                            pB = mfma16(w0, qb[4 * grp + 2 * pq], pB);
                            pA = mfma16(w1, qa[4 * grp + 2 * pq + 1], pA);
                            pB = mfma16(w1, qb[4 * grp + 2 * pq + 1], pB);
                            if (pq == 1) {
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    sA[e] += sc[e][grp] * pA[e];
                                    sB[e] += sc[e][grp] * pB[e];
                                }
                            }
                        }
                        if (u + PF < 10) kr[sl] = lds_load<u32x4>(st + unit_off(u + PF));
                    }
                    __builtin_amdgcn_sched_group_barrier(0x100, PF + 4, 0);
#pragma unroll
                    for (int u = 0; u < 10 - PF; ++u) {
                        if (u < 2)
                            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                        else
                            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 4 * PF, 0);
                    }

                    // ---- mask, reference, softmax weights (base 2)
                    float sv[8];  // [0..3]: headA, tokens tokC + e; [4..7]: headB
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sv[e] = vc[e] >= 0 ? sA[e] * a.scale_log2 : -INFINITY;
                        sv[4 + e] = vc[e] >= 0 ? sB[e] * a.scale_log2 : -INFINITY;
                    }
                    float mA = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
                    float mB = fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7]));
                    mA = head_max(mA);
                    mB = head_max(mB);
                    swap_post(mA, mB, k + 2);
                    // The weights against the references, and their P copies.  The
                    // denominator sums the fp32 weights; the PV product takes them
                    // rounded to bf16 once (for fp8 rows after multiplying by the
                    // token's scale of each 128-group, one copy per group).
                    float psA = 0.f, psB = 0.f;
                    lds_u8* const pbuf = p_mine + (k & 1) * PBUF;  // headA; headB at + pb_off
                    auto weights = [&](float muA, float muB) {
                        float pf[8];
                        psA = 0.f;
                        psB = 0.f;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            pf[e] = __builtin_amdgcn_exp2f(sv[e] - muA);
                            pf[4 + e] = __builtin_amdgcn_exp2f(sv[4 + e] - muB);
                            psA += pf[e];
                            psB += pf[4 + e];
                        }
                        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
#pragma unroll
                            for (int grp = 0; grp < 4; ++grp) {
                                bf16x4 wa, wb;
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    wa[e] = (__bf16)(pf[e] * sc[e][grp]);
                                    wb[e] = (__bf16)(pf[4 + e] * sc[e][grp]);
                                }
                                *(lds_bf16x4*)(pbuf + grp * kPBytesPerCopy) = wa;
                                *(lds_bf16x4*)(pbuf + grp * kPBytesPerCopy + pb_off) = wb;
                            }
                    };
                    // Once the references are set, the weights are taken against them
                    // while the partner's maxima are on their way; they are redone in
                    // the rare step that raises a reference (the PV waves read P only
                    // after the step's barrier).  Until then, the first tile with a
                    // valid token sets the references from both halves' maxima.
                    if (ref_set) weights(mrA, mrB);
                    {
                        float oA, oB;
                        swap_wait(k + 2, oA, oB);
                        mA = fmaxf(mA, oA);  // the tile's maximum of headA over both halves
                        mB = fmaxf(mB, oB);
                    }
                    bool redo = false;
                    if (!ref_set) {
                        // first tile with a valid token (the same tile for every head and wave)
                        const bool any_valid = vc[0] >= 0 || vc[1] >= 0 || vc[2] >= 0 || vc[3] >= 0 || vo[0] >= 0 ||
                                               vo[1] >= 0 || vo[2] >= 0 || vo[3] >= 0;
                        if (__any(any_valid)) {
                            mrA = mA;
                            mrB = mB;
                            ref_set = true;
                        }
                        redo = true;
                    } else if (__any(mA > mrA + kMaxRise || mB > mrB + kMaxRise)) {  // rare: raise the references
                        const bool upA = mA > mrA + kMaxRise, upB = mB > mrB + kMaxRise;
                        const float alA = upA ? __builtin_amdgcn_exp2f(mrA - mA) : 1.f;
                        const float alB = upB ? __builtin_amdgcn_exp2f(mrB - mB) : 1.f;
                        mrA = upA ? mA : mrA;
                        mrB = upB ? mB : mrB;
                        lA *= alA;
                        lB *= alB;
                        if (half == 0 && g == 0) {
                            __attribute__((address_space(3))) float* al =
                                (__attribute__((address_space(3))) float*)(aux + AUX_ALPHA + (k & 1) * (kHeads * 4));
                            al[headA] = alA;
                            al[headB] = alB;
                        }
                        raised = 1;
                        redo = true;
                    }
                    if (redo) weights(ref_set ? mrA : 0.f, ref_set ? mrB : 0.f);
                    lA += psA;
                    lB += psB;
                }
                if (half == 0 && lane == 0)
                    *(__attribute__((address_space(3))) i32x2*)(aux + AUX_FLAG + 16 * (k & 1) + 8 * hp) = i32x2{raised, raised};
                if (k == ntiles) {
                    // ---- denominators and lse of headA and headB: final since step
                    // ntiles - 1, published in the last step (the PV waves still add
                    // the last tile), so the barrier that ends it makes them visible
                    float tA = head_sum(lA), tB = head_sum(lB);
                    float oA, oB;
                    swap_post(tA, tB, ntiles + 2);
                    swap_wait(ntiles + 2, oA, oB);
                    if (half == 0 && g == 0) {
                        tA += oA;
                        tB += oB;
                        __attribute__((address_space(3))) float* dn = (__attribute__((address_space(3))) float*)(aux + AUX_DENOM);
                        dn[headA] = ref_set ? tA : 0.f;
                        dn[headB] = ref_set ? tB : 0.f;
                        lbase[headA] = ref_set ? (mrA + log2f(tA)) * kLn2 : -INFINITY;
                        lbase[headB] = ref_set ? (mrB + log2f(tB)) * kLn2 : -INFINITY;
                    }
                }
                if (LPT_QK > 0 && k + 1 < ntiles) wait_tiles<LPT_QK>(min(NST - 2, ntiles - 2 - k));  // its part of tile k+1 has landed
                __syncthreads();  // E_k
            }

            __syncthreads();  // the PV waves have staged every head
            store_all();
        } else {
            // =================== QK waves: heads [16q, 16q + 16) ===================
            const int q = wave;
            const int head = 16 * q + i16;
            // Q of `head` as the B operand of S^T = K . Q^T (8 dims of k-step kk per
            // lane).  (v4 rows: the 16-byte run of nope group u feeds k-steps 2u
            // and 2u+1; k-steps 14 and 15 are the rope values.)
            constexpr int NQ = FMT == 2 ? 16 : 18;
            bf16x8 qreg[NQ];
            // The wave's 16 query rows are staged in LDS (`q_copy`) between T1 and
            // B0 (see the row table) and read from there in operand order after B0.
            // They go to the stages of tiles 2 .. (and the P buffers), which are
            // empty until P0.  (Loading the operands directly, 16 rows 1152 bytes
            // apart in every instruction, took about a microsecond to issue and held
            // B0 up.)
            static_assert(2 * STAGE + 4 * NQ * 1024 <= NST * STAGE + 2 * PBUF && NST >= 3,
                          "the query staging area exceeds the stages of tiles 2.. and the P buffers");
            __syncthreads();  // T1
            q_copy(16 * q, lds0 + (unsigned)(2 * STAGE + q * NQ * 1024));
            __syncthreads();  // B0
            wait_vmcnt<0>();
            {
                const lds_u8* xq = lds + 2 * STAGE + q * NQ * 1024;
#pragma unroll
                for (int kk = 0; kk < NQ; ++kk) {
                    const int d = FMT == 0  ? 32 * kk + 8 * g
                                  : kk < 14 ? 64 * (kk >> 1) + 16 * g + 8 * (kk & 1)
                                            : kNopeV4 + 32 * (kk - 14) + 8 * g;
                    qreg[kk] = q_read(xq, d);
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before P0 (tile 2 is gathered there after it)
            }
#pragma unroll
            for (int kk = 0; kk < NQ; ++kk) asm volatile("" : "+v"(qreg[kk]));  // loads done; no waits in the loop

            // K operand rows of the two 16-token blocks: tokens i16 and 16 + i16.
            // Accumulator entry e of a lane: tokens 4g + e (block 0), 16 + 4g + e (block 1).
            const int tokA0 = i16, tokA1 = 16 + i16;
            const int tokC0 = 4 * g, tokC1 = 16 + 4 * g;
            int qk0[2], qk1[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                qk0[e] = tokA0 * 128 + (((4 * e + g) ^ swz(tokA0)) << 4);
                qk1[e] = tokA1 * 128 + (((4 * e + g) ^ swz(tokA1)) << 4);
            }
            // v4: this lane's chunk of the half band (rope values 32 + 8g .. 32 + 8g + 7)
            const int qh0 = HALF_OFF + tokA0 * 64 + ((g ^ swz4(tokA0)) << 4);
            const int qh1 = HALF_OFF + tokA1 * 64 + ((g ^ swz4(tokA1)) << 4);
            // P slot of this lane: (block q, group g, lane i16): its 8 weights are
            // the k-slots 8g .. 8g + 7 of the PV B operand, i.e. tokens
            // 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3.
            lds_u8* const p_mine = aux + ((q * 4 + g) * 16 + i16) * 16;  // + buffer (+ group copy for fp8)

            // Online softmax of `head`, base 2.  Weights are taken against a
            // reference maximum m_ref, set at the first tile with a valid token;
            // it is raised only when a tile's maximum exceeds it by more than
            // kMaxRise (weights up to 2^kMaxRise stay finite in fp32 and bf16), and
            // then the denominator here and the output accumulators of the PV waves
            // are rescaled by alpha = 2^(old - new).
            constexpr float kMaxRise = 32.f;
            float m_ref = -INFINITY;  // the same in the four lanes of the head
            float l_run = 0.f;        // this lane's share of the denominator
            bool ref_set = false;     // the same in every lane of the wave
            const int pro = min(NST - 1, ntiles);  // tiles issued before the loop
            if (LPT_QK > 0) {
                for (int t = 0; t < pro; ++t) {
                    const Gather gt = prepare(t);
#pragma unroll
                    for (int i = 0; i < LPT_QK; ++i) issue_one(gt, i);
                }
                if (ntiles > 0) wait_tiles<LPT_QK>(pro - 1);  // this wave's part of tile 0 has landed
            }
            __syncthreads();  // P0
            for (int k = 0; k <= ntiles; ++k) {
                int raised = 0;
                // tile k + NST - 1 goes into the stage of tile k - 1 (free since E_{k-1})
                if (LPT_QK > 0 && k + NST - 1 < ntiles) {
                    const Gather gt = prepare(k + NST - 1);
#pragma unroll
                    for (int i = 0; i < LPT_QK; ++i) issue_one(gt, i);
                }
                if (k < ntiles) {
                    const lds_u8* st = lds + (k % NST) * STAGE;
                    const lds_u8* rt = rowtab + 4 * k * kTile;
                    const i32x4 v0 = lds_load<i32x4>(rt + 4 * tokC0);
                    const i32x4 v1 = lds_load<i32x4>(rt + 4 * tokC1);

                    // ---- S^T = K . Q^T for the tile's 32 tokens, in two 16-token blocks
                    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
                    if (FMT == 0) {
                        constexpr int PF = 4;  // k-steps of K operands in flight
                        bf16x8 ka[PF], kb[PF];
#pragma unroll
                        for (int kk = 0; kk < PF; ++kk) {
                            ka[kk] = lds_load<bf16x8>(st + qk0[kk & 1] + (kk >> 1) * kTile * 128);
                            kb[kk] = lds_load<bf16x8>(st + qk1[kk & 1] + (kk >> 1) * kTile * 128);
                        }
#pragma unroll
                        for (int kk = 0; kk < 18; ++kk) {
                            const int sl = kk % PF;
                            s0 = mfma16(ka[sl], qreg[kk], s0);
                            s1 = mfma16(kb[sl], qreg[kk], s1);
                            if (kk + PF < 18) {
                                const int kn = kk + PF;
                                ka[sl] = lds_load<bf16x8>(st + qk0[kn & 1] + (kn >> 1) * kTile * 128);
                                kb[sl] = lds_load<bf16x8>(st + qk1[kn & 1] + (kn >> 1) * kTile * 128);
                            }
                        }
                        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
                        for (int i = 0; i < 18 - PF; ++i) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                        }
                        __builtin_amdgcn_sched_group_barrier(0x008, 2 * PF, 0);
                    } else {
                        // 9 load units per block: nope groups 0..6 (16 e4m3 values of this
                        // lane's token, two k-steps, widened with the token's scale of
                        // that group), then rope values 0..31 and 32..63 (bf16)
                        constexpr int PF = 3;
                        u32x4 ka[PF], kb[PF];
                        auto unit_off = [&](int u, int blk) {
                            const int* qo = blk == 0 ? qk0 : qk1;
                            return u < 8 ? qo[u & 1] + (u >> 1) * kTile * 128 : (blk == 0 ? qh0 : qh1);
                        };
#pragma unroll
                        for (int u = 0; u < PF; ++u) {
                            ka[u] = lds_load<u32x4>(st + unit_off(u, 0));
                            kb[u] = lds_load<u32x4>(st + unit_off(u, 1));
                        }
                        const i32x2 ra = lds_load<i32x2>(st + REC_OFF + kScaleRecBytesV4 * tokA0);
                        const i32x2 rb = lds_load<i32x2>(st + REC_OFF + kScaleRecBytesV4 * tokA1);
#pragma unroll
                        for (int u = 0; u < 9; ++u) {
                            const int sl = u % PF;
                            if (u < 7) {
                                const float fa = ue8m0_scale(ra, u), fb = ue8m0_scale(rb, u);
                                s0 = mfma16(e4m3x8_scaled_to_bf16(ka[sl][0], ka[sl][1], fa), qreg[2 * u], s0);
                                s1 = mfma16(e4m3x8_scaled_to_bf16(kb[sl][0], kb[sl][1], fb), qreg[2 * u], s1);
                                s0 = mfma16(e4m3x8_scaled_to_bf16(ka[sl][2], ka[sl][3], fa), qreg[2 * u + 1], s0);
                                s1 = mfma16(e4m3x8_scaled_to_bf16(kb[sl][2], kb[sl][3], fb), qreg[2 * u + 1], s1);
                            } else {
                                s0 = mfma16(__builtin_bit_cast(bf16x8, ka[sl]), qreg[7 + u], s0);
                                s1 = mfma16(__builtin_bit_cast(bf16x8, kb[sl]), qreg[7 + u], s1);
                            }
                            if (u + PF < 9) {
                                ka[sl] = lds_load<u32x4>(st + unit_off(u + PF, 0));
                                kb[sl] = lds_load<u32x4>(st + unit_off(u + PF, 1));
                            }
                        }
                    }

                    // ---- mask, reference, softmax weights (base 2)
                    float sv[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sv[e] = v0[e] >= 0 ? s0[e] * a.scale_log2 : -INFINITY;
                        sv[4 + e] = v1[e] >= 0 ? s1[e] * a.scale_log2 : -INFINITY;
                    }
                    float mx = sv[0];
#pragma unroll
                    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
                    if (!ref_set) {
                        // first tile with a valid token (the same tile for every head and wave)
                        const bool any_valid = v0[0] >= 0 || v0[1] >= 0 || v0[2] >= 0 || v0[3] >= 0 || v1[0] >= 0 ||
                                               v1[1] >= 0 || v1[2] >= 0 || v1[3] >= 0;
                        if (__any(any_valid)) {
                            mx = fmaxf(mx, __shfl_xor(mx, 16));
                            mx = fmaxf(mx, __shfl_xor(mx, 32));
                            m_ref = mx;
                            ref_set = true;
                        }
                    } else if (__any(mx > m_ref + kMaxRise)) {  // rare: raise the references of this wave's heads
                        mx = fmaxf(mx, __shfl_xor(mx, 16));
                        mx = fmaxf(mx, __shfl_xor(mx, 32));
                        const bool up = mx > m_ref + kMaxRise;
                        const float alpha = up ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.f;
                        m_ref = up ? mx : m_ref;
                        l_run *= alpha;
                        if (g == 0) *(__attribute__((address_space(3))) float*)(aux + AUX_ALPHA + (k & 1) * (kHeads * 4) + 4 * head) = alpha;
                        raised = 1;
                    }
                    const float m_use = ref_set ? m_ref : 0.f;
                    // The denominator sums the fp32 weights; the PV product takes them
                    // rounded to bf16 once (for v4 rows after multiplying by the
                    // token's scale of each 64-group, one copy per group).
                    float pf[8];
                    float psum = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        pf[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
                        psum += pf[e];
                    }
                    l_run += psum;
                    lds_u8* const pbuf = p_mine + (k & 1) * PBUF;
                    if (FMT == 0) {
                        bf16x8 pb;
#pragma unroll
                        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)pf[e];
                        *(__attribute__((address_space(3))) bf16x8*)pbuf = pb;
                    } else {
                        // copies 0..6: the weights times each token's scale of nope group c;
                        // copy 7 (rope values): the weights
                        const lds_u8* rec = lds + (k % NST) * STAGE + REC_OFF;
                        const i32x4 c0a = lds_load<i32x4>(rec + kScaleRecBytesV4 * tokC0);
                        const i32x4 c0b = lds_load<i32x4>(rec + kScaleRecBytesV4 * tokC0 + 16);
                        const i32x4 c1a = lds_load<i32x4>(rec + kScaleRecBytesV4 * tokC1);
                        const i32x4 c1b = lds_load<i32x4>(rec + kScaleRecBytesV4 * tokC1 + 16);
                        const i32x2 rc[8] = {i32x2{c0a[0], c0a[1]}, i32x2{c0a[2], c0a[3]}, i32x2{c0b[0], c0b[1]},
                                             i32x2{c0b[2], c0b[3]}, i32x2{c1a[0], c1a[1]}, i32x2{c1a[2], c1a[3]},
                                             i32x2{c1b[0], c1b[1]}, i32x2{c1b[2], c1b[3]}};
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            bf16x8 pg;
#pragma unroll
                            for (int e = 0; e < 8; ++e) pg[e] = (__bf16)(c < 7 ? pf[e] * ue8m0_scale(rc[e], c) : pf[e]);
                            *(__attribute__((address_space(3))) bf16x8*)(pbuf + c * kPBytesPerCopy) = pg;
                        }
                    }
                }
                if (lane == 0) *(__attribute__((address_space(3))) int*)(aux + AUX_FLAG + 16 * (k & 1) + 4 * q) = raised;
                if (k == ntiles) {
                    // ---- denominator and lse of `head`: final since step ntiles - 1,
                    // published in the last step (the PV waves still add the last
                    // tile), so the barrier that ends it makes them visible
                    float l_tot = l_run;
                    l_tot += __shfl_xor(l_tot, 16);
                    l_tot += __shfl_xor(l_tot, 32);
                    if (g == 0) {
                        *(__attribute__((address_space(3))) float*)(aux + AUX_DENOM + 4 * head) = ref_set ? l_tot : 0.f;
                        const float lse_v = ref_set ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
                        lbase[head] = lse_v;
                    }
                }
                if (LPT_QK > 0 && k + 1 < ntiles) wait_tiles<LPT_QK>(min(NST - 2, ntiles - 2 - k));  // its part of tile k+1 has landed
                __syncthreads();  // E_k
            }

            __syncthreads();  // the PV waves have staged every head
            store_all();
        }
    } else {
        // ========= PV waves: value dims [128p, 128p + 128), all heads =========
        const int p = wave - 4;
        build_row_table();
        __syncthreads();  // B0

        // V^T operand offsets: the k-slots 8g .. 8g + 7 of a lane are the tokens
        // 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3 (the P operand order).
        //   bf16: bands 2p, 2p + 1; lane i16 addresses token tok + (i16 >> 2), 4 dims
        //         at 4(i16 & 3) of 16-dim block m; the transpose read hands lane i dim i.
        //   fp8 : band p (the scale group), 16-dim block c; lane i16 addresses token
        //         slot j = i16 >> 1, 8 dims at 8(i16 & 1).
        //   v4  : as fp8 (band p = nope groups 2p, 2p+1); wave 7 (p = 3) has nope
        //         group 6 in blocks 0..3 and the bf16 rope values in blocks 4..7
        //         (band 3 bytes 64..127, then the half band), read as for bf16.
        int pv[8];
        if (FMT == 0) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int ta = 16 * blk + 4 * g + (i16 >> 2);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    pv[4 * blk + m] = (2 * p * kTile + ta) * 128 + (((2 * m + ((i16 & 3) >> 1)) ^ swz(ta)) << 4) +
                                      8 * (i16 & 1);
            }
        } else {
            const int j = i16 >> 1;
            const int ta = j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
#pragma unroll
            for (int c = 0; c < 8; ++c) pv[c] = (p * kTile + ta) * 128 + ((c ^ swz(ta)) << 4) + 8 * (i16 & 1);
        }
        // P copies of this wave: fp8 rows copy p; v4 rows copies 2p (blocks 0..3) and 2p+1 (blocks 4..7)
        const lds_u8* const p_read = aux + (FMT == 0 ? 0 : FMT == 1 ? p : 2 * p) * kPBytesPerCopy + lane * 16;
        const bool rope_wave = FMT == 2 && p == 3;  // v4: blocks 4..7 are bf16 rope values

        f32x4 oacc[8][4];  // O^T [16-dim block of this wave's 128 dims][16-head block]
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                oacc[i][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
                asm volatile("" : "+v"(oacc[i][hb]));
            }
        // This wave's V^T slice of a tile is copied from LDS into registers in
        // the step that gathers the tile, so the stage is free again at the end
        // of that step although the product runs one step later.  Two register
        // buffers alternate: a step first copies tile k (the QK waves' MFMAs
        // run meanwhile), then multiplies tile k-1 (overlapping the QK waves'
        // softmax).  v4 rows hold twice the P operands, and there one buffer
        // is used: the step multiplies tile k-1, then copies tile k.
        constexpr bool DBUF = FMT != 2;
        //   bf16: va/vb[db] = transpose reads of 16-dim block db, tokens of block 0 / 1
        //   fp8 : vr[db] = 8-bit transpose read of 16-dim block db
        //   v4  : as fp8; in the rope wave, rope block j = db - 4 is held as
        //         vr[db] (tokens of block 0, bit-cast) and vx[j] (block 1)
        struct VSlice {
            bf16x4 va[8], vb[8];
            i32x2 vr[8];
            bf16x4 vx[4];
        };
        // v4 rope block j (values 16j .. 16j + 15), token block blk: transpose-read address
        auto rope_off = [&](int j, int blk) {
            const int ta = 16 * blk + 4 * g + (i16 >> 2);
            const int x = (i16 & 3) >> 1;
            if (j < 2) return (3 * kTile + ta) * 128 + (((2 * (2 + j) + x) ^ swz(ta)) << 4) + 8 * (i16 & 1);
            return HALF_OFF + ta * 64 + (((2 * (j - 2) + x) ^ swz4(ta)) << 4) + 8 * (i16 & 1);
        };
        auto load_v = [&](VSlice& v, const lds_u8* st) {
            if (FMT == 0) {
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    v.va[db] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (__attribute__((address_space(3))) bf16x4*)(st + pv[db & 3] + (db >> 2) * kTile * 128));
                    v.vb[db] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (__attribute__((address_space(3))) bf16x4*)(st + pv[4 + (db & 3)] + (db >> 2) * kTile * 128));
                }
            } else if (FMT == 2 && rope_wave) {
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    v.vr[db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(st + pv[db]));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v.vr[4 + j] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (__attribute__((address_space(3))) bf16x4*)(st + rope_off(j, 0))));
                    v.vx[j] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (__attribute__((address_space(3))) bf16x4*)(st + rope_off(j, 1)));
                }
            } else {
#pragma unroll
                for (int db = 0; db < 8; ++db)
                    v.vr[db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(st + pv[db]));
            }
        };

        // step k: `cur` holds tile k-1's slice, `nxt` receives tile k's; `gt` is
        // the prepared refill of this step (tile k + NST - 1 into the stage of
        // tile k - 1, free since E_{k-1}), `gt_next` receives the next step's.
        // LDS reads are ordered so that the MFMAs wait only for P: the flags
        // and P first, then the copy of tile k's V slice.
        auto step = [&](int k, VSlice& cur, VSlice& nxt, const Gather& gt, Gather& gt_next) {
            const bool refill = k + NST - 1 < ntiles;
            const int kp = (k - 1) & 1;
            i32x4 fl = i32x4{0, 0, 0, 0};
            constexpr int NPB = FMT == 2 ? 8 : 4;  // P operands: [copy][16-head block]
            bf16x8 pbh[NPB];
            if (k >= 1) {
                fl = lds_load<i32x4>(aux + AUX_FLAG + 16 * kp);
                const lds_u8* pr = p_read + kp * PBUF;
#pragma unroll
                for (int i = 0; i < NPB; ++i) pbh[i] = lds_load<bf16x8>(pr + (i >> 2) * kPBytesPerCopy + (i & 3) * 1024);
                // heads whose reference was raised at tile k-1: rescale their accumulators first
                if (fl[0] | fl[1] | fl[2] | fl[3]) {
#pragma unroll
                    for (int hb = 0; hb < 4; ++hb)
                        if (fl[hb]) {
                            const float al = lds_load<float>(aux + AUX_ALPHA + kp * (kHeads * 4) + 4 * (16 * hb + i16));
#pragma unroll
                            for (int db = 0; db < 8; ++db) oacc[db][hb] *= al;
                        }
                }
            }
            if (DBUF && k < ntiles) load_v(nxt, lds + (k % NST) * STAGE);
            if (k >= 1) {
                // ---- O^T[this wave's 128 dims, all heads] += V^T . P^T over tile k-1,
                // with the refill DMAs between its MFMAs
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    // (bf16: the bf16-typed transpose read; rebuilding the operand element
                    // by element from the i16-typed form is miscompiled)
                    bf16x8 av;
                    if (FMT == 0)
                        av = __builtin_shufflevector(cur.va[db], cur.vb[db], 0, 1, 2, 3, 4, 5, 6, 7);
                    else if (FMT == 2 && db >= 4 && rope_wave)
                        av = __builtin_shufflevector(__builtin_bit_cast(bf16x4, cur.vr[db]), cur.vx[db - 4], 0, 1, 2, 3,
                                                     4, 5, 6, 7);
                    else
                        av = e4m3x8_to_bf16((unsigned)cur.vr[db][0], (unsigned)cur.vr[db][1]);
                    const int pc = FMT == 2 ? 4 * (db >> 2) : 0;  // P copy of this block
#pragma unroll
                    for (int hb = 0; hb < 4; ++hb) oacc[db][hb] = mfma16(av, pbh[pc + hb], oacc[db][hb]);
                    if (refill && db < LPT_PV) issue_one(gt, db);
                }
                if (refill) {
#pragma unroll
                    for (int i = 8; i < LPT_PV; ++i) issue_one(gt, i);
                }
            } else if (refill) {
#pragma unroll
                for (int i = 0; i < LPT_PV; ++i) issue_one(gt, i);
            }
            if (!DBUF && k < ntiles) load_v(nxt, lds + (k % NST) * STAGE);  // (nxt is cur)
            if (k + NST < ntiles) gt_next = prepare(k + NST);
            if (k + 1 < ntiles) wait_tiles<LPT_PV>(min(NST - 2, ntiles - 2 - k));  // its part of tile k+1 has landed
            __syncthreads();  // E_k
        };

        // Only the first two tiles are gathered before P0, so that tile 0
        // competes with fewer gathers of the other workgroups; the rest of the
        // first NST - 1 follow P0, in order, before step 0's refill (the PV
        // waves have nothing else to do at step 0 before it).
        const int pro = min(NST - 1, ntiles);
        const int pro0 = min(2, pro);  // tiles issued before P0
        for (int t = 0; t < pro0; ++t) {
            const Gather gt = prepare(t);
#pragma unroll
            for (int i = 0; i < LPT_PV; ++i) issue_one(gt, i);
        }
        if (ntiles > 0) wait_tiles<LPT_PV>(pro0 - 1);  // this wave's part of tile 0 has landed
        __syncthreads();  // P0
        for (int t = pro0; t < pro; ++t) {
            const Gather gt = prepare(t);
#pragma unroll
            for (int i = 0; i < LPT_PV; ++i) issue_one(gt, i);
        }
        Gather ga, gb;
        if (NST - 1 < ntiles) ga = prepare(NST - 1);
        VSlice v0, v1;
        VSlice& w1 = DBUF ? v1 : v0;
        int k = 0;
        for (; k + 1 <= ntiles; k += 2) {
            step(k, w1, v0, ga, gb);
            step(k + 1, v0, w1, gb, ga);
        }
        if (k <= ntiles) step(k, w1, v0, ga, gb);
        // (the denominators were published in the last step: E_ntiles orders them)
        // every head block's denominator is read before any staging write (a
        // wait for a later read would otherwise also wait for earlier writes);
        // lane (head, g) holds dims 16 db + 4g .. + 3 of block db, rounded to
        // bf16 here, once
        float lt[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) lt[hb] = lds_load<float>(aux + AUX_DENOM + 4 * (16 * hb + i16));
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            const int h = 16 * hb + i16;
            const float inv = lt[hb] == 0.f ? 0.f : 1.f / lt[hb];
            lds_u8* row = lds + h * kRowPitch + 2 * (128 * p + 4 * g);
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const f32x4 x = oacc[db][hb] * inv;
                bf16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (__bf16)x[e];
                *(__attribute__((address_space(3))) i32x2*)(row + 32 * db) = __builtin_bit_cast(i32x2, v);
            }
        }
        __syncthreads();  // every head is staged
        store_all();
    }
}

template <int FMT, bool NTG>
hipError_t launch_partial(const PartialArgs& args, int grid, size_t lds_bytes, hipStream_t stream) {
    static std::mutex mu;
    static bool configured[64] = {false};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (dev < 0 || dev >= 64 || !configured[dev]) {
            e = hipFuncSetAttribute((const void*)partial_kernel<FMT, NTG>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
            if (e != hipSuccess) return e;
            if (dev >= 0 && dev < 64) configured[dev] = true;
        }
    }
    hipLaunchKernelGGL((partial_kernel<FMT, NTG>), dim3(grid), dim3(kThreads), lds_bytes, stream, args);
    return hipGetLastError();
}

}  // namespace
}  // namespace smla

namespace smla {
namespace {

// Host checks shared by smla_decode_partial and smla_decode_run; on success
// the partial kernel is enqueued (which, with one part, writes the final
// result).
smla_status_t enqueue_partial(const smla_plan_t* plan, const void* q, const void* kv_cache, int64_t num_kv_blocks,
                              const int32_t* block_table, const int32_t* indices, const int32_t* seq_lens,
                              float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, PartialArgs* args_out) {
    if (!plan) return SMLA_ERR_INVALID_ARG;
    // The plan must be exactly what smla_decode_plan gives for its problem.
    smla_plan_t check;
    if (plan->prob.num_cus <= 0) return SMLA_ERR_INVALID_ARG;
    smla_status_t st = smla_decode_plan(&plan->prob, &check);
    if (st != SMLA_OK) return st;
    if (std::memcmp(&check, plan, sizeof(check)) != 0) return SMLA_ERR_INVALID_ARG;
    if (plan->rows == 0) return SMLA_OK;
    if (!q || !block_table || !out || !lse) return SMLA_ERR_INVALID_ARG;
    if (!indices && plan->prob.topk > 0) return SMLA_ERR_INVALID_ARG;
    // alignment of the kernels' vector accesses
    if (((uintptr_t)q & 15) || ((uintptr_t)kv_cache & 15) || ((uintptr_t)out & 15) || ((uintptr_t)lse & 3) ||
        ((uintptr_t)block_table & 3) || ((uintptr_t)indices & 3) || ((uintptr_t)seq_lens & 3))
        return SMLA_ERR_INVALID_ARG;
    if (num_kv_blocks < 0 || (num_kv_blocks > 0 && !kv_cache)) return SMLA_ERR_INVALID_ARG;
    if (num_kv_blocks > (int64_t)(INT32_MAX / kBlock)) return SMLA_ERR_UNSUPPORTED;
    if (!std::isfinite(softmax_scale)) return SMLA_ERR_INVALID_ARG;
    if (plan->workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan->workspace_bytes) return SMLA_ERR_WORKSPACE_TOO_SMALL;
        if (((uintptr_t)workspace & 255) != 0) return SMLA_ERR_INVALID_ARG;
    }

    PartialArgs& args = *args_out;
    args.q = (const uint16_t*)q;
    args.kv = (const uint8_t*)kv_cache;
    args.block_table = block_table;
    args.indices = indices;
    args.seq_lens = seq_lens;
    args.out = (uint16_t*)out;
    args.lse = lse;
    const int S = plan->num_splits;
    const int64_t pairs = (int64_t)plan->rows * kHeads;
    args.part_out = S > 1 ? (uint16_t*)workspace : nullptr;
    args.part_lse = S > 1 ? (float*)((uint16_t*)workspace + (size_t)S * pairs * kDv) : nullptr;
    args.num_kv_blocks = num_kv_blocks;
    args.rows = plan->rows;
    args.q_len = plan->prob.q_len;
    args.topk = plan->prob.topk;
    args.max_blocks = plan->prob.max_blocks_per_seq;
    args.tokens_per_split = plan->tokens_per_split;
    args.num_splits = S;
    args.scale_log2 = softmax_scale * kLog2e;
    args.num_workgroups = plan->num_workgroups;
    const int pol = plan->cache_policy;
    const bool ntg = pol == SMLA_CACHE_STREAM_ROWS || pol == SMLA_CACHE_STREAM_BOTH;
    args.stream_out = pol == SMLA_CACHE_STREAM_OUT || pol == SMLA_CACHE_STREAM_BOTH ? 1 : 0;

    const size_t lds = partial_lds_bytes(plan->prob.kv_format, plan->tokens_per_split);
    (void)hipGetLastError();  // clear an earlier, unrelated error
    hipError_t e;
    const int g = plan->num_workgroups;
    switch (plan->prob.kv_format) {
        case SMLA_KV_BF16:
            e = ntg ? launch_partial<0, true>(args, g, lds, stream) : launch_partial<0, false>(args, g, lds, stream);
            break;
        case SMLA_KV_FP8_E4M3_SCALE128:
            e = ntg ? launch_partial<1, true>(args, g, lds, stream) : launch_partial<1, false>(args, g, lds, stream);
            break;
        default:
            e = ntg ? launch_partial<2, true>(args, g, lds, stream) : launch_partial<2, false>(args, g, lds, stream);
            break;
    }
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

}  // namespace
}  // namespace smla

// ---- allocation-free variant: the split partials live in a file-scope device
// array instead of a caller's workspace.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and that address is what the kernels receive.
namespace smla {
namespace {

__device__ __attribute__((aligned(256))) unsigned char scratch[SMLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (looked up on the first
// call per device); nullptr with *err set if the lookup fails.
void* scratch_address(hipError_t* err) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {nullptr};
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

}  // namespace
}  // namespace smla

extern "C" smla_status_t smla_decode_run_noalloc(const smla_plan_t* plan, const void* q, const void* kv_cache,
                                                 int64_t num_kv_blocks, const int32_t* block_table,
                                                 const int32_t* indices, const int32_t* seq_lens, float softmax_scale,
                                                 void* out, float* lse, void* stream) {
    using namespace smla;
    if (!plan) return SMLA_ERR_INVALID_ARG;
    if (plan->workspace_bytes > (uint64_t)SMLA_NOALLOC_SCRATCH_BYTES) return SMLA_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if (plan->workspace_bytes > 0) {
        hipError_t e;
        ws = scratch_address(&e);
        if (!ws) return SMLA_ERR_DEVICE;
    }
    return smla_decode_run(plan, q, kv_cache, num_kv_blocks, block_table, indices, seq_lens, softmax_scale, out, lse,
                           ws, ws ? (size_t)SMLA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

extern "C" smla_status_t smla_decode_partial(const smla_plan_t* plan, const void* q, const void* kv_cache,
                                             int64_t num_kv_blocks, const int32_t* block_table,
                                             const int32_t* indices, const int32_t* seq_lens, float softmax_scale,
                                             void* out, float* lse, void* workspace, size_t workspace_bytes,
                                             void* stream) {
    smla::PartialArgs args;
    return smla::enqueue_partial(plan, q, kv_cache, num_kv_blocks, block_table, indices, seq_lens, softmax_scale,
                                 out, lse, workspace, workspace_bytes, (hipStream_t)stream, &args);
}

extern "C" smla_status_t smla_decode_run(const smla_plan_t* plan, const void* q, const void* kv_cache,
                                         int64_t num_kv_blocks, const int32_t* block_table,
                                         const int32_t* indices, const int32_t* seq_lens, float softmax_scale,
                                         void* out, float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream) {
    using namespace smla;
    PartialArgs args;
    smla_status_t st = enqueue_partial(plan, q, kv_cache, num_kv_blocks, block_table, indices, seq_lens,
                                       softmax_scale, out, lse, workspace, workspace_bytes, (hipStream_t)stream,
                                       &args);
    if (st != SMLA_OK || plan->rows == 0 || plan->num_splits == 1) return st;
    return launch_combine(args.part_out, args.part_lse, plan->num_splits, (int64_t)plan->rows * kHeads, out, lse,
                          (hipStream_t)stream, args.stream_out != 0);
}
