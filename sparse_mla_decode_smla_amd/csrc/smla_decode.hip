// Partial-attention kernel of head-batched sparse MLA decode, and the
// smla_decode_run entry point.
//
// One workgroup handles one query row (b, s), all 64 heads, and one part of
// that row's top-k list.  Every selected latent row is gathered from the
// paged cache into LDS once and read from there by all four waves (wave w
// owns heads [16w, 16w + 16)): the head batching of "The MMA Sparse-MLA
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
//             per-group partial scores);
//   softmax : online, base 2, running max and sum per head in registers,
//             masked tokens get -inf ("Edge Case Handling": invalid tokens
//             never enter the softmax);
//   PV      : O^T[dim, head] += V^T . P^T with the same MFMA; V^T comes from
//             the same LDS tile through transpose reads (ds_read_b64_tr_b16,
//             ds_read_b64_tr_b8); fp32 accumulation, bf16 only at the store
//             ("Design Decisions" 6).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "smla.h"
#include "smla_internal.h"

namespace smla {

smla_status_t launch_combine(const float* part_out, const float* part_lse, int num_splits, int64_t pairs,
                             void* out, float* lse, hipStream_t stream);

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
    float* part_out;
    float* part_lse;
    int64_t num_kv_blocks;
    int32_t rows, q_len, topk, max_blocks, tokens_per_split, num_splits;
    float scale_log2;
};

// 16-byte LDS-DMA load: lane l's 16 bytes from `src` land at LDS byte
// lds_base + 16*l.  Issued from inline assembly so the compiler does not
// serialise the stage ring with conservative waits; the kernel waits on
// vmcnt itself.  M0 is written only here (the kernel has no other M0 use).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* src, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

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


template <int FMT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void partial_kernel(PartialArgs a) {
    constexpr int STAGE = FMT == 0 ? kStageBytesBf16 : kStageBytesFp8;
    constexpr int NST = FMT == 0 ? kStagesBf16 : kStagesFp8;
    constexpr int ROWB = FMT == 0 ? kRowBytesBf16 : kRowBytesFp8;
    constexpr int NBANDS = FMT == 0 ? kBandsBf16 : kBandsFp8;
    static_assert(NST - 2 <= 4, "wait_tiles covers at most 4 tiles in flight after the current one");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem_generic[];
    lds_u8* lds = (lds_u8*)smem_generic;
    const unsigned lds0 = (unsigned)(uintptr_t)lds;
    constexpr int AUX_FLAG = aux_flag_offset(FMT);
    constexpr int AUX_TMAX = aux_tmax_offset(FMT);
    constexpr int AUX_DENOM = aux_denom_offset(FMT);
    lds_u8* aux = lds + NST * STAGE;
    lds_u8* rowtab = aux + aux_bytes(FMT);  // int32 per token of this part: physical row or -1

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hg = wave & 3;    // QK head group: heads [16hg, 16hg + 16)
    const int tb = wave >> 2;   // QK token half of a tile: tokens [16tb, 16tb + 16)
    const int g = lane >> 4;    // 16-lane group
    const int i16 = lane & 15;  // lane within the group
    const int head = 16 * hg + i16;  // the head of this lane in QK and softmax

    const int r = blockIdx.x / a.num_splits;
    const int sp = blockIdx.x - r * a.num_splits;
    const int b = r / a.q_len;
    const int k0 = sp * a.tokens_per_split;
    const int nk = max(0, min(a.tokens_per_split, a.topk - k0));
    const int ntiles = (nk + kTile - 1) / kTile;

    // ---- Q of head 16hg + i16, as the B operand of S^T = K . Q^T (8 dims of
    // k-step kk per lane).  For fp8 rows the c_kv dims of k-steps 2p and 2p+1
    // inside a 128-group are the two halves of one 16-byte run, so one LDS
    // read feeds two k-steps.
    bf16x8 qreg[18];
    {
        const uint16_t* qh = a.q + ((int64_t)r * kHeads + head) * kDqk;
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
            int d;
            if (FMT == 0 || kk >= 16)
                d = 32 * kk + 8 * g;
            else
                d = 128 * (kk >> 2) + 64 * ((kk >> 1) & 1) + 16 * g + 8 * (kk & 1);
            qreg[kk] = *(const bf16x8*)(qh + d);
        }
    }

    // ---- logical positions -> physical rows (masked entries -> -1)
    {
        int64_t cap = (int64_t)kBlock * a.max_blocks;
        if (a.seq_lens) cap = min(cap, (int64_t)a.seq_lens[b]);
        const int32_t* idx = a.indices + (int64_t)r * a.topk + k0;
        const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks;
        for (int i = tid; i < ntiles * kTile; i += kThreads) {
            int row = -1;
            if (i < nk) {
                const int pos = idx[i];
                if (pos >= 0 && (int64_t)pos < cap) {
                    const int blk = bt[pos / kBlock];
                    if (blk >= 0 && (int64_t)blk < a.num_kv_blocks) row = blk * kBlock + (pos % kBlock);
                }
            }
            *(__attribute__((address_space(3))) int*)(rowtab + 4 * i) = row;
        }
    }
    wait_vmcnt<0>();
    // The loads above are complete; tell the compiler so it does not place
    // vmcnt waits for them inside the loop, where the stage DMAs are in flight.
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) asm volatile("" : "+a"(qreg[kk]));
    __syncthreads();

    // ---- gather: a DMA instruction moves one 128-byte band of 8 tokens.  Wave
    // w takes the tokens [8(w%4), 8(w%4) + 8) of every tile and the bands
    //   bf16: w/4, w/4 + 2, w/4 + 4, w/4 + 6, and band 8 if w < 4  (5 or 4 DMAs)
    //   fp8 : 0, 2, 4 if w < 4; 1, 3 and the fp32 scales otherwise (3 DMAs)
    // so each wave issues a fixed number of DMAs per tile and counts them itself.
    constexpr int LPT_A = FMT == 0 ? 5 : 3;  // DMAs per tile of waves 0-3
    constexpr int LPT_B = FMT == 0 ? 4 : 3;  // DMAs per tile of waves 4-7
    auto issue = [&](int tile) {
        const unsigned sbase = lds0 + (unsigned)((tile % NST) * STAGE);
        const int t = 8 * hg + (lane >> 3);  // token of this lane within the tile
        const int row = *(const __attribute__((address_space(3))) int*)(rowtab + 4 * (tile * kTile + t));
        const int chunk = (lane & 7) ^ swz(t);
        const unsigned char* src = row >= 0 ? a.kv + (int64_t)row * ROWB + chunk * 16 : kZeroChunk;
        const int bstride = row >= 0 ? 128 : 0;
        const unsigned dst = sbase + (unsigned)(8 * hg * 128);
        if (FMT == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int bd = tb + 2 * i;
                lds_dma16(src + bd * bstride, dst + (unsigned)(bd * kTile * 128));
            }
            if (tb == 0) lds_dma16(src + 8 * bstride, dst + (unsigned)(8 * kTile * 128));
        } else {
            if (tb == 0) {
#pragma unroll
                for (int bd = 0; bd < 5; bd += 2) lds_dma16(src + bd * bstride, dst + (unsigned)(bd * kTile * 128));
            } else {
#pragma unroll
                for (int bd = 1; bd < 4; bd += 2) lds_dma16(src + bd * bstride, dst + (unsigned)(bd * kTile * 128));
                // fp32 scales: lanes 0..7 fetch the 16 bytes of tokens 8hg + lane
                const int t2 = 8 * hg + (lane & 7);
                const int row2 = *(const __attribute__((address_space(3))) int*)(rowtab + 4 * (tile * kTile + t2));
                const unsigned char* s2 = row2 >= 0 ? a.kv + (int64_t)row2 * ROWB + NBANDS * 128 : kZeroChunk;
                if (lane < 8) lds_dma16(s2, sbase + (unsigned)(NBANDS * kTile * 128 + 8 * hg * 16));
            }
        }
    };
    auto wait_for_tile = [&](int after) {
        if (wave < 4)
            wait_tiles<LPT_A>(after);
        else
            wait_tiles<LPT_B>(after);
    };

    // ---- per-lane LDS byte offsets inside a stage (loop invariant)
    // QK A operand (K): token tA = 16tb + i16, chunk (4e + g) of a band (e = k-step parity).
    const int tA = 16 * tb + i16;
    int qk[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) qk[e] = tA * 128 + (((4 * e + g) ^ swz(tA)) << 4);
    // QK accumulator entry j of this lane: token tC + j of the tile (tC = 16tb + 4g).
    const int tC = 16 * tb + 4 * g;
    // PV A operand (V^T) of dims [64w, 64w + 64): the k-slots 8g .. 8g + 7 of a
    // lane are the tokens 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3 (the order in
    // which the P operand is exchanged).
    //   bf16: band w; lane i16 addresses token tok + (i16 >> 2), 4 dims at 4(i16 & 3)
    //         of 16-dim block m; the transpose read hands lane i dim i of the block.
    //   fp8 : band w/2 (the scale group), 16-dim blocks 4(w & 1) + m; lane i16
    //         addresses token slot j = i16 >> 1, 8 dims at 8(i16 & 1).
    int pv[8];
    if (FMT == 0) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int ta = 16 * blk + 4 * g + (i16 >> 2);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                pv[4 * blk + m] = (wave * kTile + ta) * 128 + (((2 * m + ((i16 & 3) >> 1)) ^ swz(ta)) << 4) +
                                  8 * (i16 & 1);
        }
    } else {
        const int j = i16 >> 1;
        const int ta = j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            pv[m] = ((wave >> 1) * kTile + ta) * 128 + (((4 * (wave & 1) + m) ^ swz(ta)) << 4) + 8 * (i16 & 1);
    }
    // P: this lane's 4 weights (tokens tC .. tC + 3 of head `head`) go to
    // operand slot (block hg, group g, lane i16), half tb.
    lds_u8* const p_mine = aux + ((hg * 4 + g) * 16 + i16) * 16 + 8 * tb;  // + grp * kPBytesPerCopy for fp8
    const lds_u8* const p_read = aux + (FMT == 0 ? 0 : (wave >> 1) * kPBytesPerCopy) + lane * 16;  // + hb * 1024

    // Softmax state of head `head` over this wave's token half.  Exponentials
    // are taken against a reference fixed at the first tile with a valid token
    // (the max over that tile, both halves), so the accumulators are never
    // rescaled inside the loop; weights up to 2^kMaxRise stay finite in fp32
    // and bf16.  If a later score rises above the reference by more than that,
    // the workgroup restarts its part of the list with the reference raised
    // (the row table and Q stay; the accumulators of the abandoned pass are
    // discarded).
    constexpr float kMaxRise = 64.f;
    float m_ref = -INFINITY;
    float l_run;       // this lane's share of sum_j p_j
    f32x4 oacc[4][4];  // O^T of this wave: [16-dim block of its 64 dims][16-head block]

    for (;;) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                oacc[i][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
                // the accumulators live in AGPRs from the start, so the loop
                // does not move them between register files each iteration
                asm volatile("" : "+a"(oacc[i][hb]));
            }
        l_run = 0.f;
        bool have_ref = m_ref != -INFINITY;  // set by an earlier pass (the same in every lane)
        bool restart = false;

#pragma unroll
        for (int t = 0; t < NST - 1; ++t)
            if (t < ntiles) issue(t);

        for (int it = 0; it < ntiles; ++it) {
            wait_for_tile(min(NST - 2, ntiles - 1 - it));
            __syncthreads();  // tile `it` is in LDS for every wave; stage (it-1)%NST is free
            if (it + NST - 1 < ntiles) issue(it + NST - 1);

            const lds_u8* st = lds + (it % NST) * STAGE;
            const lds_u8* rt = rowtab + 4 * it * kTile;
            // validity of this lane's accumulator tokens, and of the other half's
            const i32x4 vown = lds_load<i32x4>(rt + 4 * tC);
            const i32x4 voth = lds_load<i32x4>(rt + 4 * (tC ^ 16));

            // ---- S^T = K . Q^T for the 16 tokens of this wave's half
            f32x4 s;
            f32x4 sc[4];  // fp8: sc[j][grp] = scale of group grp of accumulator token tC + j
            if (FMT == 0) {
                constexpr int PF = 6;  // K operands in flight
                bf16x8 ka[PF];
                f32x4 se = f32x4{0.f, 0.f, 0.f, 0.f}, so = se;  // even / odd k-steps (two MFMA chains)
#pragma unroll
                for (int kk = 0; kk < PF; ++kk) ka[kk] = lds_load<bf16x8>(st + qk[kk & 1] + (kk >> 1) * kTile * 128);
#pragma unroll
                for (int kk = 0; kk < 18; ++kk) {
                    const int sl = kk % PF;
                    if (kk & 1)
                        so = mfma16(ka[sl], qreg[kk], so);
                    else
                        se = mfma16(ka[sl], qreg[kk], se);
                    if (kk + PF < 18) {
                        const int kn = kk + PF;
                        ka[sl] = lds_load<bf16x8>(st + qk[kn & 1] + (kn >> 1) * kTile * 128);
                    }
                }
                // PF reads first, then MFMA / read pairs
                __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
                for (int i = 0; i < 18 - PF; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
                s = se + so;
            } else {
                // 10 load units: rope k-steps 16, 17 (bf16), then c_kv pairs (group, pair)
                constexpr int PF = 5;
                u32x4 ka[PF];
                auto unit_off = [&](int u) {
                    return u < 2 ? qk[u] + 4 * kTile * 128 : qk[(u - 2) & 1] + ((u - 2) >> 1) * kTile * 128;
                };
                const lds_u8* scl = st + NBANDS * kTile * 128;
#pragma unroll
                for (int u = 0; u < PF; ++u) ka[u] = lds_load<u32x4>(st + unit_off(u));
#pragma unroll
                for (int j = 0; j < 4; ++j) sc[j] = lds_load<f32x4>(scl + 16 * (tC + j));
                s = f32x4{0.f, 0.f, 0.f, 0.f};
                f32x4 p = s;
#pragma unroll
                for (int u = 0; u < 10; ++u) {
                    const int sl = u % PF;
                    if (u < 2) {
                        s = mfma16(__builtin_bit_cast(bf16x8, ka[sl]), qreg[16 + u], s);
                    } else {
                        const int grp = (u - 2) >> 1, pr = (u - 2) & 1;
                        if (pr == 0) p = f32x4{0.f, 0.f, 0.f, 0.f};
                        p = mfma16(e4m3x8_to_bf16(ka[sl][0], ka[sl][1]), qreg[4 * grp + 2 * pr], p);
                        p = mfma16(e4m3x8_to_bf16(ka[sl][2], ka[sl][3]), qreg[4 * grp + 2 * pr + 1], p);
                        if (pr == 1) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) s[j] += sc[j][grp] * p[j];
                        }
                    }
                    if (u + PF < 10) ka[sl] = lds_load<u32x4>(st + unit_off(u + PF));
                }
                // first PF units' reads and the scales, then per unit its MFMAs and the next unit's read
                __builtin_amdgcn_sched_group_barrier(0x100, PF + 4, 0);
#pragma unroll
                for (int u = 0; u < 10 - PF; ++u) {
                    if (u < 2)
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    else
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * PF, 0);
            }

            // ---- mask, softmax weights (base 2)
            float sv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[j] = vown[j] >= 0 ? s[j] * a.scale_log2 : -INFINITY;
            float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            bool rise = false;
            if (!have_ref) {
                // first tile with a valid token: the same tile in every wave (each
                // lane group sees 4 tokens of both halves, so the vote covers all 32)
                const bool any_valid = vown[0] >= 0 || vown[1] >= 0 || vown[2] >= 0 || vown[3] >= 0 ||
                                       voth[0] >= 0 || voth[1] >= 0 || voth[2] >= 0 || voth[3] >= 0;
                if (__any(any_valid)) {
                    mx = fmaxf(mx, __shfl_xor(mx, 16));
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    if (g == 0) *(__attribute__((address_space(3))) float*)(aux + AUX_TMAX + 4 * (tb * kHeads + head)) = mx;
                    __syncthreads();
                    m_ref = fmaxf(mx, lds_load<float>(aux + AUX_TMAX + 4 * ((tb ^ 1) * kHeads + head)));
                    have_ref = true;
                }
            } else if (mx > m_ref + kMaxRise) {  // lane-local test; the restart is decided after PV
                rise = true;
                m_ref = fmaxf(m_ref, mx);  // (reconciled across the head's lanes on restart)
            }
            const float m_use = have_ref ? m_ref : 0.f;
            // The denominator sums the fp32 weights; the PV product takes them
            // rounded to bf16 once (for fp8 rows after multiplying by the
            // token's scale of each 128-group, one copy per group).
            float pf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pf[j] = __builtin_amdgcn_exp2f(sv[j] - m_use);
            l_run += (pf[0] + pf[1]) + (pf[2] + pf[3]);
            if (FMT == 0) {
                bf16x4 pb;
#pragma unroll
                for (int j = 0; j < 4; ++j) pb[j] = (__bf16)pf[j];
                *(__attribute__((address_space(3))) bf16x4*)p_mine = pb;
            } else {
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    bf16x4 pg;
#pragma unroll
                    for (int j = 0; j < 4; ++j) pg[j] = (__bf16)(pf[j] * sc[j][grp]);
                    *(__attribute__((address_space(3))) bf16x4*)(p_mine + grp * kPBytesPerCopy) = pg;
                }
            }
            const int any_rise = __any(rise) ? 1 : 0;
            if (lane == 0) *(__attribute__((address_space(3))) int*)(aux + AUX_FLAG + 4 * wave) = any_rise;
            __syncthreads();  // P and the rise flags of every wave are visible
            const i32x4 fl0 = lds_load<i32x4>(aux + AUX_FLAG);
            const i32x4 fl1 = lds_load<i32x4>(aux + AUX_FLAG + 16);

            // ---- O^T[this wave's 64 dims, all heads] += V^T . P^T
            bf16x8 pbh[4];  // P^T of head block hb (fp8: scaled for this wave's group)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) pbh[hb] = lds_load<bf16x8>(p_read + hb * 1024);
            if (FMT == 0) {
                bf16x4 va[4], vb[4];
                auto tr = [&](int m, int blk) {
                    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (__attribute__((address_space(3))) bf16x4*)(st + pv[4 * blk + m]));
                };
#pragma unroll
                for (int m = 0; m < 4; ++m) { va[m] = tr(m, 0); vb[m] = tr(m, 1); }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    // (the bf16-typed transpose read: rebuilding the operand element
                    // by element from the i16-typed form is miscompiled)
                    const bf16x8 av = __builtin_shufflevector(va[m], vb[m], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int hb = 0; hb < 4; ++hb) oacc[m][hb] = mfma16(av, pbh[hb], oacc[m][hb]);
                }
            } else {
                i32x2 raw[4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    raw[m] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(st + pv[m]));
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bf16x8 av = e4m3x8_to_bf16((unsigned)raw[m][0], (unsigned)raw[m][1]);
#pragma unroll
                    for (int hb = 0; hb < 4; ++hb) oacc[m][hb] = mfma16(av, pbh[hb], oacc[m][hb]);
                }
            }

            if ((fl0[0] | fl0[1] | fl0[2] | fl0[3]) | (fl1[0] | fl1[1] | fl1[2] | fl1[3])) {
                restart = true;  // rare: restart with raised references
                break;
            }
        }
        if (!restart) break;
        // the head's reference: max over its lanes in this wave and the other half
        m_ref = fmaxf(m_ref, __shfl_xor(m_ref, 16));
        m_ref = fmaxf(m_ref, __shfl_xor(m_ref, 32));
        wait_vmcnt<0>();  // drain the stage DMAs still in flight
        if (g == 0) *(__attribute__((address_space(3))) float*)(aux + AUX_TMAX + 4 * (tb * kHeads + head)) = m_ref;
        __syncthreads();  // every wave has left the loop; stages may be refilled
        m_ref = fmaxf(m_ref, lds_load<float>(aux + AUX_TMAX + 4 * ((tb ^ 1) * kHeads + head)));
        __syncthreads();  // tmax is read before the next pass may write it
    }

    // ---- epilogue: denominators, lse, normalised output
    float l_half = l_run;
    l_half += __shfl_xor(l_half, 16);
    l_half += __shfl_xor(l_half, 32);
    if (g == 0) *(__attribute__((address_space(3))) float*)(aux + AUX_DENOM + 4 * (tb * kHeads + head)) = l_half;
    __syncthreads();
    if (tb == 0 && g == 0) {
        const bool empty = (m_ref == -INFINITY);
        const float l_tot = l_half + lds_load<float>(aux + AUX_DENOM + 4 * (kHeads + head));
        const float lse_v = empty ? -INFINITY : (m_ref + log2f(l_tot)) * kLn2;
        if (a.num_splits == 1)
            a.lse[(int64_t)r * kHeads + head] = lse_v;
        else
            a.part_lse[((int64_t)sp * a.rows + r) * kHeads + head] = lse_v;
    }
    // The normalised output goes through the (now idle) stage ring, 32 heads at
    // a time, so that every head's row is written to HBM with contiguous
    // 1 KB stores.  Rows are padded by 16 bytes: the staging writes of a
    // 16-lane group (16 heads, same dims) then fall on distinct banks.  (Every
    // stage DMA has landed: the last loop iteration waited for all of them.)
    constexpr int kRowPitch = 4 * kDv + 16;
    static_assert(32 * kRowPitch <= NST * STAGE, "staging area exceeds the stage ring");
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
            const int hb = 2 * half + hl;
            const int h = 16 * hb + i16;
            const float lt = lds_load<float>(aux + AUX_DENOM + 4 * h) + lds_load<float>(aux + AUX_DENOM + 4 * (kHeads + h));
            const float inv = (m_ref == -INFINITY || lt == 0.f) ? 0.f : 1.f / lt;
            lds_u8* row = lds + (h - 32 * half) * kRowPitch + 4 * (64 * wave + 4 * g);
#pragma unroll
            for (int m = 0; m < 4; ++m) *(__attribute__((address_space(3))) f32x4*)(row + 64 * m) = oacc[m][hb] * inv;
        }
        __syncthreads();
        // wave w stores heads 32*half + 4w .. 32*half + 4w + 3; lane l holds dims
        // [4l, 4l + 4) and [256 + 4l, 256 + 4l + 4)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int hl = 4 * wave + j;
            const int h = 32 * half + hl;
            const f32x4 x0 = lds_load<f32x4>(lds + hl * kRowPitch + 16 * lane);
            const f32x4 x1 = lds_load<f32x4>(lds + hl * kRowPitch + 1024 + 16 * lane);
            if (a.num_splits == 1) {
                uint16_t* o = a.out + ((int64_t)r * kHeads + h) * kDv + 4 * lane;
                bf16x4 v0, v1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v0[e] = (__bf16)x0[e];
                    v1[e] = (__bf16)x1[e];
                }
                *(bf16x4*)o = v0;
                *(bf16x4*)(o + 256) = v1;
            } else {
                float* o = a.part_out + (((int64_t)sp * a.rows + r) * kHeads + h) * kDv + 4 * lane;
                *(f32x4*)o = x0;
                *(f32x4*)(o + 256) = x1;
            }
        }
        if (half == 0) __syncthreads();  // the staging rows are free again
    }
}

template <int FMT>
hipError_t launch_partial(const PartialArgs& args, int grid, size_t lds_bytes, hipStream_t stream) {
    static std::mutex mu;
    static bool configured[64] = {false};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (dev < 0 || dev >= 64 || !configured[dev]) {
            e = hipFuncSetAttribute((const void*)partial_kernel<FMT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    kLdsLimit);
            if (e != hipSuccess) return e;
            if (dev >= 0 && dev < 64) configured[dev] = true;
        }
    }
    hipLaunchKernelGGL(partial_kernel<FMT>, dim3(grid), dim3(kThreads), lds_bytes, stream, args);
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
    args.part_out = S > 1 ? (float*)workspace : nullptr;
    args.part_lse = S > 1 ? (float*)workspace + (size_t)S * pairs * kDv : nullptr;
    args.num_kv_blocks = num_kv_blocks;
    args.rows = plan->rows;
    args.q_len = plan->prob.q_len;
    args.topk = plan->prob.topk;
    args.max_blocks = plan->prob.max_blocks_per_seq;
    args.tokens_per_split = plan->tokens_per_split;
    args.num_splits = S;
    args.scale_log2 = softmax_scale * kLog2e;

    const size_t lds = partial_lds_bytes(plan->prob.kv_format, plan->tokens_per_split);
    (void)hipGetLastError();  // clear an earlier, unrelated error
    hipError_t e = plan->prob.kv_format == SMLA_KV_BF16 ? launch_partial<0>(args, plan->num_workgroups, lds, stream)
                                                        : launch_partial<1>(args, plan->num_workgroups, lds, stream);
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

}  // namespace
}  // namespace smla

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
                          (hipStream_t)stream);
}
