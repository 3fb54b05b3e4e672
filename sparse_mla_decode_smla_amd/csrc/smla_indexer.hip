// Top-k indexer: the step that produces the index lists of the sparse
// decode ("The Pivot Point: When a 6.3x Kernel Speedup Reveals the Next
// Bottleneck", Input Knowledge Required: an indexer picks the top ~512 cache
// positions of each decode step; "The Moment of Truth: Benchmarking a Custom
// MMA Kernel for DeepSeek-V4-Flash on Blackwell", The Broader Context: it
// scores every position of the context; "The MMA Sparse-MLA Decode Kernel: A
// Deep Dive ...", Context: the scores come from a batched product of the
// indexer query with the indexer keys, in bf16 on the matrix units once the
// forced fp32 path was dropped).
//
// For query row r = (b, s) and every candidate position p of sequence b
// (p < min(seq_lens[b], 64 * max_blocks), block-table entry in range):
//     score(r, p) = q_idx[r, :] . k_idx[block_table[b][p / 64], p % 64, :]
// with bf16 operands and fp32 accumulation; the row's list is the
// min(topk, #candidates) positions of highest score (equal scores: lower
// positions first), in ascending position order, then -1.
//
// Two kernels (four for rows of more than 16,384 positions):
//   score_kernel  streams each sequence's keys once (whole 64-token blocks,
//                 16 KB contiguous) for all q_len rows of the sequence; a
//                 token's 256-byte key is spread over 16 lanes (16 bytes
//                 each, v_dot2_f32_bf16) and summed across them; fp32 scores
//                 go to the workspace [rows, 64 * max_blocks].  This is HBM
//                 streaming, not a contraction worth the matrix cores (one or
//                 two query rows per key).
//   select_kernel one 1024-thread workgroup per row, each thread owning a
//                 contiguous run of up to 16 positions held in registers: an
//                 exact radix select of the topk-th largest score over an
//                 order-preserving key (digits of 12, 12 and 8 bits, LDS
//                 histogram of 4096 bins; after the first digit only the keys
//                 in its bin, copied to LDS, take part), then one block scan
//                 that gives every thread its output slots, so the winners
//                 (and the lowest positions of the threshold's ties) are
//                 written in ascending position order with no sort.
//   Longer rows take the same selection spread over one workgroup per 4096
//   positions (each chunk's first digits counted by the score kernel or by
//   chunk_hist_kernel, then chunk_thresh_kernel and chunk_final_kernel,
//   below): a single workgroup reading a row of 65,536 scores is bound by its
//   own request rate.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "smla.h"

namespace smla_idx {
namespace {

constexpr int kDidx = 128;        // indexer key / query width
constexpr int kBlk = 64;          // tokens per cache block
constexpr int kMaxTopk = 2048;    // longest list
constexpr int kMaxQlen = 4;       // query rows per sequence held in registers by score_kernel
constexpr int kScoreWaves = 4;    // waves per score workgroup
constexpr int kBlocksPerWave = 2; // cache blocks per wave per workgroup
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 4096;       // radix histogram bins (12-bit digits)
constexpr int kCandCap = 4096;    // keys sharing the first digit kept in LDS
constexpr unsigned kNegInfKey = 0x007FFFFFu;  // order key of -inf
// chunked selection (rows of more than kChunkedFrom positions)
constexpr int kChunk = 4096;                       // positions per chunk
constexpr int kChThreads = 256;                    // threads of a chunk workgroup
constexpr int kChWaves = kChThreads / 64;
constexpr int kChPer = kChunk / kChThreads;        // positions per thread
constexpr int kCoarseBins = 256;                   // top 8 bits of a key
constexpr int kHistU16 = kCoarseBins + kBins;      // per chunk: coarse counts, then first-digit counts
constexpr int kChunkedFrom = 16 * kSelThreads;     // rows of up to this many positions: select_kernel
constexpr int kHistWaves = 8;                      // waves of a score workgroup that also counts (HIST)
// The score kernel counts the chunk histograms itself when it has at least
// this many (sequence, chunk) workgroups, one per CU of an MI355X (with fewer
// it streams the keys on too few CUs, and the histograms take a kernel of
// their own)
constexpr int kCountingFromWgs = 256;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// fp32 -> unsigned key with the same order (larger score, larger key; -0
// and +0 are the same score).
__device__ __forceinline__ unsigned order_key(float s) {
    unsigned u = __builtin_bit_cast(unsigned, s);
    u = u == 0x80000000u ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(unsigned k) {
    return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// grid (ceil(max_blocks / (W * BPW)), batch), 64 W threads: W = kScoreWaves
// waves of BPW = kBlocksPerWave blocks; with HIST (rows of more than
// kChunkedFrom positions) W = kHistWaves waves of 8 blocks, so that a
// workgroup scores one whole chunk of kChunk positions, and it also counts
// the first digits of its candidates' keys per query row into the chunk
// histograms of the chunked selection (hist, u16 [rows, nch, kHistU16]).
// QL >= q_len query rows are held in registers: one row needs 76 VGPRs (six
// waves per SIMD), four need 137 (three).
template <int QL, bool HIST>
__global__ __launch_bounds__(HIST ? 64 * kHistWaves : 64 * kScoreWaves) void score_kernel(
    const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ k_cache, int64_t num_kv_blocks,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int q_len, int max_blocks,
    float* __restrict__ scores, uint16_t* __restrict__ hist) {
    constexpr int W = HIST ? kHistWaves : kScoreWaves;
    constexpr int BPW = HIST ? kChunk / (kBlk * kHistWaves) : kBlocksPerWave;
    static_assert(!HIST || W * BPW * kBlk == kChunk, "a counting workgroup scores one chunk");
    __shared__ unsigned hf[HIST ? QL * kBins : 1];
    // (sequence, chunk) items dealt XCD by XCD: consecutive workgroup ids go
    // round-robin over the 8 XCDs, XCD x takes the x-th eighth of the items, so
    // a sequence's scores land in the L2 of the XCD whose select workgroups read
    // them (the select kernel deals its rows the same way)
    const int nchunk = (max_blocks + W * BPW - 1) / (W * BPW);
    const int nitems = (int)gridDim.x;
    const int xcd = blockIdx.x & 7, within = blockIdx.x >> 3;
    const int item = xcd * (nitems >> 3) + min(xcd, nitems & 7) + within;
    const int b = item / nchunk;
    const int chunk = item - b * nchunk;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;   // token within a group of 4
    const int c = lane & 15;   // 16-byte chunk of the key (dims 8c .. 8c+7)
    const int64_t cap = (int64_t)kBlk * max_blocks;
    const int n = (int)min((int64_t)max(seq_lens[b], 0), cap);
    const int64_t row0 = (int64_t)b * q_len;

    // this lane's 8 query dims of each row of the sequence
    bf16x2 qv[QL][4];
#pragma unroll
    for (int s = 0; s < QL; ++s) {
        if (s < q_len) {
            const u32x4 v = *(const u32x4*)(q_idx + (row0 + s) * kDidx + 8 * c);
            // (each element goes through a scalar: bit-casting a vector element in
            // place reads element 0 with this compiler)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned ve = v[e];
                qv[s][e] = __builtin_bit_cast(bf16x2, ve);
            }
        }
    }

    if (HIST) {
        for (int i = threadIdx.x; i < QL * kBins; i += 64 * W) hf[i] = 0;
        __syncthreads();
    }
#pragma unroll 1
    for (int i = 0; i < BPW; ++i) {
        const int j = (chunk * BPW + i) * W + wave;  // logical block
        if (j >= max_blocks || j * kBlk >= n) continue;
        const int blk = block_table[(int64_t)b * max_blocks + j];
        const int tok_end = min(kBlk, n - j * kBlk);
        const int mytok = 4 * c + g;  // the token whose score this lane stores
        if (blk < 0 || (int64_t)blk >= num_kv_blocks) {
            if (mytok < tok_end)
                for (int s = 0; s < q_len; ++s) scores[(row0 + s) * cap + j * kBlk + mytok] = -INFINITY;
            continue;
        }
        // all 16 loads first: token 4t + g, chunk c
        const uint8_t* base = k_cache + ((int64_t)blk * kBlk) * (2 * kDidx) + 16 * c;
        u32x4 kv[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) kv[t] = __builtin_nontemporal_load((const u32x4*)(base + (4 * t + g) * (2 * kDidx)));
#pragma unroll
        for (int s = 0; s < QL; ++s) {
            if (s >= q_len) break;
            float mine = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned ke = kv[t][e];
                    p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ke), qv[s][e], p, false);
                }
                p += __shfl_xor(p, 1);
                p += __shfl_xor(p, 2);
                p += __shfl_xor(p, 4);
                p += __shfl_xor(p, 8);
                if (c == t) mine = p;   // token 4t + g
            }
            if (mytok < tok_end) {
                scores[(row0 + s) * cap + j * kBlk + mytok] = mine;
                if (HIST) {
                    const unsigned key = order_key(mine);
                    if (key > kNegInfKey) atomicAdd(&hf[s * kBins + (key >> 20)], 1u);
                }
            }
        }
    }
    if (HIST) {
        // thread t < 256: first digits 16t .. 16t + 15 of each row, and their sum
        // (the count of top-8-bit value t)
        __syncthreads();
        const int t = threadIdx.x;
        if (t < kCoarseBins)
            for (int s = 0; s < q_len; ++s) {
                uint16_t* h = hist + ((row0 + s) * nchunk + chunk) * kHistU16;
                u16x8 lo, hi;
                unsigned coarse = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned a = hf[s * kBins + 16 * t + e], bb = hf[s * kBins + 16 * t + 8 + e];
                    lo[e] = (unsigned short)a;
                    hi[e] = (unsigned short)bb;
                    coarse += a + bb;
                }
                h[t] = (uint16_t)coarse;
                *(u16x8*)(h + kCoarseBins + 16 * t) = lo;
                *(u16x8*)(h + kCoarseBins + 16 * t + 8) = hi;
            }
    }
}

// Block-wide exclusive scan of one value per thread (NW waves); returns the
// exclusive prefix and writes the total to *total.  `tmp` holds NW ints.
template <int NW = kSelWaves>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    int wsum = 0, all = 0;
    for (int w = 0; w < NW; ++w) {
        const int t = tmp[w];
        if (w < wave) wsum += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return wsum + x - v;
}

// The same for four values per thread in one pass (one round of LDS traffic
// and two barriers): returns the exclusive prefixes, writes the totals.
// `tmp` holds 4 * NW ints.
template <int NW>
__device__ __forceinline__ i32x4 block_exclusive_scan4(i32x4 v, int* tmp, i32x4* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    i32x4 x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int xi = x[i];
            const int y = __shfl_up(xi, o);
            if (lane >= o) x[i] = xi + y;
        }
    }
    if (lane == 63)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmp[4 * wave + i] = x[i];
    __syncthreads();
    i32x4 wsum = {0, 0, 0, 0}, all = {0, 0, 0, 0};
    for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tmp[4 * w + i];
            if (w < wave) wsum[i] += t;
            all[i] += t;
        }
    __syncthreads();
    *total = all;
    return wsum + x - v;
}

// grid (rows), kSelThreads threads.  Thread t owns the contiguous positions
// [t * PER, t * PER + PER) of its row, their keys held in registers, so one
// block scan orders the output by position (rows of up to kChunkedFrom
// positions; longer rows take the chunked selection below).
//
// Radix select over digits of 12, 12 and 8 bits.  The first digit of a key
// is its top 12 bits; keys of non-candidates (<= kNegInfKey) land in digits
// 0..7 only, which are left out of the search, so the first pass adds every
// key without a test.  The keys sharing the chosen first digit (usually a few
// hundred) are then copied to LDS and the other two digits are found from
// that list.
template <int PER>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ seq_lens, int q_len,
                                                             int max_blocks, int topk, int32_t* __restrict__ out_idx,
                                                             float* __restrict__ out_score) {
    static_assert(PER > 0 && PER <= 64, "a thread's keys are held in registers");
    __shared__ unsigned hist[kBins];
    __shared__ unsigned cand[kCandCap];
    __shared__ int scan_tmp[kSelWaves];
    __shared__ unsigned res_sh[3];
    __shared__ int cand_n;

    const int nr = (int)gridDim.x, xcd = blockIdx.x & 7, within = blockIdx.x >> 3;
    const int r = xcd * (nr >> 3) + min(xcd, nr & 7) + within;  // rows dealt as the score kernel deals sequences
    const int b = r / q_len;
    const int tid = threadIdx.x;
    const int64_t cap = (int64_t)kBlk * max_blocks;
    const int n = (int)min((int64_t)max(seq_lens[b], 0), cap);
    const float* s = scores + (int64_t)r * cap;
    const int lo = min(n, tid * PER), hi = min(n, lo + PER);
    const bool mine_any = lo < hi;

    // keys of this thread's positions; 0 (a non-candidate key) past hi
    unsigned keys[PER];
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
        const int p = lo + j;  // a multiple of 4: a load that starts below n stays in the row
        const f32x4 v = p < hi ? *(const f32x4*)(s + p) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) keys[j + e] = p + e < hi ? order_key(v[e]) : 0u;
    }
    // f(position, key) over this thread's positions (those past hi carry key 0)
    auto for_mine = [&](auto f) {
#pragma unroll
        for (int j = 0; j < PER; ++j) f(lo + j, keys[j]);
    };
    // the digit of the `remaining`-th largest key in the histogram: thread t
    // holds the counts of digits dmask - 4t .. dmask - 4t - 3 (largest first);
    // digits below `dmin` are not counted.  Returns the number of counted keys.
    auto find_digit = [&](unsigned dmask, int dmin, int remaining_in) {
        int h[4], h4 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = (int)dmask - 4 * tid - j;
            h[j] = d >= dmin ? (int)hist[d] : 0;
            h4 += h[j];
        }
        int total;
        int acc = block_exclusive_scan(h4, scan_tmp, &total);  // keys with a larger digit
        const int want = remaining_in < 0 ? min(topk, total) : remaining_in;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (acc < want && acc + h[j] >= want) {
                res_sh[0] = dmask - 4u * (unsigned)tid - (unsigned)j;
                res_sh[1] = (unsigned)acc;
                res_sh[2] = (unsigned)h[j];
            }
            acc += h[j];
        }
        __syncthreads();
        return total;
    };

    // ---- first digit (bits 20..31)
    for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    if (mine_any) for_mine([&](int, unsigned k) { atomicAdd(&hist[k >> 20], 1u); });
    __syncthreads();
    const int ncand = find_digit(4095u, (int)(kNegInfKey >> 20) + 1, -1);  // all candidates
    const int kk = min(topk, ncand);
    unsigned prefix = 0, pmask = 0;
    int remaining = kk;
    if (kk > 0) {
        const unsigned d0 = res_sh[0];
        remaining -= (int)res_sh[1];
        const int c0 = (int)res_sh[2];
        prefix = d0 << 20;
        pmask = 0xFFF00000u;
        // the keys with this first digit, in LDS when they fit
        const bool listed = c0 <= kCandCap;
        if (tid == 0) cand_n = 0;
        __syncthreads();
        if (listed && mine_any)
            for_mine([&](int, unsigned k) {
                if ((k >> 20) == d0) cand[atomicAdd(&cand_n, 1)] = k;
            });
        // ---- second (bits 8..19) and third (bits 0..7) digits
#pragma unroll 1
        for (int pass = 1; pass < 3; ++pass) {
            const int shift = pass == 1 ? 8 : 0;
            const unsigned dmask = pass == 1 ? 4095u : 255u;
            for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
            __syncthreads();
            if (listed) {
                for (int i = tid; i < c0; i += kSelThreads) {
                    const unsigned k = cand[i];
                    if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
                }
            } else if (mine_any) {
                for_mine([&](int, unsigned k) {
                    if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
                });
            }
            __syncthreads();
            (void)find_digit(dmask, 0, remaining);
            prefix |= res_sh[0] << shift;
            remaining -= (int)res_sh[1];
            pmask |= dmask << shift;
            __syncthreads();
        }
    }

    int32_t* oi = out_idx + (int64_t)r * topk;
    float* os = out_score ? out_score + (int64_t)r * topk : nullptr;
    if (kk > 0) {
        // every key above the threshold tau, and the need_eq lowest positions of
        // those equal to it, written in position order
        const unsigned tau = prefix;
        const int need_eq = remaining;
        unsigned long long mg = 0, me = 0;  // this thread's keys above / equal to tau
#pragma unroll
        for (int jj = 0; jj < PER; ++jj) {
            mg |= (unsigned long long)(keys[jj] > tau) << jj;
            me |= (unsigned long long)(keys[jj] == tau) << jj;
        }
        const int ngt = __builtin_popcountll(mg), neq = __builtin_popcountll(me);
        int tot;
        const int gt_before = block_exclusive_scan(ngt, scan_tmp, &tot);
        int eq_rank = block_exclusive_scan(neq, scan_tmp, &tot);
        int j = gt_before + min(eq_rank, need_eq);
        // the keys above tau and the lowest of this thread's ties still wanted,
        // one store per set bit (the scores are read back from the row; -0 is
        // reported as +0)
        unsigned long long take = mg;
        for (int c = max(0, min(neq, need_eq - eq_rank)); c > 0; --c) {
            const unsigned long long low = me & (~me + 1ull);
            take |= low;
            me ^= low;
        }
        while (take) {
            const int jj = __builtin_ctzll(take);
            take &= take - 1;
            oi[j] = lo + jj;
            if (os) {
                const float v = s[lo + jj];
                os[j] = v == 0.f ? 0.f : v;
            }
            ++j;
        }
    }
    for (int j = kk + tid; j < topk; j += kSelThreads) {
        oi[j] = -1;
        if (os) os[j] = -INFINITY;
    }
}


// ---- chunked selection: rows of more than kChunkedFrom positions
//
// One workgroup of 256 threads per (row, chunk of kChunk positions), thread t
// owning the 16 contiguous positions kChunk c + 16 t ..; with no atomics
// between workgroups (each kernel reads what the previous one wrote):
//   score_kernel<HIST>  (one workgroup per chunk) the chunk's histogram of the
//                       first 12-bit digit of its candidates' keys (u16
//                       counts) and, from it, of the top 8 bits (16 first
//                       digits each), per query row; with fewer than
//                       kCountingFromWgs (sequence, chunk) workgroups the
//                       plain score kernel and chunk_hist_kernel instead;
//   chunk_thresh_kernel every workgroup of a row sums the row's histograms:
//                       the top 8 bits of the kk-th largest key from the
//                       coarse counts, then its first digit T from the 16
//                       fine counts under them; the keys above T and with
//                       digit T in the chunks before its own, and the
//                       chunk's keys with digit T appended, in position
//                       order, to the row's candidate list;
//   chunk_final_kernel  every workgroup of a row finds the last two digits
//                       of the kk-th largest key from the candidate list
//                       (usually a few hundred keys), counts the list's
//                       entries of the earlier chunks above and equal to it,
//                       and writes its chunk's winners at their slots.
// The winners and their order are those of select_kernel.


// (row, chunk) of this workgroup: items r * nch_max + c dealt XCD by XCD, as
// the score kernel deals a sequence's items, so a row's chunks and scores
// share an L2
__device__ __forceinline__ void chunk_item(int nch_max, int& r, int& c) {
    const int nitems = (int)gridDim.x, xcd = blockIdx.x & 7, within = blockIdx.x >> 3;
    const int item = xcd * (nitems >> 3) + min(xcd, nitems & 7) + within;
    r = item / nch_max;
    c = item - r * nch_max;
}

// this thread's 16 keys of chunk c of a row with n positions (0, a
// non-candidate key, past n)
__device__ __forceinline__ void chunk_keys(const float* s, int c, int n, unsigned (&k)[kChPer]) {
    const int p0 = c * kChunk + kChPer * (int)threadIdx.x;
#pragma unroll
    for (int j = 0; j < kChPer; j += 4) {
        const int p = p0 + j;  // a multiple of 4: a load that starts below n stays in the row
        const f32x4 v = p < n ? *(const f32x4*)(s + p) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ve = v[e];
            k[j + e] = p + e < n ? order_key(ve) : 0u;
        }
    }
}

// positions of row r (its sequence's length, at most cap)
__device__ __forceinline__ int row_positions(const int32_t* seq_lens, int r, int q_len, int64_t cap) {
    return (int)min((int64_t)max(seq_lens[r / q_len], 0), cap);
}

// sum of a histogram entry (at h, stride kHistU16) over the chunks [0, nch),
// and over [0, c): the loads are issued 16 at a time before they are used
__device__ __forceinline__ void sum_chunks(const uint16_t* h, int nch, int c, int& all, int& before) {
    for (int c0 = 0; c0 < nch; c0 += 16) {
        int v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = h[(int64_t)min(c0 + j, nch - 1) * kHistU16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int x = c0 + j < nch ? v[j] : 0;
            all += x;
            before += c0 + j < c ? x : 0;
        }
    }
}

// The chunk histograms when the score kernel does not count them (fewer
// (sequence, chunk) workgroups than kCountingFromWgs): one workgroup per
// (row, chunk) reads the chunk's scores back.
__global__ __launch_bounds__(kChThreads) void chunk_hist_kernel(const float* __restrict__ scores,
                                                                const int32_t* __restrict__ seq_lens, int q_len,
                                                                int max_blocks, int nch_max,
                                                                uint16_t* __restrict__ hist) {
    __shared__ unsigned hf[kBins];
    int r, c;
    chunk_item(nch_max, r, c);
    const int64_t cap = (int64_t)kBlk * max_blocks;
    const int n = row_positions(seq_lens, r, q_len, cap);
    if (c * kChunk >= n) return;  // no such chunk: nothing reads its histogram
    const int tid = threadIdx.x;
    unsigned k[kChPer];
    chunk_keys(scores + (int64_t)r * cap, c, n, k);
    for (int i = tid; i < kBins; i += kChThreads) hf[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kChPer; ++j)
        if (k[j] > kNegInfKey) atomicAdd(&hf[k[j] >> 20], 1u);
    __syncthreads();
    // thread t: first digits 16t .. 16t + 15, whose sum is the count of top-8-bit value t
    uint16_t* h = hist + ((int64_t)r * nch_max + c) * kHistU16;
    u16x8 lo, hi;
    unsigned coarse = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const unsigned a = hf[16 * tid + e], b = hf[16 * tid + 8 + e];
        lo[e] = (unsigned short)a;
        hi[e] = (unsigned short)b;
        coarse += a + b;
    }
    h[tid] = (uint16_t)coarse;
    *(u16x8*)(h + kCoarseBins + 16 * tid) = lo;
    *(u16x8*)(h + kCoarseBins + 16 * tid + 8) = hi;
}

__global__ __launch_bounds__(kChThreads) void chunk_thresh_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ seq_lens, int q_len,
                                                                  int max_blocks, int nch_max, int topk,
                                                                  const uint16_t* __restrict__ hist,
                                                                  int* __restrict__ cinfo, int* __restrict__ header,
                                                                  unsigned* __restrict__ cand) {
    __shared__ int scan_tmp[4 * kChWaves];
    __shared__ int sh[5];
    __shared__ int sh_fb[64];
    int r, c;
    chunk_item(nch_max, r, c);
    const int64_t cap = (int64_t)kBlk * max_blocks;
    const int n = row_positions(seq_lens, r, q_len, cap);
    const int nch = (n + kChunk - 1) / kChunk;
    if (c >= max(nch, 1)) return;  // chunk 0 writes the row's header even for an empty row
    const int tid = threadIdx.x;
    unsigned k[kChPer];
    if (c < nch) chunk_keys(scores + (int64_t)r * cap, c, n, k);
    const uint16_t* hr = hist + (int64_t)r * nch_max * kHistU16;

    // coarse counts over the row, largest top-8-bit value first (thread t: value
    // 255 - t), and over the chunks before this one; loads issued 16 at a time
    const int cb = kCoarseBins - 1 - tid;
    int tot = 0, before_cb = 0;
    sum_chunks(hr + cb, nch, c, tot, before_cb);
    int ncand;
    const int above = block_exclusive_scan<kChWaves>(tot, scan_tmp, &ncand);
    const int kk = min(topk, ncand);
    if (kk == 0) {
        if (c == 0 && tid == 0) {
            header[4 * r + 0] = 0;
            header[4 * r + 1] = 0;
            header[4 * r + 2] = 0;
            header[4 * r + 3] = 0;
        }
        return;
    }
    if (above < kk && above + tot >= kk) {
        sh[0] = cb;
        sh[1] = above;
    }
    __syncthreads();
    const int ct = sh[0], above_c = sh[1];
    // the 16 first digits under it (lane t < 16: digit 16 ct + 15 - t), in the first wave
    if (tid < 64) {
        const int fd = 16 * ct + 15 - (tid & 15);
        int ft = 0, fb = 0;
        if (tid < 16) sum_chunks(hr + kCoarseBins + fd, nch, c, ft, fb);
        sh_fb[tid] = fb;
        int x = ft;  // inclusive prefix over lanes 0..15
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int y = __shfl_up(x, o);
            if ((tid & 15) >= o) x += y;
        }
        const int want = kk - above_c, acc = x - ft;
        if (tid < 16 && acc < want && acc + ft >= want) {
            sh[2] = fd;
            sh[3] = above_c + acc;
            sh[4] = ft;
        }
    }
    __syncthreads();
    const int T = sh[2], gt_total = sh[3];
    if (c == 0 && tid == 0) {
        header[4 * r + 0] = T;
        header[4 * r + 1] = gt_total;
        header[4 * r + 2] = sh[4];
        header[4 * r + 3] = kk;
    }
    if (c >= nch) return;

    // keys above T and keys with digit T in the chunks before this one
    int gtb = cb > ct ? before_cb : 0, cbe = 0;
    if (tid < 16) {
        const int fd = 16 * ct + 15 - tid;
        if (fd > T) gtb += sh_fb[tid];
        if (fd == T) cbe = sh_fb[tid];
    }
    i32x4 tot4;
    (void)block_exclusive_scan4<kChWaves>(i32x4{gtb, cbe, 0, 0}, scan_tmp, &tot4);
    const int gt_before = tot4[0], cand_before = tot4[1];

    // this chunk's keys with digit T, appended in position order
    int nt = 0;
#pragma unroll
    for (int j = 0; j < kChPer; ++j) nt += (k[j] >> 20) == (unsigned)T;
    int dummy;
    int o = cand_before + block_exclusive_scan<kChWaves>(nt, scan_tmp, &dummy);
    unsigned* cr = cand + (int64_t)r * cap;
#pragma unroll
    for (int j = 0; j < kChPer; ++j)
        if ((k[j] >> 20) == (unsigned)T && o < n) cr[o++] = k[j];  // (o < n always holds)
    if (tid == 0) {
        cinfo[4 * ((int64_t)r * nch_max + c) + 0] = gt_before;
        cinfo[4 * ((int64_t)r * nch_max + c) + 1] = cand_before;
    }
}

__global__ __launch_bounds__(kChThreads) void chunk_final_kernel(const float* __restrict__ scores,
                                                                 const int32_t* __restrict__ seq_lens, int q_len,
                                                                 int max_blocks, int nch_max, int topk,
                                                                 const int* __restrict__ cinfo,
                                                                 const int* __restrict__ header,
                                                                 const unsigned* __restrict__ cand,
                                                                 int32_t* __restrict__ out_idx,
                                                                 float* __restrict__ out_score) {
    __shared__ unsigned hist[kBins];
    __shared__ int scan_tmp[4 * kChWaves];
    __shared__ unsigned res_sh[2];
    int r, c;
    chunk_item(nch_max, r, c);
    const int64_t cap = (int64_t)kBlk * max_blocks;
    const int n = row_positions(seq_lens, r, q_len, cap);
    const int nch = (n + kChunk - 1) / kChunk;
    if (c >= max(nch, 1)) return;
    const int tid = threadIdx.x;
    // the chunk's keys, the row's header, the chunk's counts and the first
    // kCandRegs * 256 entries of the row's candidate list (entry tid + 256 j in
    // cv[j]; the list is usually a few hundred entries long, and a row has more
    // than 16,384 positions, so these reads stay in its list), all issued first
    unsigned k[kChPer];
    if (c < nch) chunk_keys(scores + (int64_t)r * cap, c, n, k);
    const unsigned* cr = cand + (int64_t)r * cap;
    constexpr int kCandRegs = 4;
    static_assert(kCandRegs * kChThreads <= kChunkedFrom, "the speculative list reads stay in the row");
    unsigned cv[kCandRegs];
#pragma unroll
    for (int j = 0; j < kCandRegs; ++j) cv[j] = cr[tid + kChThreads * j];
    const int T = header[4 * r + 0], gt_total = header[4 * r + 1], M = header[4 * r + 2], kk = header[4 * r + 3];
    const int gtb = c < nch ? cinfo[4 * ((int64_t)r * nch_max + c) + 0] : 0;
    const int cbe = c < nch ? cinfo[4 * ((int64_t)r * nch_max + c) + 1] : 0;
    int32_t* oi = out_idx + (int64_t)r * topk;
    float* os = out_score ? out_score + (int64_t)r * topk : nullptr;
    if (c == 0)
        for (int j = kk + tid; j < topk; j += kChThreads) {
            oi[j] = -1;
            if (os) os[j] = -INFINITY;
        }
    if (kk == 0 || c >= nch) return;
    // the candidate list from registers when it has at most kCandRegs * 256
    // entries, else read from the workspace in every pass
    const bool in_regs = M <= kCandRegs * kChThreads;
    auto for_cand = [&](int upto, auto f) {
        if (in_regs) {
#pragma unroll
            for (int j = 0; j < kCandRegs; ++j)
                if (tid + kChThreads * j < upto) f(cv[j]);
        } else {
            for (int i = tid; i < upto; i += kChThreads) f(cr[i]);
        }
    };

    // the last two digits (bits 8..19, then 0..7) of the remaining-th largest
    // key among the M keys with first digit T
    int remaining = kk - gt_total;
    unsigned prefix = (unsigned)T << 20, pmask = 0xFFF00000u;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 8 : 0;
        const int nb = pass == 0 ? kBins : 256;
        for (int i = tid; i < nb; i += kChThreads) hist[i] = 0;
        __syncthreads();
        for_cand(M, [&](unsigned key) {
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
        });
        __syncthreads();
        // thread t: digits nb - 1 - per t - j (largest first)
        const int per = nb / kChThreads;
        int h = 0;
        for (int j = 0; j < per; ++j) h += (int)hist[nb - 1 - per * tid - j];
        int total;
        int acc = block_exclusive_scan<kChWaves>(h, scan_tmp, &total);
        if (acc < remaining && acc + h >= remaining)
            for (int j = 0; j < per; ++j) {
                const int hj = (int)hist[nb - 1 - per * tid - j];
                if (acc < remaining && acc + hj >= remaining) {
                    res_sh[0] = (unsigned)(nb - 1 - per * tid - j);
                    res_sh[1] = (unsigned)acc;
                }
                acc += hj;
            }
        __syncthreads();
        prefix |= res_sh[0] << shift;
        remaining -= (int)res_sh[1];
        pmask |= (unsigned)(nb - 1) << shift;
        __syncthreads();
    }
    const unsigned tau = prefix;
    const int need_eq = remaining;

    // the list's keys of the earlier chunks above and equal to tau
    int g = 0, e = 0;
    for_cand(cbe, [&](unsigned key) {
        g += key > tau;
        e += key == tau;
    });
    // this thread's winners: every key above tau, and the lowest positions of
    // those equal to it while the row still wants them (one scan: the list's
    // counts summed, this thread's counts' prefixes)
    unsigned mg = 0, me = 0;
#pragma unroll
    for (int j = 0; j < kChPer; ++j) {
        mg |= (unsigned)(k[j] > tau) << j;
        me |= (unsigned)(k[j] == tau) << j;
    }
    const int ngt = __builtin_popcount(mg), neq = __builtin_popcount(me);
    i32x4 tot4;
    const i32x4 pre = block_exclusive_scan4<kChWaves>(i32x4{g, e, ngt, neq}, scan_tmp, &tot4);
    const int gsum = tot4[0], esum = tot4[1];
    const int gt_pre = pre[2];
    const int eq_rank = esum + pre[3];
    int j = gtb + gsum + gt_pre + min(eq_rank, need_eq);
    unsigned take = mg;
    for (int t = max(0, min(neq, need_eq - eq_rank)); t > 0; --t) {
        const unsigned low = me & (~me + 1u);
        take |= low;
        me ^= low;
    }
    // (a static loop over the 16 keys keeps them in registers; the score is
    // the key's inverse, -0 reported as +0)
    const int p0 = c * kChunk + kChPer * tid;
#pragma unroll
    for (int jj = 0; jj < kChPer; ++jj)
        if (((take >> jj) & 1u) && j < kk) {  // (j < kk always holds)
            oi[j] = p0 + jj;
            if (os) os[j] = key_score(k[jj]);
            ++j;
        }
}


// Byte offsets in the workspace of smla_indexer_topk: the fp32 scores [rows,
// cap], then for rows of more than kChunkedFrom positions the chunk histograms
// (u16 [rows, nch, kHistU16]), the per-chunk counts (int [rows, nch, 4]), the
// row headers (int [rows, 4]) and the candidate lists (u32 [rows, cap]); every
// part starts 16-byte aligned.
struct WsLayout {
    uint64_t hist, cinfo, header, cand, total;
};
WsLayout ws_layout(int64_t rows, int64_t cap) {
    WsLayout w{};
    uint64_t off = (uint64_t)rows * (uint64_t)cap * 4u;
    if (cap > kChunkedFrom) {
        const uint64_t nch = (uint64_t)((cap + kChunk - 1) / kChunk);
        w.hist = off;
        off += (uint64_t)rows * nch * kHistU16 * 2u;
        w.cinfo = off;
        off += (uint64_t)rows * nch * 16u;
        w.header = off;
        off += (uint64_t)rows * 16u;
        w.cand = off;
        off += (uint64_t)rows * (uint64_t)cap * 4u;
    }
    w.total = off;
    return w;
}

}  // namespace
}  // namespace smla_idx

extern "C" smla_status_t smla_indexer_workspace_size(int32_t batch, int32_t q_len, int32_t block_size,
                                                     int32_t max_blocks_per_seq, uint64_t* bytes_out) {
    if (!bytes_out || batch < 0 || q_len < 1 || block_size < 1 || max_blocks_per_seq < 1)
        return SMLA_ERR_INVALID_ARG;
    *bytes_out = smla_idx::ws_layout((int64_t)batch * q_len, (int64_t)block_size * max_blocks_per_seq).total;
    return SMLA_OK;
}

namespace smla_idx {
namespace {

// Shape and pointer checks shared by the two entry points (topk < 0: scores only).
smla_status_t check_args(const void* q_idx, int32_t d_idx, const void* k_cache, int64_t num_kv_blocks,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t batch, int32_t q_len,
                         int32_t block_size, int32_t max_blocks_per_seq) {
    if (batch < 0 || q_len < 1 || max_blocks_per_seq < 1 || num_kv_blocks < 0 || d_idx < 1 || block_size < 1)
        return SMLA_ERR_INVALID_ARG;
    if (d_idx != kDidx || block_size != kBlk || q_len > kMaxQlen) return SMLA_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)batch * q_len;
    const int64_t cap = (int64_t)kBlk * max_blocks_per_seq;
    if (rows > (1 << 24) || cap > (1 << 26) || num_kv_blocks > (int64_t)(INT32_MAX / kBlk))
        return SMLA_ERR_UNSUPPORTED;
    if (rows == 0) return SMLA_OK;
    if (!q_idx || !block_table || !seq_lens) return SMLA_ERR_INVALID_ARG;
    if (num_kv_blocks > 0 && !k_cache) return SMLA_ERR_INVALID_ARG;
    if (((uintptr_t)q_idx & 15) || ((uintptr_t)k_cache & 15) || ((uintptr_t)block_table & 3) ||
        ((uintptr_t)seq_lens & 3))
        return SMLA_ERR_INVALID_ARG;
    return SMLA_OK;
}

// hist != nullptr: the counting variant (one workgroup per chunk of kChunk positions)
smla_status_t launch_scores(const void* q_idx, const void* k_cache, int64_t num_kv_blocks,
                            const int32_t* block_table, const int32_t* seq_lens, int32_t batch, int32_t q_len,
                            int32_t max_blocks_per_seq, float* scores, uint16_t* hist, hipStream_t st) {
    const bool counting = hist != nullptr;
    const int per_wg = counting ? kChunk / kBlk : kScoreWaves * kBlocksPerWave;
    dim3 g1((unsigned)((max_blocks_per_seq + per_wg - 1) / per_wg) * (unsigned)batch);
    dim3 t1(counting ? 64 * kHistWaves : 64 * kScoreWaves);
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, g1, t1, 0, st, (const uint16_t*)q_idx, (const uint8_t*)k_cache, num_kv_blocks,
                           block_table, seq_lens, (int)q_len, (int)max_blocks_per_seq, scores, hist);
    };
    static_assert(kMaxQlen == 4, "the score kernel is instantiated for up to four query rows");
    if (q_len == 1)
        counting ? launch(score_kernel<1, true>) : launch(score_kernel<1, false>);
    else if (q_len == 2)
        counting ? launch(score_kernel<2, true>) : launch(score_kernel<2, false>);
    else
        counting ? launch(score_kernel<4, true>) : launch(score_kernel<4, false>);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

}  // namespace
}  // namespace smla_idx

extern "C" smla_status_t smla_indexer_scores(const void* q_idx, int32_t d_idx, const void* k_cache,
                                             int64_t num_kv_blocks, const int32_t* block_table,
                                             const int32_t* seq_lens, int32_t batch, int32_t q_len,
                                             int32_t block_size, int32_t max_blocks_per_seq, float* scores,
                                             void* stream) {
    using namespace smla_idx;
    smla_status_t st = check_args(q_idx, d_idx, k_cache, num_kv_blocks, block_table, seq_lens, batch, q_len,
                                  block_size, max_blocks_per_seq);
    if (st != SMLA_OK || batch == 0) return st;
    if (!scores || ((uintptr_t)scores & 3)) return SMLA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return launch_scores(q_idx, k_cache, num_kv_blocks, block_table, seq_lens, batch, q_len, max_blocks_per_seq,
                         scores, nullptr, (hipStream_t)stream);
}

extern "C" smla_status_t smla_indexer_topk(const void* q_idx, int32_t d_idx, const void* k_cache,
                                           int64_t num_kv_blocks, const int32_t* block_table,
                                           const int32_t* seq_lens, int32_t batch, int32_t q_len,
                                           int32_t block_size, int32_t max_blocks_per_seq, int32_t topk,
                                           int32_t* out_indices, float* out_scores, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    using namespace smla_idx;
    if (topk < 0) return SMLA_ERR_INVALID_ARG;
    smla_status_t st = check_args(q_idx, d_idx, k_cache, num_kv_blocks, block_table, seq_lens, batch, q_len,
                                  block_size, max_blocks_per_seq);
    if (st != SMLA_OK) return st;
    if (topk > kMaxTopk) return SMLA_ERR_UNSUPPORTED;
    if (batch == 0 || topk == 0) return SMLA_OK;
    if (!out_indices || ((uintptr_t)out_indices & 3) || ((uintptr_t)out_scores & 3)) return SMLA_ERR_INVALID_ARG;
    const int64_t rows = (int64_t)batch * q_len;
    const int64_t cap = (int64_t)kBlk * max_blocks_per_seq;
    const WsLayout wl = ws_layout(rows, cap);
    if (!workspace || workspace_bytes < wl.total) return SMLA_ERR_WORKSPACE_TOO_SMALL;
    if ((uintptr_t)workspace & 15) return SMLA_ERR_INVALID_ARG;
    const int64_t nch = (cap + kChunk - 1) / kChunk;
    if (cap > kChunkedFrom && rows * nch > INT32_MAX) return SMLA_ERR_UNSUPPORTED;

    (void)hipGetLastError();
    hipStream_t hs = (hipStream_t)stream;
    float* scores = (float*)workspace;
    uint8_t* wb = (uint8_t*)workspace;
    const bool chunked = cap > kChunkedFrom;
    const bool counting = chunked && (int64_t)batch * nch >= kCountingFromWgs;
    uint16_t* hist = chunked ? (uint16_t*)(wb + wl.hist) : nullptr;
    st = launch_scores(q_idx, k_cache, num_kv_blocks, block_table, seq_lens, batch, q_len, max_blocks_per_seq,
                       scores, counting ? hist : nullptr, hs);
    if (st != SMLA_OK) return st;
    if (chunked) {
        // long rows: the chunk histograms (counted by the score kernel, or by a
        // kernel of their own), then the threshold digit and candidate lists,
        // then the winners
        int* cinfo = (int*)(wb + wl.cinfo);
        int* header = (int*)(wb + wl.header);
        unsigned* cand = (unsigned*)(wb + wl.cand);
        const dim3 g((unsigned)(rows * nch)), t(kChThreads);
        if (!counting)
            hipLaunchKernelGGL(chunk_hist_kernel, g, t, 0, hs, scores, seq_lens, (int)q_len,
                               (int)max_blocks_per_seq, (int)nch, hist);
        hipLaunchKernelGGL(chunk_thresh_kernel, g, t, 0, hs, scores, seq_lens, (int)q_len, (int)max_blocks_per_seq,
                           (int)nch, (int)topk, hist, cinfo, header, cand);
        hipLaunchKernelGGL(chunk_final_kernel, g, t, 0, hs, scores, seq_lens, (int)q_len, (int)max_blocks_per_seq,
                           (int)nch, (int)topk, cinfo, header, cand, out_indices, out_scores);
        return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
    }
    // shorter rows keep their scores in registers, PER of them per thread (the
    // smallest that covers the row)
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, hs, scores, seq_lens, (int)q_len,
                           (int)max_blocks_per_seq, (int)topk, out_indices, out_scores);
    };
    static_assert(kChunkedFrom == 16 * kSelThreads, "select_kernel<16> covers every row up to kChunkedFrom");
    if (cap <= 8 * kSelThreads)
        launch(select_kernel<8>);
    else
        launch(select_kernel<16>);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}
