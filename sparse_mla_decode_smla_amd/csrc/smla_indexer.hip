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
// Two kernels:
//   score_kernel  streams each sequence's keys once (whole 64-token blocks,
//                 16 KB contiguous) for all q_len rows of the sequence; a
//                 token's 256-byte key is spread over 16 lanes (16 bytes
//                 each, v_dot2_f32_bf16) and summed across them; fp32 scores
//                 go to the workspace [rows, 64 * max_blocks].  This is HBM
//                 streaming, not a contraction worth the matrix cores (one or
//                 two query rows per key).
//   select_kernel one 1024-thread workgroup per row, each thread owning a
//                 contiguous run of positions (held in registers for rows of
//                 up to 65536 positions): an exact radix select of the
//                 topk-th largest score over an order-preserving key (digits
//                 of 12, 12 and 8 bits, LDS histogram of 4096 bins; after the
//                 first digit only the keys in its bin, copied to LDS, take
//                 part), then one block scan that gives every thread its
//                 output slots, so the winners (and the lowest positions of
//                 the threshold's ties) are written in ascending position
//                 order with no sort.
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
constexpr int kRegPer = 64;       // most positions per select thread held in registers
constexpr int kBins = 4096;       // radix histogram bins (12-bit digits)
constexpr int kCandCap = 4096;    // keys sharing the first digit kept in LDS
constexpr unsigned kNegInfKey = 0x007FFFFFu;  // order key of -inf

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// grid (ceil(max_blocks / (kScoreWaves * kBlocksPerWave)), batch), 256 threads.
// QL >= q_len query rows are held in registers: one row needs 76 VGPRs (six
// waves per SIMD), four need 137 (three).
template <int QL>
__global__ __launch_bounds__(64 * kScoreWaves) void score_kernel(const uint16_t* __restrict__ q_idx,
                                                                  const uint8_t* __restrict__ k_cache,
                                                                  int64_t num_kv_blocks,
                                                                  const int32_t* __restrict__ block_table,
                                                                  const int32_t* __restrict__ seq_lens, int q_len,
                                                                  int max_blocks, float* __restrict__ scores) {
    // (sequence, chunk) items dealt XCD by XCD: consecutive workgroup ids go
    // round-robin over the 8 XCDs, XCD x takes the x-th eighth of the items, so
    // a sequence's scores land in the L2 of the XCD whose select workgroups read
    // them (the select kernel deals its rows the same way)
    const int nchunk = (max_blocks + kScoreWaves * kBlocksPerWave - 1) / (kScoreWaves * kBlocksPerWave);
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

#pragma unroll 1
    for (int i = 0; i < kBlocksPerWave; ++i) {
        const int j = (chunk * kBlocksPerWave + i) * kScoreWaves + wave;  // logical block
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
            if (mytok < tok_end) scores[(row0 + s) * cap + j * kBlk + mytok] = mine;
        }
    }
}

// Block-wide exclusive scan of one value per thread (1024 threads); returns
// the exclusive prefix and writes the total to *total.  `tmp` holds kSelWaves ints.
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
    for (int w = 0; w < kSelWaves; ++w) {
        const int t = tmp[w];
        if (w < wave) wsum += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return wsum + x - v;
}

// grid (rows), kSelThreads threads.  Thread t owns the contiguous positions
// [t * per, t * per + per) of its row, so one block scan orders the output by
// position.  PER > 0: per = PER and the row's keys stay in registers (rows of
// up to PER * kSelThreads positions); PER = 0: every pass streams the
// thread's positions from the workspace.
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
    constexpr bool REG = PER > 0;
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
    const int per = REG ? PER : (((n + kSelThreads - 1) / kSelThreads + 3) & ~3);
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    const bool mine_any = lo < hi;

    // keys of this thread's positions; 0 (a non-candidate key) past hi
    unsigned keys[REG ? PER : 1];
    if (REG) {
#pragma unroll
        for (int j = 0; j < PER; j += 4) {
            const int p = lo + j;  // a multiple of 4: a load that starts below n stays in the row
            const f32x4 v = p < hi ? *(const f32x4*)(s + p) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) keys[j + e] = p + e < hi ? order_key(v[e]) : 0u;
        }
    }
    // f(position, key) over this thread's positions (streamed for PER = 0)
    auto for_mine = [&](auto f) {
        if (REG) {
#pragma unroll
            for (int j = 0; j < (REG ? PER : 1); ++j) f(lo + j, keys[j]);
        } else {
            for (int p0 = lo; p0 < hi; p0 += 16) {
                f32x4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int p = p0 + 4 * u;
                    v[u] = p < hi ? *(const f32x4*)(s + p) : f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int p = p0 + 4 * u + e;
                        if (p < hi) f(p, order_key(v[u][e]));
                    }
            }
        }
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
        int ngt = 0, neq = 0;
        unsigned long long mg = 0, me = 0;  // REG: this thread's keys above / equal to tau
        if (REG) {
#pragma unroll
            for (int jj = 0; jj < (REG ? PER : 1); ++jj) {
                mg |= (unsigned long long)(keys[jj] > tau) << jj;
                me |= (unsigned long long)(keys[jj] == tau) << jj;
            }
            ngt = __builtin_popcountll(mg);
            neq = __builtin_popcountll(me);
        } else if (mine_any) {
            for_mine([&](int, unsigned k) {
                ngt += k > tau;
                neq += k == tau;
            });
        }
        int tot;
        const int gt_before = block_exclusive_scan(ngt, scan_tmp, &tot);
        int eq_rank = block_exclusive_scan(neq, scan_tmp, &tot);
        int j = gt_before + min(eq_rank, need_eq);
        if (REG) {
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
        } else if (mine_any) {
            for_mine([&](int p, unsigned k) {
                bool take = k > tau;
                if (k == tau) {
                    take = eq_rank < need_eq;
                    ++eq_rank;
                }
                if (take) {
                    oi[j] = p;
                    if (os) os[j] = key_score(k);
                    ++j;
                }
            });
        }
    }
    for (int j = kk + tid; j < topk; j += kSelThreads) {
        oi[j] = -1;
        if (os) os[j] = -INFINITY;
    }
}

}  // namespace
}  // namespace smla_idx

extern "C" smla_status_t smla_indexer_workspace_size(int32_t batch, int32_t q_len, int32_t block_size,
                                                     int32_t max_blocks_per_seq, uint64_t* bytes_out) {
    if (!bytes_out || batch < 0 || q_len < 1 || block_size < 1 || max_blocks_per_seq < 1)
        return SMLA_ERR_INVALID_ARG;
    *bytes_out = (uint64_t)batch * (uint64_t)q_len * (uint64_t)block_size * (uint64_t)max_blocks_per_seq * 4u;
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

smla_status_t launch_scores(const void* q_idx, const void* k_cache, int64_t num_kv_blocks,
                            const int32_t* block_table, const int32_t* seq_lens, int32_t batch, int32_t q_len,
                            int32_t max_blocks_per_seq, float* scores, hipStream_t st) {
    const int per_wg = kScoreWaves * kBlocksPerWave;
    dim3 g1((unsigned)((max_blocks_per_seq + per_wg - 1) / per_wg) * (unsigned)batch);
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, g1, dim3(64 * kScoreWaves), 0, st, (const uint16_t*)q_idx,
                           (const uint8_t*)k_cache, num_kv_blocks, block_table, seq_lens, (int)q_len,
                           (int)max_blocks_per_seq, scores);
    };
    static_assert(kMaxQlen == 4, "the score kernel is instantiated for up to four query rows");
    if (q_len == 1)
        launch(score_kernel<1>);
    else if (q_len == 2)
        launch(score_kernel<2>);
    else
        launch(score_kernel<4>);
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
                         scores, (hipStream_t)stream);
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
    const uint64_t need = (uint64_t)rows * (uint64_t)kBlk * (uint64_t)max_blocks_per_seq * 4u;
    if (!workspace || workspace_bytes < need) return SMLA_ERR_WORKSPACE_TOO_SMALL;
    if ((uintptr_t)workspace & 15) return SMLA_ERR_INVALID_ARG;

    (void)hipGetLastError();
    hipStream_t hs = (hipStream_t)stream;
    float* scores = (float*)workspace;
    st = launch_scores(q_idx, k_cache, num_kv_blocks, block_table, seq_lens, batch, q_len, max_blocks_per_seq,
                       scores, hs);
    if (st != SMLA_OK) return st;
    // rows of up to kRegPer * kSelThreads positions keep their scores in
    // registers, PER of them per thread (the smallest that covers the row)
    const int64_t cap = (int64_t)kBlk * max_blocks_per_seq;
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, hs, scores, seq_lens, (int)q_len,
                           (int)max_blocks_per_seq, (int)topk, out_indices, out_scores);
    };
    if (cap <= 8 * kSelThreads)
        launch(select_kernel<8>);
    else if (cap <= 16 * kSelThreads)
        launch(select_kernel<16>);
    else if (cap <= 32 * kSelThreads)
        launch(select_kernel<32>);
    else if (cap <= (int64_t)kRegPer * kSelThreads)
        launch(select_kernel<kRegPer>);
    else
        launch(select_kernel<0>);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}
