// Host side of the library: the launch plan and status strings.
//
// The split count follows the occupancy argument of "The Moment of Truth:
// Analyzing a Custom MMA Kernel's Performance on Blackwell GPUs" ("The
// Occupancy Problem: A Deeper Dive", "The Split-K Solution: Reasoning About
// the Fix"): one workgroup per row leaves most of the GPU idle at small
// batch, so the top-k list of each row is cut into parts; here the count
// minimises a cost model of both kernels (more parts fill more compute units
// but write and re-read more partial results), and it depends only on the
// problem shape so that a captured launch stays valid for its batch bucket.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "smla.h"
#include "smla_internal.h"

namespace {

int query_cu_count(int* out) {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 64 && cached[dev] > 0) {
        *out = cached[dev];
        return 0;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
    if (dev < 64) cached[dev] = n;
    *out = n;
    return 0;
}

// Estimated time (us) of one call with S parts per row, from a model fitted
// to split sweeps of the two kernels on MI355X (256 CUs):
//   - a workgroup gathers its part at about 35 GB/s per CU, and the whole
//     launch at most at about 5 TB/s; a 32-token tile costs about 0.9 us of
//     pipelined compute (bf16 rows), 1.7 us (fp8 rows, widened in registers)
//     or 1.6 us (the pages' layout); every round of workgroups (one per CU)
//     pays about 7.5 us of launch, prologue and epilogue;
//   - with S > 1 every part writes 64 x 512 bf16 outputs (64 KiB) per row at
//     about 5 TB/s; the combine kernel pays about 2.3 us, and a call about
//     1 us more per 3 MB of partial results (their read-back and the wait
//     between the two kernels, as timed on whole calls), but a (row, head)
//     pair's S rows of 1 KiB come in at no more than about 40 GB/s per
//     workgroup, and 0.25 us per round of 16 part loads.
double estimate_us(const smla_problem_t& p, int rows, int tiles, int S, int cus) {
    const double row_bytes = smla::gathered_bytes_per_token(p.kv_format);
    const double t_tile = p.kv_format == SMLA_KV_BF16 ? 0.9 : p.kv_format == SMLA_KV_FP8_E4M3_SCALE128 ? 1.7 : 1.6;
    const int tps = (tiles + S - 1) / S;
    const double wgs = (double)rows * S;
    const double rounds = std::ceil(wgs / cus);
    const double gathered = (double)rows * p.topk * row_bytes;       // upper bound: every entry valid
    const double per_wg = (double)tps * smla::kTile * row_bytes;
    const double t_gather = std::max(per_wg / 35e3 * rounds, gathered / 5e6);  // bytes / (bytes per us)
    const double t_compute = t_tile * tps * rounds;
    const double partial = S > 1 ? wgs * smla::kHeads * smla::kDv * 2.0 : 0.0;
    double t = 7.5 * rounds + std::max(t_gather, t_compute) + partial / 5e6;
    if (S > 1) {
        const double pairs = (double)rows * smla::kHeads;
        const double pair_rounds = std::ceil(pairs / (8.0 * cus));
        t += 2.3 + std::max(partial / 3e6, S * 1024.0 / 40e3 * pair_rounds) + 0.25 * std::ceil(S / 16.0);
    }
    return t;
}

// Streaming (non-temporal) outputs when a call writes 4 MiB or more of
// results, and then streaming row gathers too; streaming row gathers alone
// when it may gather 64 MiB or more.  Measured on MI355X with the benchmark's
// workloads (cold cache, HIP graphs, us per call, cached -> chosen):
// batch 16 bf16 21.7 -> 20.9, batch 64 bf16 41.5 -> 39.1, fp8 batch 128
// 111.7 -> 109.6, pages' layout batch 64 24.1 -> 22.3; the batch-1 calls,
// which write 1 to 2 MB, were as fast or faster with cached accesses.
// Streaming rows with cached outputs made the batch-16 call slower (23.2 us):
// the combine kernel then reads the parts with ordinary loads.
int choose_cache_policy(const smla_problem_t& p, int rows, int splits) {
    const double gathered = (double)rows * p.topk * smla::gathered_bytes_per_token(p.kv_format);
    const double written = (double)rows * splits * smla::kHeads * smla::kDv * 2.0;
    const bool big_out = written >= 4.0 * (1 << 20), big_rows = gathered >= 64.0 * (1 << 20);
    // results streamed too when nothing reads them back (one part); several
    // parts stay cached for the combine kernel, which reads them from the L2
    // of the XCD that wrote them
    if (big_out && splits == 1) return SMLA_CACHE_STREAM_BOTH;
    return big_out || big_rows ? SMLA_CACHE_STREAM_ROWS : SMLA_CACHE_CACHED;
}

int choose_splits(const smla_problem_t& p, int rows, int tiles, int cap_tiles, int cus) {
    if (rows <= 0 || tiles <= 1) return 1;
    const int min_s = (tiles + cap_tiles - 1) / cap_tiles;  // parts small enough for the LDS row table
    int best = min_s;
    double best_t = estimate_us(p, rows, tiles, min_s, cus);
    for (int S = min_s + 1; S <= tiles; ++S) {
        const double t = estimate_us(p, rows, tiles, S, cus);
        if (t < best_t) {
            best_t = t;
            best = S;
        }
    }
    return best;
}

}  // namespace

extern "C" smla_status_t smla_decode_plan(const smla_problem_t* prob, smla_plan_t* plan_out) {
    using namespace smla;
    if (!prob || !plan_out) return SMLA_ERR_INVALID_ARG;
    const smla_problem_t& p = *prob;
    if (p.batch < 0 || p.q_len < 1 || p.topk < 0 || p.max_blocks_per_seq < 1 || p.num_cus < 0 ||
        p.force_splits < 0 || p.cache_policy < SMLA_CACHE_AUTO || p.cache_policy > SMLA_CACHE_STREAM_BOTH)
        return SMLA_ERR_INVALID_ARG;
    if (p.kv_format != SMLA_KV_BF16 && p.kv_format != SMLA_KV_FP8_E4M3_SCALE128 &&
        p.kv_format != SMLA_KV_FP8_NOPE_UE8M0)
        return SMLA_ERR_UNSUPPORTED;
    const int want_dqk = p.kv_format == SMLA_KV_FP8_NOPE_UE8M0 ? kDqkV4 : kDqk;
    if (p.num_heads != kHeads || p.d_qk != want_dqk || p.d_v != kDv || p.block_size != kBlock)
        return SMLA_ERR_UNSUPPORTED;
    const int64_t rows64 = (int64_t)p.batch * p.q_len;
    if (rows64 > (1 << 24)) return SMLA_ERR_UNSUPPORTED;
    if ((int64_t)p.max_blocks_per_seq * kBlock > INT32_MAX) return SMLA_ERR_UNSUPPORTED;

    int cus = p.num_cus;
    if (cus == 0 && query_cu_count(&cus) != 0) return SMLA_ERR_DEVICE;

    const int rows = (int)rows64;
    const int tiles = (p.topk + kTile - 1) / kTile;  // 0 when topk == 0
    const int cap_tiles = max_tokens_per_split(p.kv_format) / kTile;

    int splits;
    if (p.force_splits > 0) {
        splits = p.force_splits;
    } else {
        splits = choose_splits(p, rows, tiles, cap_tiles, cus);
    }
    if (splits > tiles) splits = tiles;
    if (splits < 1) splits = 1;
    int tiles_per_split = tiles > 0 ? (tiles + splits - 1) / splits : 1;
    if (tiles_per_split > cap_tiles) tiles_per_split = cap_tiles;
    if (tiles_per_split < 1) tiles_per_split = 1;
    const int tps = tiles_per_split * kTile;
    splits = p.topk > 0 ? (p.topk + tps - 1) / tps : 1;  // every part non-empty

    smla_plan_t plan;
    std::memset(&plan, 0, sizeof(plan));
    plan.prob = p;
    plan.prob.num_cus = cus;
    plan.rows = rows;
    plan.num_splits = splits;
    plan.tokens_per_split = tps;
    plan.tile_tokens = kTile;
    plan.heads_per_group = kHeads;
    plan.num_workgroups = rows * splits;
    plan.workspace_bytes =
        splits > 1 ? (uint64_t)splits * (uint64_t)rows * kHeads * (kDv * 2 + 4) : 0;
    plan.cache_policy = p.cache_policy != SMLA_CACHE_AUTO ? p.cache_policy : choose_cache_policy(p, rows, splits);
    *plan_out = plan;
    return SMLA_OK;
}

extern "C" const char* smla_status_string(smla_status_t status) {
    // A caller may pass any int through the C ABI; reading the bits as an int keeps a value outside the
    // enumeration well defined here (loading it as the enum type would not be).
    int32_t code;
    static_assert(sizeof(code) == sizeof(status), "status codes are 32-bit");
    std::memcpy(&code, &status, sizeof(code));
    switch (code) {
        case SMLA_OK: return "ok";
        case SMLA_ERR_INVALID_ARG: return "invalid argument";
        case SMLA_ERR_UNSUPPORTED: return "unsupported problem shape";
        case SMLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SMLA_ERR_LAUNCH: return "kernel launch failed";
        case SMLA_ERR_DEVICE: return "device query failed";
    }
    return "unknown status";
}
