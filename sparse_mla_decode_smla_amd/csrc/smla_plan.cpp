// Host side of the library: the launch plan and status strings.
//
// The split count follows the occupancy argument of "The Moment of Truth:
// Analyzing a Custom MMA Kernel's Performance on Blackwell GPUs" ("The
// Occupancy Problem: A Deeper Dive", "The Split-K Solution: Reasoning About
// the Fix"): one workgroup per (row, head group) leaves most of the GPU idle
// at small batch, so the top-k list of each row is cut into parts until the
// grid covers the compute units, and the choice depends only on the problem
// shape so that a captured launch stays valid for its batch bucket.
#include <hip/hip_runtime.h>

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

}  // namespace

extern "C" smla_status_t smla_decode_plan(const smla_problem_t* prob, smla_plan_t* plan_out) {
    using namespace smla;
    if (!prob || !plan_out) return SMLA_ERR_INVALID_ARG;
    const smla_problem_t& p = *prob;
    if (p.batch < 0 || p.q_len < 1 || p.topk < 0 || p.max_blocks_per_seq < 1 || p.num_cus < 0 ||
        p.force_splits < 0 || p.reserved != 0)
        return SMLA_ERR_INVALID_ARG;
    if (p.num_heads != kHeads || p.d_qk != kDqk || p.d_v != kDv || p.block_size != kBlock)
        return SMLA_ERR_UNSUPPORTED;
    if (p.kv_format != SMLA_KV_BF16 && p.kv_format != SMLA_KV_FP8_E4M3_SCALE128) return SMLA_ERR_UNSUPPORTED;
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
        // Enough parts for about one workgroup per compute unit, never more
        // parts than tiles.
        splits = rows > 0 ? (cus + rows - 1) / rows : 1;
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
        splits > 1 ? (uint64_t)splits * (uint64_t)rows * kHeads * (kDv + 1) * sizeof(float) : 0;
    *plan_out = plan;
    return SMLA_OK;
}

extern "C" const char* smla_status_string(smla_status_t status) {
    switch (status) {
        case SMLA_OK: return "ok";
        case SMLA_ERR_INVALID_ARG: return "invalid argument";
        case SMLA_ERR_UNSUPPORTED: return "unsupported problem shape";
        case SMLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SMLA_ERR_LAUNCH: return "kernel launch failed";
        case SMLA_ERR_DEVICE: return "device query failed";
    }
    return "unknown status";
}
