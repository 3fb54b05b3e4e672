/*
 * smla.h -- head-batched sparse Multi-head Latent Attention decode for AMD
 * Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (per query row r = (b, s) and head h):
 *   L      = the valid entries of indices[b, s, :] (logical token positions);
 *   K_p    = the latent row of token p: c_kv (d_v values) followed by k_rope
 *            (d_qk - d_v values); V_p = its c_kv part;
 *   score  = softmax_scale * Q[r, h, :] . K_p           for p in L;
 *   out    = sum_p softmax(score)_p * V_p,  lse = ln sum_p exp(score_p).
 * Each selected latent row is read from the cache once and shared by all
 * heads; the top-k list is cut into num_splits parts computed by separate
 * workgroups, whose partial (out, lse) pairs are merged by a log-sum-exp
 * combine kernel.
 *
 * Sources (page title, then section):
 *   - "The MMA Sparse-MLA Decode Kernel: A Deep Dive into AI Inference
 *     Optimization on Blackwell GPUs", Agent Reasoning: "Kernel Structure
 *     Analysis" (query parts, latent rows as keys and values), "Cache Layout
 *     Understanding" (paged per-token latent cache, fp8 part with per-group
 *     scales, bf16 rope part), "Design Decisions" 1 (one program serves a
 *     group of heads with one KV load), 3 (split-K over top-k with a combine
 *     kernel), 6 (fp32 accumulation, bf16 only at the store), "Edge Case
 *     Handling" (tokens past the valid length are excluded), "Validation
 *     Strategy" (results are the output and the log-sum-exp).
 *   - "The Moment of Truth: Analyzing a Custom MMA Kernel's Performance on
 *     Blackwell GPUs": "The Occupancy Problem: A Deeper Dive" (a grid of
 *     batch x head-groups starves the GPU at small batch) and "The Split-K
 *     Solution: Reasoning About the Fix" (split count fixed per batch
 *     bucket so the launch is graph-safe; deterministic scratch size).
 *
 * Conventions:
 *   - Every buffer is owned by the caller.  The library allocates no device
 *     memory and keeps no mutable global state (the CU count of each device
 *     is cached), except the fixed scratch array of smla_decode_run_noalloc,
 *     part of the library's device image.  Pointers are device pointers
 *     unless marked "host".
 *   - smla_decode_run and smla_combine are asynchronous on `stream` (a
 *     hipStream_t; NULL = the null stream): no host synchronisation, no
 *     allocation, a launch geometry that depends only on the plan.
 *   - Errors are returned as smla_status_t; nothing throws or aborts.  Host
 *     checks cover null pointers, sizes and the workspace size.  Bad index
 *     values on the device are not errors: they are masked (see
 *     smla_decode_run).
 *   - All tensors are dense row-major with the shapes given.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SMLA_OK = 0,
    SMLA_ERR_INVALID_ARG = 1,          /* null pointer, negative or inconsistent size */
    SMLA_ERR_UNSUPPORTED = 2,          /* a shape this library does not implement */
    SMLA_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < plan->workspace_bytes */
    SMLA_ERR_LAUNCH = 4,               /* the HIP runtime rejected a launch */
    SMLA_ERR_DEVICE = 5                /* the HIP runtime failed a device query */
} smla_status_t;

typedef enum {
    /* bf16 latent rows: d_qk bf16 values (c_kv then k_rope), 2*d_qk bytes. */
    SMLA_KV_BF16 = 0,
    /* fp8 latent rows: d_v OCP e4m3fn bytes (c_kv), then (d_qk-d_v) bf16
     * k_rope values, then d_v/128 little-endian fp32 scales; c_kv element d
     * is e4m3(byte d) * scale[d/128].  656 bytes for d_qk=576, d_v=512. */
    SMLA_KV_FP8_E4M3_SCALE128 = 1,
    /* The paged layout of "The MMA Sparse-MLA Decode Kernel: A Deep Dive into
     * AI Inference Optimization on Blackwell GPUs" (Agent Reasoning, "Cache
     * Layout Understanding", "Kernel Structure Analysis"): d_qk = d_v = 512.
     * A token's row is 448 "nope" values as OCP e4m3fn bytes, then 64 rope
     * values as bf16 (576 bytes); a block of 64 tokens is its 64 rows, then
     * 64 scale records of 8 bytes: 7 UE8M0 exponents (scale 2^(e-127) of nope
     * values 64g .. 64g+63) and a pad byte; 37376 bytes per block (584 per
     * token).  K = V = the whole 512-wide row: the output carries the rope
     * part too.  Supported scale codes: 1..254. */
    SMLA_KV_FP8_NOPE_UE8M0 = 2
} smla_kv_format_t;

/* Cache policy of the partial-attention kernel's memory traffic.  "Streaming"
 * marks the accesses non-temporal (the nt bit of gfx950 loads and stores: no
 * reuse expected, so the caches keep other data).  Rows: the gathered latent
 * rows; out: the per-part results (or the output with one part), which the
 * combine kernel of smla_decode_run then reads with non-temporal loads.  The
 * arithmetic, and so every result, is the same under every policy.
 * SMLA_CACHE_AUTO lets the plan choose from the problem shape: streaming rows
 * when the call writes at least 4 MiB of results or may gather at least 64 MiB;
 * streaming the output too when it writes at least 4 MiB with one part (with
 * several parts the combine kernel reads them from the cache); else cached
 * (thresholds set by measurement on MI355X). */
typedef enum {
    SMLA_CACHE_AUTO = 0,
    SMLA_CACHE_CACHED = 1,          /* rows and outputs through the caches as ordinary accesses */
    SMLA_CACHE_STREAM_ROWS = 2,     /* streaming row gathers, cached outputs */
    SMLA_CACHE_STREAM_OUT = 3,      /* cached row gathers, streaming outputs */
    SMLA_CACHE_STREAM_BOTH = 4      /* streaming row gathers and outputs */
} smla_cache_policy_t;

/* Problem description (host).  Supported: num_heads = 64, d_v = 512,
 * block_size = 64, d_qk = 576 (kv_format 0, 1) or 512 (kv_format 2); any
 * batch >= 0, q_len >= 1, topk >= 0. */
typedef struct {
    int32_t batch;               /* B: sequences */
    int32_t q_len;               /* query tokens per sequence, each with its own top-k list */
    int32_t num_heads;           /* H */
    int32_t d_qk;                /* latent row width used by QK^T (c_kv + rope) */
    int32_t d_v;                 /* value width (the c_kv part) */
    int32_t topk;                /* index entries per query row */
    int32_t block_size;          /* tokens per cache block */
    int32_t max_blocks_per_seq;  /* columns of the block table */
    int32_t kv_format;           /* smla_kv_format_t */
    int32_t num_cus;             /* compute units to fill; 0 = query the current device */
    int32_t force_splits;        /* 0 = choose automatically; > 0 = use this split count (clamped to the tile count) */
    int32_t cache_policy;        /* smla_cache_policy_t: 0 = choose automatically */
} smla_problem_t;

/* Plan: a pure function of the problem (identical problems give identical
 * plans), so a captured launch sequence stays valid for its batch bucket. */
typedef struct {
    smla_problem_t prob;
    int32_t rows;                /* batch * q_len */
    int32_t num_splits;          /* S: parts of the top-k list */
    int32_t tokens_per_split;    /* tokens per part (a multiple of tile_tokens, except through clamping) */
    int32_t tile_tokens;         /* tokens per gathered tile */
    int32_t heads_per_group;     /* heads served by one workgroup */
    int32_t num_workgroups;      /* workgroups of the partial-attention kernel */
    uint64_t workspace_bytes;    /* bytes of device workspace smla_decode_run needs (0 if S = 1):
                                    S * rows * H * (2 * d_v + 4) */
    int32_t cache_policy;        /* the policy in force (never SMLA_CACHE_AUTO) */
    int32_t reserved;            /* 0 */
} smla_plan_t;

/*
 * Fill *plan_out for *prob: the split count S, the part length, the
 * workspace size and the cache policy, a pure function of the problem shape
 * and the CU count, so
 * that a launch captured for a batch bucket stays valid ("The Moment of
 * Truth: Analyzing a Custom MMA Kernel's Performance on Blackwell GPUs",
 * "The Split-K Solution: Reasoning About the Fix": split count and scratch
 * size fixed per batch bucket; "The Occupancy Problem: A Deeper Dive": one
 * program per row leaves most of the GPU idle at small batch).  Host only;
 * touches the device only when prob->num_cus == 0 (to read the current
 * device's CU count).
 * Returns SMLA_ERR_INVALID_ARG for null pointers, negative sizes or a
 * cache_policy outside smla_cache_policy_t,
 * SMLA_ERR_UNSUPPORTED for shapes outside the supported set,
 * SMLA_ERR_DEVICE if the CU count cannot be read.
 */
smla_status_t smla_decode_plan(const smla_problem_t *prob, smla_plan_t *plan_out);

/*
 * Sparse MLA decode ("The MMA Sparse-MLA Decode Kernel: A Deep Dive into AI
 * Inference Optimization on Blackwell GPUs", Agent Reasoning: "Kernel
 * Structure Analysis" for the operation, "Design Decisions" 1 and 3 for the
 * head batching and the split over the top-k list, "Edge Case Handling" for
 * the masking; "Validation Strategy": the results are out and lse).
 * Shapes (R = batch * q_len, H = num_heads):
 *   q            bf16  [batch, q_len, H, d_qk]
 *   kv_cache     bytes [num_kv_blocks, block bytes of kv_format]
 *   block_table  int32 [batch, max_blocks_per_seq]: physical block of each
 *                logical block of a sequence
 *   indices      int32 [batch, q_len, topk]: logical token positions; -1 pads
 *                (may be NULL when topk == 0)
 *   seq_lens     int32 [batch] or NULL
 *   out          bf16  [batch, q_len, H, d_v]   (fp32 accumulation, rounded to nearest even)
 *   lse          fp32  [batch, q_len, H]        natural-log log-sum-exp of the scaled scores
 *   workspace    >= plan->workspace_bytes bytes, 256-byte aligned (may be NULL if 0)
 * q, kv_cache and out must be 16-byte aligned, lse, block_table, indices and
 * seq_lens 4-byte aligned (else SMLA_ERR_INVALID_ARG).
 * An index entry p of sequence b is masked (takes no part) when p < 0,
 * p >= block_size * max_blocks_per_seq, p >= seq_lens[b] (if given), or its
 * block-table entry lies outside [0, num_kv_blocks).  A row with no valid
 * entry gets out = 0 and lse = -inf.  Repeated entries count once each.
 * Returns SMLA_OK after enqueueing the kernels on `stream`.
 */
smla_status_t smla_decode_run(const smla_plan_t *plan, const void *q, const void *kv_cache,
                              int64_t num_kv_blocks, const int32_t *block_table, const int32_t *indices,
                              const int32_t *seq_lens, float softmax_scale, void *out, float *lse,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * smla_decode_run for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as smla_decode_run,
 * without workspace: the split partial results go into a scratch array of
 * SMLA_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * per device, for the life of the process.  Plans whose workspace_bytes
 * exceed SMLA_NOALLOC_SCRATCH_BYTES are rejected with
 * SMLA_ERR_WORKSPACE_TOO_SMALL (use smla_decode_run with a workspace then).
 * The first call on a device looks up that device's array (SMLA_ERR_DEVICE
 * if the lookup fails).  Nothing in the array needs clearing: every call
 * writes all the partial results it reads.  All calls on one device share
 * its array, so calls that overlap in time on one device (other streams,
 * other threads) race and may return wrong results; calls ordered on one
 * stream are safe.  Allocates nothing; asynchronous on `stream`.
 */
#define SMLA_NOALLOC_SCRATCH_BYTES (16u << 20)
smla_status_t smla_decode_run_noalloc(const smla_plan_t *plan, const void *q, const void *kv_cache,
                                      int64_t num_kv_blocks, const int32_t *block_table, const int32_t *indices,
                                      const int32_t *seq_lens, float softmax_scale, void *out, float *lse,
                                      void *stream);

/*
 * The first half of smla_decode_run: the partial-attention kernel alone, with
 * the same arguments and checks.  With plan->num_splits == 1 it writes the
 * final out and lse (the whole decode).  Otherwise it leaves the per-part
 * results in the workspace, for smla_combine (or an exchange between devices
 * first: parts computed on different devices over disjoint index lists merge
 * the same way; "The Moment of Truth: Analyzing a Custom MMA Kernel's
 * Performance on Blackwell GPUs", "The Split-K Solution: Reasoning About the
 * Fix"), laid out as
 *   part_out = (uint16_t *)workspace                bf16 [S, R, H, d_v]
 *   part_lse = (float *)(part_out + S * R * H * d_v) fp32 [S, R, H]
 * with S = plan->num_splits; out and lse are then not written.  An empty
 * part has part_lse = -inf and part_out = 0.  The partial outputs are
 * rounded to bf16 (fp32 accumulation, one rounding more than the final
 * output; the combine adds them in fp32): half the bytes of fp32 partials.
 */
smla_status_t smla_decode_partial(const smla_plan_t *plan, const void *q, const void *kv_cache,
                                  int64_t num_kv_blocks, const int32_t *block_table, const int32_t *indices,
                                  const int32_t *seq_lens, float softmax_scale, void *out, float *lse,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Log-sum-exp merge of partial attention results over disjoint parts of a
 * list ("The Moment of Truth: Analyzing a Custom MMA Kernel's Performance
 * on Blackwell GPUs", "The Split-K Solution: Reasoning About the Fix").
 *   part_out  bf16 [num_splits, rows, num_heads, d_v]: per-part normalised outputs
 *   part_lse  fp32 [num_splits, rows, num_heads]: per-part lse, -inf for an empty part
 *   out       bf16 [rows, num_heads, d_v];  lse fp32 [rows, num_heads]
 * out = sum_i exp(lse_i - lse) * part_out_i with lse = ln sum_i exp(lse_i), in fp32;
 * parts with lse_i = -inf carry no weight and their part_out values are
 * ignored (even NaN); if every part is empty, out = 0 and lse = -inf.
 * Supported: d_v = 512 (else SMLA_ERR_UNSUPPORTED), num_splits >= 1,
 * rows * num_heads < 2^31; part_out and out 16-byte aligned (else
 * SMLA_ERR_INVALID_ARG).  Asynchronous on `stream`; allocates nothing.
 */
smla_status_t smla_combine(const void *part_out, const float *part_lse, int32_t num_splits, int32_t rows,
                           int32_t num_heads, int32_t d_v, void *out, float *lse, void *stream);

/*
 * Top-k indexer: the step that produces the index lists ("The Pivot Point:
 * When a 6.3x Kernel Speedup Reveals the Next Bottleneck", Input Knowledge
 * Required: an indexer selects the top ~512 cache positions of each decode
 * step; "The Moment of Truth: Benchmarking a Custom MMA Kernel for
 * DeepSeek-V4-Flash on Blackwell", The Broader Context: it scores every
 * position of the context; "The MMA Sparse-MLA Decode Kernel: A Deep Dive
 * into AI Inference Optimization on Blackwell GPUs", Context: a batched
 * product of the indexer query with the indexer keys).
 *   q_idx        bf16  [batch, q_len, d_idx]
 *   k_cache      bf16  [num_kv_blocks, block_size, d_idx]: indexer keys, paged
 *                with the same block table as the latent cache
 *   block_table  int32 [batch, max_blocks_per_seq];  seq_lens int32 [batch] (required)
 *   out_indices  int32 [batch, q_len, topk]: logical positions, ready to be
 *                the `indices` of smla_decode_run
 *   out_scores   fp32  [batch, q_len, topk] or NULL
 *   workspace    >= smla_indexer_workspace_size(...) bytes, 16-byte aligned:
 *                fp32 scores [batch * q_len, block_size * max_blocks_per_seq]
 *                first; for rows of more than 16,384 positions it also holds
 *                the selection's per-chunk histograms, counts and candidate
 *                lists (about 2.5x the scores in all)
 * For row (b, s) the candidates are the positions p < min(seq_lens[b],
 * block_size * max_blocks_per_seq) whose block-table entry lies in
 * [0, num_kv_blocks); score(p) = q_idx[b, s, :] . key(p), bf16 products
 * accumulated in fp32.  The row's list is the min(topk, #candidates)
 * positions of highest score (among equal scores the lower positions), in
 * ascending position order, then -1 (out_scores -inf).  Scores must be
 * finite (finite inputs).
 * Supported: d_idx = 128, block_size = 64, 1 <= q_len <= 4,
 * 0 <= topk <= 2048 (else SMLA_ERR_UNSUPPORTED).  Pointer alignment: q_idx
 * and k_cache 16 bytes, the int32/fp32 arrays 4 bytes (else
 * SMLA_ERR_INVALID_ARG).  Kernels on `stream`: the scores, then the
 * selection (one kernel, or two or three when block_size *
 * max_blocks_per_seq exceeds 16,384); asynchronous; allocates nothing; the
 * launch geometry depends only on the sizes.
 */
smla_status_t smla_indexer_workspace_size(int32_t batch, int32_t q_len, int32_t block_size,
                                          int32_t max_blocks_per_seq, uint64_t *bytes_out);
/* The first half of smla_indexer_topk alone: the scores of every candidate
 * into scores fp32 [batch * q_len, block_size * max_blocks_per_seq] (caller's
 * buffer, 4-byte aligned): position p < min(seq_lens[b], block_size *
 * max_blocks_per_seq) gets its score, or -inf if its block-table entry is out
 * of range; later positions are not written.  Same shape and pointer rules. */
smla_status_t smla_indexer_scores(const void *q_idx, int32_t d_idx, const void *k_cache, int64_t num_kv_blocks,
                                  const int32_t *block_table, const int32_t *seq_lens, int32_t batch, int32_t q_len,
                                  int32_t block_size, int32_t max_blocks_per_seq, float *scores, void *stream);
smla_status_t smla_indexer_topk(const void *q_idx, int32_t d_idx, const void *k_cache, int64_t num_kv_blocks,
                                const int32_t *block_table, const int32_t *seq_lens, int32_t batch, int32_t q_len,
                                int32_t block_size, int32_t max_blocks_per_seq, int32_t topk, int32_t *out_indices,
                                float *out_scores, void *workspace, size_t workspace_bytes, void *stream);

/* Static text for a status code (host). */
const char *smla_status_string(smla_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
