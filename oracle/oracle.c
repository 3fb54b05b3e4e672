/*
 * oracle.c -- plain fp64 CPU reference for head-batched sparse MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the GPU library; the two meet only at the byte
 * layout of the inputs, which both sides implement separately.
 *
 * What is computed (the plain definition, no blocking, no online softmax):
 *   For every query row r = (b, s) and head h, over the list L of valid
 *   selected token positions of that row,
 *       score_j = scale * sum_{d < d_qk} Q[r,h,d] * K_{L_j}[d]
 *       m       = max_j score_j,   Z = sum_j exp(score_j - m)
 *       lse     = m + ln Z                         (natural log)
 *       out[d]  = sum_j exp(score_j - m) * V_{L_j}[d] / Z,   d < d_v
 *   K is the whole latent row of a token (the c_kv part followed by the rope
 *   part) and V is its first d_v values: the c_kv part for kv_formats 0 and
 *   1 (d_v < d_qk), the whole row, rope included, for kv_format 2
 *   (d_v = d_qk).
 *   Sources:
 *   - "The MMA Sparse-MLA Decode Kernel: A Deep Dive into AI Inference
 *     Optimization on Blackwell GPUs", Agent Reasoning, "Kernel Structure
 *     Analysis": the query carries a non-positional and a rotary part, and
 *     the cached latent rows serve as both keys and values for all heads.
 *   - same page, "Cache Layout Understanding": a paged per-token latent
 *     cache, partly fp8 with per-group scales, partly bf16 rope.
 *   - same page, "Edge Case Handling": tokens past the valid length take no
 *     part in the softmax.
 *   - same page, "Validation Strategy": the kernel's results are the output
 *     and the log-sum-exp per head.
 *   - "The Moment of Truth: Analyzing a Custom MMA Kernel's Performance on
 *     Blackwell GPUs", "The Split-K Solution: Reasoning About the Fix": the
 *     top-k list may be cut into chunks whose partial results are merged by
 *     a combine step (oracle_lse_combine below).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - an index is a logical position in its sequence; the block table maps
 *     position p to physical block table[b][p / block_size], slot
 *     p % block_size;
 *   - an index is invalid (masked) if it is negative, >= seq_lens[b] (when
 *     seq_lens is given), >= block_size * max_blocks_per_seq, or if its
 *     block-table entry is outside [0, num_kv_blocks);
 *   - the list is a multiset: a repeated index counts once per occurrence;
 *   - a row with no valid index yields out = 0 and lse = -inf.
 *
 * Byte layout of the cache (blocks of block_size tokens are contiguous):
 *   kv_format 0 (bf16):  a block is block_size token rows of d_qk bf16
 *                        values, 2*d_qk bytes each.
 *   kv_format 1 (fp8):   a block is block_size token rows of d_v OCP e4m3fn
 *                        bytes (the c_kv part), then (d_qk-d_v) bf16 rope
 *                        values, then d_v/128 fp32 scales; c_kv element d is
 *                        e4m3(byte d) * scale[d/128].
 *   kv_format 2 (the pages' paged layout, "Cache Layout Understanding" and
 *                "Kernel Structure Analysis"): d_qk = d_v = 512.  A token's
 *                latent row is 448 "nope" values stored as OCP e4m3fn bytes
 *                followed by 64 rope values stored as bf16 (576 bytes); the
 *                nope values carry one UE8M0 scale per group of 64 (7 scale
 *                bytes, padded to 8).  A block holds the 576-byte rows of all
 *                its tokens first, then the 8-byte scale records of all its
 *                tokens (584 bytes per token slot).  Element d < 448 of the
 *                row is e4m3(byte d) * ue8m0(scale byte d/64); the values V
 *                are the whole 512-wide row, rope included.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

/* bf16: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits. */
double oracle_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int m = h & 0x7f;
    double v;
    if (e == 0xff)
        v = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)m, -133);            /* m/128 * 2^(1-127) */
    else
        v = ldexp(1.0 + m / 128.0, e - 127);
    return sign ? -v : v;
}

/* OCP fp8 e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN. */
double oracle_e4m3fn_to_f64(uint8_t x)
{
    int sign = (x >> 7) & 1;
    int e = (x >> 3) & 0xf;
    int m = x & 0x7;
    double v;
    if (e == 0xf && m == 0x7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);              /* m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* UE8M0 (the OCP microscaling scale format): 8 exponent bits, no sign, no
 * mantissa; code e is 2^(e-127) and code 255 is NaN. */
double oracle_ue8m0_to_f64(uint8_t e)
{
    return e == 0xff ? NAN : ldexp(1.0, (int)e - 127);
}

/* IEEE binary32 stored little-endian. */
double oracle_f32_le_to_f64(const uint8_t *p)
{
    uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
    int sign = (u >> 31) & 1;
    int e = (u >> 23) & 0xff;
    uint32_t m = u & 0x7fffff;
    double v;
    if (e == 0xff)
        v = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)m, -149);
    else
        v = ldexp(1.0 + m / 8388608.0, e - 127);
    return sign ? -v : v;
}

static uint16_t load_u16_le(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* n little-endian binary32 values (4 bytes each) -> f64. */
void oracle_f32_array_to_f64(int64_t n, const uint8_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_le_to_f64(in + 4 * i);
}

void oracle_bf16_array_to_f64(int64_t n, const uint16_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(in[i]);
}

void oracle_e4m3fn_array_to_f64(int64_t n, const uint8_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3fn_to_f64(in[i]);
}

void oracle_ue8m0_array_to_f64(int64_t n, const uint8_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_ue8m0_to_f64(in[i]);
}

/* kv_format 2: widths of the pages' layout. */
#define V4_NOPE 448          /* e4m3fn values per token */
#define V4_ROPE 64           /* bf16 values per token */
#define V4_GROUP 64          /* nope values per scale */
#define V4_DATA_BYTES (V4_NOPE + 2 * V4_ROPE)   /* 576 */
#define V4_SCALE_BYTES 8     /* 7 scales + 1 pad byte */

/* Bytes per token slot (for kv_format 2: row plus scale record); -1 if the
 * format does not fit the widths. */
int64_t oracle_row_bytes(int32_t kv_format, int32_t d_qk, int32_t d_v)
{
    if (kv_format == 0) return 2 * (int64_t)d_qk;
    if (kv_format == 1) return (int64_t)d_v + 2 * (int64_t)(d_qk - d_v) + 4 * (int64_t)(d_v / 128);
    if (kv_format == 2) return (d_qk == V4_NOPE + V4_ROPE && d_v == d_qk) ? V4_DATA_BYTES + V4_SCALE_BYTES : -1;
    return -1;
}

/* Bytes of one cache block of block_size tokens. */
int64_t oracle_block_bytes(int32_t kv_format, int32_t block_size, int32_t d_qk, int32_t d_v)
{
    int64_t rb = oracle_row_bytes(kv_format, d_qk, d_v);
    return rb < 0 ? -1 : rb * block_size;
}

/* Decode the token in slot `slot` of the block at `block` into K[0..d_qk). */
static void decode_token(int32_t kv_format, int32_t d_qk, int32_t d_v, int32_t block_size, const uint8_t *block,
                         int slot, double *k)
{
    if (kv_format == 0) {
        const uint8_t *row = block + (int64_t)slot * oracle_row_bytes(0, d_qk, d_v);
        for (int d = 0; d < d_qk; ++d) k[d] = oracle_bf16_to_f64(load_u16_le(row + 2 * d));
    } else if (kv_format == 1) {
        const uint8_t *row = block + (int64_t)slot * oracle_row_bytes(1, d_qk, d_v);
        const uint8_t *rope = row + d_v;
        const uint8_t *scales = row + d_v + 2 * (d_qk - d_v);
        for (int d = 0; d < d_v; ++d) k[d] = oracle_e4m3fn_to_f64(row[d]) * oracle_f32_le_to_f64(scales + 4 * (d / 128));
        for (int d = d_v; d < d_qk; ++d) k[d] = oracle_bf16_to_f64(load_u16_le(rope + 2 * (d - d_v)));
    } else {
        const uint8_t *row = block + (int64_t)slot * V4_DATA_BYTES;
        const uint8_t *scales = block + (int64_t)block_size * V4_DATA_BYTES + (int64_t)slot * V4_SCALE_BYTES;
        for (int d = 0; d < V4_NOPE; ++d)
            k[d] = oracle_e4m3fn_to_f64(row[d]) * oracle_ue8m0_to_f64(scales[d / V4_GROUP]);
        for (int d = V4_NOPE; d < d_qk; ++d)
            k[d] = oracle_bf16_to_f64(load_u16_le(row + V4_NOPE + 2 * (d - V4_NOPE)));
    }
}

typedef struct {
    int32_t batch, q_len, num_heads, d_qk, d_v, topk, block_size, max_blocks_per_seq, kv_format;
    int64_t num_kv_blocks;
    const uint16_t *q;
    const uint8_t *kv_cache;
    const int32_t *block_table;
    const int32_t *indices;
    const int32_t *seq_lens;
    double scale;
    double *out;
    double *lse;
    int32_t head_parts;   /* each row's heads are cut into this many contiguous ranges */
    int64_t next_item;    /* work item i: row i / head_parts, head range i % head_parts */
    int error;
    pthread_mutex_t lock;
} decode_job;

/* Physical row of logical position p in sequence b, or -1 if p is masked. */
static int64_t physical_row(const decode_job *J, int b, int32_t p)
{
    int64_t cap = (int64_t)J->block_size * J->max_blocks_per_seq;
    if (J->seq_lens && (int64_t)J->seq_lens[b] < cap) cap = J->seq_lens[b];
    if (p < 0 || (int64_t)p >= cap) return -1;
    int32_t blk = J->block_table[(int64_t)b * J->max_blocks_per_seq + p / J->block_size];
    if (blk < 0 || (int64_t)blk >= J->num_kv_blocks) return -1;
    return (int64_t)blk * J->block_size + p % J->block_size;
}

/* Heads [h0, h1) of query row r.  The valid list is decoded once per call and
 * shared by those heads; the arithmetic of a (row, head) pair does not depend
 * on how the heads are grouped. */
static void decode_one_row(decode_job *J, int64_t r, int h0, int h1, double *kbuf, double *score, double *qrow)
{
    const int H = J->num_heads, DQK = J->d_qk, DV = J->d_v;
    const int b = (int)(r / J->q_len);
    const int64_t block_bytes = oracle_block_bytes(J->kv_format, J->block_size, DQK, DV);
    const int32_t *idx = J->indices + r * J->topk;

    /* Valid list L, decoded once and shared by all heads. */
    int n = 0;
    for (int j = 0; j < J->topk; ++j) {
        int64_t pr = physical_row(J, b, idx[j]);
        if (pr < 0) continue;
        decode_token(J->kv_format, DQK, DV, J->block_size, J->kv_cache + (pr / J->block_size) * block_bytes,
                     (int)(pr % J->block_size), kbuf + (int64_t)n * DQK);
        ++n;
    }

    for (int h = h0; h < h1; ++h) {
        double *o = J->out + (r * H + h) * DV;
        const uint16_t *qh = J->q + (r * H + h) * DQK;
        if (n == 0) {
            for (int d = 0; d < DV; ++d) o[d] = 0.0;
            J->lse[r * H + h] = -INFINITY;
            continue;
        }
        for (int d = 0; d < DQK; ++d) qrow[d] = oracle_bf16_to_f64(qh[d]);
        double m = -INFINITY;
        for (int j = 0; j < n; ++j) {
            const double *k = kbuf + (int64_t)j * DQK;
            double acc = 0.0;
            for (int d = 0; d < DQK; ++d) acc += qrow[d] * k[d];
            score[j] = J->scale * acc;
            if (score[j] > m) m = score[j];
        }
        double z = 0.0;
        for (int j = 0; j < n; ++j) {
            score[j] = exp(score[j] - m);      /* now the unnormalised weight */
            z += score[j];
        }
        for (int d = 0; d < DV; ++d) o[d] = 0.0;
        for (int j = 0; j < n; ++j) {
            const double *v = kbuf + (int64_t)j * DQK;  /* V = first d_v of K */
            for (int d = 0; d < DV; ++d) o[d] += score[j] * v[d];
        }
        for (int d = 0; d < DV; ++d) o[d] /= z;
        J->lse[r * H + h] = m + log(z);
    }
}

static void *decode_worker(void *arg)
{
    decode_job *J = (decode_job *)arg;
    double *kbuf = (double *)malloc(sizeof(double) * (size_t)(J->topk > 0 ? J->topk : 1) * J->d_qk);
    double *score = (double *)malloc(sizeof(double) * (size_t)(J->topk > 0 ? J->topk : 1));
    double *qrow = (double *)malloc(sizeof(double) * (size_t)J->d_qk);
    if (!kbuf || !score || !qrow) {
        pthread_mutex_lock(&J->lock);
        J->error = ORACLE_NO_MEMORY;
        pthread_mutex_unlock(&J->lock);
        free(kbuf); free(score); free(qrow);
        return NULL;
    }
    const int64_t items = (int64_t)J->batch * J->q_len * J->head_parts;
    const int per = (J->num_heads + J->head_parts - 1) / J->head_parts;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t i = J->next_item++;
        pthread_mutex_unlock(&J->lock);
        if (i >= items) break;
        const int part = (int)(i % J->head_parts);
        const int h0 = part * per;
        const int h1 = h0 + per < J->num_heads ? h0 + per : J->num_heads;
        if (h0 < h1) decode_one_row(J, i / J->head_parts, h0, h1, kbuf, score, qrow);
    }
    free(kbuf); free(score); free(qrow);
    return NULL;
}

/*
 * q:           bf16 [batch, q_len, num_heads, d_qk]
 * kv_cache:    bytes [num_kv_blocks, block_bytes] (layout above)
 * block_table: int32 [batch, max_blocks_per_seq]
 * indices:     int32 [batch, q_len, topk]
 * seq_lens:    int32 [batch] or NULL
 * out:         f64 [batch, q_len, num_heads, d_v]
 * lse:         f64 [batch, q_len, num_heads]
 * Work items (a query row and a contiguous range of its heads; a row's heads
 * are cut into ranges only when there are fewer rows than threads) are split
 * over num_threads POSIX threads (<= 0 means 1); the arithmetic of a (row,
 * head) pair does not depend on the thread count.
 */
int oracle_sparse_mla_decode(int32_t batch, int32_t q_len, int32_t num_heads, int32_t d_qk, int32_t d_v,
                             int32_t topk, int32_t block_size, int32_t max_blocks_per_seq,
                             int64_t num_kv_blocks, int32_t kv_format,
                             const uint16_t *q, const uint8_t *kv_cache, const int32_t *block_table,
                             const int32_t *indices, const int32_t *seq_lens, double scale,
                             double *out, double *lse, int32_t num_threads)
{
    if (batch < 0 || q_len <= 0 || num_heads <= 0 || d_v <= 0 || d_qk < d_v || topk < 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_kv_blocks < 0)
        return ORACLE_BAD_ARG;
    if (kv_format != 0 && kv_format != 1 && kv_format != 2) return ORACLE_BAD_ARG;
    if (kv_format == 1 && d_v % 128 != 0) return ORACLE_BAD_ARG;
    if (oracle_row_bytes(kv_format, d_qk, d_v) < 0) return ORACLE_BAD_ARG;
    if ((int64_t)batch * q_len == 0) return ORACLE_OK;
    if (!q || !kv_cache || !block_table || !indices || !out || !lse) return ORACLE_BAD_ARG;

    decode_job J;
    memset(&J, 0, sizeof(J));
    J.batch = batch; J.q_len = q_len; J.num_heads = num_heads; J.d_qk = d_qk; J.d_v = d_v;
    J.topk = topk; J.block_size = block_size; J.max_blocks_per_seq = max_blocks_per_seq;
    J.kv_format = kv_format; J.num_kv_blocks = num_kv_blocks;
    J.q = q; J.kv_cache = kv_cache; J.block_table = block_table; J.indices = indices;
    J.seq_lens = seq_lens; J.scale = scale; J.out = out; J.lse = lse;
    J.next_item = 0; J.error = ORACLE_OK;
    pthread_mutex_init(&J.lock, NULL);

    int nt = num_threads <= 0 ? 1 : num_threads;
    if (nt > 256) nt = 256;
    {
        const int64_t rows = (int64_t)batch * q_len;
        int64_t hp = rows >= nt ? 1 : (nt + rows - 1) / rows;
        J.head_parts = (int32_t)(hp > num_heads ? num_heads : hp);
    }
    if (nt == 1) {
        decode_worker(&J);
    } else {
        pthread_t th[256];
        int started = 0;
        for (int i = 0; i < nt; ++i)
            if (pthread_create(&th[i], NULL, decode_worker, &J) == 0) ++started;
        if (started == 0) decode_worker(&J);
        for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    }
    pthread_mutex_destroy(&J.lock);
    return J.error;
}

/*
 * Merge of partial attention results over disjoint parts of one list
 * ("The Split-K Solution: Reasoning About the Fix": partial results over
 * chunks of the top-k dimension are reduced by a combine step; the pages'
 * kernel-design page also names the log-sum-exp as the quantity carried).
 * For each of n (row, head) pairs, given S partial outputs o_i (normalised
 * over part i) and their log-sum-exps lse_i:
 *     M = max_i lse_i;  if M = -inf the result is (0, -inf);
 *     lse = M + ln sum_i exp(lse_i - M);  out = sum_i exp(lse_i - lse) * o_i.
 * part_out: f64 [S, n, d_v]; part_lse: f64 [S, n]; out: f64 [n, d_v]; lse: f64 [n].
 */
int oracle_lse_combine(int32_t num_splits, int64_t n, int32_t d_v, const double *part_out,
                       const double *part_lse, double *out, double *lse)
{
    if (num_splits <= 0 || n < 0 || d_v <= 0) return ORACLE_BAD_ARG;
    if (n == 0) return ORACLE_OK;
    if (!part_out || !part_lse || !out || !lse) return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) {
        double M = -INFINITY;
        for (int s = 0; s < num_splits; ++s) {
            double v = part_lse[(int64_t)s * n + i];
            if (v > M) M = v;
        }
        double *o = out + i * d_v;
        for (int d = 0; d < d_v; ++d) o[d] = 0.0;
        if (M == -INFINITY) {
            lse[i] = -INFINITY;
            continue;
        }
        double z = 0.0;
        for (int s = 0; s < num_splits; ++s) z += exp(part_lse[(int64_t)s * n + i] - M);
        double total = M + log(z);
        for (int s = 0; s < num_splits; ++s) {
            if (part_lse[(int64_t)s * n + i] == -INFINITY) continue;   /* an empty part has zero weight */
            double w = exp(part_lse[(int64_t)s * n + i] - total);
            const double *po = part_out + ((int64_t)s * n + i) * d_v;
            for (int d = 0; d < d_v; ++d) o[d] += w * po[d];
        }
        lse[i] = total;
    }
    return ORACLE_OK;
}

/*
 * Top-k indexer: the step that produces the index lists.
 *
 * Sources: "The Pivot Point: When a 6.3x Kernel Speedup Reveals the Next
 * Bottleneck", Input Knowledge Required (an indexer selects the top ~512
 * cache positions of each decode step; the attention reads only those) and
 * the note on the bf16 indexer product (the top-512 selection is sensitive
 * to the precision of the scores); "The Moment of Truth: Benchmarking a
 * Custom MMA Kernel for DeepSeek-V4-Flash on Blackwell", The Broader
 * Context (the indexer scores every position of the context, each decode
 * step); "The MMA Sparse-MLA Decode Kernel: A Deep Dive ...", Context (the
 * indexer's scores come from a batched matrix product).
 *
 * Reading (the pages give no formula): for query row r = (b, s) the score
 * of position p is the dot product of the row's indexer query and the
 * indexer key of token p, both bf16 vectors of d_idx values, the keys paged
 * with the same block table as the latent cache:
 *     score(r, p) = sum_{d < d_idx} q_idx[r, d] * k_idx[block_table[b][p / bs], p % bs, d]
 * over the candidate positions of sequence b: 0 <= p < min(seq_lens[b],
 * bs * max_blocks_per_seq) whose block-table entry lies in [0, num_kv_blocks).
 * The selection is the min(topk, #candidates) positions of highest score
 * (among equal scores the lower positions first), listed in ascending
 * position order (the pages give no order; the attention that consumes the
 * list does not depend on it); the rest of the row's list is -1.
 */

static double indexer_score(const uint16_t *q, const uint8_t *kcache, int64_t row_bytes, int64_t phys, int32_t d_idx,
                            double *abs_sum)
{
    const uint8_t *k = kcache + phys * row_bytes;
    double acc = 0.0, a = 0.0;
    for (int d = 0; d < d_idx; ++d) {
        double t = oracle_bf16_to_f64(q[d]) * oracle_bf16_to_f64(load_u16_le(k + 2 * d));
        acc += t;
        a += fabs(t);
    }
    if (abs_sum) *abs_sum = a;
    return acc;
}

/* Physical row of position p of sequence b for the indexer, or -1. */
static int64_t indexer_phys(const int32_t *block_table, const int32_t *seq_lens, int32_t b, int32_t block_size,
                            int32_t max_blocks, int64_t num_kv_blocks, int64_t p)
{
    int64_t cap = (int64_t)block_size * max_blocks;
    if ((int64_t)seq_lens[b] < cap) cap = seq_lens[b];
    if (p < 0 || p >= cap) return -1;
    int32_t blk = block_table[(int64_t)b * max_blocks + p / block_size];
    if (blk < 0 || (int64_t)blk >= num_kv_blocks) return -1;
    return (int64_t)blk * block_size + p % block_size;
}

/*
 * Scores of every position p < block_size * max_blocks_per_seq:
 * scores [batch, q_len, cap] fp64 (-inf where p is not a candidate) and
 * abs_sums [batch, q_len, cap] = sum_d |q_d * k_d| (0 where not a candidate;
 * may be NULL).
 * q_idx: bf16 [batch, q_len, d_idx]; k_cache: bf16 [num_kv_blocks, block_size, d_idx].
 */
int oracle_indexer_scores(int32_t batch, int32_t q_len, int32_t d_idx, int32_t block_size,
                          int32_t max_blocks_per_seq, int64_t num_kv_blocks, const uint16_t *q_idx,
                          const uint8_t *k_cache, const int32_t *block_table, const int32_t *seq_lens,
                          double *scores, double *abs_sums)
{
    if (batch < 0 || q_len <= 0 || d_idx <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_kv_blocks < 0)
        return ORACLE_BAD_ARG;
    if ((int64_t)batch * q_len == 0) return ORACLE_OK;
    if (!q_idx || !block_table || !seq_lens || !scores) return ORACLE_BAD_ARG;
    if (num_kv_blocks > 0 && !k_cache) return ORACLE_BAD_ARG;
    const int64_t cap = (int64_t)block_size * max_blocks_per_seq;
    const int64_t row_bytes = 2 * (int64_t)d_idx;
    for (int32_t b = 0; b < batch; ++b) {
        for (int32_t s = 0; s < q_len; ++s) {
            const int64_t r = (int64_t)b * q_len + s;
            for (int64_t p = 0; p < cap; ++p) {
                int64_t phys = indexer_phys(block_table, seq_lens, b, block_size, max_blocks_per_seq, num_kv_blocks, p);
                double a = 0.0;
                scores[r * cap + p] = phys < 0 ? -INFINITY
                                               : indexer_score(q_idx + r * d_idx, k_cache, row_bytes, phys, d_idx, &a);
                if (abs_sums) abs_sums[r * cap + p] = a;
            }
        }
    }
    return ORACLE_OK;
}

/* Does (sa, pa) come before (sb, pb) in the selection order? */
static int ranks_before(double sa, int64_t pa, double sb, int64_t pb)
{
    return sa > sb || (sa == sb && pa < pb);
}

/*
 * The selection: out_idx [batch, q_len, topk] int32 positions in ascending
 * order and out_score [batch, q_len, topk] fp64 (or NULL), -1 / -inf past
 * the candidates.  A plain selection: repeatedly the best candidate not yet
 * taken (O(topk * cap) per row; test sizes only), then the taken positions
 * in ascending order.
 */
int oracle_indexer_topk(int32_t batch, int32_t q_len, int32_t d_idx, int32_t block_size, int32_t max_blocks_per_seq,
                        int64_t num_kv_blocks, const uint16_t *q_idx, const uint8_t *k_cache,
                        const int32_t *block_table, const int32_t *seq_lens, int32_t topk, int32_t *out_idx,
                        double *out_score)
{
    if (topk < 0) return ORACLE_BAD_ARG;
    if ((int64_t)batch * q_len == 0 || topk == 0) return ORACLE_OK;
    if (!out_idx) return ORACLE_BAD_ARG;
    const int64_t cap = (int64_t)block_size * max_blocks_per_seq;
    const int64_t rows = (int64_t)batch * q_len;
    double *sc = (double *)malloc(sizeof(double) * (size_t)(rows * cap));
    unsigned char *taken = (unsigned char *)malloc((size_t)cap);
    if (!sc || !taken) {
        free(sc); free(taken);
        return ORACLE_NO_MEMORY;
    }
    int rc = oracle_indexer_scores(batch, q_len, d_idx, block_size, max_blocks_per_seq, num_kv_blocks, q_idx,
                                   k_cache, block_table, seq_lens, sc, NULL);
    for (int64_t r = 0; rc == ORACLE_OK && r < rows; ++r) {
        const double *s = sc + r * cap;
        memset(taken, 0, (size_t)cap);
        for (int32_t j = 0; j < topk; ++j) {
            int64_t best = -1;
            for (int64_t p = 0; p < cap; ++p) {
                if (taken[p] || s[p] == -INFINITY) continue;
                if (best < 0 || ranks_before(s[p], p, s[best], best)) best = p;
            }
            if (best < 0) break;
            taken[best] = 1;
        }
        int32_t j = 0;
        for (int64_t p = 0; p < cap; ++p) {
            if (!taken[p]) continue;
            out_idx[r * topk + j] = (int32_t)p;
            if (out_score) out_score[r * topk + j] = s[p];
            ++j;
        }
        for (; j < topk; ++j) {
            out_idx[r * topk + j] = -1;
            if (out_score) out_score[r * topk + j] = -INFINITY;
        }
    }
    free(sc);
    free(taken);
    return rc;
}
