"""Seeded synthetic inputs for sparse MLA decode (shared by the GPU path and the oracle).

This module only produces input bytes; it holds none of the attention
arithmetic.  Both the GPU library and the CPU oracle receive exactly the bytes
made here.

Workloads have the shape of the pages' decode step -- 64 query heads sharing
one latent KV row per token, a top-k list of selected positions per query
token, a paged cache ("The MMA Sparse-MLA Decode Kernel: A Deep Dive into AI
Inference Optimization on Blackwell GPUs", Agent Reasoning, "Kernel Structure
Analysis" and "Cache Layout Understanding") -- at five sizes from batch 1 to
batch 128.  The latent row is 512 c_kv values followed by 64 rope values.

Recipe (seed 0 unless given; numpy PCG64 streams from ``SeedSequence(seed).spawn``):

* sequence lengths: fixed, or uniform integers in [lo, hi];
* block table: each sequence owns ceil(N_b / 64) physical blocks; physical ids
  are one random permutation over all sequences ("paged"), or the identity
  ("contiguous"); unused table entries are 0;
* indices: per query row, ``choice(N_b, topk, replace=False)`` in generated
  order; when N_b < topk the first N_b entries are a random permutation of
  [0, N_b) and the rest are -1;
* q and KV values: float32 N(0, 1) rounded to bf16 (round to nearest even);
* fp8 cache rows: c_kv quantised per group of 128 values with fp32 scale
  amax/448 to OCP e4m3fn (round to nearest even, via torch), rope in bf16,
  row bytes = [512 e4m3][64 bf16 rope][4 fp32 scales] = 656 bytes;
* the pages' paged layout (kv_format 2, "Cache Layout Understanding"): 448
  nope values per token drawn as N(0, 1) * 2^u with u uniform in {-3..0} per
  group of 64 (so the groups' scales differ), quantised per group with the
  power-of-two scale 2^e, e = ceil(log2(amax / 448)), to OCP e4m3fn (round to
  nearest even), e stored as the UE8M0 byte e + 127; 64 rope values N(0, 1)
  in bf16.  A 64-token block is the 64 token rows [448 e4m3][64 bf16] (576
  bytes each) followed by the 64 scale records [7 UE8M0][1 zero pad byte];
* softmax scale: fp32(1/sqrt(d_qk)) (576, or 512 for kv_format 2).

Large caches are filled only at the rows some index selects ("selected"
fill); the other rows stay zero.  Small caches are filled completely.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

KV_BF16 = 0
KV_FP8 = 1
KV_FP8_NOPE_UE8M0 = 2

# kv_format 2 widths
V4_NOPE = 448
V4_ROPE = 64
V4_GROUP = 64
V4_DATA_BYTES = V4_NOPE + 2 * V4_ROPE   # 576
V4_SCALE_BYTES = 8

FILL_ALL_MAX_BYTES = 256 << 20


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    topk: int
    kv_format: int
    paged: bool
    seq_len: Optional[int] = None          # fixed N per sequence
    seq_len_range: Optional[tuple] = None  # (lo, hi) inclusive, uniform per sequence
    num_heads: int = 64
    d_qk: int = 576
    d_v: int = 512
    block_size: int = 64

    @property
    def rows(self) -> int:
        return self.batch * self.q_len

    @property
    def max_seq_len(self) -> int:
        return self.seq_len if self.seq_len is not None else self.seq_len_range[1]

    @property
    def row_bytes(self) -> int:
        """Bytes per token slot (for kv_format 2: the row plus its scale record)."""
        return kv_row_bytes(self.kv_format, self.d_qk, self.d_v)

    @property
    def block_bytes(self) -> int:
        return self.block_size * self.row_bytes


def kv_row_bytes(kv_format: int, d_qk: int = 576, d_v: int = 512) -> int:
    if kv_format == KV_BF16:
        return 2 * d_qk
    if kv_format == KV_FP8:
        return d_v + 2 * (d_qk - d_v) + 4 * (d_v // 128)
    if kv_format == KV_FP8_NOPE_UE8M0:
        if d_qk != V4_NOPE + V4_ROPE or d_v != d_qk:
            raise ValueError("kv_format 2 has d_qk = d_v = 512")
        return V4_DATA_BYTES + V4_SCALE_BYTES
    raise ValueError(f"unknown kv_format {kv_format}")


WORKLOADS = [
    Workload("b1_topk512_n4096_contiguous_bf16", batch=1, q_len=1, topk=512, kv_format=KV_BF16,
             paged=False, seq_len=4096),
    Workload("b1_topk2048_n32768_paged_bf16", batch=1, q_len=1, topk=2048, kv_format=KV_BF16,
             paged=True, seq_len=32768),
    Workload("b16_topk2048_n65536_paged_bf16", batch=16, q_len=1, topk=2048, kv_format=KV_BF16,
             paged=True, seq_len=65536),
    Workload("b64_topk2048_n1k-128k_paged_bf16", batch=64, q_len=1, topk=2048, kv_format=KV_BF16,
             paged=True, seq_len_range=(1024, 131072)),
    Workload("b128_q2_topk2048_n65536_paged_fp8", batch=128, q_len=2, topk=2048, kv_format=KV_FP8,
             paged=True, seq_len=65536),
    # the pages' own cache layout and decode step: top-512 selection, contexts
    # up to 8192 tokens, batch 1 and the batch-64 serving point
    Workload("b1_topk512_n8192_paged_v4fp8", batch=1, q_len=1, topk=512, kv_format=KV_FP8_NOPE_UE8M0,
             paged=True, seq_len=8192, d_qk=512, d_v=512),
    Workload("b64_topk512_n8192_paged_v4fp8", batch=64, q_len=1, topk=512, kv_format=KV_FP8_NOPE_UE8M0,
             paged=True, seq_len=8192, d_qk=512, d_v=512),
]
WORKLOADS_BY_NAME = {w.name: w for w in WORKLOADS}


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: np.ndarray             # uint16 [B, q_len, H, d_qk] bf16 bits
    kv_cache: np.ndarray      # uint8 [num_blocks, block_size, row_bytes]; kv_format 2: [num_blocks, block_bytes]
    block_table: np.ndarray   # int32 [B, max_blocks]
    indices: np.ndarray       # int32 [B, q_len, topk]
    seq_lens: np.ndarray      # int32 [B]
    softmax_scale: float
    fill: str                 # "all" or "selected"
    filled_rows: np.ndarray   # int64 physical rows holding generated values
    extra_indices: list       # further index sets over the same cache (benchmark rotation)

    @property
    def num_kv_blocks(self) -> int:
        return int(self.kv_cache.shape[0])

    def valid_count(self, indices: Optional[np.ndarray] = None, seq_lens: Optional[np.ndarray] = None) -> int:
        """Number of index entries that select a token (the gathered-token count).

        `indices` [b, q_len, topk] and `seq_lens` [b] may be a subset of the sequences."""
        idx = self.indices if indices is None else indices
        sl = self.seq_lens if seq_lens is None else seq_lens
        cap = np.minimum(sl.astype(np.int64), self.workload.block_size * self.block_table.shape[1])
        return int(((idx >= 0) & (idx < cap[:, None, None])).sum())


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def _e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.clip(x, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def encode_rows(w: Workload, values: np.ndarray) -> np.ndarray:
    """Cache bytes uint8 [n, row_bytes] of float32 latent rows [n, d_qk] in the workload's format.

    For kv_format 2 a returned row is the token's 576-byte row followed by its
    8-byte scale record; the two go to different places of the block."""
    values = np.ascontiguousarray(values, dtype=np.float32)
    n = values.shape[0]
    if w.kv_format == KV_BF16:
        return bf16_bits_rne(values).view(np.uint8).reshape(n, w.row_bytes)
    if w.kv_format == KV_FP8_NOPE_UE8M0:
        groups = values[:, :V4_NOPE].reshape(n, V4_NOPE // V4_GROUP, V4_GROUP)
        amax = np.abs(groups).max(axis=2).astype(np.float64)
        e = np.where(amax > 0, np.ceil(np.log2(np.maximum(amax, 1e-300) / 448.0)), 0.0)
        e = np.clip(e, -126, 127).astype(np.int32)
        codes = _e4m3fn_codes(groups / np.ldexp(1.0, e)[:, :, None].astype(np.float32))
        out = np.zeros((n, w.row_bytes), dtype=np.uint8)
        out[:, :V4_NOPE] = codes.reshape(n, V4_NOPE)
        out[:, V4_NOPE:V4_DATA_BYTES] = bf16_bits_rne(values[:, V4_NOPE:]).view(np.uint8).reshape(n, -1)
        out[:, V4_DATA_BYTES:V4_DATA_BYTES + V4_NOPE // V4_GROUP] = (e + 127).astype(np.uint8)
        return out
    c = values[:, : w.d_v]
    rope = bf16_bits_rne(values[:, w.d_v:])
    groups = c.reshape(n, w.d_v // 128, 128)
    amax = np.abs(groups).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = _e4m3fn_codes(groups / scale[:, :, None]).reshape(n, w.d_v)
    out = np.empty((n, w.row_bytes), dtype=np.uint8)
    out[:, : w.d_v] = codes
    out[:, w.d_v: w.d_v + 2 * (w.d_qk - w.d_v)] = rope.view(np.uint8).reshape(n, -1)
    out[:, w.d_v + 2 * (w.d_qk - w.d_v):] = scale.view(np.uint8).reshape(n, -1)
    return out


def _row_values(w: Workload, rng: np.random.Generator, n: int) -> np.ndarray:
    """Bytes of n token rows, uint8 [n, row_bytes]."""
    if w.kv_format == KV_BF16:
        return encode_rows(w, rng.standard_normal((n, w.d_qk), dtype=np.float32))
    if w.kv_format == KV_FP8_NOPE_UE8M0:
        nope = rng.standard_normal((n, V4_NOPE // V4_GROUP, V4_GROUP), dtype=np.float32)
        u = rng.integers(-3, 1, size=(n, V4_NOPE // V4_GROUP, 1))
        nope = (nope * np.ldexp(1.0, u)).astype(np.float32).reshape(n, V4_NOPE)
        rope = rng.standard_normal((n, V4_ROPE), dtype=np.float32)
        return encode_rows(w, np.concatenate([nope, rope], axis=1))
    c = rng.standard_normal((n, w.d_v), dtype=np.float32)
    rope = rng.standard_normal((n, w.d_qk - w.d_v), dtype=np.float32)
    return encode_rows(w, np.concatenate([c, rope], axis=1))


def _index_set(w: Workload, rng: np.random.Generator, seq_lens: np.ndarray) -> np.ndarray:
    idx = np.full((w.batch, w.q_len, w.topk), -1, dtype=np.int32)
    for b in range(w.batch):
        n_b = int(seq_lens[b])
        for s in range(w.q_len):
            if n_b >= w.topk:
                idx[b, s] = rng.choice(n_b, size=w.topk, replace=False).astype(np.int32)
            else:
                idx[b, s, :n_b] = rng.permutation(n_b).astype(np.int32)
    return idx


def make_inputs(w: Workload, seed: int = 0, fill: Optional[str] = None, index_sets: int = 1) -> Inputs:
    """Inputs for workload ``w``; ``index_sets`` > 1 adds extra index sets over the same cache."""
    streams = [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(6)]
    r_len, r_blk, r_idx, r_q, r_kv, r_extra = streams
    B = w.batch
    if w.seq_len is not None:
        seq_lens = np.full(B, w.seq_len, dtype=np.int32)
    else:
        lo, hi = w.seq_len_range
        seq_lens = r_len.integers(lo, hi + 1, size=B).astype(np.int32)
    bs = w.block_size
    max_blocks = (w.max_seq_len + bs - 1) // bs
    nblk = (seq_lens.astype(np.int64) + bs - 1) // bs
    total_blocks = int(nblk.sum())
    block_table = np.zeros((B, max_blocks), dtype=np.int32)
    phys = r_blk.permutation(total_blocks) if w.paged else np.arange(total_blocks)
    off = 0
    for b in range(B):
        block_table[b, : nblk[b]] = phys[off: off + nblk[b]]
        off += int(nblk[b])

    indices = _index_set(w, r_idx, seq_lens)
    extra = [_index_set(w, r_extra, seq_lens) for _ in range(index_sets - 1)]

    q = bf16_bits_rne(r_q.standard_normal((B, w.q_len, w.num_heads, w.d_qk), dtype=np.float32))

    rb = w.row_bytes
    cache_bytes = total_blocks * bs * rb
    if fill is None:
        fill = "all" if cache_bytes <= FILL_ALL_MAX_BYTES else "selected"
    kv = np.zeros((total_blocks, bs, rb) if w.kv_format != KV_FP8_NOPE_UE8M0 else (total_blocks, bs * rb),
                  dtype=np.uint8)
    if fill == "all":
        rows = np.arange(total_blocks * bs, dtype=np.int64)
    elif fill == "selected":
        sel = []
        for idx in [indices] + extra:
            bb = np.broadcast_to(np.arange(B)[:, None, None], idx.shape)
            ok = idx >= 0
            p = idx[ok].astype(np.int64)
            sel.append(block_table[bb[ok], p // bs].astype(np.int64) * bs + p % bs)
        rows = np.unique(np.concatenate(sel)) if sel else np.zeros(0, np.int64)
    else:
        raise ValueError(f"fill must be 'all' or 'selected', not {fill!r}")
    chunk = 1 << 18
    if w.kv_format == KV_FP8_NOPE_UE8M0:
        data = kv[:, : bs * V4_DATA_BYTES].reshape(total_blocks, bs, V4_DATA_BYTES)
        recs = kv[:, bs * V4_DATA_BYTES:].reshape(total_blocks, bs, V4_SCALE_BYTES)
        for start in range(0, rows.size, chunk):
            part = rows[start: start + chunk]
            vals = _row_values(w, r_kv, part.size)
            data[part // bs, part % bs] = vals[:, :V4_DATA_BYTES]
            recs[part // bs, part % bs] = vals[:, V4_DATA_BYTES:]
    else:
        flat = kv.reshape(-1, rb)
        for start in range(0, rows.size, chunk):
            part = rows[start: start + chunk]
            flat[part] = _row_values(w, r_kv, part.size)

    scale = float(np.float32(1.0 / math.sqrt(w.d_qk)))
    return Inputs(workload=w, q=q, kv_cache=kv, block_table=block_table, indices=indices,
                  seq_lens=seq_lens, softmax_scale=scale, fill=fill, filled_rows=rows,
                  extra_indices=extra)


def small_inputs(batch=2, q_len=1, topk=96, seq_len=256, kv_format=KV_BF16, paged=True, seed=0,
                 num_heads=64, seq_len_range=None) -> Inputs:
    """A small workload of the same structure, for tests that the oracle runs in seconds."""
    fmt_name = {KV_BF16: "bf16", KV_FP8: "fp8", KV_FP8_NOPE_UE8M0: "v4fp8"}[kv_format]
    d_qk = 512 if kv_format == KV_FP8_NOPE_UE8M0 else 576
    w = Workload(f"small_b{batch}_q{q_len}_topk{topk}_n{seq_len}_{fmt_name}",
                 batch=batch, q_len=q_len, topk=topk, kv_format=kv_format, paged=paged,
                 seq_len=None if seq_len_range else seq_len, seq_len_range=seq_len_range,
                 num_heads=num_heads, d_qk=d_qk, d_v=512)
    return make_inputs(w, seed=seed, fill="all")


# ----------------------------------------------------------------- top-k indexer inputs
#
# The indexer scores every position of a sequence with the dot product of the
# row's indexer query and the token's indexer key and keeps the top-k
# positions.  Recipe: seed 0 streams as above; q_idx and the keys are N(0, 1)
# rounded to bf16; keys are paged like the latent cache (64-token blocks, one
# random block permutation over all sequences); the cache is filled completely.

@dataclasses.dataclass(frozen=True)
class IndexerWorkload:
    name: str
    batch: int
    q_len: int
    topk: int
    seq_len: Optional[int] = None
    seq_len_range: Optional[tuple] = None
    d_idx: int = 128
    block_size: int = 64

    @property
    def rows(self) -> int:
        return self.batch * self.q_len

    @property
    def max_seq_len(self) -> int:
        return self.seq_len if self.seq_len is not None else self.seq_len_range[1]


INDEXER_WORKLOADS = [
    # the pages' decode step after the context cap: top-512 over 8192-token contexts at batch 64
    IndexerWorkload("idx_b64_topk512_n8192", batch=64, q_len=1, topk=512, seq_len=8192),
    # the latent-cache workloads' sizes: top-2048 over 65536-token contexts at batch 16
    IndexerWorkload("idx_b16_topk2048_n65536", batch=16, q_len=1, topk=2048, seq_len=65536),
]
INDEXER_WORKLOADS_BY_NAME = {w.name: w for w in INDEXER_WORKLOADS}


@dataclasses.dataclass
class IndexerInputs:
    workload: IndexerWorkload
    q_idx: np.ndarray        # uint16 [B, q_len, d_idx] bf16 bits
    k_cache: np.ndarray      # uint16 [num_blocks, block_size, d_idx] bf16 bits
    block_table: np.ndarray  # int32 [B, max_blocks]
    seq_lens: np.ndarray     # int32 [B]

    def candidate_count(self) -> int:
        return int(np.minimum(self.seq_lens.astype(np.int64),
                              self.workload.block_size * self.block_table.shape[1]).sum())


def make_indexer_inputs(w: IndexerWorkload, seed: int = 0) -> IndexerInputs:
    streams = [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(4)]
    r_len, r_blk, r_q, r_k = streams
    B, bs = w.batch, w.block_size
    if w.seq_len is not None:
        seq_lens = np.full(B, w.seq_len, dtype=np.int32)
    else:
        lo, hi = w.seq_len_range
        seq_lens = r_len.integers(lo, hi + 1, size=B).astype(np.int32)
    max_blocks = (w.max_seq_len + bs - 1) // bs
    nblk = (seq_lens.astype(np.int64) + bs - 1) // bs
    total = int(nblk.sum())
    block_table = np.zeros((B, max_blocks), dtype=np.int32)
    phys = r_blk.permutation(total)
    off = 0
    for b in range(B):
        block_table[b, : nblk[b]] = phys[off: off + nblk[b]]
        off += int(nblk[b])
    q_idx = bf16_bits_rne(r_q.standard_normal((B, w.q_len, w.d_idx), dtype=np.float32))
    k_cache = np.empty((total, bs, w.d_idx), dtype=np.uint16)
    flat = k_cache.reshape(-1, w.d_idx)
    chunk = 1 << 18
    for start in range(0, flat.shape[0], chunk):
        n = min(chunk, flat.shape[0] - start)
        flat[start: start + n] = bf16_bits_rne(r_k.standard_normal((n, w.d_idx), dtype=np.float32))
    return IndexerInputs(workload=w, q_idx=q_idx, k_cache=k_cache, block_table=block_table, seq_lens=seq_lens)


def small_indexer_inputs(batch=2, q_len=1, topk=64, seq_len=300, seed=0, seq_len_range=None,
                         d_idx=128) -> IndexerInputs:
    w = IndexerWorkload(f"small_idx_b{batch}_q{q_len}_topk{topk}_n{seq_len}", batch=batch, q_len=q_len, topk=topk,
                        seq_len=None if seq_len_range else seq_len, seq_len_range=seq_len_range, d_idx=d_idx)
    return make_indexer_inputs(w, seed=seed)
