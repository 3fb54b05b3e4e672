"""The seeded input generator: determinism, formats and the workload recipe (CPU only)."""
import hashlib

import numpy as np
import torch

from sparse_mla_decode_smla_amd import inputs as I


def _digest(inp):
    h = hashlib.sha256()
    for a in (inp.q, inp.kv_cache, inp.block_table, inp.indices, inp.seq_lens):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    a = I.small_inputs(batch=2, topk=64, seq_len=200, kv_format=I.KV_FP8, seed=5)
    b = I.small_inputs(batch=2, topk=64, seq_len=200, kv_format=I.KV_FP8, seed=5)
    c = I.small_inputs(batch=2, topk=64, seq_len=200, kv_format=I.KV_FP8, seed=6)
    assert _digest(a) == _digest(b)
    assert _digest(a) != _digest(c)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 10
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.bf16_bits_rne(x), ref)


def test_fp8_row_layout():
    inp = I.small_inputs(batch=1, topk=32, seq_len=128, kv_format=I.KV_FP8, seed=1)
    rows = inp.kv_cache.reshape(-1, 656)
    scales = np.ascontiguousarray(rows[:, 640:656]).view(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(rows[:, :512])).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    # each group of 128 was scaled so that its largest magnitude maps to 448
    amax = np.abs(codes.reshape(-1, 4, 128)).max(axis=2)
    assert np.all(amax == 448.0)
    assert np.all(scales > 0)
    assert not np.isnan(codes).any()


def test_workload_recipe():
    w = I.WORKLOADS_BY_NAME["b1_topk2048_n32768_paged_bf16"]
    inp = I.make_inputs(w)
    assert inp.fill == "all" and inp.kv_cache.shape == (512, 64, 1152)
    row = inp.indices[0, 0]
    assert len(np.unique(row)) == 2048 and row.min() >= 0 and row.max() < 32768
    assert sorted(inp.block_table[0].tolist()) == list(range(512))
    assert inp.block_table[0].tolist() != list(range(512)), "paged cache must be shuffled"
    w1 = I.WORKLOADS_BY_NAME["b1_topk512_n4096_contiguous_bf16"]
    inp1 = I.make_inputs(w1)
    assert inp1.block_table[0].tolist() == list(range(64))


def test_padding_for_short_sequences():
    w = I.Workload("short", batch=3, q_len=1, topk=300, kv_format=I.KV_BF16, paged=True,
                   seq_len_range=(100, 500))
    inp = I.make_inputs(w, seed=3)
    for b in range(3):
        n_b = int(inp.seq_lens[b])
        row = inp.indices[b, 0]
        if n_b < 300:
            assert sorted(row[:n_b].tolist()) == list(range(n_b)) and np.all(row[n_b:] == -1)
        else:
            assert row.min() >= 0 and len(np.unique(row)) == 300


def test_selected_fill_covers_every_selected_row():
    w = I.Workload("sel", batch=2, q_len=2, topk=50, kv_format=I.KV_FP8, paged=True, seq_len=4096)
    inp = I.make_inputs(w, seed=2, fill="selected", index_sets=3)
    rows = inp.kv_cache.reshape(-1, w.row_bytes)
    bs = w.block_size
    for idx in [inp.indices] + inp.extra_indices:
        for b in range(2):
            p = idx[b].reshape(-1).astype(np.int64)
            phys = inp.block_table[b, p // bs].astype(np.int64) * bs + p % bs
            assert np.all(rows[phys, 640:656].view(np.float32) > 0), "a selected row was left unfilled"


def test_v4_block_layout_and_quantisation():
    # kv_format 2: per block, 64 rows of [448 e4m3][64 bf16] then 64 records of [7 UE8M0][pad]
    inp = I.small_inputs(batch=2, topk=64, seq_len=256, kv_format=I.KV_FP8_NOPE_UE8M0, seed=3)
    nb = inp.kv_cache.shape[0]
    assert inp.kv_cache.shape == (nb, 64 * 584)
    data = inp.kv_cache[:, : 64 * 576].reshape(-1, 576)
    rec = inp.kv_cache[:, 64 * 576:].reshape(-1, 8)
    assert np.all(rec[:, 7] == 0), "pad byte must be zero"
    e = rec[:, :7].astype(np.int64) - 127
    assert e.min() >= -126 and e.max() <= 127
    assert len(np.unique(e)) >= 3, "group scales should differ"
    codes = torch.from_numpy(np.ascontiguousarray(data[:, :448])).view(torch.float8_e4m3fn).to(torch.float64)
    codes = codes.numpy().reshape(-1, 7, 64)
    assert not np.isnan(codes).any()
    amax = np.abs(codes).max(axis=2)
    # a power-of-two scale leaves each group's largest magnitude in (224, 448]
    assert np.all(amax <= 448.0) and np.all(amax > 224.0 * (1 - 2 ** -4))
    rope = np.ascontiguousarray(data[:, 448:]).view(np.uint16)
    assert rope.shape[1] == 64 and np.isfinite(
        torch.from_numpy(rope.view(np.int16)).view(torch.bfloat16).float().numpy()).all()
    assert abs(inp.softmax_scale - 1 / np.sqrt(512)) < 1e-7


def test_v4_selected_fill():
    w = I.WORKLOADS_BY_NAME["b1_topk512_n8192_paged_v4fp8"]
    inp = I.make_inputs(w, fill="selected")
    bs = w.block_size
    nb = inp.kv_cache.shape[0]
    rec = inp.kv_cache[:, bs * 576:].reshape(nb, bs, 8)
    p = inp.indices[0, 0].astype(np.int64)
    blk = inp.block_table[0, p // bs]
    assert np.all(rec[blk, p % bs, :7] > 0), "a selected token's scale record was left unfilled"


def test_indexer_inputs_recipe():
    w = I.INDEXER_WORKLOADS_BY_NAME["idx_b64_topk512_n8192"]
    a = I.make_indexer_inputs(w)
    assert a.q_idx.shape == (64, 1, 128) and a.k_cache.shape == (64 * 128, 64, 128)
    assert sorted(a.block_table.reshape(-1).tolist()) == list(range(64 * 128)), "paged: one permutation"
    assert a.candidate_count() == 64 * 8192
    b = I.make_indexer_inputs(w)
    assert np.array_equal(a.k_cache[:3], b.k_cache[:3]) and np.array_equal(a.q_idx, b.q_idx)
