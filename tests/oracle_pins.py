"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError if
the oracle disagrees with:

* textbook dense attention written with numpy matrix products and an
  independent numpy/torch decoding of the cache bytes (when the top-k list
  covers every token of the sequence);
* invariances of the definition: order of the index list, split of the list
  into parts merged by the log-sum-exp combine, placement of blocks in the
  paged cache, masking by -1 / out-of-range entries;
* closed forms: a single selected token, a zero query, identical rows,
  repeated indices, and the combine's own special cases;
* library conversions (torch) of every bf16, e4m3fn and UE8M0 bit pattern;
* for the top-k indexer: numpy matmul scores over keys decoded here, a numpy
  lexsort selection, a closed form with ties, masking and block placement.

kv_format 2 (the pages' paged layout: per block, the 576-byte token rows,
then the 8-byte scale records) is decoded here with numpy slicing of the
block and torch's float8_e4m3fn / float8_e8m0fnu conversions.

The same battery is run against deliberately broken copies of the oracle
source to show that plausible mistakes are caught.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from sparse_mla_decode_smla_amd import inputs as I

# ----------------------------------------------------------------- helpers


def np_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 via the fp32 upper-half definition."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def np_ue8m0(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e8m0fnu)
    return t.to(torch.float64).numpy()


def token_rows(inp: I.Inputs, b: int, positions: np.ndarray) -> np.ndarray:
    """Decoded latent rows K [n, d_qk] (float64) of logical positions of sequence b."""
    w = inp.workload
    bs, rb = w.block_size, w.row_bytes
    positions = np.asarray(positions, dtype=np.int64)
    if w.kv_format == I.KV_FP8_NOPE_UE8M0:
        nb = inp.kv_cache.shape[0]
        blocks = inp.kv_cache.reshape(nb, -1)
        blk = inp.block_table[b, positions // bs].astype(np.int64)
        slot = positions % bs
        data = blocks[:, : bs * 576].reshape(nb, bs, 576)[blk, slot]       # [n, 576]
        rec = blocks[:, bs * 576:].reshape(nb, bs, 8)[blk, slot]           # [n, 8]
        nope = np_e4m3(data[:, :448]) * np.repeat(np_ue8m0(rec[:, :7]), 64, axis=1)
        rope = np_bf16(np.ascontiguousarray(data[:, 448:]).view(np.uint16))
        return np.concatenate([nope, rope], axis=1)
    flat = inp.kv_cache.reshape(-1, rb)
    phys = inp.block_table[b, positions // bs].astype(np.int64) * bs + positions % bs
    raw = flat[phys]
    if w.kv_format == I.KV_BF16:
        return np_bf16(np.ascontiguousarray(raw).view(np.uint16).reshape(len(positions), w.d_qk))
    dr = w.d_qk - w.d_v
    c = np_e4m3(raw[:, : w.d_v])
    scales = np.ascontiguousarray(raw[:, w.d_v + 2 * dr:]).view(np.float32).astype(np.float64)
    c = c * np.repeat(scales, 128, axis=1)
    rope = np_bf16(np.ascontiguousarray(raw[:, w.d_v: w.d_v + 2 * dr]).view(np.uint16))
    return np.concatenate([c, rope], axis=1)


def dense_attention(inp: I.Inputs, b: int, s: int, positions: np.ndarray):
    """Textbook softmax(Q K^T * scale) V over the given positions (numpy matmuls)."""
    w = inp.workload
    K = token_rows(inp, b, positions)
    Q = np_bf16(inp.q[b, s])                         # [H, d_qk]
    S = (Q @ K.T) * inp.softmax_scale                # [H, n]
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    Z = P.sum(axis=1, keepdims=True)
    out = (P @ K[:, : w.d_v]) / Z
    lse = (m + np.log(Z))[:, 0]
    return out, lse


def assert_close(got, ref, rtol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    scale = max(1.0, float(np.abs(ref).max())) if ref.size else 1.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {scale:.3g}"


def run_rows(orc, inp: I.Inputs, indices: np.ndarray, with_seq_lens=True):
    return orc.decode_inputs(inp, indices=indices, with_seq_lens=with_seq_lens)


# ----------------------------------------------------------------- decode tables


def pin_bf16_table(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all(), "bf16 NaN patterns differ"
    assert np.array_equal(got[~nan], ref[~nan]), "bf16 decode differs from torch"


def pin_e4m3_table(orc):
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    ref = np_e4m3(codes)
    got = orc.e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2, "torch should report exactly two e4m3fn NaN codes"
    assert (np.isnan(got) == nan).all(), "e4m3fn NaN codes differ"
    assert np.array_equal(got[~nan], ref[~nan]), "e4m3fn decode differs from torch"


def pin_ue8m0_table(orc):
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    ref = np_ue8m0(codes)
    got = orc.ue8m0_to_f64(codes)
    assert np.isnan(ref[255]) and np.isnan(ref).sum() == 1, "torch should report code 255 as the only NaN"
    assert np.isnan(got[255]) and not np.isnan(got[:255]).any(), "UE8M0 NaN code differs"
    assert np.array_equal(got[:255], ref[:255]), "UE8M0 decode differs from torch"


# ----------------------------------------------------------------- dense brute force


def _dense_pin(orc, inp: I.Inputs):
    out, lse = orc.decode_inputs(inp)
    w = inp.workload
    for b in range(w.batch):
        n_b = int(inp.seq_lens[b])
        for s in range(w.q_len):
            row = inp.indices[b, s]
            assert sorted(row[row >= 0].tolist()) == list(range(n_b)), "test setup: list must cover the sequence"
            ref_o, ref_l = dense_attention(inp, b, s, np.arange(n_b))
            assert_close(out[b, s], ref_o, 1e-12, f"dense out b{b} s{s}")
            assert_close(lse[b, s], ref_l, 1e-12, f"dense lse b{b} s{s}")


def pin_dense_bf16(orc):
    _dense_pin(orc, I.small_inputs(batch=2, q_len=2, topk=256, seq_len=256, kv_format=I.KV_BF16, seed=1))


def pin_dense_fp8(orc):
    _dense_pin(orc, I.small_inputs(batch=2, q_len=2, topk=256, seq_len=256, kv_format=I.KV_FP8, seed=2))


def pin_dense_v4(orc):
    _dense_pin(orc, I.small_inputs(batch=2, q_len=2, topk=256, seq_len=256, kv_format=I.KV_FP8_NOPE_UE8M0,
                                   seed=15))


def pin_dense_ragged_padded(orc):
    # lengths 60..200 with top-k 200: every list covers its sequence, short ones padded with -1
    _dense_pin(orc, I.small_inputs(batch=4, q_len=1, topk=200, seq_len_range=(60, 200), kv_format=I.KV_BF16,
                                   seed=3))


# ----------------------------------------------------------------- invariances


def pin_permutation(orc):
    inp = I.small_inputs(batch=2, q_len=2, topk=160, seq_len=512, kv_format=I.KV_FP8, seed=4)
    out, lse = orc.decode_inputs(inp)
    rng = np.random.default_rng(40)
    perm_idx = inp.indices.copy()
    for b in range(perm_idx.shape[0]):
        for s in range(perm_idx.shape[1]):
            perm_idx[b, s] = rng.permutation(perm_idx[b, s])
    out2, lse2 = orc.decode_inputs(inp, indices=perm_idx)
    assert_close(out2, out, 1e-12, "permuted out")
    assert_close(lse2, lse, 1e-12, "permuted lse")


def pin_split_combine(orc):
    inp = I.small_inputs(batch=2, q_len=1, topk=150, seq_len=512, kv_format=I.KV_BF16, seed=5)
    out, lse = orc.decode_inputs(inp)
    rng = np.random.default_rng(50)
    topk = inp.indices.shape[2]
    for S in (2, 3, 5):
        cuts = np.sort(rng.integers(0, topk + 1, size=S - 1))
        if S == 5:
            cuts[1] = cuts[0]      # one empty part
        bounds = [0, *cuts.tolist(), topk]
        parts_o, parts_l = [], []
        for a, c in zip(bounds[:-1], bounds[1:]):
            o, l = orc.decode_inputs(inp, indices=np.ascontiguousarray(inp.indices[:, :, a:c]))
            parts_o.append(o)
            parts_l.append(l)
        co, cl = orc.lse_combine(np.stack(parts_o), np.stack(parts_l))
        assert_close(co, out, 1e-12, f"combine of {S} parts, out")
        assert_close(cl, lse, 1e-12, f"combine of {S} parts, lse")


def pin_paging(orc):
    _paging_pin(orc, I.small_inputs(batch=3, q_len=1, topk=100, seq_len=320, kv_format=I.KV_FP8, seed=6))


def pin_paging_v4(orc):
    _paging_pin(orc, I.small_inputs(batch=3, q_len=1, topk=100, seq_len=320, kv_format=I.KV_FP8_NOPE_UE8M0,
                                    seed=16))


def _paging_pin(orc, inp):
    out, lse = orc.decode_inputs(inp)
    w = inp.workload
    bs = w.block_size
    nblk = (inp.seq_lens.astype(np.int64) + bs - 1) // bs
    cache2 = np.zeros_like(inp.kv_cache)
    bt2 = np.zeros_like(inp.block_table)
    off = 0
    for b in range(w.batch):
        for j in range(nblk[b]):
            cache2[off + j] = inp.kv_cache[inp.block_table[b, j]]
            bt2[b, j] = off + j
        off += int(nblk[b])
    out2, lse2 = orc.sparse_mla_decode(inp.q, cache2, bt2, inp.indices, inp.seq_lens, inp.softmax_scale,
                                       d_v=w.d_v, kv_format=w.kv_format, block_size=bs)
    assert np.array_equal(out2, out) and np.array_equal(lse2, lse), "block placement changed the result"


def pin_masking(orc):
    inp = I.small_inputs(batch=2, q_len=2, topk=120, seq_len=300, kv_format=I.KV_BF16, seed=7)
    w = inp.workload
    rng = np.random.default_rng(70)
    cap = w.block_size * inp.block_table.shape[1]
    idx = inp.indices.copy()
    seq_lens = inp.seq_lens.copy()
    seq_lens[1] = 250                                  # positions 250..299 of sequence 1 become invalid
    bt = inp.block_table.copy()
    bt[0, 2] = -5                                      # positions 128..191 of sequence 0: bad block id
    bt[1, 0] = inp.kv_cache.shape[0] + 3               # positions 0..63 of sequence 1: block id past the cache
    for b in range(w.batch):
        for s in range(w.q_len):
            pos = rng.choice(idx.shape[2], size=30, replace=False)
            kinds = rng.integers(0, 3, size=30)
            idx[b, s, pos[kinds == 0]] = -1
            idx[b, s, pos[kinds == 1]] = -7
            idx[b, s, pos[kinds == 2]] = cap + 11
    out, lse = orc.sparse_mla_decode(inp.q, inp.kv_cache, bt, idx, seq_lens, inp.softmax_scale,
                                     d_v=w.d_v, kv_format=w.kv_format, block_size=w.block_size)
    for b in range(w.batch):
        for s in range(w.q_len):
            row = idx[b, s]
            keep = (row >= 0) & (row < min(cap, seq_lens[b]))
            blk_ok = np.zeros_like(keep)
            blk_ok[keep] = [(0 <= bt[b, p // w.block_size] < inp.kv_cache.shape[0]) for p in row[keep]]
            keep &= blk_ok
            sub = np.ascontiguousarray(row[keep][None, None, :])
            o1, l1 = orc.sparse_mla_decode(inp.q[b:b + 1, s:s + 1], inp.kv_cache, bt[b:b + 1], sub,
                                           seq_lens[b:b + 1], inp.softmax_scale, d_v=w.d_v,
                                           kv_format=w.kv_format, block_size=w.block_size)
            assert np.array_equal(out[b, s], o1[0, 0]) and np.array_equal(lse[b, s], l1[0, 0]), \
                f"masked entries changed row ({b}, {s})"


def pin_seq_lens_mask(orc):
    inp = I.small_inputs(batch=2, q_len=1, topk=256, seq_len=256, kv_format=I.KV_FP8, seed=8)
    seq_lens = np.array([256, 100], dtype=np.int32)
    w = inp.workload
    out, lse = orc.sparse_mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.indices, seq_lens,
                                     inp.softmax_scale, d_v=w.d_v, kv_format=w.kv_format,
                                     block_size=w.block_size)
    ref_o, ref_l = dense_attention(inp, 1, 0, np.arange(100))
    assert_close(out[1, 0], ref_o, 1e-12, "seq_lens-limited out")
    assert_close(lse[1, 0], ref_l, 1e-12, "seq_lens-limited lse")


def pin_empty_row(orc):
    inp = I.small_inputs(batch=2, q_len=1, topk=64, seq_len=128, kv_format=I.KV_BF16, seed=9)
    idx = inp.indices.copy()
    idx[1] = -1
    out, lse = orc.decode_inputs(inp, indices=idx)
    assert np.all(out[1] == 0.0), "an empty row must give out = 0"
    assert np.all(lse[1] == -np.inf), "an empty row must give lse = -inf"
    assert np.isfinite(lse[0]).all()


# ----------------------------------------------------------------- closed forms


def pin_single_token(orc):
    inp = I.small_inputs(batch=2, q_len=2, topk=48, seq_len=256, kv_format=I.KV_FP8, seed=10)
    idx = np.full_like(inp.indices, -1)
    rng = np.random.default_rng(100)
    for b in range(2):
        for s in range(2):
            idx[b, s, rng.integers(0, 48)] = rng.integers(0, 256)
    out, lse = orc.decode_inputs(inp, indices=idx)
    w = inp.workload
    for b in range(2):
        for s in range(2):
            p = int(idx[b, s][idx[b, s] >= 0][0])
            K = token_rows(inp, b, np.array([p]))[0]
            assert np.array_equal(out[b, s], np.broadcast_to(K[: w.d_v], out[b, s].shape)), \
                "one token: out must equal its V row exactly"
            ref_l = (np_bf16(inp.q[b, s]) @ K) * inp.softmax_scale
            assert_close(lse[b, s], ref_l, 1e-12, "one token: lse = scaled score")


def pin_single_token_v4(orc):
    inp = I.small_inputs(batch=1, q_len=2, topk=40, seq_len=256, kv_format=I.KV_FP8_NOPE_UE8M0, seed=17)
    idx = np.full_like(inp.indices, -1)
    idx[0, 0, 5] = 200
    idx[0, 1, 39] = 3
    out, lse = orc.decode_inputs(inp, indices=idx)
    for s, p in ((0, 200), (1, 3)):
        K = token_rows(inp, 0, np.array([p]))[0]
        assert np.array_equal(out[0, s], np.broadcast_to(K, out[0, s].shape)), \
            "one token: out must equal its whole row (rope included) exactly"
        assert_close(lse[0, s], (np_bf16(inp.q[0, s]) @ K) * inp.softmax_scale, 1e-12, "one token: lse")


def pin_fp32_scale_table(orc):
    """The oracle's binary32 decoder (the fp8 rows' scales) against numpy's float32 -> float64 widening
    over every exponent field, zero / smallest / random / largest mantissas and both signs: subnormals,
    normals, infinities and NaNs."""
    rng = np.random.default_rng(40)
    words = []
    for e in range(256):
        for m in (0, 1, int(rng.integers(2, 1 << 23)), (1 << 23) - 1):
            for sign in (0, 1):
                words.append((sign << 31) | (e << 23) | m)
    words = np.array(words, dtype=np.uint32)
    got = orc.f32_to_f64(words)
    ref = words.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "binary32 decode differs from numpy's float32 widening"


def pin_fp32_scale_rows(orc):
    """fp8 rows whose four per-128 scales are a subnormal, the smallest normal, 1.0 and a large normal:
    with one selected token per query row, out must be that token's V row exactly as decoded here
    (numpy float32 view of the scale bytes) and lse its scaled score."""
    inp = I.small_inputs(batch=1, q_len=4, topk=1, seq_len=256, kv_format=I.KV_FP8, seed=41)
    w = inp.workload
    scales = np.array([0x00000123, 0x00800000, 0x3F800000, 0x7E967699], dtype=np.uint32)
    flat = inp.kv_cache.reshape(-1, w.row_bytes)
    positions = [7, 64, 130, 255]
    idx = np.full_like(inp.indices, -1)
    for s, p in enumerate(positions):
        phys = int(inp.block_table[0, p // w.block_size]) * w.block_size + p % w.block_size
        words = np.roll(scales, s)                       # each scale value on each 128-group once
        flat[phys, w.row_bytes - 16:] = words.astype("<u4").view(np.uint8)
        idx[0, s, 0] = p
    out, lse = orc.decode_inputs(inp, indices=idx)
    for s, p in enumerate(positions):
        K = token_rows(inp, 0, np.array([p]))[0]
        assert np.array_equal(out[0, s], np.broadcast_to(K[: w.d_v], out[0, s].shape)), \
            "one token with special scales: out must equal its V row exactly"
        ref_l = (np_bf16(inp.q[0, s]) @ K) * inp.softmax_scale
        assert np.allclose(lse[0, s], ref_l, rtol=1e-13, atol=0), "one token with special scales: lse"


def pin_zero_query(orc):
    inp = I.small_inputs(batch=1, q_len=1, topk=77, seq_len=256, kv_format=I.KV_BF16, seed=11)
    q0 = np.zeros_like(inp.q)
    w = inp.workload
    out, lse = orc.sparse_mla_decode(q0, inp.kv_cache, inp.block_table, inp.indices, inp.seq_lens,
                                     inp.softmax_scale, d_v=w.d_v, kv_format=w.kv_format,
                                     block_size=w.block_size)
    K = token_rows(inp, 0, inp.indices[0, 0])
    ref = np.broadcast_to(K[:, : w.d_v].mean(axis=0), out[0, 0].shape)
    assert_close(out[0, 0], ref, 1e-13, "zero query: out = mean of V rows")
    assert_close(lse[0, 0], np.full(w.num_heads, math.log(77)), 1e-14, "zero query: lse = ln n")


def pin_identical_rows(orc):
    inp = I.small_inputs(batch=1, q_len=1, topk=90, seq_len=256, kv_format=I.KV_FP8, seed=12)
    kv = inp.kv_cache.copy()
    kv[:] = kv[0, 0]                                    # every token row identical
    w = inp.workload
    out, lse = orc.sparse_mla_decode(inp.q, kv, inp.block_table, inp.indices, inp.seq_lens,
                                     inp.softmax_scale, d_v=w.d_v, kv_format=w.kv_format,
                                     block_size=w.block_size)
    inp2 = I.Inputs(**{**inp.__dict__, "kv_cache": kv})
    K = token_rows(inp2, 0, np.array([0]))[0]
    assert_close(out[0, 0], np.broadcast_to(K[: w.d_v], out[0, 0].shape), 1e-13, "identical rows: out = V")
    s = (np_bf16(inp.q[0, 0]) @ K) * inp.softmax_scale
    assert_close(lse[0, 0], s + math.log(90), 1e-12, "identical rows: lse = s + ln n")


def pin_identical_rows_v4(orc):
    inp = I.small_inputs(batch=1, q_len=1, topk=70, seq_len=192, kv_format=I.KV_FP8_NOPE_UE8M0, seed=18)
    nb = inp.kv_cache.shape[0]
    kv = inp.kv_cache.copy()
    data = kv[:, : 64 * 576].reshape(nb, 64, 576)
    rec = kv[:, 64 * 576:].reshape(nb, 64, 8)
    data[:] = data[1, 7].copy()                          # every token row and scale record identical
    rec[:] = rec[1, 7].copy()
    w = inp.workload
    out, lse = orc.sparse_mla_decode(inp.q, kv, inp.block_table, inp.indices, inp.seq_lens,
                                     inp.softmax_scale, d_v=w.d_v, kv_format=w.kv_format,
                                     block_size=w.block_size)
    inp2 = I.Inputs(**{**inp.__dict__, "kv_cache": kv})
    K = token_rows(inp2, 0, np.array([0]))[0]
    assert_close(out[0, 0], np.broadcast_to(K, out[0, 0].shape), 1e-13, "identical rows: out = V")
    s = (np_bf16(inp.q[0, 0]) @ K) * inp.softmax_scale
    assert_close(lse[0, 0], s + math.log(70), 1e-12, "identical rows: lse = s + ln n")


def pin_duplicates(orc):
    inp = I.small_inputs(batch=1, q_len=1, topk=3, seq_len=128, kv_format=I.KV_BF16, seed=13)
    idx = np.array([[[17, 17, 90]]], dtype=np.int32)
    out, lse = orc.decode_inputs(inp, indices=idx)
    w = inp.workload
    K = token_rows(inp, 0, np.array([17, 90]))
    sc = (np_bf16(inp.q[0, 0]) @ K.T) * inp.softmax_scale      # [H, 2]
    wts = np.exp(sc) * np.array([2.0, 1.0])
    ref = (wts @ K[:, : w.d_v]) / wts.sum(axis=1, keepdims=True)
    assert_close(out[0, 0], ref, 1e-12, "repeated index counts twice: out")
    assert_close(lse[0, 0], np.log(wts.sum(axis=1)), 1e-12, "repeated index counts twice: lse")


def pin_combine_closed_forms(orc):
    rng = np.random.default_rng(14)
    o = rng.standard_normal((1, 3, 5, 8))
    l = rng.standard_normal((1, 3, 5))
    co, cl = orc.lse_combine(o, l)
    assert np.array_equal(co, o[0]) and np.array_equal(cl, l[0]), "one part: combine is the identity"
    o2 = rng.standard_normal((2, 4, 8))
    l2 = np.stack([np.full(4, 0.7), np.full(4, 0.7)])
    co, cl = orc.lse_combine(o2, l2)
    assert_close(co, (o2[0] + o2[1]) / 2, 1e-15, "equal lse: average")
    assert_close(cl, np.full(4, 0.7 + math.log(2)), 1e-15, "equal lse: lse + ln 2")
    l3 = np.array([[-np.inf, 1.5], [2.0, -np.inf]])
    o3 = rng.standard_normal((2, 2, 8))
    o3[0, 0] = np.nan                                  # an empty part's values carry no weight
    co, cl = orc.lse_combine(o3, l3)
    assert np.array_equal(co[0], o3[1, 0]) and cl[0] == 2.0
    assert np.array_equal(co[1], o3[0, 1]) and cl[1] == 1.5
    co, cl = orc.lse_combine(np.ones((3, 2, 8)), np.full((3, 2), -np.inf))
    assert np.all(co == 0.0) and np.all(cl == -np.inf), "all parts empty: (0, -inf)"


# ----------------------------------------------------------------- top-k indexer


def _np_indexer_scores(inp):
    """Scores [B, q_len, cap] by a numpy matmul over keys decoded here; -inf where not a candidate."""
    w = inp.workload
    bs, mb = w.block_size, inp.block_table.shape[1]
    cap = bs * mb
    K = np_bf16(inp.k_cache)                                  # [blocks, bs, d]
    out = np.full((w.batch, w.q_len, cap), -np.inf)
    for b in range(w.batch):
        n = min(int(inp.seq_lens[b]), cap)
        pos = np.arange(n)
        blk = inp.block_table[b, pos // bs]
        ok = (blk >= 0) & (blk < inp.k_cache.shape[0])
        Kb = K[blk[ok], pos[ok] % bs]                         # [n_ok, d]
        out[b][:, pos[ok]] = np_bf16(inp.q_idx[b]) @ Kb.T
    return out


def _np_topk(scores, k):
    """Positions of the k highest scores (ties: lower position first) in ascending order, -1 past the candidates."""
    B, Q, cap = scores.shape
    idx = np.full((B, Q, k), -1, dtype=np.int64)
    for b in range(B):
        for q in range(Q):
            s = scores[b, q]
            cand = np.nonzero(np.isfinite(s))[0]
            order = cand[np.lexsort((cand, -s[cand]))]      # primary: score descending, then position
            take = np.sort(order[:k])
            idx[b, q, : len(take)] = take
    return idx


def pin_indexer_scores_dense(orc):
    inp = I.small_indexer_inputs(batch=3, q_len=2, topk=40, seq_len_range=(50, 300), seed=20)
    sc, ab = orc.indexer_scores(inp.q_idx, inp.k_cache, inp.block_table, inp.seq_lens)
    ref = _np_indexer_scores(inp)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(sc), fin), "candidate positions differ"
    assert_close(sc[fin], ref[fin], 1e-13, "indexer scores")
    assert np.all(ab[fin] >= np.abs(sc[fin]) - 1e-9) and np.all(ab[~fin] == 0)


def pin_indexer_abs_sums(orc):
    """The indexer's per-score sums of |q_d * k_d| (the bound the GPU score check is scaled by) against a
    numpy matmul of |q| and |k| over keys decoded here; with operands of one sign the sum is |score|."""
    inp = I.small_indexer_inputs(batch=3, q_len=2, topk=40, seq_len_range=(50, 300), seed=26)
    sc, ab = orc.indexer_scores(inp.q_idx, inp.k_cache, inp.block_table, inp.seq_lens)
    w = inp.workload
    bs, mb = w.block_size, inp.block_table.shape[1]
    K = np.abs(np_bf16(inp.k_cache))
    fin = np.isfinite(sc)
    for b in range(w.batch):
        n = min(int(inp.seq_lens[b]), bs * mb)
        pos = np.arange(n)
        blk = inp.block_table[b, pos // bs]
        ref = np.abs(np_bf16(inp.q_idx[b])) @ K[blk, pos % bs].T          # [q_len, n]
        assert_close(ab[b][:, :n][fin[b][:, :n]], ref[fin[b][:, :n]], 1e-13, "indexer abs sums")
    # one sign: q >= 0 and k >= 0 give abs_sum == score; q <= 0 gives abs_sum == -score
    qp = (inp.q_idx & 0x7FFF).astype(np.uint16)
    kp = (inp.k_cache & 0x7FFF).astype(np.uint16)
    sc2, ab2 = orc.indexer_scores(qp, kp, inp.block_table, inp.seq_lens)
    f2 = np.isfinite(sc2)
    assert np.array_equal(ab2[f2], sc2[f2]), "non-negative operands: abs sum must equal the score"
    sc3, ab3 = orc.indexer_scores((qp | 0x8000).astype(np.uint16), kp, inp.block_table, inp.seq_lens)
    assert np.array_equal(ab3[f2], -sc3[f2]), "non-positive query: abs sum must equal -score"


def pin_indexer_topk_matches_sort(orc):
    for seed, k in ((21, 64), (22, 300)):                    # 300 > some sequences: -1 padding
        inp = I.small_indexer_inputs(batch=3, q_len=2, topk=k, seq_len_range=(100, 400), seed=seed)
        idx, sc = orc.indexer_topk(inp.q_idx, inp.k_cache, inp.block_table, inp.seq_lens, k)
        ref_scores = _np_indexer_scores(inp)
        ref = _np_topk(ref_scores, k)
        assert np.array_equal(idx, ref), f"selection differs from a sort of numpy scores (k={k})"
        fin = ref >= 0
        got = np.take_along_axis(ref_scores, np.maximum(ref, 0), axis=2)
        assert_close(sc[fin], got[fin], 1e-13, "selected scores")
        assert np.all(np.isneginf(sc[~fin]))


def pin_indexer_ties_and_closed_form(orc):
    # q = e_0 and key[p][0] = v(p): the scores are the v(p) exactly; repeated values tie
    inp = I.small_indexer_inputs(batch=1, q_len=1, topk=10, seq_len=128, seed=23)
    q = np.zeros_like(inp.q_idx)
    q[0, 0, 0] = 0x3F80                                       # 1.0
    k = np.zeros_like(inp.k_cache)
    vals = np.array([(p * 37) % 11 for p in range(128)], dtype=np.float32)   # 0..10, many ties
    bs = 64
    for p in range(128):
        k[inp.block_table[0, p // bs], p % bs, 0] = I.bf16_bits_rne(vals[p:p + 1])[0]
    idx, sc = orc.indexer_topk(q, k, inp.block_table, inp.seq_lens, 25)
    expect = sorted(sorted(range(128), key=lambda p: (-vals[p], p))[:25])
    assert idx[0, 0].tolist() == expect, "ties must go to the lower position"
    assert np.array_equal(sc[0, 0], vals[expect].astype(np.float64))


def pin_indexer_masking_and_paging(orc):
    inp = I.small_indexer_inputs(batch=2, q_len=1, topk=80, seq_len=256, seed=24)
    bt = inp.block_table.copy()
    sl = inp.seq_lens.copy()
    sl[0] = 150                                               # positions 150.. of sequence 0 excluded
    bt[1, 1] = -3                                             # positions 64..127 of sequence 1 excluded
    bt[1, 3] = inp.k_cache.shape[0] + 2                       # positions 192..255 too
    idx, _ = orc.indexer_topk(inp.q_idx, inp.k_cache, bt, sl, 200)
    assert (idx[0, 0] >= 0).sum() == 150 and idx[0, 0, :150].max() < 150 and np.all(idx[0, 0, 150:] == -1)
    v1 = idx[1, 0][idx[1, 0] >= 0]
    assert len(v1) == 128 and not np.any((v1 >= 64) & (v1 < 128)) and not np.any(v1 >= 192)
    # moving the blocks and their table entries together changes nothing
    nb = inp.k_cache.shape[0]
    perm = np.random.default_rng(25).permutation(nb)
    k2 = np.empty_like(inp.k_cache)
    k2[perm] = inp.k_cache
    bt2 = perm[inp.block_table].astype(np.int32)
    a = orc.indexer_topk(inp.q_idx, inp.k_cache, inp.block_table, inp.seq_lens, 80)
    c = orc.indexer_topk(inp.q_idx, k2, bt2, inp.seq_lens, 80)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1]), "block placement changed the selection"
    e = orc.indexer_topk(inp.q_idx, inp.k_cache, inp.block_table, np.zeros_like(inp.seq_lens), 5)
    assert np.all(e[0] == -1), "no candidates: all -1"


ALL_PINS = [
    pin_bf16_table, pin_e4m3_table, pin_ue8m0_table, pin_dense_bf16, pin_dense_fp8, pin_dense_v4,
    pin_dense_ragged_padded, pin_permutation, pin_split_combine, pin_paging, pin_paging_v4, pin_masking,
    pin_seq_lens_mask, pin_empty_row, pin_single_token, pin_single_token_v4, pin_fp32_scale_table,
    pin_fp32_scale_rows, pin_zero_query,
    pin_identical_rows, pin_identical_rows_v4, pin_duplicates, pin_combine_closed_forms,
    pin_indexer_scores_dense, pin_indexer_abs_sums, pin_indexer_topk_matches_sort, pin_indexer_ties_and_closed_form,
    pin_indexer_masking_and_paging,
]
