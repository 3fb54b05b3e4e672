"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Bar (fp32 accumulation of bf16 inputs): max |out - ref| <= 2e-2 and
max |out - ref| / max |ref| <= 1e-2 over rows with a finite reference lse,
max |lse - ref| <= 1e-3; rows with no valid index must give out = 0 and
lse = -inf exactly.  Index handling is exact by construction (the same
bytes go to both sides).
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import oracle_pins
from sparse_mla_decode_smla_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

OUT_ABS, OUT_REL, LSE_ABS = 2e-2, 1e-2, 1e-3


def B():
    from sparse_mla_decode_smla_amd import binding
    return binding


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(out_gpu, lse_gpu, out_ref, lse_ref, what):
    o = out_gpu.float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse_ref)
    assert np.all(lg[~fin] == -np.inf), f"{what}: empty rows must give lse = -inf"
    assert np.all(o[~fin] == 0.0), f"{what}: empty rows must give out = 0"
    if not fin.any():
        return
    err = float(np.abs(o[fin] - out_ref[fin]).max())
    ref_max = float(np.abs(out_ref[fin]).max())
    lerr = float(np.abs(lg[fin] - lse_ref[fin]).max())
    note(f"  {what}: out abs err {err:.3e} (rel {err / ref_max:.3e}), lse abs err {lerr:.3e}")
    assert err <= OUT_ABS and err <= OUT_REL * ref_max, f"{what}: out err {err:.3e}, max|ref| {ref_max:.3e}"
    assert lerr <= LSE_ABS, f"{what}: lse err {lerr:.3e}"


def run_gpu(inp, indices=None, force_splits=0, with_seq_lens=True, block_table=None, cache_policy=0):
    w = inp.workload
    q, kv, bt, idx, sl = B().to_device(inp, indices=indices)
    if block_table is not None:
        bt = torch.from_numpy(block_table).cuda()
    out, lse = B().sparse_mla_decode(q, kv, bt, idx, sl if with_seq_lens else None, inp.softmax_scale,
                                     kv_format=w.kv_format, force_splits=force_splits, cache_policy=cache_policy)
    torch.cuda.synchronize()
    return out, lse


FORMATS = [I.KV_BF16, I.KV_FP8, I.KV_FP8_NOPE_UE8M0]
FMT_IDS = ["bf16", "fp8", "v4fp8"]


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("splits", [1, 3])
def test_cache_policies_give_identical_results(fmt, splits):
    """The cache policy changes only the cache hints of the row loads and result stores: every policy
    gives the same bits, and those match the oracle."""
    inp = I.small_inputs(batch=3, q_len=1, topk=300, seq_len=900, kv_format=fmt, seed=150 + fmt)
    runs = [run_gpu(inp, force_splits=splits, cache_policy=pol) for pol in (1, 2, 3, 4)]
    for out, lse in runs[1:]:
        assert torch.equal(out, runs[0][0]) and torch.equal(lse, runs[0][1])
    ref_o, ref_l = oracle.decode_inputs(inp, threads=8)
    check(runs[0][0], runs[0][1], ref_o, ref_l, f"fmt{fmt} S={splits} policies")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("splits", [0, 1, 2, 7])
def test_small_parity(fmt, splits):
    # top-k 200 = 6 full tiles of 32 + a ragged tail of 8; q_len 2; paged, shuffled blocks
    inp = I.small_inputs(batch=3, q_len=2, topk=200, seq_len=700, kv_format=fmt, seed=11 + fmt)
    note(f"small parity fmt={fmt} splits={splits}")
    ref_o, ref_l = oracle.decode_inputs(inp, threads=8)
    out, lse = run_gpu(inp, force_splits=splits)
    check(out, lse, ref_o, ref_l, f"fmt{fmt} S{splits}")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("topk,seq_len", [(100, 600), (700, 1500)], ids=["topk100", "topk700"])
def test_masking_edge_cases(fmt, topk, seq_len):
    # top-k 700 in one part: 704 row-table entries, translated four per lane at a time
    # (the last round ragged), with the same masked entries as the short lists
    inp = I.small_inputs(batch=4, q_len=2, topk=topk, seq_len=seq_len, kv_format=fmt, seed=21 + fmt + topk)
    w = inp.workload
    rng = np.random.default_rng(5)
    idx = inp.indices.copy()
    cap = 64 * inp.block_table.shape[1]
    # row (0,0): scattered -1, negatives and positions past the table
    pos = rng.choice(topk, size=40, replace=False)
    idx[0, 0, pos[:15]] = -1
    idx[0, 0, pos[15:30]] = -123
    idx[0, 0, pos[30:]] = cap + 5
    idx[0, 1] = -1                                   # fully masked row
    idx[1, 0] = -1
    idx[1, 0, 57] = 333                              # a single valid index
    idx[1, 1, :10] = idx[1, 1, 10]                   # repeated index
    bt = inp.block_table.copy()
    bt[2, 3] = -4                                    # bad block ids mask their positions
    bt[3, 1] = inp.kv_cache.shape[0] + 9
    note(f"masking edge cases fmt={fmt} topk={topk}")
    ref_o, ref_l = oracle.default().sparse_mla_decode(inp.q, inp.kv_cache, bt, idx, inp.seq_lens,
                                                      inp.softmax_scale, d_v=w.d_v, kv_format=fmt,
                                                      block_size=64, threads=8)
    assert np.isinf(ref_l[0, 1]).all() and np.isfinite(ref_l[1, 0]).all()
    for splits in (0, 1, 3):
        out, lse = run_gpu(inp, indices=idx, force_splits=splits, block_table=bt)
        check(out, lse, ref_o, ref_l, f"masks fmt{fmt} S{splits}")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_unaligned_lists_and_table_rows(fmt):
    # top-k 702 and 259-entry block-table rows: the index list of row 1 and the table rows of sequences
    # 1 and 2 start 8, 12 and 8 bytes past a 16-byte boundary, so their whole 256-entry chunks are copied
    # entry by entry, while the others take the 16-byte copies; parts of 702 and of 352 entries
    inp = I.small_inputs(batch=3, q_len=1, topk=702, seq_len=259 * 64 - 10, kv_format=fmt, seed=70 + fmt)
    assert inp.block_table.shape[1] == 259
    note(f"unaligned lists and table rows fmt={fmt}")
    ref_o, ref_l = oracle.decode_inputs(inp, threads=8)
    for splits in (1, 2):
        out, lse = run_gpu(inp, force_splits=splits)
        check(out, lse, ref_o, ref_l, f"unaligned fmt{fmt} S{splits}")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_seq_lens_optional(fmt):
    inp = I.small_inputs(batch=2, q_len=1, topk=96, seq_len=256, kv_format=fmt, seed=31)
    sl = np.array([256, 120], dtype=np.int32)
    inp.seq_lens[:] = sl
    ref_o, ref_l = oracle.decode_inputs(inp)
    out, lse = run_gpu(inp)
    check(out, lse, ref_o, ref_l, "with seq_lens")
    ref_o2, ref_l2 = oracle.decode_inputs(inp, with_seq_lens=False)
    out2, lse2 = run_gpu(inp, with_seq_lens=False)
    check(out2, lse2, ref_o2, ref_l2, "without seq_lens")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_long_block_table_rows(fmt):
    """Contexts past 4096 blocks of 64 tokens: the block-table row is too long to
    be staged in LDS, so each position's block is looked up in global memory."""
    d_qk = 512 if fmt == I.KV_FP8_NOPE_UE8M0 else 576
    w = I.Workload(f"long_b2_topk200_{FMT_IDS[fmt]}", batch=2, q_len=1, topk=200, kv_format=fmt, paged=True,
                   seq_len_range=(270_000, 300_000), d_qk=d_qk, d_v=512)
    inp = I.make_inputs(w, seed=41 + fmt, fill="selected")
    assert inp.block_table.shape[1] > 4096
    idx = inp.indices.copy()
    idx[0, 0, 5] = int(inp.seq_lens[0]) + 3      # past seq_lens, inside the table: masked
    idx[1, 0, 7] = -1
    bt = inp.block_table.copy()
    bt[1, int(idx[1, 0, 9]) // 64] = -2          # a bad block id masks its positions
    note(f"long block table fmt={fmt} max_blocks={bt.shape[1]} seq_lens={inp.seq_lens.tolist()}")
    ref_o, ref_l = oracle.default().sparse_mla_decode(inp.q, inp.kv_cache, bt, idx, inp.seq_lens,
                                                      inp.softmax_scale, d_v=w.d_v, kv_format=fmt,
                                                      block_size=64, threads=8)
    for splits in (0, 3):
        out, lse = run_gpu(inp, indices=idx, force_splits=splits, block_table=bt)
        check(out, lse, ref_o, ref_l, f"long table fmt{fmt} S{splits}")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_part_at_the_row_table_cap(fmt):
    """A part as long as the LDS row table allows, then a short one (a single
    part was asked for; the plan splits the list at the cap)."""
    d_qk = 512 if fmt == I.KV_FP8_NOPE_UE8M0 else 576
    cap = B().decode_plan(1, 1, 16384, 1, fmt, d_qk=d_qk, force_splits=1).tokens_per_split
    topk = cap + 96
    plan = B().decode_plan(1, 1, topk, (topk + 600 + 63) // 64, fmt, d_qk=d_qk, force_splits=1)
    assert (plan.num_splits, plan.tokens_per_split) == (2, cap)
    inp = I.small_inputs(batch=1, q_len=1, topk=topk, seq_len=topk + 600, kv_format=fmt, seed=51 + fmt)
    note(f"row-table cap fmt={fmt}: part of {cap} tokens, top-k {topk}")
    ref_o, ref_l = oracle.decode_inputs(inp, threads=8)
    out, lse = run_gpu(inp, force_splits=1)
    check(out, lse, ref_o, ref_l, f"cap fmt{fmt}")


def _bf16_times_pow2(bits, factor):
    """bf16 bit patterns times a power of two (exact while the result stays in range)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_query_magnitudes(fmt):
    """Queries far from unit size, a zero head, 128x outliers and groups 2^12 apart in one head.
    The contraction must hold fp32 accuracy whatever the spread of the products: an fp8 MFMA over the
    cached codes with Q split into two exact e4m3 halves loses bits of the small products next to a large
    one, and puts the outlier head's lse 3e-3 off at 128x (1.5e-3 at 64x)."""
    base = I.small_inputs(batch=2, q_len=1, topk=200, seq_len=700, kv_format=fmt, seed=41 + fmt)
    cases = []
    for k in (-30, 30):  # Q * 2^k with the softmax scale * 2^-k: the same scores
        scale = float(np.float32(base.softmax_scale) * np.float32(2.0 ** -k))
        cases.append((f"Q*2^{k}", dataclasses.replace(base, q=_bf16_times_pow2(base.q, 2.0 ** k),
                                                      softmax_scale=scale)))
    q = base.q.copy()
    q[:, :, 5, :] = 0                                                   # a zero head
    q[:, :, 6, 0:448:64] = _bf16_times_pow2(np.full_like(q[:, :, 6, 0:448:64], 0x3F80), 128.0)  # outliers 128
    q[:, :, 7, 128:384] = _bf16_times_pow2(q[:, :, 7, 128:384], 2.0 ** -12)   # two small groups
    q[:, :, 8, :] = _bf16_times_pow2(q[:, :, 8, :], 2.0 ** -100)               # a tiny head
    cases.append(("mixed heads", dataclasses.replace(base, q=q)))
    for what, inp in cases:
        note(f"query magnitudes fmt={fmt}: {what}")
        ref_o, ref_l = oracle.decode_inputs(inp, threads=8)
        out, lse = run_gpu(inp)
        check(out, lse, ref_o, ref_l, f"fmt{fmt} {what}")


@pytest.mark.parametrize("fmt", FORMATS[:2], ids=FMT_IDS[:2])
@pytest.mark.parametrize("pos", [230, 250], ids=["tokens0-15", "tokens16-31"])
def test_late_large_scores_restart(fmt, pos):
    # A token near the end of each list gets a score far above the first tiles' max
    # (the rope part of its K row is a large multiple of head 0's rope query; its V
    # part stays as generated), so the kernel must raise its softmax reference after
    # accumulating; forced splits keep several tiles per part.  The token sits in
    # the first or the second half of its tile (list position 230 or 250: for fp8
    # rows the two halves belong to different QK waves, which must raise together).
    inp = I.small_inputs(batch=2, q_len=1, topk=256, seq_len=512, kv_format=fmt, seed=90)
    w = inp.workload
    kv = inp.kv_cache.reshape(-1, w.row_bytes).copy()
    for b in range(2):
        p = int(inp.indices[b, 0, pos])
        row = int(inp.block_table[b, p // 64]) * 64 + p % 64
        qf = (inp.q[b, 0, 0].astype(np.uint32) << 16).view(np.float32)
        kf = oracle_pins.token_rows(inp, b, np.array([p]))[0].astype(np.float32)
        kf[w.d_v:] = qf[w.d_v:] * np.float32(60.0)
        kv[row] = I.encode_rows(w, kf[None, :])[0]
    inp2 = I.Inputs(**{**inp.__dict__, "kv_cache": kv.reshape(inp.kv_cache.shape)})
    ref_o, ref_l = oracle.decode_inputs(inp2)
    # head 0 must sit far (> 64 in log2 units) above the first tiles: about 130 nats here
    assert ref_l[:, 0, 0].min() > 100, "the planted token must dominate head 0"
    for splits in (1, 2):
        out, lse = run_gpu(inp2, force_splits=splits)
        check(out, lse, ref_o, ref_l, f"late large score S{splits}")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_first_valid_token_in_one_half_of_a_tile(fmt):
    """The softmax reference is set at the first tile with a valid token.  For fp8 rows the two
    halves of a tile (tokens 0-15, 16-31) belong to two QK waves that must set it together: rows
    whose first valid tokens all lie in one half of a tile, or in one token of a later tile."""
    inp = I.small_inputs(batch=4, q_len=1, topk=128, seq_len=600, kv_format=fmt, seed=160 + fmt)
    idx = inp.indices.copy()
    idx[0, 0, 0:16] = -1          # tile 0: only tokens 16..31 valid
    idx[1, 0, 16:32] = -1         # tile 0: only tokens 0..15 valid
    idx[2, 0, 0:52] = -1          # tiles 0, 1 masked but token 52 (tile 1, second half) ...
    idx[2, 0, 53:64] = -1         # ... alone in tile 1
    idx[3, 0, 0:32] = -1          # tile 0 masked, tile 1 only token 33 (first half)
    idx[3, 0, 34:64] = -1
    idx[3, 0, 32] = -1
    ref_o, ref_l = oracle.default().sparse_mla_decode(inp.q, inp.kv_cache, inp.block_table, idx, inp.seq_lens,
                                                      inp.softmax_scale, d_v=inp.workload.d_v, kv_format=fmt,
                                                      block_size=64, threads=8)
    assert np.isfinite(ref_l).all()
    for splits in (1, 2):
        note(f"first valid token in one half fmt={fmt} S={splits}")
        out, lse = run_gpu(inp, indices=idx, force_splits=splits)
        check(out, lse, ref_o, ref_l, f"one-half first tile fmt{fmt} S{splits}")


def test_late_large_scores_v4():
    # The pages' layout: V is the whole row, so a large K row would also be a large V
    # row; instead head 0's query is set to 8 x the row of a token late in each list,
    # which lifts that token's score 40 to 100 (log2 units) above the first tile's max
    # with rows of ordinary size.
    inp = I.small_inputs(batch=2, q_len=1, topk=256, seq_len=512, kv_format=I.KV_FP8_NOPE_UE8M0, seed=91)
    q = inp.q.copy()
    for b in range(2):
        p = int(inp.indices[b, 0, 250])
        kf = oracle_pins.token_rows(inp, b, np.array([p]))[0]
        q[b, 0, 0] = I.bf16_bits_rne((8.0 * kf).astype(np.float32))
    inp2 = I.Inputs(**{**inp.__dict__, "q": q})
    ref_o, ref_l = oracle.decode_inputs(inp2)
    assert ref_l[:, 0, 0].min() > 30, "the chosen token must dominate head 0"
    for splits in (1, 2):
        out, lse = run_gpu(inp2, force_splits=splits)
        check(out, lse, ref_o, ref_l, f"v4 late large score S{splits}")


@pytest.mark.parametrize("topk", [1, 31, 33, 64])
def test_short_lists(topk):
    inp = I.small_inputs(batch=2, q_len=2, topk=topk, seq_len=300, kv_format=I.KV_BF16, seed=40 + topk)
    ref_o, ref_l = oracle.decode_inputs(inp)
    out, lse = run_gpu(inp)
    check(out, lse, ref_o, ref_l, f"topk {topk}")


def test_topk_zero_and_empty_batch():
    inp = I.small_inputs(batch=2, q_len=1, topk=4, seq_len=128, kv_format=I.KV_BF16, seed=3)
    idx0 = np.zeros((2, 1, 0), dtype=np.int32)
    q, kv, bt, _, sl = B().to_device(inp)
    out, lse = B().sparse_mla_decode(q, kv, bt, torch.from_numpy(idx0).cuda(), sl, inp.softmax_scale)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    out, lse = B().sparse_mla_decode(q[:0], kv, bt[:0], torch.zeros((0, 1, 4), dtype=torch.int32).cuda(),
                                     sl[:0], inp.softmax_scale)
    assert out.shape[0] == 0 and lse.shape[0] == 0


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_paging_invariance_bit_exact(fmt):
    inp = I.small_inputs(batch=2, q_len=1, topk=150, seq_len=512, kv_format=fmt, seed=50)
    w = inp.workload
    nblk = 512 // 64
    cache2 = np.zeros_like(inp.kv_cache)
    bt2 = np.zeros_like(inp.block_table)
    for b in range(2):
        for j in range(nblk):
            cache2[b * nblk + j] = inp.kv_cache[inp.block_table[b, j]]
            bt2[b, j] = b * nblk + j
    out1, lse1 = run_gpu(inp, force_splits=3)
    inp2 = I.Inputs(**{**inp.__dict__, "kv_cache": cache2, "block_table": bt2})
    out2, lse2 = run_gpu(inp2, force_splits=3)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_deterministic():
    inp = I.small_inputs(batch=2, q_len=2, topk=300, seq_len=1000, kv_format=I.KV_FP8, seed=60)
    a = run_gpu(inp, force_splits=4)
    b = run_gpu(inp, force_splits=4)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# (S, rows): up to 512 (row, head) pairs the combine runs four waves per pair, beyond that one;
# with up to 64 parts one lse read per lane serves all weights, past 64 the parts are looped over;
# a wave's parts go in batches of 16, 8, 4 and 1
@pytest.mark.parametrize("S,rows", [(1, 3), (5, 3), (70, 3), (64, 3), (40, 9), (17, 9)])
def test_combine_kernel_alone(S, rows):
    rng = np.random.default_rng(70 + S)
    H, dv = 64, 512
    po = rng.standard_normal((S, rows, H, dv)).astype(np.float32)
    pl = (rng.standard_normal((S, rows, H)) * 3).astype(np.float32)
    if S > 1:
        pl[1, 0, :] = -np.inf
        po[1, 0, :, :] = np.nan                 # an empty part's values are ignored
    pl[:, 2, 5] = -np.inf                       # every part of one pair empty
    # the partial outputs are bf16: the oracle merges exactly the same (decoded) values
    po_bits = I.bf16_bits_rne(np.nan_to_num(po))
    if S > 1:
        po_bits[1, 0, :, :] = 0x7FC0            # bf16 NaN
    po_ref = oracle_pins.np_bf16(po_bits)
    po_ref[np.isnan(po_ref)] = 0.0
    ref_o, ref_l = oracle.lse_combine(po_ref, pl.astype(np.float64))
    out = torch.empty((rows, H, dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows, H), dtype=torch.float32, device="cuda")
    po_dev = torch.from_numpy(po_bits.view(np.int16)).view(torch.bfloat16).cuda()
    B().combine(po_dev, torch.from_numpy(pl).cuda(), out, lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    lg = lse.cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.all(o[~fin] == 0) and np.all(np.isneginf(lg[~fin]))
    assert np.abs(o[fin] - ref_o[fin]).max() <= 2 ** -8 * np.abs(ref_o[fin]).max() + 1e-6
    assert np.abs(lg[fin] - ref_l[fin]).max() <= 1e-5 * max(1.0, np.abs(ref_l[fin]).max())


@pytest.mark.parametrize("splits", [1, 3])
def test_partial_then_combine_equals_run(splits):
    """smla_decode_partial + smla_combine is smla_decode_run, bit for bit."""
    inp = I.small_inputs(batch=2, q_len=1, topk=300, seq_len=900, kv_format=I.KV_BF16, seed=81)
    w = inp.workload
    q, kv, bt, idx, sl = B().to_device(inp)
    plan = B().decode_plan(w.batch, w.q_len, w.topk, inp.block_table.shape[1], w.kv_format, force_splits=splits)
    out_a = torch.empty((w.batch, w.q_len, w.num_heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    lse_a = torch.empty((w.batch, w.q_len, w.num_heads), dtype=torch.float32, device="cuda")
    out_b, lse_b = torch.empty_like(out_a), torch.empty_like(lse_a)
    ws = B().alloc_workspace(plan, "cuda")
    B().decode_run(plan, q, kv, bt, idx, sl, inp.softmax_scale, out_a, lse_a, ws)
    torch.cuda.synchronize()
    ws2 = B().alloc_workspace(plan, "cuda")
    B().decode_partial(plan, q, kv, bt, idx, sl, inp.softmax_scale, out_b, lse_b, ws2)
    if plan.num_splits > 1:
        po, pl = B().workspace_parts(plan, ws2)
        B().combine(po, pl, out_b.view(plan.rows, w.num_heads, w.d_v), lse_b.view(plan.rows, w.num_heads))
    torch.cuda.synchronize()
    assert plan.num_splits == splits
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)


def test_runs_on_a_side_stream():
    inp = I.small_inputs(batch=2, q_len=1, topk=128, seq_len=512, kv_format=I.KV_BF16, seed=80)
    ref_o, ref_l = oracle.decode_inputs(inp)
    q, kv, bt, idx, sl = B().to_device(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = B().sparse_mla_decode(q, kv, bt, idx, sl, inp.softmax_scale)
    s.synchronize()
    check(out, lse, ref_o, ref_l, "side stream")


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_multi_token_verify(fmt):
    """Four query tokens per sequence (speculative-decode verify), each with its own top-k list:
    rows (b, s) are independent; the block table and the cache are shared by a sequence's tokens."""
    inp = I.small_inputs(batch=3, q_len=4, topk=160, seq_len=700, kv_format=fmt, seed=90)
    ref_o, ref_l = oracle.decode_inputs(inp)
    for splits in (0, 1, 3):
        out, lse = run_gpu(inp, force_splits=splits)
        check(out, lse, ref_o, ref_l, f"q_len=4 splits={splits}")


@pytest.mark.parametrize("splits", [1, 4])
def test_graph_capture_replays(splits):
    """run (partial + combine) captured once in a HIP graph and replayed three times, the inputs
    rewritten in place by eager work between replays; every replay matches the oracle."""
    inp = I.small_inputs(batch=2, q_len=1, topk=256, seq_len=1024, kv_format=I.KV_BF16, seed=95)
    w = inp.workload
    q, kv, bt, idx, sl = B().to_device(inp)
    plan = B().decode_plan(w.batch, w.q_len, w.topk, inp.block_table.shape[1], w.kv_format, force_splits=splits)
    out = torch.empty((w.batch, w.q_len, w.num_heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.q_len, w.num_heads), dtype=torch.float32, device="cuda")
    ws = B().alloc_workspace(plan, "cuda")
    stream = torch.cuda.Stream()
    B().decode_run(plan, q, kv, bt, idx, sl, inp.softmax_scale, out, lse, ws)  # warm (per-device setup)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            B().decode_run(plan, q, kv, bt, idx, sl, inp.softmax_scale, out, lse, ws, stream=stream)
    rng = np.random.default_rng(96)
    for rep in range(3):
        # new index lists and query values for this replay, written in place (eager work)
        new_idx = np.stack([rng.permutation(1024)[:256] for _ in range(2)]).astype(np.int32).reshape(2, 1, 256)
        new_idx[1, 0, rng.choice(256, size=40, replace=False)] = -1
        new_q = I.bf16_bits_rne(rng.standard_normal(inp.q.shape).astype(np.float32)).astype(np.uint16)
        idx.copy_(torch.from_numpy(new_idx))
        q.copy_(torch.from_numpy(new_q.view(np.int16)).view(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        inp_r = I.Inputs(**{**inp.__dict__, "q": new_q, "indices": new_idx})
        ref_o, ref_l = oracle.decode_inputs(inp_r)
        check(out, lse, ref_o, ref_l, f"graph replay {rep} splits={plan.num_splits}")


# ---------------------------------------------------------------- full workloads

@pytest.fixture(scope="module")
def workload_cache():
    return {}


@pytest.mark.parametrize("w", I.WORKLOADS, ids=lambda w: w.name)
def test_workload_parity_all_rows(w):
    """Every query row of each full-size workload, in the launch configuration the benchmark times (the
    automatic plan), against the oracle over all its sequences (16 host threads)."""
    note(f"workload {w.name}: generating")
    inp = I.make_inputs(w, seed=0)
    plan = B().decode_plan(w.batch, w.q_len, w.topk, inp.block_table.shape[1], w.kv_format, d_qk=w.d_qk)
    note(f"workload {w.name}: plan splits={plan.num_splits} tps={plan.tokens_per_split} wgs={plan.num_workgroups}")
    out, lse = run_gpu(inp)
    note(f"workload {w.name}: oracle on all {w.rows} query rows")
    ref_o, ref_l = oracle.default().sparse_mla_decode(
        inp.q, inp.kv_cache, inp.block_table, inp.indices, inp.seq_lens, inp.softmax_scale, d_v=w.d_v,
        kv_format=w.kv_format, block_size=w.block_size, threads=16)
    check(out, lse, ref_o, ref_l, f"{w.name} all {w.rows} rows")


def test_graph_capture_replays_v4():
    """The pages' layout: run (partial + combine) captured once, replayed with new lists and queries."""
    inp = I.small_inputs(batch=2, q_len=2, topk=192, seq_len=1024, kv_format=I.KV_FP8_NOPE_UE8M0, seed=97)
    w = inp.workload
    q, kv, bt, idx, sl = B().to_device(inp)
    plan = B().decode_plan(w.batch, w.q_len, w.topk, inp.block_table.shape[1], w.kv_format, d_qk=w.d_qk,
                           force_splits=3)
    out = torch.empty((w.batch, w.q_len, w.num_heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.q_len, w.num_heads), dtype=torch.float32, device="cuda")
    ws = B().alloc_workspace(plan, "cuda")
    stream = torch.cuda.Stream()
    B().decode_run(plan, q, kv, bt, idx, sl, inp.softmax_scale, out, lse, ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            B().decode_run(plan, q, kv, bt, idx, sl, inp.softmax_scale, out, lse, ws, stream=stream)
    rng = np.random.default_rng(98)
    for rep in range(3):
        new_idx = np.stack([rng.permutation(1024)[:192] for _ in range(4)]).astype(np.int32).reshape(2, 2, 192)
        new_idx[1, 1, rng.choice(192, size=30, replace=False)] = -1
        new_q = I.bf16_bits_rne(rng.standard_normal(inp.q.shape).astype(np.float32)).astype(np.uint16)
        idx.copy_(torch.from_numpy(new_idx))
        q.copy_(torch.from_numpy(new_q.view(np.int16)).view(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        inp_r = I.Inputs(**{**inp.__dict__, "q": new_q, "indices": new_idx})
        ref_o, ref_l = oracle.decode_inputs(inp_r)
        check(out, lse, ref_o, ref_l, f"v4 graph replay {rep}")
