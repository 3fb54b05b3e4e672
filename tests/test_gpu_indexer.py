"""Top-k indexer (smla_indexer_topk) vs the fp64 oracle, through the C ABI (needs an MI355X).

The scores are bf16 products summed in fp32, so they match the oracle's fp64
scores to within the fp32 summation bound 2^-16 * sum_d |q_d k_d| (twice the
textbook n*u bound for n = 128 terms).  The selection is a decision taken on
those fp32 scores: it must equal, element for element, a numpy top-k over the
kernel's own fp32 scores (ties to the lower position; the list in ascending
position order), and the selected set must be a valid top-k of the oracle's
scores up to that bound.
"""
import sys

import numpy as np
import pytest

import oracle
from sparse_mla_decode_smla_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

EPS_REL = 2.0 ** -16


def B():
    from sparse_mla_decode_smla_amd import binding
    return binding


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_indexer(inp, topk, block_table=None, seq_lens=None):
    q, k, bt, sl = B().indexer_to_device(inp)
    if block_table is not None:
        bt = torch.from_numpy(np.ascontiguousarray(block_table)).cuda()
    if seq_lens is not None:
        sl = torch.from_numpy(np.ascontiguousarray(seq_lens)).cuda()
    Bn, Q, _ = inp.q_idx.shape
    mb = bt.shape[1]
    ws = torch.empty(max(B().indexer_workspace_size(Bn, Q, mb), 16), dtype=torch.uint8, device="cuda")
    idx, sc = B().indexer_topk(q, k, bt, sl, topk, workspace=ws)
    torch.cuda.synchronize()
    ws_scores = ws[: Bn * Q * 64 * mb * 4].view(torch.float32).view(Bn, Q, 64 * mb)
    return idx.cpu().numpy(), sc.cpu().numpy(), ws_scores.cpu().numpy()


def check(inp, topk, idx_g, sc_g, ws_g, what, block_table=None, seq_lens=None, rows=None):
    bt = inp.block_table if block_table is None else block_table
    sl = inp.seq_lens if seq_lens is None else seq_lens
    ref_s, ref_a = oracle.indexer_scores(inp.q_idx, inp.k_cache, bt, sl)
    Bn, Q, cap = ref_s.shape
    worst = 0.0
    exact_rows = 0
    for b in range(Bn):
        n = min(max(int(sl[b]), 0), cap)
        for q in range(Q):
            if rows is not None and (b, q) not in rows:
                continue
            s_ref, a_ref = ref_s[b, q, :n], ref_a[b, q, :n]
            s_gpu = ws_g[b, q, :n].astype(np.float64)
            cand = np.isfinite(s_ref)
            # (a) scores of every candidate within the fp32 bound; -inf exactly where not a candidate
            assert np.array_equal(np.isfinite(s_gpu), cand), f"{what}: candidate set differs in row ({b},{q})"
            eps = EPS_REL * a_ref + 1e-30
            err = np.abs(s_gpu[cand] - s_ref[cand])
            assert np.all(err <= eps[cand]), f"{what}: score error {err.max():.3e} in row ({b},{q})"
            if cand.any():
                worst = max(worst, float((err / np.maximum(a_ref[cand], 1e-30)).max()))
            # (b) the selection equals a top-k over the kernel's own fp32 scores, element for element
            s32 = ws_g[b, q, :n]
            pos = np.nonzero(cand)[0]
            order = np.sort(pos[np.lexsort((pos, -s32[pos]))][:topk])
            kk = len(order)
            assert np.array_equal(idx_g[b, q, :kk], order), f"{what}: selection differs in row ({b},{q})"
            assert np.all(idx_g[b, q, kk:] == -1), f"{what}: padding in row ({b},{q})"
            assert np.array_equal(sc_g[b, q, :kk], s32[order]), f"{what}: returned scores in row ({b},{q})"
            assert np.all(np.diff(idx_g[b, q, :kk]) > 0), f"{what}: list not in ascending position order"
            assert np.all(np.isneginf(sc_g[b, q, kk:]))
            # (c) a valid top-k of the oracle's scores up to the bound
            chosen = np.zeros(n, dtype=bool)
            chosen[order] = True
            rest = cand & ~chosen
            if kk and rest.any():
                assert (s_ref[chosen] + eps[chosen]).min() >= (s_ref[rest] - eps[rest]).max(), \
                    f"{what}: not a top-k of the oracle's scores in row ({b},{q})"
            ref_order = np.sort(pos[np.lexsort((pos, -s_ref[pos]))][:topk])
            exact_rows += int(np.array_equal(ref_order, order))
    note(f"  {what}: worst score error / sum|q k| = {worst:.2e}; rows equal to the oracle's own order: {exact_rows}")


def test_indexer_small_ragged():
    inp = I.small_indexer_inputs(batch=3, q_len=2, topk=100, seq_len_range=(40, 700), seed=31)
    note(f"indexer small: seq_lens {inp.seq_lens.tolist()}")
    idx, sc, ws = run_indexer(inp, 100)
    check(inp, 100, idx, sc, ws, "small ragged")


@pytest.mark.parametrize("topk", [1, 63, 64, 2048])
def test_indexer_topk_sizes(topk):
    inp = I.small_indexer_inputs(batch=2, q_len=1, topk=topk, seq_len_range=(1500, 3000), seed=40 + topk)
    idx, sc, ws = run_indexer(inp, topk)
    check(inp, topk, idx, sc, ws, f"topk {topk}")


def test_indexer_masking_and_short_rows():
    inp = I.small_indexer_inputs(batch=4, q_len=4, topk=200, seq_len=640, seed=33)
    bt = inp.block_table.copy()
    sl = inp.seq_lens.copy()
    sl[0] = 0                                    # no candidates
    sl[1] = 130                                  # fewer candidates than topk, last block partial
    bt[2, 3] = -1                                # a bad block id masks its 64 positions
    bt[3, 0] = inp.k_cache.shape[0] + 5
    idx, sc, ws = run_indexer(inp, 200, block_table=bt, seq_lens=sl)
    assert np.all(idx[0] == -1) and np.all(np.isneginf(sc[0]))
    assert np.all((idx[1] >= 0).sum(axis=1) == 130)
    check(inp, 200, idx, sc, ws, "masks", block_table=bt, seq_lens=sl)


def test_indexer_exact_ties_go_to_lower_positions():
    # keys repeat with period 7: every score value occurs many times, bit-identical in fp32
    inp = I.small_indexer_inputs(batch=2, q_len=1, topk=45, seq_len=448, seed=34)
    flat = inp.k_cache.reshape(-1, 128)
    k2 = inp.k_cache.copy()
    for b in range(2):
        for p in range(448):
            phys = inp.block_table[b, p // 64] * 64 + p % 64
            src = inp.block_table[b, (p % 7) // 64] * 64 + (p % 7) % 64
            k2.reshape(-1, 128)[phys] = flat[src]
    inp2 = I.IndexerInputs(workload=inp.workload, q_idx=inp.q_idx, k_cache=k2, block_table=inp.block_table,
                           seq_lens=inp.seq_lens)
    idx, sc, ws = run_indexer(inp2, 45)
    check(inp2, 45, idx, sc, ws, "ties")
    ref, _ = oracle.indexer_topk(inp2.q_idx, inp2.k_cache, inp2.block_table, inp2.seq_lens, 45)
    assert np.array_equal(idx, ref), "with exact ties the selection must be the oracle's"


def _periodic_keys(inp, period):
    """A copy of the key cache in which position p of every sequence holds the key of position p % period,
    so every score value occurs many times, bit-identical in fp32."""
    k2 = inp.k_cache.copy().reshape(-1, 128)
    flat = inp.k_cache.reshape(-1, 128)
    bt = inp.block_table
    for b in range(bt.shape[0]):
        p = np.arange(bt.shape[1] * 64)
        phys = bt[b, p // 64].astype(np.int64) * 64 + p % 64
        src = bt[b, (p % period) // 64].astype(np.int64) * 64 + (p % period) % 64
        k2[phys] = flat[src]
    return k2.reshape(inp.k_cache.shape)


# Chunked selection: batches of a few sequences have the chunk histograms counted by a kernel of their
# own; from 256 (sequence, chunk) workgroups on (here batch 52 or 64) the score kernel counts them.
@pytest.mark.parametrize("batch", [3, 64])
def test_indexer_chunked_ties_across_chunks(batch):
    # rows of 20480 (five whole chunks of 4096), 20481 (one position in a sixth) and 17000 positions,
    # each score value repeated every 7 positions: the threshold's ties spread over every chunk, and the
    # lowest positions among them must win, as in the oracle
    inp = I.small_indexer_inputs(batch=batch, q_len=1, topk=2048, seq_len=20481, seed=44)
    sl = np.full(batch, 20481, dtype=np.int32)
    sl[[0, 2]] = [20480, 17000]
    inp2 = I.IndexerInputs(workload=inp.workload, q_idx=inp.q_idx, k_cache=_periodic_keys(inp, 7),
                           block_table=inp.block_table, seq_lens=sl)
    note(f"indexer chunked ties: seq_lens {sl.tolist()}")
    idx, sc, ws = run_indexer(inp2, 2048)
    check(inp2, 2048, idx, sc, ws, "chunked ties")
    ref, _ = oracle.indexer_topk(inp2.q_idx, inp2.k_cache, inp2.block_table, inp2.seq_lens, 2048)
    assert np.array_equal(idx, ref), "with exact ties the selection must be the oracle's"


@pytest.mark.parametrize("batch", [4, 52])
def test_indexer_chunked_masks_and_short_rows(batch):
    # rows long enough for the chunked selection: an empty row, a row with fewer candidates than the list
    # (its last chunk one position long), bad block ids inside chunks
    inp = I.small_indexer_inputs(batch=batch, q_len=2, topk=1000, seq_len=18000, seed=45)
    bt = inp.block_table.copy()
    sl = inp.seq_lens.copy()
    sl[0] = 0                                    # no candidates
    sl[1] = 16385                                # five chunks, the last one position long
    bt[1, 5:250] = -1                            # ... and most blocks masked: fewer candidates than topk
    bt[2, 70] = -3                               # one bad block in the middle of chunk 1
    bt[3, 0] = inp.k_cache.shape[0] + 7          # the first block past the cache
    idx, sc, ws = run_indexer(inp, 1000, block_table=bt, seq_lens=sl)
    assert np.all(idx[0] == -1) and np.all(np.isneginf(sc[0]))
    assert np.all((idx[1] >= 0).sum(axis=1) == 5 * 64 + (16385 - 250 * 64))
    check(inp, 1000, idx, sc, ws, "chunked masks", block_table=bt, seq_lens=sl)


@pytest.mark.parametrize("q_len,batch", [(3, 2), (4, 2), (3, 52)])
def test_indexer_chunked_multi_token_rows(q_len, batch):
    # three and four query rows per sequence on rows long enough for the chunked selection (at batch 52
    # the score kernel counts each row's chunk histograms, its four-row instantiation serving three);
    # the second sequence's blocks are all out of range, so its rows have positions but no candidates
    inp = I.small_indexer_inputs(batch=batch, q_len=q_len, topk=500, seq_len=17500, seed=46 + q_len)
    bt = inp.block_table.copy()
    bt[1, :] = -1
    note(f"indexer chunked q_len={q_len}")
    idx, sc, ws = run_indexer(inp, 500, block_table=bt)
    assert np.all(idx[1] == -1) and np.all(np.isneginf(sc[1]))
    check(inp, 500, idx, sc, ws, f"chunked q_len={q_len}", block_table=bt)


@pytest.mark.parametrize("topk", [1, 63])
@pytest.mark.parametrize("batch", [2, 52])
def test_indexer_chunked_short_lists(topk, batch):
    # the chunked selection with lists far shorter than a chunk's candidates: top-1 (the row's maximum,
    # wherever it lies) and 63, with the histograms counted by their own kernel (batch 2) and by the
    # score kernel (batch 52)
    inp = I.small_indexer_inputs(batch=batch, q_len=1, topk=topk, seq_len=17000, seed=48 + topk)
    idx, sc, ws = run_indexer(inp, topk)
    check(inp, topk, idx, sc, ws, f"chunked top-{topk} batch {batch}")


def test_indexer_rows_longer_than_registers():
    # more than 65536 positions per row: the selection streams the row from the workspace each pass
    inp = I.small_indexer_inputs(batch=2, q_len=1, topk=300, seq_len_range=(66000, 70000), seed=37)
    note(f"indexer long rows: seq_lens {inp.seq_lens.tolist()}")
    idx, sc, ws = run_indexer(inp, 300)
    check(inp, 300, idx, sc, ws, "long rows")


@pytest.mark.parametrize("seq_len_range", [(9000, 16000), (20000, 32000)], ids=["per16", "per32"])
def test_indexer_register_sizes(seq_len_range):
    # rows of up to 16384 and 32768 positions: 16 and 32 keys per select thread
    inp = I.small_indexer_inputs(batch=2, q_len=2, topk=2048, seq_len_range=seq_len_range, seed=42)
    note(f"indexer rows {seq_len_range}: seq_lens {inp.seq_lens.tolist()}")
    idx, sc, ws = run_indexer(inp, 2048)
    check(inp, 2048, idx, sc, ws, f"rows {seq_len_range}")


@pytest.mark.parametrize("seq_len", [2000, 40000])
def test_indexer_one_outlier_key(seq_len):
    # one key equal to 64 q: its score is far above all others, so the keys
    # near the row's largest are fewer than the list needs and the selection
    # counts the rest as well
    inp = I.small_indexer_inputs(batch=2, q_len=1, topk=300, seq_len=seq_len, seed=43)
    k2 = inp.k_cache.copy()
    p0 = seq_len // 3
    q = inp.q_idx[0, 0].view(np.uint16).astype(np.uint32) << 16
    big = (q.view(np.float32) * np.float32(64.0)).view(np.uint32) >> 16      # exact: a power of two
    k2.reshape(-1, 128)[inp.block_table[0, p0 // 64] * 64 + p0 % 64] = big.astype(np.uint16)
    inp2 = I.IndexerInputs(workload=inp.workload, q_idx=inp.q_idx, k_cache=k2, block_table=inp.block_table,
                           seq_lens=inp.seq_lens)
    idx, sc, ws = run_indexer(inp2, 300)
    assert p0 in idx[0, 0]
    check(inp2, 300, idx, sc, ws, f"outlier n={seq_len}")


@pytest.mark.parametrize("name", [w.name for w in I.INDEXER_WORKLOADS])
def test_indexer_workloads(name):
    w = I.INDEXER_WORKLOADS_BY_NAME[name]
    note(f"indexer workload {name}: generating")
    inp = I.make_indexer_inputs(w)
    idx, sc, ws = run_indexer(inp, w.topk)
    rng = np.random.default_rng(7)
    rows = {(0, 0), (w.batch - 1, w.q_len - 1)} | {(int(b), 0) for b in rng.choice(w.batch, size=3, replace=False)}
    sub = sorted({b for b, _ in rows})
    note(f"indexer workload {name}: oracle on sequences {sub}")
    small = I.IndexerInputs(workload=w, q_idx=inp.q_idx[sub], k_cache=inp.k_cache, block_table=inp.block_table[sub],
                            seq_lens=inp.seq_lens[sub])
    check(small, w.topk, idx[sub], sc[sub], ws[sub], name)


def test_indexer_feeds_decode():
    """The indexer's lists drive smla_decode_run directly (same block table, same positions)."""
    lat = I.small_inputs(batch=2, q_len=1, topk=128, seq_len=1000, kv_format=I.KV_BF16, seed=35)
    rng = np.random.default_rng(36)
    q_idx = I.bf16_bits_rne(rng.standard_normal((2, 1, 128)).astype(np.float32))
    nb = lat.kv_cache.shape[0]
    k_cache = I.bf16_bits_rne(rng.standard_normal((nb, 64, 128)).astype(np.float32))
    ix = I.IndexerInputs(workload=I.IndexerWorkload("feed", 2, 1, 128, seq_len=1000), q_idx=q_idx, k_cache=k_cache,
                         block_table=lat.block_table, seq_lens=lat.seq_lens)
    idx, _, _ = run_indexer(ix, 128)
    ref_o, ref_l = oracle.decode_inputs(lat, indices=idx.astype(np.int32))
    q, kv, bt, _, sl = B().to_device(lat)
    out, lse = B().sparse_mla_decode(q, kv, bt, torch.from_numpy(idx).cuda(), sl, lat.softmax_scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    err = float(np.abs(o - ref_o).max())
    lerr = float(np.abs(lse.cpu().numpy() - ref_l).max())
    note(f"  indexer -> decode: out err {err:.3e}, lse err {lerr:.3e}")
    assert err <= 2e-2 and err <= 1e-2 * np.abs(ref_o).max() and lerr <= 1e-3


def test_indexer_graph_capture_replays():
    """smla_indexer_topk captured once and replayed with new queries written in place between replays."""
    inp = I.small_indexer_inputs(batch=3, q_len=2, topk=150, seq_len_range=(200, 900), seed=38)
    q, k, bt, sl = B().indexer_to_device(inp)
    mb = bt.shape[1]
    ws = torch.empty(B().indexer_workspace_size(3, 2, mb), dtype=torch.uint8, device="cuda")
    idx = torch.empty((3, 2, 150), dtype=torch.int32, device="cuda")
    sc = torch.empty((3, 2, 150), dtype=torch.float32, device="cuda")
    B().indexer_topk(q, k, bt, sl, 150, out_indices=idx, out_scores=sc, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            B().indexer_topk(q, k, bt, sl, 150, out_indices=idx, out_scores=sc, workspace=ws, stream=stream)
    rng = np.random.default_rng(39)
    for rep in range(3):
        new_q = I.bf16_bits_rne(rng.standard_normal(inp.q_idx.shape).astype(np.float32))
        q.copy_(torch.from_numpy(new_q.view(np.int16)).view(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        inp_r = I.IndexerInputs(workload=inp.workload, q_idx=new_q, k_cache=inp.k_cache,
                                block_table=inp.block_table, seq_lens=inp.seq_lens)
        ws_scores = ws[: 3 * 2 * 64 * mb * 4].view(torch.float32).view(3, 2, 64 * mb)
        check(inp_r, 150, idx.cpu().numpy(), sc.cpu().numpy(), ws_scores.cpu().numpy(), f"indexer graph replay {rep}")
