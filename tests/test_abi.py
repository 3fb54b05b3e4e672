"""The C ABI of libsmla.so without a GPU: exports, struct layout, plan logic, argument checks."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_mla_decode_smla_amd import binding as B
from sparse_mla_decode_smla_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libsmla.so not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(smla_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"smla_decode_plan", "smla_decode_run", "smla_decode_partial", "smla_combine",
                          "smla_status_string", "smla_indexer_workspace_size", "smla_indexer_topk",
                          "smla_indexer_scores"}
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in smla.h but not exported"


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "smla.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(smla_problem_t), sizeof(smla_plan_t),
         offsetof(smla_plan_t, rows), offsetof(smla_plan_t, num_workgroups), offsetof(smla_plan_t, workspace_bytes),
         offsetof(smla_problem_t, cache_policy), offsetof(smla_plan_t, cache_policy));
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [ctypes.sizeof(B.Problem), ctypes.sizeof(B.Plan), B.Plan.rows.offset,
                   B.Plan.num_workgroups.offset, B.Plan.workspace_bytes.offset, B.Problem.cache_policy.offset,
                   B.Plan.cache_policy.offset]


def test_status_strings():
    for code in range(6):
        assert B.status_string(code) and B.status_string(code) != "unknown status"
    assert B.status_string(99) == "unknown status"


# split counts the plan's cost model chooses for the workloads on 256 CUs
PLANNED_SPLITS = {"b1_topk512_n4096_contiguous_bf16": 16, "b1_topk2048_n32768_paged_bf16": 32,
                  "b16_topk2048_n65536_paged_bf16": 8, "b64_topk2048_n1k-128k_paged_bf16": 3,
                  "b128_q2_topk2048_n65536_paged_fp8": 1, "b1_topk512_n8192_paged_v4fp8": 16,
                  "b64_topk512_n8192_paged_v4fp8": 4}


# cache policies the plan chooses automatically: streaming rows and outputs from 4 MiB of results written
# by the partial kernel, streaming rows alone from 64 MiB of gathered rows (upper bound rows * topk * row
# bytes), else cached
PLANNED_POLICY = {"b1_topk512_n4096_contiguous_bf16": B.CACHE_CACHED, "b1_topk2048_n32768_paged_bf16": B.CACHE_CACHED,
                  "b16_topk2048_n65536_paged_bf16": B.CACHE_STREAM_ROWS,
                  "b64_topk2048_n1k-128k_paged_bf16": B.CACHE_STREAM_ROWS,
                  "b128_q2_topk2048_n65536_paged_fp8": B.CACHE_STREAM_BOTH,
                  "b1_topk512_n8192_paged_v4fp8": B.CACHE_CACHED, "b64_topk512_n8192_paged_v4fp8": B.CACHE_STREAM_ROWS}


@pytest.mark.parametrize("w", I.WORKLOADS, ids=lambda w: w.name)
def test_plan_cache_policy(w):
    mb = (w.max_seq_len + 63) // 64
    p = B.decode_plan(w.batch, w.q_len, w.topk, mb, w.kv_format, d_qk=w.d_qk, num_cus=256)
    assert p.prob.cache_policy == B.CACHE_AUTO and p.cache_policy == PLANNED_POLICY[w.name]
    for pol in (B.CACHE_CACHED, B.CACHE_STREAM_ROWS, B.CACHE_STREAM_OUT, B.CACHE_STREAM_BOTH):
        q = B.decode_plan(w.batch, w.q_len, w.topk, mb, w.kv_format, d_qk=w.d_qk, num_cus=256, cache_policy=pol)
        assert q.cache_policy == pol and q.num_splits == p.num_splits and q.workspace_bytes == p.workspace_bytes


def test_plan_cache_policy_thresholds():
    # bf16 rows (1152 bytes): 64 MiB of rows = 58254 selected tokens; one part of 64 KiB per row
    rows = B.decode_plan(29, 1, 2048, 64, num_cus=256, force_splits=1)     # 65.3 MiB rows, 1.8 MiB out
    assert rows.cache_policy == B.CACHE_STREAM_ROWS
    below = B.decode_plan(28, 1, 2048, 64, num_cus=256, force_splits=1)    # 63.0 MiB rows
    assert below.cache_policy == B.CACHE_CACHED
    tiny = B.decode_plan(2, 1, 2048, 64, num_cus=256, force_splits=1)      # 4.7 MB rows, 128 KiB out
    assert tiny.cache_policy == B.CACHE_CACHED
    out = B.decode_plan(64, 1, 32, 64, num_cus=256, force_splits=1)        # 2.4 MB rows, 4 MiB out
    assert out.cache_policy == B.CACHE_STREAM_BOTH
    out_below = B.decode_plan(63, 1, 32, 64, num_cus=256, force_splits=1)  # 4 MiB - 64 KiB out
    assert out_below.cache_policy == B.CACHE_CACHED
    # several parts: the parts stay cached for the combine; rows streamed from 4 MiB of parts
    parts = B.decode_plan(32, 1, 64, 64, num_cus=256, force_splits=2)      # 2 x 32 parts: 4 MiB
    assert parts.num_splits == 2 and parts.cache_policy == B.CACHE_STREAM_ROWS
    parts_below = B.decode_plan(31, 1, 64, 64, num_cus=256, force_splits=2)
    assert parts_below.cache_policy == B.CACHE_CACHED
    many = B.decode_plan(29, 1, 2048, 64, num_cus=256, force_splits=2)     # 65.3 MiB rows, 3.6 MiB of parts
    assert many.cache_policy == B.CACHE_STREAM_ROWS
    big = B.decode_plan(64, 1, 2048, 64, num_cus=256, force_splits=2)      # 144 MiB rows, 8 MiB of parts
    assert big.cache_policy == B.CACHE_STREAM_ROWS                         # parts cached whatever the rows
    for bad in (-1, 5):
        with pytest.raises(B.SmlaError):
            B.decode_plan(1, 1, 64, 4, num_cus=256, cache_policy=bad)


@pytest.mark.parametrize("w", I.WORKLOADS, ids=lambda w: w.name)
def test_plan_covers_the_list(w):
    mb = (w.max_seq_len + 63) // 64
    p = B.decode_plan(w.batch, w.q_len, w.topk, mb, w.kv_format, d_qk=w.d_qk, num_cus=256)
    assert p.rows == w.rows
    assert p.num_workgroups == p.rows * p.num_splits
    assert p.tokens_per_split % p.tile_tokens == 0
    # every part non-empty, the parts together cover the list
    assert (p.num_splits - 1) * p.tokens_per_split < w.topk <= p.num_splits * p.tokens_per_split
    if p.num_splits > 1:
        assert p.workspace_bytes == p.num_splits * p.rows * 64 * (512 * 2 + 4)
    else:
        assert p.workspace_bytes == 0
    assert p.num_splits == PLANNED_SPLITS[w.name]


# further shapes, each planned at the split count that measured fastest of the
# two a cost-model change moved between (µs/call on MI355X, cold cache):
# (batch, top-k, kv_format) -> S
MEASURED_BEST_SPLITS = {(4, 2048, B.KV_BF16): 16,    # 17.3 against 18.2 at S=32
                        (16, 512, B.KV_BF16): 4,     # 17.1 against 17.4 at S=8
                        (32, 2048, B.KV_BF16): 5,    # 29.2 against 29.8 at S=6
                        (64, 512, B.KV_BF16): 2,     # 22.5 against 23.1 at S=3
                        (128, 1024, B.KV_BF16): 1,   # 41.8 against 46.7 at S=2
                        (8, 2048, B.KV_FP8_E4M3_SCALE128): 16}  # 20.8 against 22.2 at S=22


@pytest.mark.parametrize("shape", sorted(MEASURED_BEST_SPLITS), ids=str)
def test_plan_picks_the_measured_best_split(shape):
    batch, topk, fmt = shape
    p = B.decode_plan(batch, 1, topk, 1024, fmt, num_cus=256)
    assert p.num_splits == MEASURED_BEST_SPLITS[shape]


def test_plan_splits_small_batches_more():
    """Fewer rows -> more parts per row (the occupancy argument), never more parts than tiles."""
    s = [B.decode_plan(b, 1, 2048, 1024, num_cus=256).num_splits for b in (1, 4, 16, 64, 256)]
    assert all(x >= y for x, y in zip(s, s[1:])), s
    assert s[0] > 1 and s[-1] <= 2
    assert B.decode_plan(1, 1, 64, 8, num_cus=256).num_splits <= 2


def test_plan_is_deterministic_and_data_independent():
    a = B.decode_plan(16, 1, 2048, 1024, num_cus=256)
    b = B.decode_plan(16, 1, 2048, 1024, num_cus=256)
    assert bytes(a) == bytes(b)


def test_forced_splits_and_edge_shapes():
    p = B.decode_plan(1, 1, 200, 8, num_cus=256, force_splits=7)
    assert p.num_splits == 7 and p.tokens_per_split == 32
    p = B.decode_plan(1, 1, 200, 8, num_cus=256, force_splits=1000)
    assert p.num_splits == 7                      # never more parts than tiles
    p = B.decode_plan(1, 1, 0, 8, num_cus=256)
    assert p.num_splits == 1 and p.workspace_bytes == 0
    p = B.decode_plan(0, 1, 64, 8, num_cus=256)
    assert p.rows == 0 and p.num_workgroups == 0
    p = B.decode_plan(1, 1, 100000, 4096, num_cus=256, force_splits=1)
    assert p.num_splits > 1, "a part must fit the LDS row table"


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=32), 2), (dict(d_qk=512), 2), (dict(d_v=448), 2), (dict(block_size=32), 2),
    (dict(kv_format=7), 2), (dict(q_len=0), 1), (dict(topk=-1), 1), (dict(max_blocks_per_seq=0), 1),
    (dict(kv_format=2), 2),                        # the pages' layout is 512 wide
    (dict(kv_format=2, d_qk=512, d_v=448), 2),
])
def test_plan_rejects(kw, status):
    args = dict(batch=2, q_len=1, topk=64, max_blocks_per_seq=8, kv_format=0, num_cus=256)
    args.update(kw)
    with pytest.raises(B.SmlaError) as e:
        B.decode_plan(**args)
    assert e.value.status == status


ENTRY = "smla_decode_run"


def _run(plan, **kw):
    lib = B.load()
    args = dict(q=1 << 20, kv=1 << 21, nb=16, bt=1 << 22, idx=1 << 23, sl=None, scale=0.04, out=1 << 24,
                lse=1 << 25, ws=None, wsb=0)
    args.update(kw)
    return getattr(lib, ENTRY)(ctypes.byref(plan) if plan is not None else None, args["q"], args["kv"], args["nb"],
                               args["bt"], args["idx"], args["sl"], args["scale"], args["out"], args["lse"],
                               args["ws"], args["wsb"], None)


@pytest.mark.parametrize("entry", ["smla_decode_run", "smla_decode_partial"])
def test_run_argument_checks_need_no_gpu(entry, monkeypatch):
    monkeypatch.setitem(globals(), "ENTRY", entry)
    plan = B.decode_plan(2, 1, 256, 8, num_cus=256)
    assert plan.workspace_bytes > 0
    assert _run(None) == 1
    assert _run(plan, q=None) == 1
    assert _run(plan, nb=-1) == 1
    assert _run(plan, kv=None) == 1
    assert _run(plan, scale=float("nan")) == 1
    assert _run(plan) == 3                                   # no workspace
    assert _run(plan, ws=1 << 26, wsb=plan.workspace_bytes - 1) == 3
    assert _run(plan, ws=(1 << 26) + 16, wsb=plan.workspace_bytes) == 1   # misaligned
    bad = B.Plan.from_buffer_copy(bytes(plan))
    bad.num_splits += 1
    assert _run(bad) == 1                                    # edited plan
    empty = B.decode_plan(0, 1, 256, 8, num_cus=256)
    assert _run(empty, q=None, out=None) == 0                # nothing to do
    ws = dict(ws=1 << 26, wsb=plan.workspace_bytes)
    for name, off in (("q", 8), ("kv", 4), ("out", 8), ("lse", 2), ("bt", 2), ("idx", 1), ("sl", 2)):
        base = {"sl": 1 << 27}.get(name, None)
        base = base if base is not None else {"q": 1 << 20, "kv": 1 << 21, "bt": 1 << 22, "idx": 1 << 23,
                                              "out": 1 << 24, "lse": 1 << 25}[name]
        assert _run(plan, **{name: base + off}, **ws) == 1, f"misaligned {name} accepted"
    v4 = B.decode_plan(2, 1, 256, 8, B.KV_FP8_NOPE_UE8M0, d_qk=512, num_cus=256)
    assert v4.prob.kv_format == 2 and _run(v4, q=None) == 1


def test_noalloc_argument_checks_need_no_gpu():
    lib = B.load()

    def run(plan, q=1 << 20):
        return lib.smla_decode_run_noalloc(ctypes.byref(plan) if plan is not None else None, q, 1 << 21, 16,
                                           1 << 22, 1 << 23, None, 0.04, 1 << 24, 1 << 25, None)
    assert run(None) == 1
    one = B.decode_plan(2, 1, 256, 8, num_cus=256, force_splits=1)
    assert one.workspace_bytes == 0 and run(one, q=None) == 1          # checked like smla_decode_run
    big = B.decode_plan(256, 1, 2048, 1024, num_cus=256, force_splits=2)
    assert big.workspace_bytes > (16 << 20) and run(big) == 3           # beyond the scratch array


def test_combine_argument_checks_need_no_gpu():
    lib = B.load()
    assert lib.smla_combine(1 << 20, 1 << 21, 0, 1, 64, 512, 1 << 22, 1 << 23, None) == 1
    assert lib.smla_combine(1 << 20, 1 << 21, 2, 1, 64, 510, 1 << 22, 1 << 23, None) == 2
    assert lib.smla_combine(None, None, 2, 0, 64, 512, None, None, None) == 0
    assert lib.smla_combine(None, 1 << 21, 2, 1, 64, 512, 1 << 22, 1 << 23, None) == 1
    assert lib.smla_combine((1 << 20) + 8, 1 << 21, 2, 1, 64, 512, 1 << 22, 1 << 23, None) == 1  # misaligned
    assert lib.smla_combine(1 << 20, 1 << 21, 2, 1, 64, 512, (1 << 22) + 8, 1 << 23, None) == 1


def test_indexer_argument_checks_need_no_gpu():
    lib = B.load()
    assert B.indexer_workspace_size(3, 2, 10) == 3 * 2 * 640 * 4
    assert B.indexer_workspace_size(1, 1, 256) == 16384 * 4              # the one-kernel selection
    # rows of more than 16,384 positions: scores, then per chunk of 4096 positions a histogram of 4352
    # u16 counts and 16 bytes of counts, 16 bytes per row, and a candidate list as long as the row
    rows, cap, nch = 2, 300 * 64, 5
    assert B.indexer_workspace_size(2, 1, 300) == rows * cap * 4 + rows * nch * (4352 * 2 + 16) + rows * 16 + rows * cap * 4
    n = ctypes.c_uint64(0)
    assert lib.smla_indexer_workspace_size(-1, 1, 64, 10, ctypes.byref(n)) == 1
    assert lib.smla_indexer_workspace_size(1, 1, 64, 10, None) == 1

    def call(**kw):
        a = dict(q=1 << 20, d=128, k=1 << 21, nb=16, bt=1 << 22, sl=1 << 23, B=2, Q=1, bs=64, mb=8, topk=64,
                 oi=1 << 24, os=1 << 25, ws=1 << 26, wsb=2 * 512 * 4)
        a.update(kw)
        return lib.smla_indexer_topk(a["q"], a["d"], a["k"], a["nb"], a["bt"], a["sl"], a["B"], a["Q"], a["bs"],
                                     a["mb"], a["topk"], a["oi"], a["os"], a["ws"], a["wsb"], None)
    assert call(d=64) == 2 and call(bs=32) == 2 and call(topk=4096) == 2 and call(Q=5) == 2
    assert call(topk=-1) == 1 and call(mb=0) == 1 and call(nb=-1) == 1
    assert call(q=None) == 1 and call(sl=None) == 1 and call(oi=None) == 1
    assert call(wsb=2 * 512 * 4 - 1) == 3 and call(ws=None) == 3
    long_ws = B.indexer_workspace_size(2, 1, 300)                       # chunked selection: its buffers count
    assert call(mb=300, wsb=long_ws - 1) == 3 and call(mb=300, wsb=2 * 300 * 64 * 4) == 3
    assert call(q=(1 << 20) + 8) == 1 and call(k=(1 << 21) + 4) == 1 and call(oi=(1 << 24) + 2) == 1
    assert call(B=0, q=None, oi=None) == 0 and call(topk=0, oi=None) == 0   # nothing to do
    assert call(topk=0, q=None) == 1                                          # still checked
    assert lib.smla_indexer_scores(1 << 20, 128, 1 << 21, 16, 1 << 22, 1 << 23, 2, 1, 64, 8, None, None) == 1
    assert lib.smla_indexer_scores(1 << 20, 128, 1 << 21, 16, 1 << 22, 1 << 23, 2, 1, 64, 8, (1 << 24) + 2,
                                   None) == 1
    assert lib.smla_indexer_scores(1 << 20, 96, 1 << 21, 16, 1 << 22, 1 << 23, 2, 1, 64, 8, 1 << 24, None) == 2
