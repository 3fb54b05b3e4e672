#!/usr/bin/env python3
"""Benchmark: head-batched sparse MLA decode on one MI355X.

One step = one ``smla_decode_run`` call (partial-attention kernel, plus the
log-sum-exp combine kernel when the plan splits the top-k list) over one
batch of synthetic, seeded inputs already resident in HBM.  The default
workload is the largest one that fits one GPU: batch 128 with 2 query tokens
each (256 query rows), 64 heads, top-k 2048 over 65536-token paged latent
caches whose c_kv part is fp8 e4m3 with one fp32 scale per 128 values
(656-byte rows).

Timing: W eager warm-up steps, then K steps captured in one HIP graph.  The
graph is replayed several times between torch.cuda.synchronize() calls, each
replay timed with events on the stream the kernels run on, and the median
replay is reported (the graph removes host launch gaps, so the time is the
GPU's).  Cold cache: consecutive steps cycle over R copies of the cache
(R * gathered bytes >= 1 GiB, four times the 256 MB Infinity Cache), and
1 GiB of another buffer is read on the same stream before every timed
replay, so no step finds its rows cached, whatever K is.  A hot figure (every step on the same
cache copy, no flush) is reported separately and labelled.

Output: one JSON line.  ``value`` = gathered-KV GB/s of the whole call
(gathered bytes = valid selected tokens * row bytes).  ``roofline`` is for
the partial-attention kernel alone, timed the same way from a graph of K
``smla_decode_partial`` calls (the combine kernel is timed from a graph of
K ``smla_combine`` calls).  ``cpu_baseline`` times the fp64 oracle on the
host for a bounded sample.

``--workload idx_...`` measures the top-k indexer instead (one step = one
``smla_indexer_topk`` call: the score kernel streams every candidate's
indexer key, the select kernel picks the top-k per row): ``value`` = key
bytes / call time, ``roofline`` for the score kernel alone (timed from a
graph of ``smla_indexer_scores`` calls), cold cache by rotating copies of the
key cache the same way.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode µs/call + gathered-KV HBM GB/s (% peak), B=1..128, H=64"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "b128_q2_topk2048_n65536_paged_fp8"
ROTATION_BYTES = 1 << 30
FLUSH_BYTES = 1 << 30        # read before every cold replay (4x the Infinity Cache)
N_REPLAYS = 5                # timed replays of each graph; the median is reported
WARM_SECONDS = 0.05          # untimed replays of each graph before timing it
MFMA_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA peak of MI355X (both products run on bf16 MFMA)
HOST_THREADS = 16            # host cores the CPU baseline may use (the box's share per GPU)
MAX_COPY_BYTES = 48 << 30
INDEXER_METRIC = "top-k indexer µs/call + indexer-key HBM GB/s (% peak)"
KERNEL_SOURCES = ["sparse_mla_decode_smla_amd/csrc/smla_decode.hip",
                  "sparse_mla_decode_smla_amd/csrc/smla_combine.hip",
                  "sparse_mla_decode_smla_amd/csrc/smla_internal.h",
                  "sparse_mla_decode_smla_amd/csrc/smla_plan.cpp"]
INDEXER_SOURCES = ["sparse_mla_decode_smla_amd/csrc/smla_indexer.hip"]


def is_indexer(workload: str) -> bool:
    return workload.startswith("idx_")


def _code_only(text: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed (the
    sources hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(workload: str = DEFAULT_WORKLOAD) -> str:
    """Hash of the code of the kernel sources (comments and layout do not count)."""
    h = hashlib.sha256()
    for f in (INDEXER_SOURCES if is_indexer(workload) else KERNEL_SOURCES):
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(workload: str):
    """HBM bytes per partial-kernel launch from the committed counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return rec.get("bytes_per_launch")


def measured_counters(workload: str):
    """MFMA / VALU activity of the partial kernel from the committed counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return {k: rec[k] for k in ("mfma_busy_frac", "valu_busy_frac", "mfma_flops_frac_of_busy") if k in rec}


PARTIAL_KERNEL = "partial_kernel"
SCORE_KERNEL = "score_kernel"
COPY_PROBE_BYTES = 1 << 30


def copy_probe() -> int:
    """A plain streaming kernel of known size (reads and writes COPY_PROBE_BYTES each) to scale counters."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe": "bitwise_not uint8", "bytes_read": COPY_PROBE_BYTES,
                      "bytes_written": COPY_PROBE_BYTES}), flush=True)
    return 0


def _counter_means(csv_dir: str, counter: str, name_part: str) -> tuple[float, int]:
    """Mean per-dispatch value of `counter` over dispatches whose kernel name contains `name_part`."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {csv_dir}")
    per_dispatch = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                    key = (f, r["Dispatch_Id"])
                    per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    if not per_dispatch:
        raise ValueError(f"no {counter} rows for kernels matching {name_part!r} under {csv_dir}")
    vals = list(per_dispatch.values())
    return sum(vals) / len(vals), len(vals)


def traffic_summary(workload: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str,
                    copy_write_dir: str, command: str) -> int:
    """Turn FETCH_SIZE / WRITE_SIZE counter runs (KiB per dispatch) into HBM bytes per partial launch."""
    kernel = SCORE_KERNEL if is_indexer(workload) else PARTIAL_KERNEL
    fetch_kib, nf = _counter_means(fetch_dir, "FETCH_SIZE", kernel)
    write_kib, nw = _counter_means(write_dir, "WRITE_SIZE", kernel)
    # the probe's own dispatches only (not the fill that creates its input)
    cf_kib, _ = _counter_means(copy_fetch_dir, "FETCH_SIZE", "bitwise_not")
    cw_kib, _ = _counter_means(copy_write_dir, "WRITE_SIZE", "bitwise_not")
    f_scale = COPY_PROBE_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_PROBE_BYTES / (cw_kib * 1024.0)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    rec = {"workload": workload, "kernel": kernel, "kernel_source_hash": kernel_source_hash(workload),
           "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
           "bytes_per_launch": round(fetch_b + write_b), "dispatches": {"fetch": nf, "write": nw},
           "raw_kib_per_dispatch": {"FETCH_SIZE": fetch_kib, "WRITE_SIZE": write_kib},
           "copy_probe": {"bytes": COPY_PROBE_BYTES, "FETCH_SIZE_kib": cf_kib, "WRITE_SIZE_kib": cw_kib,
                          "fetch_scale": f_scale, "write_scale": w_scale},
           "command": command}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec), flush=True)
    return 0


def _counter_dispatches(csv_dir: str, name_part: str) -> dict:
    """{dispatch id: {counter: value summed over its dimensions, '_us': duration}} for matching kernels."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {csv_dir}")
    per = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if name_part not in r["Kernel_Name"]:
                    continue
                d = per.setdefault((f, r["Dispatch_Id"]), {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                d["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    if not per:
        raise ValueError(f"no dispatches of kernels matching {name_part!r} under {csv_dir}")
    return per


MI355X_XCDS = 8           # GRBM_GUI_ACTIVE is summed over the XCDs
MI355X_SIMDS = 1024       # 256 CUs x 4 SIMDs
MI355X_CUS = 256


def counter_summary(workload: str, dir_a: str, dir_b: str, command: str) -> int:
    """Activity counters of the partial kernel (two rocprofv3 --pmc passes) -> profiles/counters_<workload>.*

    Fractions follow AMD's derived metrics: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x active
    cycles), VALU busy = 4 x SQ_ACTIVE_INST_VALU (quad-cycles) / (SIMDs x active cycles), where active
    cycles = GRBM_GUI_ACTIVE / XCDs.  Means over the profiled dispatches."""
    kernel = PARTIAL_KERNEL
    a = list(_counter_dispatches(dir_a, kernel).values())
    b = list(_counter_dispatches(dir_b, kernel).values())

    def mean(rows, f):
        return sum(f(r) for r in rows) / len(rows)
    cyc = lambda r: r["GRBM_GUI_ACTIVE"] / MI355X_XCDS
    rec = {
        "workload": workload, "kernel": kernel, "kernel_source_hash": kernel_source_hash(workload),
        "dispatches": {"pass_a": len(a), "pass_b": len(b)},
        "kernel_us": round(mean(a, lambda r: r["_us"]), 3),
        "active_cycles_per_us": round(mean(a, lambda r: cyc(r) / r["_us"]), 1),
        "mfma_busy_frac": round(mean(a, lambda r: r["SQ_VALU_MFMA_BUSY_CYCLES"] / (MI355X_SIMDS * cyc(r))), 4),
        "valu_busy_frac": round(mean(a, lambda r: 4 * r["SQ_ACTIVE_INST_VALU"] / (MI355X_SIMDS * cyc(r))), 4),
        "mfma_flops_per_launch": round(mean(a, lambda r: 512 * r["SQ_INSTS_VALU_MFMA_MOPS_BF16"])),
        "mfma_flops_frac_of_busy": None,
        "insts_per_launch": {"valu": round(mean(a, lambda r: r["SQ_INSTS_VALU"])),
                             "mfma": round(mean(a, lambda r: r["SQ_INSTS_MFMA"])),
                             "valu_cvt": round(mean(b, lambda r: r["SQ_INSTS_VALU_CVT"])),
                             "lds": round(mean(b, lambda r: r["SQ_INSTS_LDS"]))},
        "lds_busy_frac": round(mean(b, lambda r: r["SQ_LDS_IDX_ACTIVE"] / (MI355X_CUS * cyc(r))), 4),
        "lds_bank_conflict_per_access": round(mean(b, lambda r: r["SQ_LDS_BANK_CONFLICT"] /
                                                   max(1.0, r["SQ_LDS_IDX_ACTIVE"] - r["SQ_LDS_BANK_CONFLICT"])), 4),
        "wave_wait_any_frac": round(mean(b, lambda r: r["SQ_WAIT_ANY"] / max(1.0, r["SQ_WAVE_CYCLES"]))
                                    if "SQ_WAVE_CYCLES" in b[0] else
                                    mean(b, lambda r: r["SQ_WAIT_ANY"] / max(1.0, r["SQ_ACTIVE_INST_ANY"] +
                                                                            r["SQ_WAIT_ANY"])), 4),
        "command": command,
    }
    # flops the busy MFMA cycles would deliver at the dense bf16 rate (16 cycles per 16x16x32 MFMA)
    busy = mean(a, lambda r: r["SQ_VALU_MFMA_BUSY_CYCLES"])
    rec["mfma_flops_frac_of_busy"] = round(rec["mfma_flops_per_launch"] / max(1.0, busy / 16 * 16384), 4)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"counters_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec), flush=True)
    return 0


def cpu_baseline(inp, gathered_bytes: int, seconds: float) -> dict:
    """The fp64 oracle on the host over a bounded sample of whole sequences of the workload, on all the
    host cores it may use (it splits its work over (query row, head range) items, so one row fills them)."""
    import oracle
    w = inp.workload
    nproc = os.cpu_count() or 1
    threads = max(1, min(nproc, HOST_THREADS))
    # bounded sample: whole sequences (all their query rows), enough of them for the threads
    nseq = max(1, min(w.batch, threads))
    sel = list(range(nseq))
    rows = nseq * w.q_len
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.default().sparse_mla_decode(inp.q[sel], inp.kv_cache, inp.block_table[sel], inp.indices[sel],
                                           inp.seq_lens[sel], inp.softmax_scale, d_v=w.d_v,
                                           kv_format=w.kv_format, block_size=w.block_size,
                                           threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    sample_bytes = inp.valid_count(inp.indices[sel], inp.seq_lens[sel]) * w.row_bytes * reps
    # one thread: the first sequence's rows, for about a fifth of the time
    t0 = time.perf_counter()
    reps1 = 0
    while True:
        oracle.default().sparse_mla_decode(inp.q[:1], inp.kv_cache, inp.block_table[:1], inp.indices[:1],
                                           inp.seq_lens[:1], inp.softmax_scale, d_v=w.d_v,
                                           kv_format=w.kv_format, block_size=w.block_size, threads=1)
        reps1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= seconds / 5 or reps1 >= 1000:
            break
    bytes1 = inp.valid_count(inp.indices[:1], inp.seq_lens[:1]) * w.row_bytes * reps1
    return {"value": round(sample_bytes / el / 1e9, 6), "unit": "GB/s", "cores": threads, "host_nproc": nproc,
            "kind": "oracle", "value_1_thread": round(bytes1 / el1 / 1e9, 6),
            "sample": f"{reps} x {nseq} sequence(s) ({rows} query rows, all 64 heads) of the workload, "
                      f"{el:.1f} s fp64 on {threads} host threads; one thread: {reps1} x sequence 0, {el1:.1f} s"}


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def _graph_timer(torch, stream, K, flush_buf=None, warm_seconds=WARM_SECONDS):
    """capture(fn) records fn(0..K-1) in one graph; time_graph(g, cold) replays it N_REPLAYS times, each
    timed with events on `stream` (with cold, `flush_buf` is read on that stream first), and
    returns (median us per step, [us per step of each replay])."""
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(K):
                    fn(i)
        return g

    def time_graph(g, cold: bool = True):
        # (a written flush would leave dirty lines whose write-back lands in the timed replay)
        # untimed replays for at least WARM_SECONDS first, each run exactly as a timed one (flush, then
        # replay): the clock and the translation caches settle under the same alternation of the
        # flush and the steps.  (With back-to-back replays alone, the first timed replays of the
        # compute-bound fp8 workload ran 10-25% slower at 20 steps per replay.)
        t0 = time.perf_counter()
        n = 0
        while n < 1 or (time.perf_counter() - t0 < warm_seconds and n < 1000):
            with torch.cuda.stream(stream):
                if cold and flush_buf is not None:
                    torch.sum(flush_buf)
                g.replay()
            torch.cuda.synchronize()
            n += 1
        per = []
        for rep in range(N_REPLAYS):
            with torch.cuda.stream(stream):
                if cold and flush_buf is not None:
                    torch.sum(flush_buf)  # reads only: the caches hold clean lines of it afterwards
                s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s0.record(stream)
                g.replay()
                s1.record(stream)
            torch.cuda.synchronize()
            per.append(s0.elapsed_time(s1) * 1e3 / K)
        return _median(per), per
    return capture, time_graph


def gather_probe(nbytes: int = 16 << 30, ntiles: int = 64, reps: int = 3) -> int:
    """Random 1152-byte rows gathered into LDS by LDS-DMA with four instruction patterns, and the kernel's
    pattern with non-temporal loads (libsmla_probe.so, no compute), at 128, 192 and 256 workgroups; one JSON
    line per (mode, workgroups) with the best of `reps`."""
    import ctypes
    import numpy as np
    import torch
    from sparse_mla_decode_smla_amd import build as Bd
    lib = ctypes.CDLL(Bd.PROBE_PATH)
    lib.smla_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    lib.smla_probe_gather.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    nrows = nbytes // 1152
    buf = torch.ones(nrows * 1152, dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(0)
    names = {0: "8 rows x 128 B, 8 lanes per row (band-major, as the kernel)", 1: "1 row x 1024 B (row-major)",
             2: "8 rows x 128 B, lanes by half band", 3: "8 rows x 128 B, lanes interleaved by row",
             4: "band-major, non-temporal loads (nt)"}
    for grid in (128, 192, 256):
        rows = torch.from_numpy(rng.integers(0, nrows, size=grid * ntiles * 32, dtype=np.int32)).to(dev)
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
        stream = torch.cuda.current_stream().cuda_stream
        for mode in range(5):
            best = float("inf")
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                rc = lib.smla_probe_gather(buf.data_ptr(), rows.data_ptr(), ntiles, mode, sink.data_ptr(), grid,
                                           stream)
                e1.record()
                torch.cuda.synchronize()
                if rc != 0:
                    raise RuntimeError(f"gather probe failed: {rc}")
                best = min(best, e0.elapsed_time(e1) * 1e-3)
            moved = grid * ntiles * 32 * 1152
            print(json.dumps({"gather_probe": names[mode], "mode": mode, "workgroups": grid, "rows": grid * ntiles * 32,
                              "us": round(best * 1e6, 1), "tb_per_s": round(moved / best / 1e12, 3),
                              "gb_per_s_per_workgroup": round(moved / grid / best / 1e9, 2)}), flush=True)
    return 0


def launch_probe(K: int = 200) -> int:
    """Time of one kernel node in a HIP graph of K back-to-back launches of an almost empty kernel
    (libsmla_probe.so: thread 0 of each workgroup stores one word): the floor that every launch of the
    decode path pays.  One JSON line per (workgroups, threads), the best of five replays."""
    import ctypes
    import torch
    from sparse_mla_decode_smla_amd import build as Bd
    lib = ctypes.CDLL(Bd.PROBE_PATH)
    lib.smla_probe_empty.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_uint, ctypes.c_void_p]
    lib.smla_probe_empty.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    for grid, threads in ((1, 64), (64, 256), (256, 512)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(K):
                    rc = lib.smla_probe_empty(sink.data_ptr(), grid, threads, i, stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"launch probe failed: {rc}")
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / K)
        print(json.dumps({"launch_probe": "graph of back-to-back almost empty kernels", "workgroups": grid,
                          "threads": threads, "us_per_kernel_node": round(best, 3)}), flush=True)
    return 0


def stream_read_gbs(torch, dev, nbytes: int = 4 << 30, grid: int = 8192) -> tuple[float, str]:
    """Measured read bandwidth of a plain streaming kernel (libsmla_probe.so: one pass of 16-byte
    non-temporal loads over nbytes), the best of five timed calls: a second denominator next to the
    8 TB/s peak."""
    import ctypes
    from sparse_mla_decode_smla_amd import build as Bd
    lib = ctypes.CDLL(Bd.PROBE_PATH)
    lib.smla_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p]
    lib.smla_probe_stream_read.restype = ctypes.c_int
    x = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(grid * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.smla_probe_stream_read(x.data_ptr(), nbytes, sink.data_ptr(), grid, stream)
        if rc != 0:
            raise RuntimeError(f"stream-read probe failed: {rc}")
    launch()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del x, sink
    return nbytes / best / 1e9, f"stream-read probe over {nbytes >> 20} MiB ({grid} x 256 lanes), best of 5"


def bench_indexer(args) -> int:
    import numpy as np
    import torch

    from sparse_mla_decode_smla_amd import binding as B
    from sparse_mla_decode_smla_amd import inputs as I

    w = I.INDEXER_WORKLOADS_BY_NAME[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name}")
    inp = I.make_indexer_inputs(w)
    key_bytes = inp.candidate_count() * 2 * w.d_idx          # each candidate's key, read once per sequence
    q, k, bt, sl = B.indexer_to_device(inp, device=dev)
    mb = bt.shape[1]
    R = max(2, min(math.ceil(ROTATION_BYTES / key_bytes), MAX_COPY_BYTES // max(k.numel() * 2, 1), 64))
    log(f"[bench] key bytes {key_bytes}, key-cache copies for rotation: {R}")
    copies = [k] + [k.clone() for _ in range(R - 1)]
    idx = torch.empty((w.batch, w.q_len, w.topk), dtype=torch.int32, device=dev)
    sc = torch.empty((w.batch, w.q_len, w.topk), dtype=torch.float32, device=dev)
    ws = torch.empty(B.indexer_workspace_size(w.batch, w.q_len, mb), dtype=torch.uint8, device=dev)
    scores = ws.view(torch.float32)

    def step(i):
        B.indexer_topk(q, copies[i % R], bt, sl, w.topk, out_indices=idx, out_scores=sc, workspace=ws)

    def step_scores(i):
        B.indexer_scores(q, copies[i % R], bt, sl, scores)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ref_idx = idx.clone()
    K = args.steps
    stream = torch.cuda.Stream(device=dev)
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    capture, time_graph = _graph_timer(torch, stream, K, flush_buf, args.warm_seconds)
    g = capture(step)
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(idx, ref_idx):
        log("[bench] graph replay result differs from the eager result")
        return 1
    call_us, _ = time_graph(g)
    del g
    score_us, _ = time_graph(capture(step_scores))
    gbs = key_bytes / (call_us * 1e-6) / 1e9
    kernel_gbs = key_bytes / (score_us * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle  # the CPU baseline leg only
        log("[bench] timing the oracle on the host")
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.indexer_topk(inp.q_idx[:1], inp.k_cache, inp.block_table[:1], inp.seq_lens[:1], w.topk)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or reps >= 1000:
                break
        sample = int(min(inp.seq_lens[0], 64 * mb)) * 2 * w.d_idx * w.q_len * reps
        cpu = {"value": round(sample / el / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} x sequence 0 ({w.q_len} query row(s)) of the workload, {el:.1f} s fp64 on the "
                         "host (scores and selection)"}
    line = {
        "metric": INDEXER_METRIC,
        "value": round(gbs, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(call_us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_len": w.q_len, "topk": w.topk, "d_idx": w.d_idx,
                   "seq_len": w.seq_len if w.seq_len else list(w.seq_len_range), "key_bytes": key_bytes,
                   "cache": f"cold: steps cycle over {R} key-cache copies ({min(K, R)} per replay), "
                            f"{FLUSH_BYTES >> 20} MiB read before each timed replay"},
        "us_per_call": round(call_us, 3),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "kernels_us": {"score": round(score_us, 3), "select (call minus score)": round(call_us - score_us, 3)},
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kernel_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--warm-seconds", type=float, default=WARM_SECONDS,
                    help="untimed replays of each graph before its timed replays (clock and caches settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--force-splits", type=int, default=0, help="override the planned split count (sweeps)")
    ap.add_argument("--cache-policy", default="auto", choices=["auto", "cached", "stream-rows", "stream-out",
                                                                "stream-both"],
                    help="cache hints of the row gathers and result stores (auto: the plan's choice)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain streaming kernel of known size (counter calibration)")
    ap.add_argument("--launch-probe", action="store_true",
                    help="time one node of a HIP graph of almost empty kernels (the per-launch floor)")
    ap.add_argument("--gather-probe", action="store_true",
                    help="run only the row-gather probe (LDS-DMA instruction patterns, no compute)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                            "COPY_WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc csv output directories")
    ap.add_argument("--traffic-command", default="", help="the profiling command, recorded in the summary")
    ap.add_argument("--counter-summary", nargs=2, metavar=("PASS_A_DIR", "PASS_B_DIR"),
                    help="write profiles/counters_<workload>.json from the two rocprofv3 --pmc activity passes")
    args = ap.parse_args()

    if args.traffic_summary:
        return traffic_summary(args.workload, *args.traffic_summary, command=args.traffic_command)
    if args.counter_summary:
        return counter_summary(args.workload, *args.counter_summary, command=args.traffic_command)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2
    if args.copy_probe:
        return copy_probe()
    if args.gather_probe:
        return gather_probe()
    if args.launch_probe:
        return launch_probe()

    import numpy as np
    import torch

    from sparse_mla_decode_smla_amd import binding as B
    from sparse_mla_decode_smla_amd import inputs as I

    if is_indexer(args.workload):
        return bench_indexer(args)
    w = I.WORKLOADS_BY_NAME[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name}")
    inp = I.make_inputs(w, seed=0)
    gathered = inp.valid_count() * w.row_bytes
    q, kv, bt, idx, sl = B.to_device(inp, device=dev)
    plan = B.decode_plan(w.batch, w.q_len, w.topk, inp.block_table.shape[1], w.kv_format, d_qk=w.d_qk,
                         force_splits=args.force_splits, cache_policy=B.CACHE_POLICY_NAMES[args.cache_policy])
    out = torch.empty((w.batch, w.q_len, w.num_heads, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.q_len, w.num_heads), dtype=torch.float32, device=dev)
    ws = B.alloc_workspace(plan, dev)

    cache_bytes = kv.numel()
    R = max(2, math.ceil(ROTATION_BYTES / max(gathered, 1)))
    R = min(R, max(2, MAX_COPY_BYTES // max(cache_bytes, 1)), 1024)
    log(f"[bench] plan splits={plan.num_splits} tokens/split={plan.tokens_per_split} "
        f"workgroups={plan.num_workgroups}; cache copies for rotation: {R}")
    copies = [kv] + [kv.clone() for _ in range(R - 1)]
    scale = inp.softmax_scale

    def step(i):
        B.decode_run(plan, q, copies[i % R], bt, idx, sl, scale, out, lse, ws)

    def step_partial(i):
        B.decode_partial(plan, q, copies[i % R], bt, idx, sl, scale, out, lse, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()

    # eager per-call time (includes host launch gaps), for reference only
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_eager = min(args.steps, 100)
    e0.record()
    for i in range(n_eager):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / n_eager

    K = args.steps
    stream = torch.cuda.Stream(device=dev)
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    capture, time_graph = _graph_timer(torch, stream, K, flush_buf, args.warm_seconds)

    graph = capture(step)
    graph.replay()
    torch.cuda.synchronize()
    if not (torch.equal(out, ref_out) and torch.equal(lse, ref_lse)):
        log("[bench] graph replay result differs from the eager result")
        return 1
    call_us, call_reps = time_graph(graph)
    del graph

    # the partial-attention kernel alone (the dominant kernel), then the combine alone
    partial_us, partial_reps = time_graph(capture(step_partial))
    combine_us = 0.0
    if plan.num_splits > 1:
        part_out, part_lse = B.workspace_parts(plan, ws)
        out2 = torch.empty_like(out).view(plan.rows, w.num_heads, w.d_v)
        lse2 = torch.empty_like(lse).view(plan.rows, w.num_heads)
        combine_us, _ = time_graph(capture(lambda i: B.combine(part_out, part_lse, out2, lse2)))
    # hot: every step on the same cache copy, no flush (the rows stay in the caches)
    hot_call_us, _ = time_graph(capture(lambda i: B.decode_run(plan, q, kv, bt, idx, sl, scale, out, lse, ws)),
                                cold=False)
    hot_partial_us, _ = time_graph(capture(lambda i: B.decode_partial(plan, q, kv, bt, idx, sl, scale, out, lse,
                                                                       ws)), cold=False)
    del copies
    read_gbs, read_how = stream_read_gbs(torch, dev)

    gbs = gathered / (call_us * 1e-6) / 1e9
    kernel_gbs = gathered / (partial_us * 1e-6) / 1e9
    traffic = measured_traffic(w.name)
    flops = inp.valid_count() * 2 * w.num_heads * (w.d_qk + w.d_v)   # QK^T + PV per valid (row, token)
    kernel_tflops = flops / (partial_us * 1e-6) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        cpu = cpu_baseline(inp, gathered, args.cpu_seconds)

    fmt_name = {I.KV_BF16: "bf16", I.KV_FP8: "fp8e4m3+bf16",
                I.KV_FP8_NOPE_UE8M0: "fp8e4m3(ue8m0/64)+bf16 rope, 584 B/token pages"}[w.kv_format]
    touched = min(K, R)
    line = {
        "metric": METRIC,
        "value": round(gbs, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(call_us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_format == I.KV_BF16 else "fp8e4m3/bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_len": w.q_len, "heads": w.num_heads,
                   "topk": w.topk, "seq_len": w.seq_len if w.seq_len else list(w.seq_len_range),
                   "kv_format": fmt_name, "row_bytes": w.row_bytes, "gathered_bytes": gathered,
                   "splits": plan.num_splits, "tokens_per_split": plan.tokens_per_split,
                   "workgroups": plan.num_workgroups,
                   "cache_policy": {v: k for k, v in B.CACHE_POLICY_NAMES.items()}[plan.cache_policy],
                   "cache": f"cold: steps cycle over {R} cache copies ({touched} per replay), "
                            f"{FLUSH_BYTES >> 20} MiB read before each timed replay"},
        "us_per_call": round(call_us, 3),
        "us_per_call_replays": [round(x, 3) for x in call_reps],
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_call_eager": round(eager_us, 3),
        "kernels_us": {"partial": round(partial_us, 3), "combine": round(combine_us, 3)},
        "partial_us_replays": [round(x, 3) for x in partial_reps],
        "hot": {"us_per_call": round(hot_call_us, 3), "partial_us": round(hot_partial_us, 3),
                "note": "every step on the same cache copy, no flush: rows served from the caches"},
        "stream_read": {"gbs": round(read_gbs, 1), "how": read_how,
                        "partial_frac": round(kernel_gbs / read_gbs, 4)},
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kernel_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "mfma": {"achieved": round(kernel_tflops, 3), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(kernel_tflops / MFMA_PEAK_TFLOPS, 4),
                              "counters": measured_counters(w.name)}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
