"""ctypes binding of ``libsmla.so`` (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
turns torch tensors into the pointers and sizes of the C ABI declared in
``include/smla.h`` and raises ``SmlaError`` on a non-OK status.  Names follow
the C entry points: ``decode_plan``, ``decode_run``, ``combine``.  If the
library has not been built, loading fails with an error that says so; there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmla.so")

KV_BF16 = 0
KV_FP8_E4M3_SCALE128 = 1
KV_FP8_NOPE_UE8M0 = 2

# smla_cache_policy_t
CACHE_AUTO = 0
CACHE_CACHED = 1
CACHE_STREAM_ROWS = 2
CACHE_STREAM_OUT = 3
CACHE_STREAM_BOTH = 4
CACHE_POLICY_NAMES = {"auto": CACHE_AUTO, "cached": CACHE_CACHED, "stream-rows": CACHE_STREAM_ROWS,
                      "stream-out": CACHE_STREAM_OUT, "stream-both": CACHE_STREAM_BOTH}

STATUS = {0: "SMLA_OK", 1: "SMLA_ERR_INVALID_ARG", 2: "SMLA_ERR_UNSUPPORTED",
          3: "SMLA_ERR_WORKSPACE_TOO_SMALL", 4: "SMLA_ERR_LAUNCH", 5: "SMLA_ERR_DEVICE"}


class SmlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("kv_format", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("force_splits", ctypes.c_int32), ("cache_policy", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("prob", Problem), ("rows", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("tokens_per_split", ctypes.c_int32), ("tile_tokens", ctypes.c_int32),
                ("heads_per_group", ctypes.c_int32), ("num_workgroups", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("cache_policy", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_ if f != "prob"}
        d["prob"] = {f: getattr(self.prob, f) for f, _ in Problem._fields_}
        return d


_lib = None


def load(path: Optional[str] = None):
    """Load the GPU library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m sparse_mla_decode_smla_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.smla_decode_plan.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Plan)]
    lib.smla_decode_plan.restype = ctypes.c_int
    lib.smla_decode_run.argtypes = [ctypes.POINTER(Plan), P, P, ctypes.c_int64, P, P, P, ctypes.c_float,
                                    P, P, P, ctypes.c_size_t, P]
    lib.smla_decode_run.restype = ctypes.c_int
    lib.smla_decode_run_noalloc.argtypes = [ctypes.POINTER(Plan), P, P, ctypes.c_int64, P, P, P, ctypes.c_float,
                                            P, P, P]
    lib.smla_decode_run_noalloc.restype = ctypes.c_int
    lib.smla_decode_partial.argtypes = lib.smla_decode_run.argtypes
    lib.smla_decode_partial.restype = ctypes.c_int
    lib.smla_combine.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P]
    lib.smla_combine.restype = ctypes.c_int
    lib.smla_indexer_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.POINTER(ctypes.c_uint64)]
    lib.smla_indexer_workspace_size.restype = ctypes.c_int
    lib.smla_indexer_topk.argtypes = [P, ctypes.c_int32, P, ctypes.c_int64, P, P, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_size_t, P]
    lib.smla_indexer_topk.restype = ctypes.c_int
    lib.smla_indexer_scores.argtypes = [P, ctypes.c_int32, P, ctypes.c_int64, P, P, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, P, P]
    lib.smla_indexer_scores.restype = ctypes.c_int
    lib.smla_status_string.argtypes = [ctypes.c_int]
    lib.smla_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().smla_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise SmlaError(status, where)


def decode_plan(batch: int, q_len: int, topk: int, max_blocks_per_seq: int, kv_format: int = KV_BF16, *,
                num_heads: int = 64, d_qk: int = 576, d_v: int = 512, block_size: int = 64,
                num_cus: int = 0, force_splits: int = 0, cache_policy: int = CACHE_AUTO) -> Plan:
    prob = Problem(batch, q_len, num_heads, d_qk, d_v, topk, block_size, max_blocks_per_seq, kv_format,
                   num_cus, force_splits, cache_policy)
    plan = Plan()
    _check(load().smla_decode_plan(ctypes.byref(prob), ctypes.byref(plan)), "smla_decode_plan")
    return plan


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def decode_run(plan: Plan, q, kv_cache, block_table, indices, seq_lens, softmax_scale: float, out, lse,
               workspace=None, stream=None) -> None:
    """Enqueue smla_decode_run on `stream` (default: torch's current stream)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    num_blocks = kv_cache.shape[0] if kv_cache is not None else 0
    _check(load().smla_decode_run(ctypes.byref(plan), _ptr(q), _ptr(kv_cache), num_blocks, _ptr(block_table),
                                  _ptr(indices), _ptr(seq_lens), float(softmax_scale), _ptr(out), _ptr(lse),
                                  _ptr(workspace), ws_bytes, _stream(stream)),
           "smla_decode_run")


def decode_run_noalloc(plan: Plan, q, kv_cache, block_table, indices, seq_lens, softmax_scale: float, out, lse,
                       stream=None) -> None:
    """Enqueue smla_decode_run_noalloc (split partials in the library's own device scratch array)."""
    num_blocks = kv_cache.shape[0] if kv_cache is not None else 0
    _check(load().smla_decode_run_noalloc(ctypes.byref(plan), _ptr(q), _ptr(kv_cache), num_blocks,
                                          _ptr(block_table), _ptr(indices), _ptr(seq_lens), float(softmax_scale),
                                          _ptr(out), _ptr(lse), _stream(stream)),
           "smla_decode_run_noalloc")


def decode_partial(plan: Plan, q, kv_cache, block_table, indices, seq_lens, softmax_scale: float, out, lse,
                   workspace=None, stream=None) -> None:
    """Enqueue smla_decode_partial (the partial-attention kernel alone)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    num_blocks = kv_cache.shape[0] if kv_cache is not None else 0
    _check(load().smla_decode_partial(ctypes.byref(plan), _ptr(q), _ptr(kv_cache), num_blocks, _ptr(block_table),
                                      _ptr(indices), _ptr(seq_lens), float(softmax_scale), _ptr(out), _ptr(lse),
                                      _ptr(workspace), ws_bytes, _stream(stream)),
           "smla_decode_partial")


def workspace_parts(plan: Plan, workspace):
    """Views (part_out bf16 [S, rows, H, d_v], part_lse fp32 [S, rows, H]) of a split plan's workspace."""
    import torch
    S, rows, H, dv = plan.num_splits, plan.rows, plan.prob.num_heads, plan.prob.d_v
    n_out = S * rows * H * dv
    po = workspace[: 2 * n_out].view(torch.bfloat16).view(S, rows, H, dv)
    pl = workspace[2 * n_out: 2 * n_out + 4 * S * rows * H].view(torch.float32).view(S, rows, H)
    return po, pl


def combine(part_out, part_lse, out, lse, stream=None) -> None:
    """Enqueue smla_combine: part_out [S, rows, H, d_v] bf16, part_lse [S, rows, H] fp32."""
    S, rows, H, d_v = part_out.shape
    _check(load().smla_combine(_ptr(part_out), _ptr(part_lse), S, rows, H, d_v, _ptr(out), _ptr(lse),
                               _stream(stream)),
           "smla_combine")


def alloc_workspace(plan: Plan, device):
    """A workspace tensor of the plan's size (torch allocates it; 256-byte aligned)."""
    import torch
    n = int(plan.workspace_bytes)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def to_device(inp, device="cuda", indices=None):
    """Device tensors of a generated ``inputs.Inputs`` (selected-fill caches are scattered on the device)."""
    import numpy as np
    import torch
    w = inp.workload
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(device)
    if inp.fill == "all" or w.kv_format == KV_FP8_NOPE_UE8M0:
        # (kv_format 2 blocks interleave rows and scale records: copied whole)
        kv = torch.from_numpy(inp.kv_cache).to(device)
    else:
        kv = torch.zeros(inp.kv_cache.shape, dtype=torch.uint8, device=device)
        rows = inp.filled_rows
        flat = inp.kv_cache.reshape(-1, w.row_bytes)
        step = 1 << 18
        kv_flat = kv.view(-1, w.row_bytes)
        for s in range(0, rows.size, step):
            r = torch.from_numpy(rows[s:s + step]).to(device)
            kv_flat[r] = torch.from_numpy(np.ascontiguousarray(flat[rows[s:s + step]])).to(device)
    bt = torch.from_numpy(inp.block_table).to(device)
    idx = torch.from_numpy(inp.indices if indices is None else indices).to(device)
    sl = torch.from_numpy(inp.seq_lens).to(device)
    return q, kv, bt, idx, sl


def sparse_mla_decode(q, kv_cache, block_table, indices, seq_lens, softmax_scale: float,
                      kv_format: int = KV_BF16, force_splits: int = 0, stream=None, cache_policy: int = CACHE_AUTO):
    """Plan, allocate (torch) and run; returns (out bf16 [B, q_len, H, d_v], lse fp32 [B, q_len, H])."""
    import torch
    B, q_len, H, d_qk = q.shape
    topk = indices.shape[2]
    plan = decode_plan(B, q_len, topk, block_table.shape[1], kv_format, num_heads=H, d_qk=d_qk,
                       force_splits=force_splits, cache_policy=cache_policy)
    out = torch.empty((B, q_len, H, plan.prob.d_v), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, q_len, H), dtype=torch.float32, device=q.device)
    ws = alloc_workspace(plan, q.device)
    decode_run(plan, q, kv_cache, block_table, indices, seq_lens, softmax_scale, out, lse, ws, stream)
    return out, lse


# ----------------------------------------------------------------- top-k indexer


def indexer_workspace_size(batch: int, q_len: int, max_blocks_per_seq: int, block_size: int = 64) -> int:
    n = ctypes.c_uint64(0)
    _check(load().smla_indexer_workspace_size(batch, q_len, block_size, max_blocks_per_seq, ctypes.byref(n)),
           "smla_indexer_workspace_size")
    return int(n.value)


def indexer_topk(q_idx, k_cache, block_table, seq_lens, topk: int, out_indices=None, out_scores=None,
                 workspace=None, stream=None, with_scores: bool = True):
    """Enqueue smla_indexer_topk; returns (indices int32 [B, q_len, topk], scores fp32 or None).

    q_idx bf16 [B, q_len, d_idx]; k_cache bf16 [num_blocks, 64, d_idx]; block_table int32 [B, max_blocks];
    seq_lens int32 [B].  Output and workspace tensors are allocated with torch when not given."""
    import torch
    B, q_len, d_idx = q_idx.shape
    mb = block_table.shape[1]
    if out_indices is None:
        out_indices = torch.empty((B, q_len, topk), dtype=torch.int32, device=q_idx.device)
    if out_scores is None and with_scores:
        out_scores = torch.empty((B, q_len, topk), dtype=torch.float32, device=q_idx.device)
    if workspace is None:
        workspace = torch.empty(max(indexer_workspace_size(B, q_len, mb, k_cache.shape[1]), 16), dtype=torch.uint8,
                                device=q_idx.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().smla_indexer_topk(_ptr(q_idx), d_idx, _ptr(k_cache), k_cache.shape[0], _ptr(block_table),
                                    _ptr(seq_lens), B, q_len, k_cache.shape[1], mb, topk, _ptr(out_indices),
                                    _ptr(out_scores), _ptr(workspace), ws_bytes, _stream(stream)),
           "smla_indexer_topk")
    return out_indices, out_scores


def indexer_scores(q_idx, k_cache, block_table, seq_lens, scores, stream=None) -> None:
    """Enqueue smla_indexer_scores into `scores` fp32 [B * q_len, 64 * max_blocks]."""
    B, q_len, d_idx = q_idx.shape
    _check(load().smla_indexer_scores(_ptr(q_idx), d_idx, _ptr(k_cache), k_cache.shape[0], _ptr(block_table),
                                      _ptr(seq_lens), B, q_len, k_cache.shape[1], block_table.shape[1],
                                      _ptr(scores), _stream(stream)),
           "smla_indexer_scores")


def indexer_to_device(inp, device="cuda"):
    """Device tensors (q_idx, k_cache, block_table, seq_lens) of ``inputs.IndexerInputs``."""
    import numpy as np
    import torch
    q = torch.from_numpy(inp.q_idx.view(np.int16)).view(torch.bfloat16).to(device)
    k = torch.from_numpy(inp.k_cache.view(np.int16)).view(torch.bfloat16).to(device)
    bt = torch.from_numpy(inp.block_table).to(device)
    sl = torch.from_numpy(inp.seq_lens).to(device)
    return q, k, bt, sl
