"""Python access to the fp64 CPU oracle (``oracle.c``).

Test infrastructure only: the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it; the GPU library never does.  Everything here is
argument marshalling around the C functions, plus ``build()`` which compiles
``oracle.c`` with gcc into ``liboracle.so`` next to it.

Functions (see ``oracle.c`` for the definitions and the passages they follow):

* ``bf16_to_f64``, ``e4m3fn_to_f64``, ``ue8m0_to_f64`` -- exact decoding of
  the input formats;
* ``sparse_mla_decode`` -- out/lse of sparse softmax attention per head;
* ``lse_combine`` -- merge of partial (out, lse) pairs over parts of a list;
* ``indexer_scores``, ``indexer_topk`` -- the top-k indexer that produces the
  index lists (scores of every position, and the selection).

``Oracle(path)`` wraps any compiled copy of the source (the tests use this to
show that planted mistakes are caught); the module-level functions use the
library built from ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

KV_BF16 = 0
KV_FP8 = 1
KV_FP8_NOPE_UE8M0 = 2


def build(force: bool = True, src: str = SOURCE, out_path: str = LIB_PATH, sanitize: bool = False) -> str:
    """Compile an oracle source (IEEE arithmetic: no fast-math, no FMA contraction).  With sanitize,
    AddressSanitizer and UndefinedBehaviorSanitizer instrument it (the runtime must be preloaded into the
    process that loads it)."""
    if force or not os.path.exists(out_path):
        tmp = out_path + ".tmp"
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               *(san if sanitize else []), "-o", tmp, src, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out_path)
    return out_path


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_f32_array_to_f64.argtypes = [i64, P, P]
    lib.oracle_f32_array_to_f64.restype = None
    lib.oracle_bf16_array_to_f64.argtypes = [i64, P, P]
    lib.oracle_bf16_array_to_f64.restype = None
    lib.oracle_e4m3fn_array_to_f64.argtypes = [i64, P, P]
    lib.oracle_e4m3fn_array_to_f64.restype = None
    lib.oracle_ue8m0_array_to_f64.argtypes = [i64, P, P]
    lib.oracle_ue8m0_array_to_f64.restype = None
    lib.oracle_row_bytes.argtypes = [i32, i32, i32]
    lib.oracle_row_bytes.restype = i64
    lib.oracle_block_bytes.argtypes = [i32, i32, i32, i32]
    lib.oracle_block_bytes.restype = i64
    lib.oracle_sparse_mla_decode.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i64, i32,
                                             P, P, P, P, P, f64, P, P, i32]
    lib.oracle_sparse_mla_decode.restype = ctypes.c_int
    lib.oracle_lse_combine.argtypes = [i32, i64, i32, P, P, P, P]
    lib.oracle_lse_combine.restype = ctypes.c_int
    lib.oracle_indexer_scores.argtypes = [i32, i32, i32, i32, i32, i64, P, P, P, P, P, P]
    lib.oracle_indexer_scores.restype = ctypes.c_int
    lib.oracle_indexer_topk.argtypes = [i32, i32, i32, i32, i32, i64, P, P, P, P, i32, P, P]
    lib.oracle_indexer_topk.restype = ctypes.c_int
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """The oracle functions of one compiled oracle library."""

    def __init__(self, path: str):
        self.path = path
        self.lib = _bind(path)

    def f32_to_f64(self, words: np.ndarray) -> np.ndarray:
        """Little-endian binary32 bit patterns (uint32) -> float64, by the oracle's own decoder."""
        words = np.ascontiguousarray(words, dtype='<u4')
        out = np.empty(words.shape, dtype=np.float64)
        self.lib.oracle_f32_array_to_f64(words.size, _ptr(words), _ptr(out))
        return out

    def bf16_to_f64(self, bits: np.ndarray) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.oracle_bf16_array_to_f64(bits.size, _ptr(bits), _ptr(out))
        return out

    def e4m3fn_to_f64(self, codes: np.ndarray) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(codes.shape, dtype=np.float64)
        self.lib.oracle_e4m3fn_array_to_f64(codes.size, _ptr(codes), _ptr(out))
        return out

    def ue8m0_to_f64(self, codes: np.ndarray) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(codes.shape, dtype=np.float64)
        self.lib.oracle_ue8m0_array_to_f64(codes.size, _ptr(codes), _ptr(out))
        return out

    def row_bytes(self, kv_format: int, d_qk: int, d_v: int) -> int:
        return int(self.lib.oracle_row_bytes(kv_format, d_qk, d_v))

    def block_bytes(self, kv_format: int, block_size: int, d_qk: int, d_v: int) -> int:
        return int(self.lib.oracle_block_bytes(kv_format, block_size, d_qk, d_v))

    def sparse_mla_decode(self, q_bits, kv_cache, block_table, indices, seq_lens, softmax_scale, *,
                          d_v: int, kv_format: int, block_size: int, threads: int = 1):
        """fp64 (out [B, q_len, H, d_v], lse [B, q_len, H]).

        q_bits: uint16 [B, q_len, H, d_qk] (bf16 bit patterns); kv_cache: uint8
        [num_blocks, ...] with block_bytes per block; block_table: int32 [B,
        max_blocks]; indices: int32 [B, q_len, topk]; seq_lens: int32 [B] or None.
        """
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        B, q_len, H, d_qk = q_bits.shape
        kv_cache = np.ascontiguousarray(kv_cache, dtype=np.uint8)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        indices = np.ascontiguousarray(indices, dtype=np.int32)
        if indices.ndim != 3 or indices.shape[:2] != (B, q_len):
            raise ValueError(f"indices shape {indices.shape} does not match q {q_bits.shape}")
        if block_table.ndim != 2 or block_table.shape[0] != B:
            raise ValueError(f"block_table shape {block_table.shape} does not match batch {B}")
        bb = self.block_bytes(kv_format, block_size, d_qk, d_v)
        if bb < 0 or kv_cache.ndim < 2 or kv_cache[0].size != bb:
            raise ValueError(f"kv_cache shape {kv_cache.shape} does not match {bb} bytes per block "
                             f"(format {kv_format}, block_size {block_size})")
        if seq_lens is not None:
            seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
            if seq_lens.shape != (B,):
                raise ValueError("seq_lens must have shape [B]")
        topk = indices.shape[2]
        out = np.empty((B, q_len, H, d_v), dtype=np.float64)
        lse = np.empty((B, q_len, H), dtype=np.float64)
        rc = self.lib.oracle_sparse_mla_decode(B, q_len, H, d_qk, d_v, topk, block_size, block_table.shape[1],
                                               kv_cache.shape[0], kv_format, _ptr(q_bits), _ptr(kv_cache),
                                               _ptr(block_table), _ptr(indices), _ptr(seq_lens),
                                               float(softmax_scale), _ptr(out), _ptr(lse), int(threads))
        if rc != 0:
            raise RuntimeError(f"oracle_sparse_mla_decode failed with code {rc}")
        return out, lse

    def lse_combine(self, part_out, part_lse):
        """Merge S partial results: part_out [S, ..., d_v], part_lse [S, ...] -> (out, lse) in fp64."""
        part_out = np.ascontiguousarray(part_out, dtype=np.float64)
        part_lse = np.ascontiguousarray(part_lse, dtype=np.float64)
        S = part_out.shape[0]
        d_v = part_out.shape[-1]
        if part_lse.shape != part_out.shape[:-1]:
            raise ValueError("part_lse must match part_out without its last axis")
        n = int(np.prod(part_out.shape[1:-1], dtype=np.int64))
        out = np.empty(part_out.shape[1:], dtype=np.float64)
        lse = np.empty(part_lse.shape[1:], dtype=np.float64)
        rc = self.lib.oracle_lse_combine(S, n, d_v, _ptr(part_out), _ptr(part_lse), _ptr(out), _ptr(lse))
        if rc != 0:
            raise RuntimeError(f"oracle_lse_combine failed with code {rc}")
        return out, lse

    def _indexer_args(self, q_idx, k_cache, block_table, seq_lens, block_size):
        q_idx = np.ascontiguousarray(q_idx, dtype=np.uint16)
        B, q_len, d_idx = q_idx.shape
        k_cache = np.ascontiguousarray(k_cache, dtype=np.uint16)
        if k_cache.ndim != 3 or k_cache.shape[1] != block_size or k_cache.shape[2] != d_idx:
            raise ValueError(f"k_cache shape {k_cache.shape} does not match block_size {block_size}, d_idx {d_idx}")
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        if block_table.ndim != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
            raise ValueError("block_table [B, max_blocks] and seq_lens [B] required")
        return q_idx, k_cache, block_table, seq_lens, B, q_len, d_idx

    def indexer_scores(self, q_idx, k_cache, block_table, seq_lens, *, block_size: int = 64):
        """fp64 (scores, abs_sums) [B, q_len, block_size * max_blocks]; -inf / 0 where not a candidate."""
        q_idx, k_cache, block_table, seq_lens, B, q_len, d_idx = self._indexer_args(q_idx, k_cache, block_table,
                                                                                    seq_lens, block_size)
        cap = block_size * block_table.shape[1]
        sc = np.empty((B, q_len, cap), dtype=np.float64)
        ab = np.empty((B, q_len, cap), dtype=np.float64)
        rc = self.lib.oracle_indexer_scores(B, q_len, d_idx, block_size, block_table.shape[1], k_cache.shape[0],
                                            _ptr(q_idx), _ptr(k_cache), _ptr(block_table), _ptr(seq_lens),
                                            _ptr(sc), _ptr(ab))
        if rc != 0:
            raise RuntimeError(f"oracle_indexer_scores failed with code {rc}")
        return sc, ab

    def indexer_topk(self, q_idx, k_cache, block_table, seq_lens, topk: int, *, block_size: int = 64):
        """(indices int32 [B, q_len, topk], scores fp64 [B, q_len, topk]); -1 / -inf past the candidates."""
        q_idx, k_cache, block_table, seq_lens, B, q_len, d_idx = self._indexer_args(q_idx, k_cache, block_table,
                                                                                    seq_lens, block_size)
        idx = np.empty((B, q_len, topk), dtype=np.int32)
        sc = np.empty((B, q_len, topk), dtype=np.float64)
        rc = self.lib.oracle_indexer_topk(B, q_len, d_idx, block_size, block_table.shape[1], k_cache.shape[0],
                                          _ptr(q_idx), _ptr(k_cache), _ptr(block_table), _ptr(seq_lens), int(topk),
                                          _ptr(idx), _ptr(sc))
        if rc != 0:
            raise RuntimeError(f"oracle_indexer_topk failed with code {rc}")
        return idx, sc

    def decode_inputs(self, inp, indices=None, threads: int = 1, with_seq_lens: bool = True):
        """Oracle on an ``Inputs`` object of the seeded generator."""
        w = inp.workload
        return self.sparse_mla_decode(inp.q, inp.kv_cache, inp.block_table,
                                      inp.indices if indices is None else indices,
                                      inp.seq_lens if with_seq_lens else None, inp.softmax_scale,
                                      d_v=w.d_v, kv_format=w.kv_format, block_size=w.block_size,
                                      threads=threads)


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (rebuilt when the source is newer than the library)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
            build(force=True)
        _default = Oracle(LIB_PATH)
    return _default


def bf16_to_f64(bits):
    return default().bf16_to_f64(bits)


def e4m3fn_to_f64(codes):
    return default().e4m3fn_to_f64(codes)


def ue8m0_to_f64(codes):
    return default().ue8m0_to_f64(codes)


def row_bytes(kv_format, d_qk, d_v):
    return default().row_bytes(kv_format, d_qk, d_v)


def block_bytes(kv_format, block_size, d_qk, d_v):
    return default().block_bytes(kv_format, block_size, d_qk, d_v)


def sparse_mla_decode(*args, **kwargs):
    return default().sparse_mla_decode(*args, **kwargs)


def lse_combine(part_out, part_lse):
    return default().lse_combine(part_out, part_lse)


def decode_inputs(inp, indices=None, threads: int = 1, with_seq_lens: bool = True):
    return default().decode_inputs(inp, indices=indices, threads=threads, with_seq_lens=with_seq_lens)


def indexer_scores(*args, **kwargs):
    return default().indexer_scores(*args, **kwargs)


def indexer_topk(*args, **kwargs):
    return default().indexer_topk(*args, **kwargs)
