"""The oracle's result does not depend on how its work is spread over threads.

Work items are a query row and a range of its heads; with fewer rows than
threads a row's heads are cut into ranges.  Each (row, head) pair is computed
by the same arithmetic whatever the split, so the outputs must be identical
bit for bit.
"""
import numpy as np

from sparse_mla_decode_smla_amd import inputs as I


def test_thread_count_does_not_change_results(oracle_lib):
    for fmt, batch, q_len in ((I.KV_BF16, 1, 1), (I.KV_FP8, 2, 2), (I.KV_FP8_NOPE_UE8M0, 1, 3)):
        inp = I.small_inputs(batch=batch, q_len=q_len, topk=70, seq_len=256, kv_format=fmt, seed=50 + fmt)
        ref_o, ref_l = oracle_lib.decode_inputs(inp, threads=1)
        for threads in (3, 8, 64, 200):
            o, l = oracle_lib.decode_inputs(inp, threads=threads)
            assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l), (fmt, threads)
