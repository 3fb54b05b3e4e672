"""smla_decode_run_noalloc against smla_decode_run (GPU).

The allocation-free entry point runs the same kernels with the split partial
results in the library's own device scratch array instead of a caller's
workspace, so its output must equal smla_decode_run's bit for bit.  Calls
follow one another on one stream, each with a different (and the second a
smaller) problem, so a later call reads only what it wrote itself.
"""
import pytest
import torch

from sparse_mla_decode_smla_amd import binding as B
from sparse_mla_decode_smla_amd import inputs as I

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20


def _run_both(inp, force_splits):
    w = inp.workload
    dev = torch.device("cuda:0")
    q, kv, bt, idx, sl = B.to_device(inp, device=dev)
    plan = B.decode_plan(w.batch, w.q_len, w.topk, inp.block_table.shape[1], w.kv_format, d_qk=w.d_qk,
                         force_splits=force_splits)
    assert plan.workspace_bytes <= SCRATCH_BYTES
    shape_o, shape_l = (w.batch, w.q_len, w.num_heads, w.d_v), (w.batch, w.q_len, w.num_heads)
    out_a = torch.full(shape_o, float("nan"), dtype=torch.bfloat16, device=dev)
    lse_a = torch.full(shape_l, float("nan"), dtype=torch.float32, device=dev)
    out_b, lse_b = torch.full_like(out_a, float("nan")), torch.full_like(lse_a, float("nan"))
    ws = B.alloc_workspace(plan, dev)
    B.decode_run(plan, q, kv, bt, idx, sl, inp.softmax_scale, out_a, lse_a, ws)
    B.decode_run_noalloc(plan, q, kv, bt, idx, sl, inp.softmax_scale, out_b, lse_b)
    torch.cuda.synchronize()
    return plan, (out_a, lse_a), (out_b, lse_b)


@pytest.mark.parametrize("fmt", [I.KV_BF16, I.KV_FP8, I.KV_FP8_NOPE_UE8M0])
def test_noalloc_matches_run_on_two_calls(fmt):
    torch.cuda.set_device(0)
    # first call: 64 query rows in 3 parts (12.6 MB of partial results), then a smaller one
    big = I.small_inputs(batch=32, q_len=2, topk=1024, seq_len=2048, kv_format=fmt, seed=60 + fmt)
    small = I.small_inputs(batch=1, q_len=1, topk=300, seq_len=512, kv_format=fmt, seed=70 + fmt)
    for inp, splits in ((big, 3), (small, 5)):
        plan, (oa, la), (ob, lb) = _run_both(inp, splits)
        assert plan.num_splits == splits and plan.workspace_bytes > 0
        assert torch.equal(oa, ob), f"out differs (format {fmt}, rows {plan.rows}, parts {splits})"
        assert torch.equal(la, lb), f"lse differs (format {fmt}, rows {plan.rows}, parts {splits})"
        assert torch.isfinite(la).all()


def test_noalloc_one_part_and_too_large_plan():
    torch.cuda.set_device(0)
    inp = I.small_inputs(batch=2, q_len=1, topk=200, seq_len=640, kv_format=I.KV_BF16, seed=80)
    plan, (oa, la), (ob, lb) = _run_both(inp, 1)
    assert plan.num_splits == 1 and plan.workspace_bytes == 0
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    # a plan whose partial results exceed the scratch array is refused before anything runs
    big = B.decode_plan(256, 1, 2048, 1024, I.KV_BF16, force_splits=2)
    assert big.workspace_bytes > SCRATCH_BYTES
    dev = torch.device("cuda:0")
    t = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(B.SmlaError) as e:
        B.decode_run_noalloc(big, t, t, t.view(torch.int32), t.view(torch.int32), None, 1.0, t,
                             t.view(torch.float32))
    assert e.value.status == 3
