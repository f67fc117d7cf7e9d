"""GPU test of the allocation-free decode entry point
(``hipdecode_paged_attn_noalloc``), through the C ABI.

Its split partials and arrival counters live in the library's static device
array instead of a caller workspace.  Two calls in a row on one stream, the
second with a smaller batch and shorter contexts, must each give exactly what
``hipdecode_paged_attn`` gives on the same inputs with a workspace of its own
(the same kernels run in both), and so meet the oracle at the decode bars.
Both calls split every context into several partitions, so the partials and
the counters are really used, and the second call reuses the array the first
one left behind.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_gqa_amd as hd
from tests.gpu_util import DeviceCase, compare, log
from workloads import make_case

pytestmark = pytest.mark.gpu


def params_of(case, max_context_len, partition_tokens=0):
    return hd.make_params(num_seqs=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv, num_pages=case.num_pages,
                          max_blocks_per_seq=case.block_table.shape[1], max_context_len=max_context_len,
                          scale=case.scale, partition_tokens=partition_tokens,
                          out_dtype=hd.HIPDECODE_F32 if case.out_dtype == "f32" else hd.HIPDECODE_BF16)


def with_workspace(dc, params):
    c = dc.case
    out = torch.full((c.B, c.Hq, c.D), 7.0, dtype=dc.out_dtype, device="cuda")
    lse = torch.full((c.B, c.Hq), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(hd.hipdecode_workspace_bytes(params), 16) // 4 + 4, dtype=torch.int32, device="cuda")
    hd.hipdecode_paged_attn(params, dc.q, dc.k, dc.v, dc.table, dc.ctx, out, lse, ws)
    return out, lse


def test_noalloc_matches_workspace_entry_point_twice():
    big = make_case([9000, 28672, 513, 4097, 0, 16000, 1, 20000], seed=91, pool_pages=5300, poison=True)
    small = make_case([3000, 17, 2049], seed=92, pool_pages=400, poison=True)
    cases = [(big, big.max_context_len, 1024), (small, small.max_context_len, 256)]
    devs = [DeviceCase(c) for c, _, _ in cases]
    outs = []
    # both allocation-free calls back to back on one stream, no host sync between them
    for dc, (c, mcl, part) in zip(devs, cases):
        p = params_of(c, mcl, part)
        assert hd.hipdecode_partition_tokens(p) == part and hd.hipdecode_workspace_bytes(p) > 0
        out = torch.full((c.B, c.Hq, c.D), 7.0, dtype=dc.out_dtype, device="cuda")
        lse = torch.full((c.B, c.Hq), 7.0, dtype=torch.float32, device="cuda")
        log(f"[noalloc] call B={c.B} max_ctx={mcl} partition={part}")
        hd.hipdecode_paged_attn_noalloc(p, dc.q, dc.k, dc.v, dc.table, dc.ctx, out, lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    for i, (dc, (c, mcl, part), (out, lse)) in enumerate(zip(devs, cases, outs)):
        ref_o, ref_l = with_workspace(dc, params_of(c, mcl, part))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                           ref_o.view(torch.int16) if ref_o.dtype == torch.bfloat16 else ref_o.view(torch.int32)), \
            f"call {i}: out differs from hipdecode_paged_attn"
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"call {i}: lse differs"
        o_ref, l_ref = oracle.run_case(c)
        err, lerr = compare(out, lse, o_ref, l_ref, what=f"noalloc call {i}")
        log(f"[noalloc] call {i}: bit-equal to the workspace entry point; max|dout|={err:.2e} "
            f"max rel dlse={lerr:.2e}")


def test_noalloc_refuses_past_its_limits():
    c = make_case([64], seed=93, pool_pages=8)
    dc = DeviceCase(c)
    out = torch.empty((c.B, c.Hq, c.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    # 513 requests x 8 KV heads: more (request, KV head) pairs than the counter region holds
    p = hd.make_params(num_seqs=513, num_q_heads=16, num_kv_heads=8, num_pages=c.num_pages,
                       max_blocks_per_seq=c.block_table.shape[1], max_context_len=16, scale=c.scale)
    with pytest.raises(hd.HipDecodeError) as ei:
        hd.hipdecode_paged_attn_noalloc(p, dc.q, dc.k, dc.v, dc.table, dc.ctx, out, lse)
    assert ei.value.status == hd.HIPDECODE_ERR_WORKSPACE
    # partials past the array: 64 requests split 1024 ways
    p = hd.make_params(num_seqs=64, num_q_heads=16, num_kv_heads=8, num_pages=c.num_pages,
                       max_blocks_per_seq=4096, max_context_len=65536, scale=c.scale, partition_tokens=64)
    assert hd.hipdecode_check_params(p) == hd.HIPDECODE_OK
    with pytest.raises(hd.HipDecodeError) as ei:
        hd.hipdecode_paged_attn_noalloc(p, dc.q, dc.k, dc.v, dc.table, dc.ctx, out, lse)
    assert ei.value.status == hd.HIPDECODE_ERR_WORKSPACE
    log("[noalloc] calls past the static scratch refused")


def test_noalloc_graph_replays_between_other_calls():
    """The allocation-free call captured in a HIP graph and replayed three times
    with new context lengths, an eager allocation-free call of another shape
    between the replays (it shares the static array); every replay bit-equal to
    the same call made eagerly, and within the decode bars of the oracle."""
    case = make_case([9000, 9000, 9000], seed=94, pool_pages=1800)
    other = make_case([5000, 300, 12000, 64, 7000], seed=95, pool_pages=1600)
    dc, do = DeviceCase(case), DeviceCase(other)
    p = params_of(case, 9000)
    po = params_of(other, other.max_context_len)
    out = torch.empty((case.B, case.Hq, case.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.B, case.Hq), dtype=torch.float32, device="cuda")
    ctx_dev = dc.ctx.clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up outside the graph
        hd.hipdecode_paged_attn_noalloc(p, dc.q, dc.k, dc.v, dc.table, ctx_dev, out, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hd.hipdecode_paged_attn_noalloc(p, dc.q, dc.k, dc.v, dc.table, ctx_dev, out, lse)
    torch.cuda.synchronize()
    o_other = torch.empty((other.B, other.Hq, other.D), dtype=torch.bfloat16, device="cuda")
    l_other = torch.empty((other.B, other.Hq), dtype=torch.float32, device="cuda")
    ref_other = oracle.run_case(other)
    for it, lens in enumerate([[4000, 9000, 100], [8191, 17, 0], [9000, 2500, 4096]]):
        log(f"[noalloc] graph replay {it}: {lens}")
        ctx_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_case = make_case([9000, 9000, 9000], seed=94, pool_pages=1800)
        ref_case.context_lens = np.array(lens, dtype=np.int32)
        ref_out, ref_lse = oracle.run_case(ref_case)
        compare(out, lse, ref_out, ref_lse, what=f"noalloc graph replay {it}")
        eager_out = torch.empty_like(out)
        eager_lse = torch.empty_like(lse)
        hd.hipdecode_paged_attn_noalloc(p, dc.q, dc.k, dc.v, dc.table, ctx_dev, eager_out, eager_lse)
        torch.cuda.synchronize()
        assert torch.equal(eager_out, out) and torch.equal(eager_lse, lse), "replay differs from eager"
        # another shape on the same static array between the replays
        hd.hipdecode_paged_attn_noalloc(po, do.q, do.k, do.v, do.table, do.ctx, o_other, l_other)
        torch.cuda.synchronize()
        compare(o_other, l_other, *ref_other, what=f"noalloc other shape after replay {it}")
