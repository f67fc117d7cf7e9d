"""Pools past 4 GiB, on the GPU, through the C ABI.

A small case's pages are copied to the top of pools of 140,000 pages (4.6 GB
each), and its block table is shifted to match, so every page the kernels
touch sits more than 4 GiB into its pool.  Decode (three kernel variants),
the KV append, the fused append-and-attend and chunked prefill run on the big
pools; each is compared with the fp64 oracle on the small case (same logical
content, original page ids), to the same bars as the other GPU tests.  The
V rows written by the append, with no rounding in between, are compared bit
for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_gqa_amd as hd
from tests.gpu_util import DeviceCase, bits_to_bf16, compare, log, run_hip
from tests.test_gpu_prefill import check_full, run_gpu as run_prefill
from workloads import make_append_inputs, make_case, make_prefill_case

pytestmark = pytest.mark.gpu

BIG_PAGES = 140_000


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hd.library()   # fail loudly if the HIP library is missing


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def on_big_pools(case, dc: DeviceCase) -> int:
    """Move dc's pools to the top of BIG_PAGES-page pools; returns the page offset."""
    off = BIG_PAGES - case.num_pages
    page_bytes = case.page * case.Hkv * case.D * 2
    assert off * page_bytes > 2 ** 32, "the case's pages must start past 4 GiB"
    shape = (BIG_PAGES, case.page, case.Hkv, case.D)
    big_k = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    big_v = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    big_k[off:] = dc.k
    big_v[off:] = dc.v
    table = case.block_table.copy()
    table[table >= 0] += off
    dc.k, dc.v = big_k, big_v
    dc.table = torch.from_numpy(table).cuda()
    log(f"[large pool] {BIG_PAGES} pages, case pages from {off} ({off * page_bytes / 2**30:.2f} GiB)")
    return off


@pytest.mark.parametrize("waves,schedule", [(4, 0), (16, 0), (4, 1)])
def test_decode_past_4gib(waves, schedule):
    case = make_case([3000, 17, 5000, 1, 0, 2048], seed=51, poison=True)
    dc = DeviceCase(case)
    on_big_pools(case, dc)
    out, lse = run_hip(dc, workgroup_waves=waves, schedule=schedule)
    ref_out, ref_lse = oracle.run_case(case)
    err, lerr = compare(out, lse, ref_out, ref_lse, what=f"decode past 4 GiB, {waves} waves, schedule {schedule}")
    log(f"[large pool] decode {waves} waves schedule {schedule}: max|dout|={err:.2e} max rel dlse={lerr:.2e}")


def test_append_and_fused_past_4gib():
    case = make_case([700, 1, 4097, 16], seed=52, pool_pages=310)
    inputs = make_append_inputs(case, None, seed=52)
    ok, ov, oq = oracle.kv_append(inputs.k_new, inputs.v_new, case.block_table, case.context_lens, case.k_pool,
                                  case.v_pool, q=inputs.q, rope=True, theta=inputs.theta)
    ref_out, ref_lse = oracle.paged_attn(oq, ok, ov, case.block_table, case.context_lens, case.scale)

    # separate append, then attend
    dc = DeviceCase(case)
    off = on_big_pools(case, dc)
    qd = bits_to_bf16(inputs.q)
    hd.kv_append(bits_to_bf16(inputs.k_new), bits_to_bf16(inputs.v_new), dc.table, dc.ctx, dc.k, dc.v, q=qd,
                 rope_theta=inputs.theta)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(dc.v[off:]), ov), "append past 4 GiB: V pool differs"
    assert not torch.any(dc.v[:off] != 0) and not torch.any(dc.k[:off] != 0), "pages below the case were written"
    dc.q = qd
    out, lse = run_hip(dc)
    err, lerr = compare(out, lse, ref_out, ref_lse, what="append then attend past 4 GiB")
    log(f"[large pool] append then attend: max|dout|={err:.2e} max rel dlse={lerr:.2e}")

    # one fused launch
    dc2 = DeviceCase(case)
    on_big_pools(case, dc2)
    out2, lse2 = hd.paged_attn_append(bits_to_bf16(inputs.q), bits_to_bf16(inputs.k_new),
                                      bits_to_bf16(inputs.v_new), dc2.k, dc2.v, dc2.table, dc2.ctx, case.scale,
                                      max_context_len=case.max_context_len, rope_theta=inputs.theta)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(dc2.v[off:]), ov), "fused past 4 GiB: V pool differs"
    err, lerr = compare(out2, lse2, ref_out, ref_lse, what="fused append and attend past 4 GiB")
    log(f"[large pool] fused: max|dout|={err:.2e} max rel dlse={lerr:.2e}")


def test_prefill_past_4gib():
    case, inp = make_prefill_case([4000, 700, 130], [1000, 700, 129], seed=53, poison=True, extra_rows=2)
    dc = DeviceCase(case)
    on_big_pools(case, dc)
    o, l = run_prefill(case, inp, dc=dc)
    check_full(case, inp, o, l, "prefill past 4 GiB")
