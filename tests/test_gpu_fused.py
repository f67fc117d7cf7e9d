"""GPU parity of the fused decode step (``hipdecode_paged_attn_append``:
append of each request's new token and attention in one launch) against the
fp64 oracle doing the two steps in turn.

The bar is the append's and the attention's own: V pools bit-exact, K pools
bit-exact up to rounding ties of the RoPE rotation, out within 1e-2 and LSE
within 1e-4 relative of the oracle (plus the rounding-level bound).  Cases
cover a last page that is partial, full, or a single token, padding rows,
contexts long enough that the last page sits in the last of many splits,
group sizes 1, 2 and 4, 4 and 16 wavefronts, fp32 output, and RoPE off.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_gqa_amd as hd
from tests.gpu_util import DeviceCase, bits_to_bf16, compare, log
from tests.test_gpu_append import check_rotated, to_bits
from workloads import make_append_inputs, make_case

pytestmark = pytest.mark.gpu

THETA = 1e6
CTX = [300, 1, 517, 4096, 0, 2049, 16, 32, 17]


def run_case(case, inputs, *, theta, waves=0, partition=0, out_dtype=None, what=""):
    dc = DeviceCase(case)
    q = bits_to_bf16(inputs.q)
    q_before = q.clone()
    out, lse = hd.paged_attn_append(q, bits_to_bf16(inputs.k_new), bits_to_bf16(inputs.v_new), dc.k, dc.v, dc.table,
                                    dc.ctx, case.scale, max_context_len=case.max_context_len, rope_theta=theta,
                                    out_dtype=out_dtype or dc.out_dtype, partition_tokens=partition,
                                    workgroup_waves=waves)
    torch.cuda.synchronize()
    assert torch.equal(q, q_before), f"{what}: q must not be modified"
    rope = theta > 0
    kp, vp, q_rot = oracle.kv_append(inputs.k_new, inputs.v_new, case.block_table, case.context_lens, case.k_pool,
                                     case.v_pool, q=inputs.q, rope=rope, theta=theta if rope else 1e6)
    ref_out, ref_lse = oracle.paged_attn(q_rot if rope else inputs.q, kp, vp, case.block_table,
                                         case.context_lens, case.scale)
    err, lerr = compare(out, lse, ref_out, ref_lse, what=what)
    gk, gv = to_bits(dc.k), to_bits(dc.v)
    assert np.array_equal(gv, vp), f"{what}: V pool differs"
    if rope:
        for b, c in enumerate(case.context_lens):
            if c == 0:
                continue
            p = int(c) - 1
            page, slot = int(case.block_table[b, p // 16]), p % 16
            check_rotated(gk[page, slot], kp[page, slot], inputs.k_new[b], p, theta, f"{what} K")
        diff = np.any(gk != kp, axis=(2, 3))
        written = {(int(case.block_table[b, (int(c) - 1) // 16]), (int(c) - 1) % 16)
                   for b, c in enumerate(case.context_lens) if c > 0}
        assert all((int(p), int(s)) in written for p, s in np.argwhere(diff)), f"{what}: K changed elsewhere"
    else:
        assert np.array_equal(gk, kp), f"{what}: K pool differs"
    log(f"[fused] {what}: max|dout|={err:.2e} max rel dlse={lerr:.2e}")


@pytest.mark.parametrize("theta", [THETA, 0.0])
def test_fused_mixed_contexts(theta):
    case = make_case(CTX, seed=71, pool_pages=800)
    run_case(case, make_append_inputs(case, None, seed=71), theta=theta, what=f"mixed theta={theta}")


@pytest.mark.parametrize("waves,partition", [(4, 0), (4, 64), (16, 0), (16, 256)])
def test_fused_splits_and_waves(waves, partition):
    case = make_case([28672, 1000, 64], seed=72, pool_pages=1900)
    run_case(case, make_append_inputs(case, None, seed=72), theta=THETA, waves=waves, partition=partition,
             what=f"waves={waves} part={partition}")


@pytest.mark.parametrize("waves", [4, 16])
def test_fused_last_page_on_every_wavefront(waves):
    """The page that takes the new token goes to the wavefront next in turn
    after the full pages: with 256-token partitions, contexts 16k + 9 and
    16k + 16 put it at every relative index, partly filled or full."""
    ctx = [16 * k + 9 for k in range(16)] + [16 * k + 16 for k in range(0, 16, 3)]
    case = make_case(ctx, seed=75, pool_pages=sum((n + 15) // 16 for n in ctx) + 5)
    run_case(case, make_append_inputs(case, None, seed=75), theta=THETA, waves=waves, partition=256,
             what=f"last page on every wavefront, {waves} waves")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 4), (32, 16)])
def test_fused_group_sizes(hq, hkv):
    case = make_case([700, 33, 1500, 16], seed=73, Hq=hq, Hkv=hkv, pool_pages=200)
    run_case(case, make_append_inputs(case, None, seed=73), theta=THETA, what=f"{hq}/{hkv}")


def test_fused_fp32_out():
    case = make_case([512, 97], seed=74, pool_pages=64)
    run_case(case, make_append_inputs(case, None, seed=74), theta=THETA, out_dtype=torch.float32, what="fp32")


@pytest.mark.parametrize("theta", [0.0, THETA])
def test_fused_context_past_bound_writes_nothing(theta):
    """A request whose context length exceeds the host bound breaks the
    contract: the kernel clamps its context, so slot ctx - 1 would be a real
    cached token.  The fused call must then leave that request's pages
    untouched, as the separate append does, while the other requests append
    normally."""
    case = make_case([300, 1000, 517], seed=75, pool_pages=120)
    inputs = make_append_inputs(case, None, seed=75)
    dc = DeviceCase(case)
    bound = 800                     # request 1 (1000 tokens) is past it
    k_before, v_before = to_bits(dc.k).copy(), to_bits(dc.v).copy()
    hd.hipdecode_contract_violations()   # clear what earlier calls left
    hd.paged_attn_append(bits_to_bf16(inputs.q), bits_to_bf16(inputs.k_new), bits_to_bf16(inputs.v_new), dc.k, dc.v,
                         dc.table, dc.ctx, case.scale, max_context_len=bound, rope_theta=theta)
    torch.cuda.synchronize()
    assert hd.hipdecode_contract_violations() == hd.HIPDECODE_VIOLATION_CONTEXT
    gk, gv = to_bits(dc.k), to_bits(dc.v)
    pages_1 = {int(p) for p in case.block_table[1, :(1000 + 15) // 16]}
    for p in pages_1:
        assert np.array_equal(gk[p], k_before[p]) and np.array_equal(gv[p], v_before[p]), \
            f"page {p} of the over-long request was written"
    # the valid requests appended exactly what the oracle appends
    valid_ctx = case.context_lens.copy()
    valid_ctx[1] = 0
    rope = theta > 0
    kp, vp, _ = oracle.kv_append(inputs.k_new, inputs.v_new, case.block_table, valid_ctx, case.k_pool, case.v_pool,
                                 q=inputs.q, rope=rope, theta=theta if rope else 1e6)
    assert np.array_equal(gv, vp), "V pool differs"
    if rope:
        for b in (0, 2):
            p = int(case.context_lens[b]) - 1
            page, slot = int(case.block_table[b, p // 16]), p % 16
            check_rotated(gk[page, slot], kp[page, slot], inputs.k_new[b], p, theta, f"K of request {b}")
        diff = {(int(p), int(s)) for p, s in np.argwhere(np.any(gk != kp, axis=(2, 3)))}
        written = {(int(case.block_table[b, (int(case.context_lens[b]) - 1) // 16]),
                    (int(case.context_lens[b]) - 1) % 16) for b in (0, 2)}
        assert diff <= written, "K changed outside the valid requests' new slots"
    else:
        assert np.array_equal(gk, kp), "K pool differs"
    log(f"[fused] context past the bound (theta={theta}): pools as the oracle's, over-long request untouched")
