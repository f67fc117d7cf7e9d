"""GPU parity of the KV-cache append (with and without RoPE) against the fp64
oracle, through the C ABI.

The bar: V rows, K rows without RoPE and every untouched byte of the pools are
bit-exact.  Rotated K and q rows equal the oracle's nearest-even bf16 of the
exact rotation; the only difference allowed is at an exact value so close to
the midpoint of two bf16 neighbours (relative 1e-9) that fp64 evaluation
order can decide it, and each such element is checked against the oracle's
unrounded fp64 rotation.
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_gqa_amd as hd
from tests.gpu_util import DeviceCase, bits_to_bf16, compare, log, run_hip
from workloads import bf16_bits_to_f32, make_append_case, make_append_config, make_append_inputs, make_case

pytestmark = pytest.mark.gpu

TIE_REL = 1e-9


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def written(case, inputs):
    """(row, request, position) of every new token, computed here from the inputs."""
    out = []
    for b, c in enumerate(case.context_lens):
        c = int(c)
        if inputs.new_start is None:
            start, n = b, (1 if c > 0 else 0)
        else:
            start, n = int(inputs.new_start[b]), int(inputs.new_start[b + 1] - inputs.new_start[b])
        for j in range(n):
            out.append((start + j, b, c - n + j))
    return out


def run_gpu_append(case, inputs, *, rope=True, q=True, max_new_tokens=None):
    k_pool = bits_to_bf16(case.k_pool)
    v_pool = bits_to_bf16(case.v_pool)
    qd = bits_to_bf16(inputs.q) if (q and inputs.q is not None) else None
    hd.kv_append(bits_to_bf16(inputs.k_new), bits_to_bf16(inputs.v_new), i32(case.block_table),
                 i32(case.context_lens), k_pool, v_pool, q=qd, new_start=i32(inputs.new_start),
                 max_new_tokens=max_new_tokens if max_new_tokens is not None else
                 (inputs.max_new_tokens if inputs.new_start is not None else None),
                 rope_theta=inputs.theta if rope else None)
    torch.cuda.synchronize()
    return to_bits(k_pool), to_bits(v_pool), None if qd is None else to_bits(qd)


def check_rotated(got: np.ndarray, want: np.ndarray, src_bits: np.ndarray, pos: int, theta: float, what: str):
    """got/want: bf16 bits [heads, D] of one rotated row; src_bits its input."""
    diff = got != want
    if not diff.any():
        return 0
    exact = oracle.rope_f64(bf16_bits_to_f32(src_bits).astype(np.float64), pos, theta)
    g = bf16_bits_to_f32(got[diff]).astype(np.float64)
    w = bf16_bits_to_f32(want[diff]).astype(np.float64)
    x = exact[diff]
    mid = (g + w) / 2
    adjacent = np.abs(got[diff].astype(np.int32) - want[diff].astype(np.int32)) == 1
    assert adjacent.all() and np.all(np.abs(x - mid) <= TIE_REL * np.abs(x)), \
        f"{what}: {int(diff.sum())} elements differ beyond a rounding tie at position {pos}"
    return int(diff.sum())


def check_append(case, inputs, *, rope=True, q=True, what=""):
    log(f"[append] {what}: B={case.B} rows={inputs.rows} rope={rope} q={q}")
    gk, gv, gq = run_gpu_append(case, inputs, rope=rope, q=q)
    ok, ov, oq = oracle.kv_append(inputs.k_new, inputs.v_new, case.block_table, case.context_lens,
                                  case.k_pool, case.v_pool, new_start=inputs.new_start,
                                  q=inputs.q if q else None, rope=rope, theta=inputs.theta)
    assert np.array_equal(gv, ov), f"{what}: V pool differs"
    ties = 0
    if not rope:
        assert np.array_equal(gk, ok), f"{what}: K pool differs"
        if gq is not None:
            assert np.array_equal(gq, inputs.q), f"{what}: q changed without RoPE"
        return
    touched = np.zeros(case.k_pool.shape[:2], dtype=bool)
    for row, b, pos in written(case, inputs):
        page = int(case.block_table[b, pos // case.page])
        slot = pos % case.page
        touched[page, slot] = True
        ties += check_rotated(gk[page, slot], ok[page, slot], inputs.k_new[row], pos, inputs.theta, f"{what} K")
        if gq is not None:
            ties += check_rotated(gq[row], oq[row], inputs.q[row], pos, inputs.theta, f"{what} q")
    assert np.array_equal(gk[~touched], case.k_pool[~touched]), f"{what}: K slots outside the append changed"
    if gq is not None:
        rows = {r for r, _, _ in written(case, inputs)}
        rest = [r for r in range(inputs.rows) if r not in rows]
        assert np.array_equal(gq[rest], inputs.q[rest]), f"{what}: q rows without a token changed"
    log(f"[append] {what}: ok ({ties} rounding ties)")


@pytest.mark.parametrize("name", ["a1", "a2"])
def test_append_named_workloads(name):
    case, inputs = make_append_config(name)
    check_append(case, inputs, what=name)


@pytest.mark.parametrize("rope", [False, True])
def test_append_ragged_chunks(rope):
    # chunks crossing page boundaries, an empty chunk, a padding row, a chunk
    # that is the whole context, one deep into a 90-minute context
    ctx = [11, 7, 20, 3, 0, 67500, 16, 33]
    new = [6, 0, 9, 3, 0, 37, 16, 1]
    case, _ = make_append_case(ctx, new, seed=21, extra_pages=5)
    inputs = make_append_inputs(case, new, seed=21, extra_rows=3)
    check_append(case, inputs, rope=rope, what=f"ragged rope={rope}")


def test_append_without_q():
    case, inputs = make_append_case([100, 2000, 5], seed=22, extra_pages=2)
    check_append(case, inputs, q=False, what="no q")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 4), (32, 8), (2, 1)])
def test_append_group_shapes(hq, hkv):
    case, _ = make_append_case([70, 1, 4096], [5, 1, 64], seed=23, Hq=hq, Hkv=hkv, extra_pages=1)
    inputs = make_append_inputs(case, [5, 1, 64], seed=23)
    check_append(case, inputs, what=f"{hq}/{hkv}")


def test_append_decode_padding_rows():
    case, inputs = make_append_case([0, 5, 0, 16, 17], seed=24, extra_pages=3)
    check_append(case, inputs, what="padding rows")


def test_append_nan_inputs():
    case, inputs = make_append_case([40, 9], [8, 2], seed=25, extra_pages=1)
    inputs.k_new[1, 0, 3] = 0x7FC0
    inputs.k_new[4, 1, 70] = 0xFFC1              # negative NaN with a payload
    inputs.v_new[2, 0, 5] = 0x7FA5               # V is copied bit for bit
    inputs.q[0, 3, 100] = 0x7FC0
    check_append(case, inputs, what="NaN inputs")


def test_append_skips_what_breaks_the_contract():
    """A last block naming no page, a page outside the pool, more new tokens
    than the context: those requests write nothing; the others are done."""
    ctx = [40, 30, 20, 50, 9]
    new = [4, 3, 2, 5, 1]
    case, _ = make_append_case(ctx, new, seed=26, extra_pages=2)
    inputs = make_append_inputs(case, new, seed=26)
    bad = case.block_table.copy()
    bad[1, (30 - 1) // 16] = -1                          # request 1: last block unmapped
    bad[2, (20 - 1) // 16] = case.num_pages + 7          # request 2: page outside the pool
    ctx_bad = case.context_lens.copy()
    ctx_bad[3] = 3                                       # request 3: 5 new tokens, context 3
    broken = replace(case, block_table=bad, context_lens=ctx_bad)
    hd.hipdecode_contract_violations()   # clear what earlier calls left
    run_gpu_append(case, inputs)
    assert hd.hipdecode_contract_violations() == 0, "a call within the contract reported a violation"
    gk, gv, gq = run_gpu_append(broken, inputs)
    # an unmapped block and a page outside the pool, and more new tokens than the context
    assert hd.hipdecode_contract_violations() == hd.HIPDECODE_VIOLATION_PAGE | hd.HIPDECODE_VIOLATION_ROWS
    # expected: only requests 0 and 4, appended one at a time by the oracle
    ek, ev, eq = case.k_pool, case.v_pool, inputs.q
    for b in (0, 4):
        s, e = int(inputs.new_start[b]), int(inputs.new_start[b + 1])
        ns = np.array([0, e - s], dtype=np.int32)
        ek, ev, qb = oracle.kv_append(inputs.k_new[s:e], inputs.v_new[s:e], case.block_table[b:b + 1],
                                      case.context_lens[b:b + 1], ek, ev, new_start=ns, q=eq[s:e], rope=True,
                                      theta=inputs.theta)
        eq = eq.copy()
        eq[s:e] = qb
    assert np.array_equal(gv, ev)
    assert np.array_equal(gk, ek)        # no rounding ties at these seeds (checked bit for bit)
    assert np.array_equal(gq, eq)


def test_append_then_attend():
    """One decode step: append the new token (RoPE on K and q), then attend."""
    ctx = [300, 1, 517, 4096, 0, 2049]
    case = make_case(ctx, seed=27, pool_pages=600)
    inputs = make_append_inputs(case, None, seed=27)
    dc = DeviceCase(case)
    qd = bits_to_bf16(inputs.q)
    hd.kv_append(bits_to_bf16(inputs.k_new), bits_to_bf16(inputs.v_new), dc.table, dc.ctx, dc.k, dc.v, q=qd,
                 rope_theta=inputs.theta)
    dc.q = qd
    out, lse = run_hip(dc)
    ok, ov, oq = oracle.kv_append(inputs.k_new, inputs.v_new, case.block_table, case.context_lens, case.k_pool,
                                  case.v_pool, q=inputs.q, rope=True, theta=inputs.theta)
    ref_out, ref_lse = oracle.paged_attn(oq, ok, ov, case.block_table, case.context_lens, case.scale)
    err, lerr = compare(out, lse, ref_out, ref_lse, what="append then attend")
    log(f"[append] then attend: max|dout|={err:.2e} max rel dlse={lerr:.2e}")


def test_append_then_attend_graph_replays():
    """A captured [append, attend] pair replayed over three decode steps, the
    contexts growing by one token per step, each replay against the oracle."""
    base = [700, 33, 1500, 16]
    steps = 3
    case = make_case([c + steps for c in base], seed=28, pool_pages=200)
    B = case.B
    dc = DeviceCase(case)
    ctx_dev = torch.zeros(B, dtype=torch.int32, device="cuda")
    k_new = torch.empty((B, case.Hkv, case.D), dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    q_dev = torch.empty((B, case.Hq, case.D), dtype=torch.bfloat16, device="cuda")
    mcl = max(base) + steps
    params = hd.make_params(num_seqs=B, num_q_heads=case.Hq, num_kv_heads=case.Hkv, num_pages=case.num_pages,
                            max_blocks_per_seq=case.max_blocks, max_context_len=mcl, scale=case.scale)
    ws = torch.zeros(hd.hipdecode_workspace_bytes(params) // 4 + 4, dtype=torch.int32, device="cuda")
    out = torch.empty((B, case.Hq, case.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, case.Hq), dtype=torch.float32, device="cuda")
    aparams = hd.make_append_params(num_seqs=B, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                                    num_pages=case.num_pages, max_blocks_per_seq=case.max_blocks, num_rows=B,
                                    rope=hd.HIPDECODE_ROPE_HALF, rope_theta=1e6)

    def step():
        hd.hipdecode_kv_append(aparams, q_dev, k_new, v_new, None, dc.table, ctx_dev, dc.k, dc.v)
        hd.hipdecode_paged_attn(params, q_dev, dc.k, dc.v, dc.table, ctx_dev, out, lse, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    ctx_dev.copy_(torch.tensor(base, dtype=torch.int32))
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):       # recorded, not run
            step()
    torch.cuda.synchronize()
    k_ref, v_ref = case.k_pool, case.v_pool
    for t in range(steps):
        ctx = np.array([c + t + 1 for c in base], dtype=np.int32)
        sub = replace_ctx(case, ctx)
        inputs = make_append_inputs(sub, None, seed=280 + t)
        ctx_dev.copy_(torch.from_numpy(ctx))
        k_new.copy_(bits_to_bf16(inputs.k_new))
        v_new.copy_(bits_to_bf16(inputs.v_new))
        q_dev.copy_(bits_to_bf16(inputs.q))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        k_ref, v_ref, q_rot = oracle.kv_append(inputs.k_new, inputs.v_new, case.block_table, ctx, k_ref, v_ref,
                                               q=inputs.q, rope=True, theta=inputs.theta)
        ref_out, ref_lse = oracle.paged_attn(q_rot, k_ref, v_ref, case.block_table, ctx, case.scale)
        err, lerr = compare(out, lse, ref_out, ref_lse, what=f"graph replay {t}")
        log(f"[append] graph replay {t}: max|dout|={err:.2e}")


def replace_ctx(case, ctx):
    return replace(case, context_lens=np.asarray(ctx, dtype=np.int32))
