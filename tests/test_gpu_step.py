"""GPU tests of the graph-replayed decode step (``hipdecode_step_runner``)
against the fp64 oracle, through the C ABI.

Each step appends one token per live request (RoPE on K and q) and attends,
layer after layer, inside one captured graph per batch bucket; padding rows
must stay untouched and read as empty.  Several steps are enqueued without any
host synchronisation, their inputs copied in on the stream between them, to
exercise the double-buffered context lengths; afterwards every layer's pools
must equal the oracle's after the same sequence of appends, and the last
step's outputs must match the oracle at the attention tolerances.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_gqa_amd as hd
from tests.gpu_util import bits_to_bf16, compare, log
from tests.test_gpu_append import check_rotated, to_bits
from workloads import f32_to_bf16_bits, make_case

pytestmark = pytest.mark.gpu

THETA = 1e6


def rows_bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


class Setup:
    """Per-layer pools and step buffers for ``bucket`` rows."""

    def __init__(self, final_ctx, layers, max_seqs, seed, Hq=16, Hkv=8, out_dtype=torch.bfloat16, lse=True):
        self.max_seqs = max_seqs
        self.bucket = hd.hipdecode_step_bucket(max_seqs, max_seqs)
        ctx_rows = list(final_ctx) + [0] * (self.bucket - len(final_ctx))
        self.cases = [make_case(ctx_rows, seed=seed + 10 * l, Hq=Hq, Hkv=Hkv,
                                pool_pages=sum((c + 15) // 16 for c in ctx_rows) + 4)
                      for l in range(layers)]
        # every layer shares one table: same pages per request, different pools
        self.table = self.cases[0].block_table
        for c in self.cases[1:]:
            c.block_table = self.table
        c0 = self.cases[0]
        self.Hq, self.Hkv, self.D = c0.Hq, c0.Hkv, c0.D
        self.scale = c0.scale
        dev = "cuda"
        self.layers = []
        for c in self.cases:
            self.layers.append(dict(
                k_pool=bits_to_bf16(c.k_pool), v_pool=bits_to_bf16(c.v_pool),
                q=torch.zeros((self.bucket, self.Hq, self.D), dtype=torch.bfloat16, device=dev),
                k_new=torch.zeros((self.bucket, self.Hkv, self.D), dtype=torch.bfloat16, device=dev),
                v_new=torch.zeros((self.bucket, self.Hkv, self.D), dtype=torch.bfloat16, device=dev),
                out=torch.full((self.bucket, self.Hq, self.D), 5.0, dtype=out_dtype, device=dev),
                lse=torch.full((self.bucket, self.Hq), 5.0, dtype=torch.float32, device=dev) if lse else None))
        self.table_dev = torch.from_numpy(self.table).to(dev)
        self.ctx_dev = torch.zeros(self.bucket, dtype=torch.int32, device=dev)
        self.max_context_len = int(max(final_ctx))
        self.runner = hd.StepRunner(self.layers, self.table_dev, self.ctx_dev, max_seqs=max_seqs,
                                    num_pages=c0.num_pages, max_context_len=self.max_context_len,
                                    scale=self.scale, rope_theta=THETA,
                                    out_dtype=hd.HIPDECODE_F32 if out_dtype == torch.float32 else hd.HIPDECODE_BF16)


def draw_step(rng, s, B):
    """Host bits of one step's new rows, per layer: q, k_new, v_new."""
    return [(rows_bits(rng, (B, s.Hq, s.D)), rows_bits(rng, (B, s.Hkv, s.D)), rows_bits(rng, (B, s.Hkv, s.D)))
            for _ in s.layers]


def test_step_runner_one_step_with_padding():
    s = Setup([300, 1, 517], layers=2, max_seqs=12, seed=61)
    rng = np.random.default_rng(62)
    B = 3
    rows = draw_step(rng, s, B)
    for layer, (q, k, v) in zip(s.layers, rows):
        layer["q"][:B].copy_(bits_to_bf16(q))
        layer["k_new"][:B].copy_(bits_to_bf16(k))
        layer["v_new"][:B].copy_(bits_to_bf16(v))
    ctx = np.array([300, 1, 517], dtype=np.int32)
    assert s.runner.bucket(B) == 4
    s.runner.step(ctx)
    torch.cuda.synchronize()
    for l, (case, layer, (q, k, v)) in enumerate(zip(s.cases, s.layers, rows)):
        kp, vp, q_rot = oracle.kv_append(k, v, s.table[:B], ctx, case.k_pool, case.v_pool, q=q, rope=True,
                                         theta=THETA)
        ref_out, ref_lse = oracle.paged_attn(q_rot, kp, vp, s.table[:B], ctx, s.scale)
        err, _ = compare(layer["out"][:B], layer["lse"][:B], ref_out, ref_lse, what=f"layer {l}")
        pad_out = layer["out"][B:4].float().cpu().numpy()
        pad_lse = layer["lse"][B:4].cpu().numpy()
        assert np.all(pad_out == 0) and np.all(np.isneginf(pad_lse)), "padding row must read as empty"
        assert np.all(layer["out"][4:].float().cpu().numpy() == 5.0), "rows past the bucket were written"
        log(f"[step] one step layer {l}: max|dout|={err:.2e}")
    s.runner.close()


def test_step_runner_pipelined_steps():
    """Five steps, batch 3, 3, 5, 1, 12 (buckets 4, 4, 8, 1, 16), enqueued
    back to back with their inputs copied in on the stream."""
    run_pipelined([700, 33, 1500, 16, 90, 1, 250, 64, 511, 1024, 7, 300], [3, 3, 5, 1, 12], max_seqs=12, seed=63)


@pytest.mark.parametrize("hq,hkv", [(16, 8), (16, 4)])
def test_step_runner_long_contexts_split(hq, hkv):
    """Long contexts in small buckets: the planner splits every request over
    many partitions, so each replayed layer runs the cross-workgroup merge
    (tickets and partials shared by the layers' launches) inside the graph."""
    base = [9000, 4000]
    params = hd.make_params(num_seqs=2, num_q_heads=hq, num_kv_heads=hkv, num_pages=1000, max_blocks_per_seq=600,
                            max_context_len=9004, scale=0.088)
    assert hd.hipdecode_partition_tokens(params) < 4000, "the requests must be split"
    run_pipelined(base, [2, 1, 2, 2], max_seqs=2, seed=65, Hq=hq, Hkv=hkv)


def test_step_runner_fp32_out_without_lse():
    """fp32 outputs and no LSE buffers (lse NULL for every layer), split contexts."""
    run_pipelined([6000, 2500], [2, 2, 1], max_seqs=2, seed=67, out_dtype=torch.float32, lse=False)


def run_pipelined(base, batches, *, max_seqs, seed, Hq=16, Hkv=8, out_dtype=torch.bfloat16, lse=True):
    final = list(base)
    for B in batches:
        for b in range(B):
            final[b] += 1
    s = Setup(final, layers=2, max_seqs=max_seqs, seed=seed, Hq=Hq, Hkv=Hkv, out_dtype=out_dtype, lse=lse)
    rng = np.random.default_rng(seed + 1)
    grown = list(base)
    plan = []
    for B in batches:
        for b in range(B):
            grown[b] += 1
        plan.append((B, np.array(grown[:B], dtype=np.int32), draw_step(rng, s, B)))
    # stage every step's rows on the device first, then run without host syncs
    staged = [[tuple(bits_to_bf16(x) for x in r) for r in rows] for _, _, rows in plan]
    torch.cuda.synchronize()
    for (B, ctx, _), dev_rows in zip(plan, staged):
        for layer, (q, k, v) in zip(s.layers, dev_rows):
            layer["q"][:B].copy_(q)
            layer["k_new"][:B].copy_(k)
            layer["v_new"][:B].copy_(v)
        s.runner.step(ctx)
    torch.cuda.synchronize()
    # the oracle replays the same appends in order
    for l, (case, layer) in enumerate(zip(s.cases, s.layers)):
        kp, vp = case.k_pool, case.v_pool
        q_rot = None
        for t, (B, ctx, rows) in enumerate(plan):
            q, k, v = rows[l]
            kp, vp, q_rot = oracle.kv_append(k, v, s.table[:B], ctx, kp, vp, q=q, rope=True, theta=THETA)
        gk, gv = to_bits(layer["k_pool"]), to_bits(layer["v_pool"])
        assert np.array_equal(gv, vp), f"layer {l}: V pool differs after {len(plan)} steps"
        diff = np.argwhere(np.any(gk != kp, axis=(2, 3)))
        for page, slot in diff:       # only rounding ties may differ
            row_pos = None
            for t, (B, ctx, rows) in enumerate(plan):
                for b in range(B):
                    p = int(ctx[b]) - 1
                    if s.table[b, p // 16] == page and p % 16 == slot:
                        row_pos = (t, b, p)
            t, b, p = row_pos
            check_rotated(gk[page, slot], kp[page, slot], plan[t][2][l][1][b], p, THETA, f"layer {l} K")
        B, ctx, _ = plan[-1]
        ref_out, ref_lse = oracle.paged_attn(q_rot, kp, vp, s.table[:B], ctx, s.scale)
        if layer["lse"] is not None:
            err, _ = compare(layer["out"][:B], layer["lse"][:B], ref_out, ref_lse, what=f"pipelined layer {l}")
        else:   # fp32 out, no LSE: the fp32 bar and a rounding-level bound on out alone
            o = layer["out"][:B].float().cpu().numpy().astype(np.float64)
            err = float(np.abs(o - ref_out).max())
            assert err <= 1e-2 and np.all(np.abs(o - ref_out) <= 1e-5 * np.abs(ref_out) + 2e-5), \
                f"pipelined layer {l}: fp32 out error {err}"
        log(f"[step] pipelined layer {l}: pools equal, max|dout|={err:.2e}")
    s.runner.close()


def test_step_runner_rejects_context_past_bound():
    """A host context length above the runner's max_context_len (or below 0)
    is refused before anything is enqueued, so no graph sized for the bound
    can clamp it and append over a cached token."""
    s = Setup([300, 1, 517], layers=1, max_seqs=4, seed=65)
    k_before = to_bits(s.layers[0]["k_pool"]).copy()
    for bad in ([300, 1, s.max_context_len + 1], [300, -1, 517]):
        with pytest.raises(hd.HipDecodeError) as ei:
            s.runner.step(np.array(bad, dtype=np.int32))
        assert ei.value.status == hd.HIPDECODE_ERR_SHAPE
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(s.layers[0]["k_pool"]), k_before), "a refused step wrote the pool"
    s.runner.close()
    log("[step] context lengths outside [0, max_context_len] refused")
