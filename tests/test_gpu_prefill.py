"""GPU parity of chunked-prefill attention against the fp64 oracle, through the
C ABI.

The bar is the decode one: |out - oracle| <= 1e-2, and |lse - oracle| <=
1e-4 * max(1, |oracle|).  On bf16 outputs 1e-2 is within reach of a
correctly rounded result only below 4 in magnitude (half the bf16 spacing is
at most 2^-7 there, 2^-5 from 4 to 8), so it binds every element with
|oracle| < 4; every element, those above 4 included, must also meet a
rounding-level bound derived from the kernel's arithmetic.  The matrix
cores take every softmax weight p as its nearest fp16 (|p~ - p| <= 2^-11 p,
the weights kept in fp16's normal range) and V exactly, while the running sum
l adds up the fp32 weights.  The result sum_i p~_i v_i / l is therefore off
by at most 2^-11 sum_i w_i |v_i| <= 2^-11 Vmax, and a bf16 output adds its
own rounding, at most 2^-8 |out|:

    |out - oracle| <= 2^-8 |oracle| (bf16 out) + 2^-11 (1 + 2^-10) Vmax + 2e-5

with 2e-5 for the fp32 scores, sums and accumulation.  Rows that no request
names must be left exactly as they were.
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_gqa_amd as hd
from tests.gpu_util import DeviceCase, bits_to_bf16, compare, log, run_hip
from workloads import (bf16_bits_to_f32, f32_to_bf16_bits, make_append_inputs, make_case, make_prefill_case,
                       make_prefill_config)

pytestmark = pytest.mark.gpu

BF16_EPS = 2.0 ** -8      # unit roundoff of bf16 (8 significant bits, nearest even)
F16_EPS = 2.0 ** -11 * (1 + 2.0 ** -10)   # fp16-rounded weights in P.V: error per unit of max |V|
OUT_ATOL = 1e-2           # max |out - oracle|, as for decode
BF16_REACH = 4.0          # below this magnitude a correctly rounded bf16 is within 2^-7 of any value
LSE_RTOL = 1e-4
SENTINEL = 7.0


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def run_gpu(case, inp, *, out_dtype=torch.bfloat16, dc=None, q=None, max_new=None):
    dc = dc or DeviceCase(case)
    q = q if q is not None else bits_to_bf16(inp.q)
    T = q.shape[0]
    out = torch.full((T, case.Hq, case.D), SENTINEL, dtype=out_dtype, device="cuda")
    lse = torch.full((T, case.Hq), SENTINEL, dtype=torch.float32, device="cuda")
    hd.prefill_attn(q, dc.k, dc.v, dc.table, dc.ctx, i32(inp.new_start), case.scale,
                    max_new_tokens=max_new or inp.max_new_tokens, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def named_rows(new_start, T):
    named = np.zeros(T, dtype=bool)
    for b in range(len(new_start) - 1):
        named[new_start[b]:new_start[b + 1]] = True
    return named


def v_max(v_pool):
    return float(np.nanmax(np.abs(bf16_bits_to_f32(v_pool))))


def rounding_bound(ref_o, vmax, bf16_out=True):
    return (BF16_EPS * np.abs(ref_o) if bf16_out else 0.0) + F16_EPS * vmax + 2e-5


def check_rows(o, l, ref_o, ref_l, what, vmax, bf16_out=True):
    err = np.abs(o - ref_o)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    max_err = float(err.max()) if err.size else 0.0
    # 1e-2 binds where a bf16 result can meet it; fp32 outputs everywhere
    bar = np.abs(ref_o) < BF16_REACH if bf16_out else np.ones(err.shape, dtype=bool)
    max_bar = float(err[bar].max()) if bar.any() else 0.0
    assert max_bar <= OUT_ATOL, f"{what}: max |out err| {max_bar} > {OUT_ATOL}"
    over = err - rounding_bound(ref_o, vmax, bf16_out)
    assert not np.any(over > 0), f"{what}: error above rounding level by {float(over.max())}"
    lerr = np.abs(l - ref_l) / np.maximum(1.0, np.abs(ref_l))
    assert np.all(lerr <= LSE_RTOL), f"{what}: lse err {float(lerr.max())}"
    log(f"[prefill] {what}: max|dout|={max_err:.2e} (|oracle|<4: {max_bar:.2e}; {int((~bar).sum())} above) "
        f"mean|dout|={float(err.mean()):.2e} max|out|={float(np.abs(ref_o).max()) if ref_o.size else 0.0:.2f} "
        f"max rel dlse={float(lerr.max()):.2e} (Vmax {vmax:.2f})")
    return max_err


def check_full(case, inp, o, l, what, bf16_out=True):
    ref_o, ref_l = oracle.prefill_attn(inp.q, case.k_pool, case.v_pool, case.block_table, case.context_lens,
                                       inp.new_start, case.scale)
    named = named_rows(inp.new_start, inp.rows)
    check_rows(o[named], l[named], ref_o[named], ref_l[named], what, v_max(case.v_pool), bf16_out)
    assert np.all(o[~named] == SENTINEL) and np.all(l[~named] == SENTINEL), f"{what}: an unnamed row was written"


RAGGED = [(300, 300), (1000, 64), (77, 5), (16, 16), (33, 1), (130, 129), (64, 0)]


def test_prefill_ragged_chunks():
    ctx = [c for c, _ in RAGGED]
    new = [n for _, n in RAGGED]
    case, inp = make_prefill_case(ctx, new, seed=41, extra_rows=3)
    o, l = run_gpu(case, inp)
    check_full(case, inp, o, l, "ragged chunks")


# Chunk lengths around the half-tile size of each group size (64 tokens at
# G = 2, 128 at G = 1, 32 at G = 4): even and odd half-tile counts, a lone
# middle half-tile, and late half-tiles whose last wavefronts hold no rows.
PAIRED = [(700, 191), (192, 192), (900, 193), (1255, 255), (256, 256), (3000, 257), (2047, 1023), (40, 33)]


@pytest.mark.parametrize("hq,hkv", [(16, 8), (8, 8), (16, 4)])
def test_prefill_half_tile_pairs(hq, hkv):
    ctx = [c for c, _ in PAIRED]
    new = [n for _, n in PAIRED]
    case, inp = make_prefill_case(ctx, new, seed=45, Hq=hq, Hkv=hkv, poison=True,
                                  pool_pages=sum((c + 15) // 16 for c in ctx) + 5)
    o, l = run_gpu(case, inp)
    check_full(case, inp, o, l, f"half-tile pairs, Hq={hq} Hkv={hkv}")


def test_prefill_poisoned_unused_slots():
    # Unused slots of last pages and unused pool pages hold NaN; keys past a
    # tile's last position are masked, and must not turn the output into NaN.
    ctx = [301, 77, 1000, 16, 129, 4097]
    new = [301, 5, 64, 16, 128, 1000]
    case, inp = make_prefill_case(ctx, new, seed=44, poison=True,
                                  pool_pages=sum((c + 15) // 16 for c in ctx) + 9)
    hd.hipdecode_contract_violations()
    o, l = run_gpu(case, inp)
    # no NaN reaches the products, so no non-finite sum is reported either
    assert hd.hipdecode_contract_violations() == 0
    check_full(case, inp, o, l, "poisoned unused slots")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 4), (4, 1), (32, 16)])
def test_prefill_group_shapes(hq, hkv):
    case, inp = make_prefill_case([200, 70, 513], [200, 33, 129], seed=42, Hq=hq, Hkv=hkv)
    o, l = run_gpu(case, inp)
    check_full(case, inp, o, l, f"{hq}/{hkv}")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prefill_rising_scores(out_dtype):
    # Keys grow with their position, so a row's maximum keeps rising past the
    # running reference: the rescale path runs on many halves, not only the
    # first, and the last few keys carry most of the weight (outputs reach
    # past 4 in magnitude).
    ctx, new = [3000, 700], [512, 700]
    case, inp = make_prefill_case(ctx, new, seed=45)
    k = bf16_bits_to_f32(case.k_pool).astype(np.float32)
    for b, n in enumerate(ctx):
        for t in range(n):
            page, slot = case.block_table[b, t // 16], t % 16
            k[page, slot] *= np.float32(1.0 + 7.0 * (t / n) ** 2)
    case = replace(case, k_pool=f32_to_bf16_bits(k))
    o, l = run_gpu(case, inp, out_dtype=out_dtype)
    f32 = out_dtype == torch.float32
    check_full(case, inp, o, l, "rising scores" + (", fp32 out" if f32 else ""), bf16_out=not f32)


def test_prefill_dominant_key():
    """One key per request takes about 88% of the weight of every row of one
    query head per KV head, and its V holds values of 2.5 to 3.9 in
    magnitude, so those rows' outputs sit in [2, 4), where bf16 rounding alone
    is up to 7.8e-3: the weights' own error must stay far below the rest of the
    1e-2 bar.  The key sits past the first 64, so the running reference is not
    its own score and its weight is not exactly 1."""
    ctx, new = [3000, 1500], [256, 128]
    case, inp = make_prefill_case(ctx, new, seed=48)
    rng = np.random.default_rng(480)
    G = case.Hq // case.Hkv
    q = bf16_bits_to_f32(inp.q).astype(np.float32)
    k = bf16_bits_to_f32(case.k_pool).astype(np.float32)
    v = bf16_bits_to_f32(case.v_pool).astype(np.float32)
    j = 100
    for b, c in enumerate(ctx):
        r0, r1 = int(inp.new_start[b]), int(inp.new_start[b + 1])
        q[r0:r1] = q[r0]                      # every chunk row asks the same question
        page, slot = case.block_table[b, j // 16], j % 16
        target = np.log(1.65 * c) + 2.0       # E exp(z) = e^0.5 for the N(0,1) scores of the other keys
        for g in range(case.Hkv):
            qh = q[r0, g * G].astype(np.float64)
            k[page, slot, g] = (qh * (target / (case.scale * np.dot(qh, qh)))).astype(np.float32)
            v[page, slot, g] = (rng.uniform(2.5, 3.9, case.D) * rng.choice([-1.0, 1.0], case.D)).astype(np.float32)
    case = replace(case, k_pool=f32_to_bf16_bits(k), v_pool=f32_to_bf16_bits(v))
    inp = replace(inp, q=f32_to_bf16_bits(q))
    o, l = run_gpu(case, inp)
    check_full(case, inp, o, l, "dominant key")
    ref_o, _ = oracle.prefill_attn(inp.q, case.k_pool, case.v_pool, case.block_table, case.context_lens,
                                   inp.new_start, case.scale)
    big = np.abs(ref_o) >= 2.0
    assert big.sum() > 1000, "the dominated rows must put outputs in [2, 4)"


def _random_prefill_shapes(seed, n):
    """Seeded random small prefill shapes: group size, KV heads, chunk and
    context lengths around the half-tile sizes, output type, scale sign and
    size, poisoned slots."""
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        G, Hkv = [(1, 8), (2, 8), (4, 4), (2, 2), (1, 1), (4, 1)][rng.integers(6)]
        reqs = []
        for _ in range(int(rng.integers(1, 5))):
            c = int(rng.choice([1, 15, 16, 17, 63, 64, 65, 127, 300, 1000, 2100]))
            n_new = int(rng.choice([c, 1, 33, 64, 129, c // 2]))
            reqs.append((c, min(c, n_new)))
        shapes.append(dict(i=i, G=G, Hkv=Hkv, reqs=reqs, f32=bool(rng.random() < 0.3),
                           scale=float(rng.choice([1 / np.sqrt(128), -0.05, 0.0, 0.3])),
                           poison=bool(rng.random() < 0.5)))
    return shapes


@pytest.mark.parametrize("shape", _random_prefill_shapes(77, 20), ids=lambda s: f"r{s['i']}")
def test_prefill_random_small_shapes(shape):
    ctx = [c for c, _ in shape["reqs"]]
    new = [n for _, n in shape["reqs"]]
    case, inp = make_prefill_case(ctx, new, seed=700 + shape["i"], Hq=shape["G"] * shape["Hkv"], Hkv=shape["Hkv"],
                                  poison=shape["poison"], pool_pages=sum((c + 15) // 16 for c in ctx) + 3,
                                  extra_rows=shape["i"] % 3)
    case = replace(case, scale=shape["scale"])
    what = (f"random {shape['i']}: G={shape['G']} Hkv={shape['Hkv']} (ctx, chunk)={shape['reqs']} "
            f"scale={shape['scale']:.3g} {'f32' if shape['f32'] else 'bf16'}{' poisoned' if shape['poison'] else ''}")
    log(f"[prefill] {what}")
    o, l = run_gpu(case, inp, out_dtype=torch.float32 if shape["f32"] else torch.bfloat16)
    check_full(case, inp, o, l, what, bf16_out=not shape["f32"])


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prefill_equal_keys(out_dtype):
    """Every key of a request the same: the softmax is uniform over the
    visible keys, and chunk row j returns the mean of V over positions
    0 .. p_j (the oracle's closed-form pin).  All of a row's fp16 weights are
    then equal, so their rounding errors all point the same way."""
    ctx, new = [700, 300], [256, 300]
    case, inp = make_prefill_case(ctx, new, seed=51)
    k = bf16_bits_to_f32(case.k_pool).astype(np.float32)
    rng = np.random.default_rng(510)
    for b, c in enumerate(ctx):
        key = rng.standard_normal((case.Hkv, case.D)).astype(np.float32)
        for t in range(c):
            k[case.block_table[b, t // 16], t % 16] = key
    case = replace(case, k_pool=f32_to_bf16_bits(k))
    o, l = run_gpu(case, inp, out_dtype=out_dtype)
    f32 = out_dtype == torch.float32
    check_full(case, inp, o, l, "equal keys" + (", fp32 out" if f32 else ""), bf16_out=not f32)


def test_prefill_fp32_out():
    case, inp = make_prefill_case([450, 97], [160, 97], seed=43)
    o, l = run_gpu(case, inp, out_dtype=torch.float32)
    check_full(case, inp, o, l, "fp32 out", bf16_out=False)


@pytest.mark.parametrize("name", ["p2", "p1"])
def test_prefill_named_workloads_full(name):
    """Every (row, query head) of the named 4,096-token chunks against the
    oracle: p1 (the last chunk of a 28,672-token prompt) and p2 (the first)."""
    case, inp = make_prefill_config(name)
    log(f"[prefill] {name}: {case.name} rows={inp.rows}")
    o, l = run_gpu(case, inp)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), f"{name}: non-finite rows"
    check_full(case, inp, o, l, f"{name} every row")


def test_prefill_last_rows_match_decode_kernel():
    """The last row of each chunk sees the whole context: the decode kernel on
    that query must agree."""
    case, inp = make_prefill_case([3000, 517, 16], [256, 100, 16], seed=45)
    dc = DeviceCase(case)
    o, l = run_gpu(case, inp, dc=dc)
    last = inp.new_start[1:] - 1
    dc.q = bits_to_bf16(inp.q[last])
    d_out, d_lse = run_hip(dc)
    d_o = d_out.float().cpu().numpy()
    d_l = d_lse.cpu().numpy()
    # both rounding-level bounds: prefill's and the decode kernel's (fp32 weights, bf16 out)
    assert np.all(np.abs(o[last] - d_o) <= rounding_bound(d_o, v_max(case.v_pool)) + 2.0 ** -8 * np.abs(d_o) + 2e-5)
    assert np.all(np.abs(l[last] - d_l) <= 2 * LSE_RTOL * np.maximum(1.0, np.abs(d_l)))


def test_prefill_without_lse():
    """lse may be NULL: out is then bit-identical to the call that writes lse."""
    case, inp = make_prefill_case([900, 300], [300, 100], seed=49)
    dc = DeviceCase(case)
    q = bits_to_bf16(inp.q)
    p = hd.make_prefill_params(num_seqs=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                               num_pages=case.num_pages, max_blocks_per_seq=case.max_blocks,
                               num_rows=q.shape[0], max_new_tokens=inp.max_new_tokens, scale=case.scale)
    starts = i32(inp.new_start)
    outs = [torch.empty((q.shape[0], case.Hq, case.D), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    lse = torch.empty((q.shape[0], case.Hq), dtype=torch.float32, device="cuda")
    hd.hipdecode_prefill_attn(p, q, dc.k, dc.v, starts, dc.table, dc.ctx, outs[0], lse)
    hd.hipdecode_prefill_attn(p, q, dc.k, dc.v, starts, dc.table, dc.ctx, outs[1], None)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_prefill_skips_what_breaks_the_contract():
    case, inp = make_prefill_case([100, 50, 40], [20, 10, 40], seed=46)
    ctx_bad = case.context_lens.copy()
    ctx_bad[1] = 5                                   # 10 chunk tokens, context 5
    broken = replace(case, context_lens=ctx_bad)
    hd.hipdecode_contract_violations()   # clear what earlier calls left
    run_gpu(case, inp)
    assert hd.hipdecode_contract_violations() == 0, "a call within the contract reported a violation"
    o, l = run_gpu(broken, inp)
    assert hd.hipdecode_contract_violations() == hd.HIPDECODE_VIOLATION_ROWS
    ok_rows = np.r_[0:20, 30:70]
    ref_o, ref_l = oracle.prefill_attn(inp.q, case.k_pool, case.v_pool, case.block_table, case.context_lens,
                                       inp.new_start, case.scale)
    check_rows(o[ok_rows], l[ok_rows], ref_o[ok_rows], ref_l[ok_rows], "valid requests", v_max(case.v_pool))
    assert np.all(o[20:30] == SENTINEL) and np.all(l[20:30] == SENTINEL), "a broken request wrote rows"


def _with_v_entries(case, value, seed):
    """A copy of the case with `value` (and -value) at 16 dims of each
    request's first key, which every chunk row attends to."""
    v = bf16_bits_to_f32(case.v_pool).astype(np.float32)
    rng = np.random.default_rng(seed)
    for b in range(case.B):
        page, slot = case.block_table[b, 0], 0
        dims = rng.choice(case.D, 16, replace=False)
        v[page, slot, :, dims[:8]] = value
        v[page, slot, :, dims[8:]] = -value
    return replace(case, v_pool=f32_to_bf16_bits(v))


def test_prefill_v_at_the_top_of_the_fp16_range():
    """V entries of +-65,280, the largest bf16 below 2^16, enter the fp16
    products exactly: a one-token context returns its V bit for bit (its
    weight is exact), the rows that attend to them match the oracle at the
    rounding-level bound, and no violation is reported.  An entry of 2^16
    sets HIPDECODE_VIOLATION_VALUE."""
    case, inp = make_prefill_case([300, 200, 1], [100, 200, 1], seed=50)
    big = _with_v_entries(case, 65280.0, 500)
    assert v_max(big.v_pool) == 65280.0
    hd.hipdecode_contract_violations()
    o, l = run_gpu(big, inp)
    assert hd.hipdecode_contract_violations() == 0
    G = case.Hq // case.Hkv
    v_one = bf16_bits_to_f32(big.v_pool)[big.block_table[2, 0], 0]          # [Hkv, D]
    assert np.array_equal(o[inp.new_start[2]], np.repeat(v_one, G, axis=0)), "a one-token context must return V"
    ref_o, ref_l = oracle.prefill_attn(inp.q, big.k_pool, big.v_pool, big.block_table, big.context_lens,
                                       inp.new_start, big.scale)
    assert np.abs(ref_o).max() > 100.0, "the large entries must reach the outputs"
    # the rounding-level bound with Vmax = 65,280: 2^-11 of it, plus bf16 rounding of out
    check_rows(o, l, ref_o, ref_l, "V at 65,280", 65280.0)
    over = _with_v_entries(case, 65536.0, 500)
    run_gpu(over, inp)
    assert hd.hipdecode_contract_violations() == hd.HIPDECODE_VIOLATION_VALUE


def test_chunked_prefill_pipeline_with_append():
    """A 700-token prompt in chunks of 256, 256 and 188: each chunk's K/V are
    appended with RoPE (K and the chunk's q rotated), then the chunk attends;
    every chunk's rows against the oracle doing the same two steps."""
    total = 700
    chunks = [256, 256, 188]
    case = make_case([total], seed=47, pool_pages=50)
    dc = DeviceCase(case)
    k_ref, v_ref = case.k_pool.copy(), case.v_pool.copy()
    done = 0
    for i, n in enumerate(chunks):
        done += n
        ctx = np.array([done], dtype=np.int32)
        sub = replace(case, context_lens=ctx)
        rows = make_append_inputs(sub, [n], seed=470 + i)
        ns = i32(rows.new_start)
        ctx_d = i32(ctx)
        q = bits_to_bf16(rows.q)
        hd.kv_append(bits_to_bf16(rows.k_new), bits_to_bf16(rows.v_new), dc.table, ctx_d, dc.k, dc.v, q=q,
                     new_start=ns, max_new_tokens=n, rope_theta=rows.theta)
        out = torch.empty((n, case.Hq, case.D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((n, case.Hq), dtype=torch.float32, device="cuda")
        hd.prefill_attn(q, dc.k, dc.v, dc.table, ctx_d, ns, case.scale, max_new_tokens=n, out=out, lse=lse)
        torch.cuda.synchronize()
        k_ref, v_ref, q_rot = oracle.kv_append(rows.k_new, rows.v_new, case.block_table, ctx, k_ref, v_ref,
                                               new_start=rows.new_start, q=rows.q, rope=True, theta=rows.theta)
        ref_o, ref_l = oracle.prefill_attn(q_rot, k_ref, v_ref, case.block_table, ctx, rows.new_start, case.scale)
        check_rows(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, f"pipeline chunk {i}", v_max(v_ref))


def test_prefill_graph_replays():
    """A captured prefill call replayed three times, with eager work and a
    changed query in between: each replay equals an eager call on the same
    inputs bit for bit, and the oracle at the prefill bars."""
    case, inp = make_prefill_case([2500, 700, 64], [600, 700, 64], seed=47)
    dc = DeviceCase(case)
    T = inp.rows
    q = bits_to_bf16(inp.q)
    new_start = i32(inp.new_start)
    out = torch.empty((T, case.Hq, case.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, case.Hq), dtype=torch.float32, device="cuda")

    def call():
        hd.prefill_attn(q, dc.k, dc.v, dc.table, dc.ctx, new_start, case.scale,
                        max_new_tokens=inp.max_new_tokens, out=out, lse=lse)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        call()                      # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    q0 = q.clone()
    for rep in range(3):
        if rep == 1:
            q.mul_(-1)              # the graph reads q through its pointer
        out.fill_(SENTINEL)
        lse.fill_(SENTINEL)
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = out.clone(), lse.clone()
        call()
        torch.cuda.synchronize()
        assert torch.equal(o_g, out) and torch.equal(l_g, lse), f"replay {rep} differs from the eager call"
        log(f"[prefill] graph replay {rep}: equal to the eager call")
    q.copy_(q0)
    g.replay()
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    check_full(case, inp, o, l, "graph replay")
