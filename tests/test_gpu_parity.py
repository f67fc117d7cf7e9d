"""HIP path against the fp64 oracle, element by element, through the C ABI.

Full-size workloads run at the planner's default partition (the launch
configuration the benchmark times) and are compared on every output.  The edge
matrix covers empty and one-token contexts, page and partition boundaries,
NaN-poisoned unused slots, split-count invariance, page relabelling,
duplicates, CFG pairs, aliased pages, the three group sizes, fp32 output,
B = 0, workspace reuse and HIP-graph replay; 24 seeded random small shapes
mix all of these parameters.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_gqa_amd as hd
from tests.gpu_util import DeviceCase, compare, log, run_hip
from workloads import make_case, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hd.library()   # fail loudly if the HIP library is missing


def _check(case, what, **kw):
    log(f"[parity] {what}: B={case.B} max_ctx={case.max_context_len} pages={case.num_pages} {kw}")
    dc = DeviceCase(case)
    out, lse = run_hip(dc, **kw)
    ref_out, ref_lse = oracle.run_case(case)
    e, le = compare(out, lse, ref_out, ref_lse, what=what)
    log(f"[parity] {what}: max|dout|={e:.3e} max rel dlse={le:.3e}")
    return out, lse


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "c3b"])
def test_workload_parity(name):
    case = make_config(name)
    _check(case, name)


@pytest.mark.parametrize("name,waves", [("c3", 4), ("c3b", 4), ("c2", 16)])
def test_workload_parity_other_waves(name, waves):
    case = make_config(name)
    _check(case, f"{name} at {waves} wavefronts", workgroup_waves=waves)


@pytest.mark.parametrize("name", ["c4", "c5"])
def test_workload_parity_explicit_schedule(name):
    case = make_config(name)
    _check(case, f"{name} on schedule 1", schedule=1)


RAGGED_CASES = {
    "edge lengths poisoned": dict(ctx=[0, 1, 15, 16, 17, 63, 64, 65, 4095, 4096, 4097, 0], poison=True),
    "one request": dict(ctx=[20000]),
    "all empty": dict(ctx=[0, 0, 0]),
    "many mixed": dict(ctx=[int(x) for x in np.random.default_rng(5).integers(0, 6000, size=100)]),
    "one long many short": dict(ctx=[50000] + [17] * 40 + [3000] * 3),
    "fp32 out": dict(ctx=[7000, 123, 2048, 9999], out_dtype="f32"),
    "G=1": dict(ctx=[5000, 700, 12000], Hq=8, Hkv=8),
    "G=4": dict(ctx=[5000, 700, 12000], Hq=16, Hkv=4),
}


@pytest.mark.parametrize("partition", [0, 64])
@pytest.mark.parametrize("name", sorted(RAGGED_CASES))
def test_ragged_batches(name, partition):
    kw = dict(RAGGED_CASES[name])
    ctx = kw.pop("ctx")
    case = make_case(ctx, seed=31, **kw)
    _check(case, f"ragged: {name}, partition {partition}", partition_tokens=partition)


@pytest.mark.parametrize("waves", [4, 16])
@pytest.mark.parametrize("partition", [0, 64, 256, 4096])
def test_edge_lengths_poisoned(partition, waves):
    ctx = [0, 1, 15, 16, 17, 63, 64, 65, 4095, 4096, 4097, 0]
    case = make_case(ctx, seed=11, poison=True, pool_pages=sum((n + 15) // 16 for n in ctx) + 7)
    _check(case, f"edge lengths, partition {partition}, {waves} waves", partition_tokens=partition,
           workgroup_waves=waves)


@pytest.mark.parametrize("waves", [4, 16])
def test_last_page_on_every_wavefront(waves):
    """A partly filled last page goes to the wavefront next in turn after the
    full pages.  With 256-token partitions (16 pages), contexts 16k + 9 for
    k = 0..15 put that page at every relative index, so on every wavefront of
    a 4- or 16-wavefront workgroup, after 0 to 3 full pages of its own; the
    unused slots hold NaN."""
    ctx = [16 * k + 9 for k in range(16)] + [256 * 3 + 16 * k + 9 for k in range(0, 16, 5)]
    case = make_case(ctx, seed=15, poison=True, pool_pages=sum((n + 15) // 16 for n in ctx) + 5)
    _check(case, f"last page on every wavefront, {waves} waves", partition_tokens=256, workgroup_waves=waves)


@pytest.mark.parametrize("waves", [4, 16])
def test_split_count_invariance(waves):
    case = make_case([200, 1000, 3333, 8191, 17], seed=12, poison=True)
    dc = DeviceCase(case)
    ref_out, ref_lse = oracle.run_case(case)
    outs = []
    for part in (64, 128, 256, 512, 1024, 2048, 4096, 0):
        log(f"[parity] split invariance, partition {part}, {waves} waves")
        out, lse = run_hip(dc, partition_tokens=part, workgroup_waves=waves)
        compare(out, lse, ref_out, ref_lse, what=f"partition {part}")
        outs.append(out.float().cpu().numpy())
    spread = max(float(np.abs(o - outs[0]).max()) for o in outs)
    assert spread <= 2e-2


def test_page_relabel_bit_identical():
    case = make_case([700, 33, 2048], seed=13, pool_pages=300)
    dc = DeviceCase(case)
    out1, lse1 = run_hip(dc)
    rng = np.random.default_rng(99)
    perm = rng.permutation(case.num_pages)
    k2 = np.empty_like(case.k_pool)
    v2 = np.empty_like(case.v_pool)
    k2[perm] = case.k_pool
    v2[perm] = case.v_pool
    t2 = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    case2 = make_case([700, 33, 2048], seed=13, pool_pages=300)
    case2.k_pool, case2.v_pool, case2.block_table = k2, v2, t2
    log("[parity] page relabel")
    out2, lse2 = run_hip(DeviceCase(case2))
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_duplicates_and_cfg_pairs():
    case = make_case([1500, 1500, 900, 900], seed=14, shared_q_pairs=True)
    # requests 2 and 3: same q (pair) and, made here, the same KV pages
    case.block_table[3] = case.block_table[2]
    out, lse = _check(case, "duplicates and CFG pairs")
    assert torch.equal(out[2], out[3]) and torch.equal(lse[2], lse[3])
    assert not torch.equal(out[0], out[1])


def test_shared_prefix_pages():
    case = make_case([600, 900, 300, 64], seed=15, shared_prefix_pages=10, poison=True)
    _check(case, "aliased prefix pages")


@pytest.mark.parametrize("hq,hkv,waves", [(8, 8, 4), (8, 8, 16), (16, 4, 4), (32, 16, 4), (32, 16, 16)])
def test_group_sizes(hq, hkv, waves):
    case = make_case([777, 3000, 1], seed=16, Hq=hq, Hkv=hkv)
    _check(case, f"Hq={hq} Hkv={hkv} waves={waves}", workgroup_waves=waves)


def test_fp32_output_long():
    case = make_case([20000, 5], seed=17, out_dtype="f32")
    _check(case, "fp32 out")


@pytest.mark.parametrize("hq,hkv", [(12, 12), (24, 12), (12, 6), (16, 8), (4, 1)])
def test_heads_mixed_across_dispatch_rounds(hq, hkv):
    """Grids of many 256-workgroup rounds, where the kernel XORs each unit's
    KV head with its round: with Hkv 12 or 6 a unit's Hkv workgroups straddle
    round boundaries, and every head must still be computed exactly once."""
    case = make_case([20000, 9000, 1], seed=23, Hq=hq, Hkv=hkv, poison=True)
    _check(case, f"heads mixed by round, {hq}/{hkv}", partition_tokens=256)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_small_lse_meets_the_relative_bar(out_dtype):
    """Two-token contexts at a small scale put every lse near ln 2 (|lse| < 1),
    where the bar 1e-4 * max(1, |lse|) is absolute; here each lse must also
    meet the relative bar 1e-4 * |lse| itself.  (The floor of 1 stays in the
    shared check for lse near 0, where the fp32 sum m + ln l of two terms of
    opposite sign can cancel and no relative bound holds.)"""
    case = make_case([2] * 12 + [3, 2, 2, 2], seed=19, out_dtype=out_dtype, scale=0.01)
    out, lse = _check(case, f"small lse, {out_dtype} out")
    _, ref_lse = oracle.run_case(case)
    l = lse.cpu().numpy().astype(np.float64)
    small = np.abs(ref_lse) < 1.0
    assert small.sum() >= 16 * 12, "the case must put most lse below 1"
    rel = np.abs(l - ref_lse)[small] / np.abs(ref_lse[small])
    assert float(rel.max()) <= 1e-4, f"relative lse error {float(rel.max())}"
    log(f"[parity] small lse: {int(small.sum())} values in (-1, 1), max relative error {float(rel.max()):.2e}")


def test_batch_zero_is_noop():
    q = torch.zeros((0, 16, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    ctx = torch.zeros((0,), dtype=torch.int32, device="cuda")
    out, lse = hd.paged_attn(q, k, k, table, ctx, 0.1, max_context_len=0)
    torch.cuda.synchronize()
    assert out.shape == (0, 16, 128) and lse.shape == (0, 16)


def test_workspace_reuse_leaves_counters_zero():
    case = make_case([5000, 12000, 64], seed=18)
    dc = DeviceCase(case)
    p = hd.make_params(num_seqs=case.B, num_q_heads=16, num_kv_heads=8, num_pages=case.num_pages,
                       max_blocks_per_seq=case.max_blocks, max_context_len=case.max_context_len,
                       scale=case.scale)
    nbytes = hd.hipdecode_workspace_bytes(p)
    ws = torch.full((nbytes // 4 + 4,), 12345, dtype=torch.int32, device="cuda")
    hd.hipdecode_workspace_init(ws)
    ref_out, ref_lse = oracle.run_case(case)
    first = None
    for it in range(3):
        log(f"[parity] workspace reuse, call {it}")
        out, lse = run_hip(dc, workspace=ws)
        compare(out, lse, ref_out, ref_lse, what=f"reuse {it}")
        assert int(ws[: case.B * 8 * 64].abs().sum().item()) == 0, "tickets must return to zero"
        if first is None:
            first = (out.clone(), lse.clone())
        else:
            assert torch.equal(out, first[0]) and torch.equal(lse, first[1]), "not deterministic"


def test_context_above_bound_is_clamped():
    # context_lens past max_context_len: the kernel uses the first max_context_len tokens
    case = make_case([3000, 1200], seed=19)
    dc = DeviceCase(case)
    log("[parity] clamp to max_context_len")
    out, lse = run_hip(dc, max_context_len=2000)
    clamped = make_case([3000, 1200], seed=19)
    clamped.context_lens = np.minimum(clamped.context_lens, 2000).astype(np.int32)
    ref_out, ref_lse = oracle.run_case(clamped)
    compare(out, lse, ref_out, ref_lse, what="clamped")


def test_graph_capture_replay():
    # every request owns pages for 9000 tokens; replays change only context_lens
    case = make_case([9000, 9000, 9000, 9000], seed=20, pool_pages=2300)
    dc = DeviceCase(case)
    p = hd.make_params(num_seqs=case.B, num_q_heads=16, num_kv_heads=8, num_pages=case.num_pages,
                       max_blocks_per_seq=case.max_blocks, max_context_len=9000, scale=case.scale)
    ws = torch.zeros(hd.hipdecode_workspace_bytes(p) // 4 + 4, dtype=torch.int32, device="cuda")
    out = torch.empty((case.B, 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.B, 16), dtype=torch.float32, device="cuda")
    ctx_dev = dc.ctx.clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up outside the graph
        hd.hipdecode_paged_attn(p, dc.q, dc.k, dc.v, dc.table, ctx_dev, out, lse, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hd.hipdecode_paged_attn(p, dc.q, dc.k, dc.v, dc.table, ctx_dev, out, lse, ws)
    torch.cuda.synchronize()
    # replay with new context lengths written into the captured buffer
    for it, lens in enumerate([[4000, 9000, 100, 0], [3999, 17, 8191, 1], [0, 9000, 4096, 2500]]):
        log(f"[parity] graph replay {it}: {lens}")
        ctx_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_case = make_case([9000, 9000, 9000, 9000], seed=20, pool_pages=2300)
        ref_case.context_lens = np.array(lens, dtype=np.int32)
        ref_out, ref_lse = oracle.run_case(ref_case)
        compare(out, lse, ref_out, ref_lse, what=f"graph replay {it}")
        eager_out, eager_lse = hd.paged_attn(dc.q, dc.k, dc.v, dc.table, ctx_dev, case.scale,
                                             max_context_len=9000)
        torch.cuda.synchronize()
        assert torch.equal(eager_out, out) and torch.equal(eager_lse, lse), "replay differs from eager"


def test_alternating_inputs_share_one_workspace():
    """Partials of one call must never leak into the next: two different inputs
    of the same shape alternate on one workspace, each checked every time."""
    case_a = make_case([30000, 9000, 333], seed=21, pool_pages=3000, max_blocks=1875)
    case_b = make_case([29000, 9000, 1000], seed=22, pool_pages=3000, max_blocks=1875)
    da, db = DeviceCase(case_a), DeviceCase(case_b)
    p = hd.make_params(num_seqs=3, num_q_heads=16, num_kv_heads=8, num_pages=3000,
                       max_blocks_per_seq=case_a.max_blocks, max_context_len=30000, scale=case_a.scale,
                       partition_tokens=256)
    ws = torch.zeros(hd.hipdecode_workspace_bytes(p) // 4 + 4, dtype=torch.int32, device="cuda")
    refs = {}
    for name, c in (("a", case_a), ("b", case_b)):
        refs[name] = oracle.run_case(c)
    first = {}
    for it in range(12):
        name, dc = ("a", da) if it % 2 == 0 else ("b", db)
        log(f"[parity] alternating call {it} ({name})")
        out, lse = run_hip(dc, partition_tokens=256, max_context_len=30000, workspace=ws)
        compare(out, lse, *refs[name], what=f"alternating {it}")
        if name in first:
            assert torch.equal(out, first[name][0]) and torch.equal(lse, first[name][1])
        else:
            first[name] = (out.clone(), lse.clone())
    assert int(ws[:3 * 8 * 64].abs().sum().item()) == 0


def test_maximum_split_count():
    # 65536 tokens at 64-token partitions: 1024 partials per (request, KV head)
    case = make_case([65536, 100], seed=23)
    _check(case, "1024 splits", partition_tokens=64)


@pytest.mark.parametrize("ctx,partition", [([3000, 700], 0), ([300, 200, 17], 4096)], ids=["split", "unsplit"])
def test_without_lse(ctx, partition):
    """lse may be NULL: out is then bit-identical to the call that writes lse,
    through the workspace and the allocation-free entry points alike."""
    case = make_case(ctx, seed=48)
    dc = DeviceCase(case)
    p = hd.make_params(num_seqs=case.B, num_q_heads=16, num_kv_heads=8, num_pages=case.num_pages,
                       max_blocks_per_seq=case.max_blocks, max_context_len=case.max_context_len, scale=case.scale,
                       partition_tokens=partition)
    ws = torch.zeros(hd.hipdecode_workspace_bytes(p) // 4 + 4, dtype=torch.int32, device="cuda")
    outs = [torch.empty((case.B, 16, 128), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    lse = torch.empty((case.B, 16), dtype=torch.float32, device="cuda")
    log(f"[parity] without lse, {len(ctx)} requests, partition {partition}")
    hd.hipdecode_paged_attn(p, dc.q, dc.k, dc.v, dc.table, dc.ctx, outs[0], lse, ws)
    hd.hipdecode_paged_attn(p, dc.q, dc.k, dc.v, dc.table, dc.ctx, outs[1], None, ws)
    hd.hipdecode_paged_attn_noalloc(p, dc.q, dc.k, dc.v, dc.table, dc.ctx, outs[2], None)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    ref_out, ref_lse = oracle.run_case(case)
    compare(outs[0], lse, ref_out, ref_lse, what="with lse")


def _violations():
    return hd.hipdecode_contract_violations()


@pytest.mark.parametrize("ctx", [[3000, 1201, 700], [3001]], ids=["batch", "single"])
def test_contract_violations_are_reported(ctx):
    """Device-side contents that break the contract are clamped or skipped,
    and reported: a clean call leaves the flags at 0; a context length past
    the bound, a negative one, and a page id outside the pool (in a full page
    and in the partly filled last page) each set their bit; the requests that
    keep the contract still match the oracle."""
    case = make_case(ctx, seed=47, pool_pages=sum((n + 15) // 16 for n in ctx) + 9)
    ref_out, ref_lse = oracle.run_case(case)
    dc = DeviceCase(case)
    _violations()   # clear what earlier calls left
    log(f"[parity] contract violations, {len(ctx)} requests: clean call")
    out, lse = run_hip(dc)
    compare(out, lse, ref_out, ref_lse, what="clean")
    assert _violations() == 0

    log("[parity] contract violations: context past the bound")
    run_hip(dc, max_context_len=2000)
    assert _violations() == hd.HIPDECODE_VIOLATION_CONTEXT

    bad_b = len(ctx) - 1
    keep = [b for b in range(len(ctx)) if b != bad_b]
    ctx_neg = case.context_lens.copy()
    ctx_neg[bad_b] = -5
    dc.ctx = torch.from_numpy(ctx_neg).cuda()
    log("[parity] contract violations: negative context length")
    out, lse = run_hip(dc)
    assert _violations() == hd.HIPDECODE_VIOLATION_CONTEXT
    if keep:
        compare(out[keep], lse[keep], ref_out[keep], ref_lse[keep], what="negative length beside")
    dc.ctx = torch.from_numpy(case.context_lens).cuda()

    b = 1 if len(ctx) > 1 else 0
    others = [x for x in range(len(ctx)) if x != b]
    for blk in (10, (ctx[b] - 1) // 16):   # a full page, then the partly filled last page
        bad = case.block_table.copy()
        bad[b, blk] = case.num_pages + 5
        dc.table = torch.from_numpy(bad).cuda()
        log(f"[parity] contract violations: page outside the pool at block {blk}")
        out, lse = run_hip(dc)
        assert _violations() == hd.HIPDECODE_VIOLATION_PAGE
        if others:
            compare(out[others], lse[others], ref_out[others], ref_lse[others], what="bad page beside")
    dc.table = torch.from_numpy(case.block_table).cuda()
    out, lse = run_hip(dc)
    assert _violations() == 0


WORK_LIST_CASES = {
    # more requests than one wavefront's lanes, so the unit scan runs over several chunks
    "65 mixed with empties": [0 if i % 9 == 4 else int(x) for i, x in
                              enumerate(np.random.default_rng(40).integers(1, 3000, size=65))],
    "130 log-uniform": [int(np.exp(x)) for x in np.random.default_rng(41).uniform(np.log(16), np.log(9000), 130)],
    "long first then short": [20000] + [40] * 70,
    "short first then long": [40] * 70 + [20000],
    "leading and trailing empties": [0, 0, 5000, 0, 129, 0, 0],
}


@pytest.mark.parametrize("partition", [0, 64, 1024])
@pytest.mark.parametrize("name", sorted(WORK_LIST_CASES))
def test_split_work_list(name, partition):
    case = make_case(WORK_LIST_CASES[name], seed=42, poison=True)
    _check(case, f"work list: {name}, partition {partition}", partition_tokens=partition)


def _random_configs(n, seed=2026):
    """Seeded random small shapes: batch, lengths, group size, wavefronts,
    schedule, partition, output type, scale sign, poisoned slots."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G, Hkv = [(1, 8), (2, 8), (4, 4), (2, 2), (1, 1), (4, 1)][rng.integers(6)]
        B = int(rng.integers(1, 9))
        ctx = [int(x) for x in rng.choice([0, 1, 15, 16, 17, 64, 65, 200, 1000, 2047, 2048, 4097, 7000], size=B)]
        draw = int(rng.choice([0, 1, 2]))   # 0 (planner) or 1 (split, explicit); 2 stands for 1
        schedule = min(draw, 1)
        waves = 16 if (G <= 2 and draw != 2 and rng.random() < 0.3) else 0
        partition = int(rng.choice([0, 64, 128, 512, 2048]))
        out_dtype = "f32" if rng.random() < 0.3 else "bf16"
        scale = float(rng.choice([1 / np.sqrt(128), -0.05, 0.0, 0.3]))
        poison = bool(rng.random() < 0.5)
        out.append(dict(i=i, G=G, Hkv=Hkv, ctx=ctx, schedule=schedule, waves=waves, partition=partition,
                        out_dtype=out_dtype, scale=scale, poison=poison))
    return out


@pytest.mark.parametrize("cfg", _random_configs(24), ids=lambda c: f"r{c['i']}")
def test_randomized_shapes(cfg):
    c = dict(cfg)
    case = make_case(c["ctx"], seed=100 + c["i"], Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"], out_dtype=c["out_dtype"],
                     scale=c["scale"], poison=c["poison"],
                     pool_pages=sum((n + 15) // 16 for n in c["ctx"]) + 3)
    _check(case, f"random r{c['i']} G={c['G']} Hkv={c['Hkv']} ctx={c['ctx']}", schedule=c["schedule"],
           workgroup_waves=c["waves"], partition_tokens=c["partition"])
