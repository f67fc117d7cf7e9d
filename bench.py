#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one decode step's attention over all 28 layers of the
Qwen3-0.6B-shaped decoder (audio.cpp "Fun-ASR-Nano Native Runtime Design",
"Decoder And Prompt": 28 layers, 16 query / 8 KV heads): 28 calls of
``hipdecode_paged_attn``, layer i reading its own KV pools.  The pools are
rotated over R distinct device copies so that every call streams from HBM
rather than from the 256 MB last-level cache.  All inputs are resident in HBM
before the timed region starts.  By default a step replays one captured HIP
graph of its 28 launches, as a serving loop replays its decode step;
``--eager`` issues the launches one by one instead.  Each pool copy is its
own allocation; ``--v-offset BYTES`` puts a copy's V pool BYTES after the end
of its K pool in one allocation instead (rows whose address has bit 8 set
stream more slowly on this GPU, so an odd multiple of 256 evens out the heads).

value   = decode tokens/s = B * steps / (timed seconds)
roofline.achieved = algorithmic bytes per call / average call duration,
          timed with HIP events on the stream the kernel runs on.
cpu_baseline = the fp64 oracle, unmodified, on this host's cores, over one
          layer's worth of (request, head) pairs, scaled to tokens/s.
configs = the default run (c4, 16 x 28,672 tokens) also times c3 (1 x 28,672),
          c3b (1 x 65,536) and c5 (32 mixed lengths up to 67,500) the same
          way, so that one line covers the metric's 28k-64k range.

``--op append`` measures the KV-cache append instead (``hipdecode_kv_append``
with RoPE on K and q): a step is 28 calls, one per layer, each writing the new
tokens of workload a1 (one token for each of 16 requests) or a2 (one
4096-token prefill chunk) into its own copy of the pools.

``--op prefill`` measures chunked-prefill attention (``hipdecode_prefill_attn``)
on workload p1 (the last 4096-token chunk of a 28672-token prompt) or p2 (the
first chunk), against the bf16 dense matrix-core peak.

``--op step`` measures the graph-replayed decode step (``hipdecode_step_runner``:
per layer, one fused launch of append with RoPE and attention, one captured
graph per batch bucket) on the latency-bound shapes s1 (one request at 512
tokens) and s2 (16 requests of 200-420 tokens), against the same fused
launches issued eagerly and against separate append and attention launches.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attn tokens/s and achieved HBM GB/s (% of peak) at 28k/64k ctx"
PEAK_HBM_GBS = 8000.0
LAYERS = 28
ROTATE_MIN_BYTES = 1.5e9
DECODE_SOURCES = ["paged_kv_decode_gqa_amd/csrc/paged_decode.hip",
                  "paged_kv_decode_gqa_amd/csrc/api.hip",
                  "paged_kv_decode_gqa_amd/csrc/internal.h",
                  "paged_kv_decode_gqa_amd/csrc/page_fold.h"]
APPEND_SOURCES = ["paged_kv_decode_gqa_amd/csrc/kv_append.hip",
                  "paged_kv_decode_gqa_amd/csrc/internal.h"]
PREFILL_SOURCES = ["paged_kv_decode_gqa_amd/csrc/prefill_attn.hip", "paged_kv_decode_gqa_amd/csrc/internal.h"]
KERNEL_NAMES = {"split": "paged_decode_kernel"}
KERNEL_SOURCES = {"paged_decode_kernel": DECODE_SOURCES,
                  "kv_append_kernel": APPEND_SOURCES, "prefill_attn_kernel": PREFILL_SOURCES}
DECODE_WORKLOADS = ("c1", "c2", "c3", "c4", "c5", "c3b")
APPEND_METRIC = "kv-cache append new tokens/s (RoPE on K and q) and achieved HBM GB/s"
PREFILL_METRIC = "chunked-prefill attention tokens/s and achieved bf16 TFLOP/s"
PEAK_BF16_TFLOPS = 2500.0


def kernel_source_hash(kernel: str = "paged_decode_kernel") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def host_cpu_model() -> str:
    """The host CPU's model name, read from /proc/cpuinfo (empty if unavailable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def shifted_pools(k, v, offset: int):
    """Copies of the K and V pools in one allocation, V starting `offset` bytes after K ends."""
    import torch
    if offset < 0 or offset % 16:
        raise ValueError("--v-offset must be a non-negative multiple of 16")
    n = k.numel() * k.element_size()
    raw = torch.empty(2 * n + offset, dtype=torch.uint8, device=k.device)
    kk = raw[:n].view(k.dtype).view(k.shape)
    vv = raw[n + offset: 2 * n + offset].view(v.dtype).view(v.shape)
    kk.copy_(k)
    vv.copy_(v)
    return kk, vv


def per_step_spread(run, stream, steps: int) -> list[float]:
    """p10, p50 and p90 of the per-call time, from `steps` more steps timed
    one by one with HIP events on the launch stream (after the main timed
    region, which they do not touch)."""
    import numpy as np
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    per_call_us = np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e3 / LAYERS
    return [round(float(np.percentile(per_call_us, q)), 3) for q in (10, 50, 90)]


def algorithmic_bytes(case, out_bytes: int) -> int:
    """Bytes the method must move per call: every cached K and V row of the
    context once, q, out, lse, the block-table entries used and the lengths."""
    import numpy as np
    ctx = case.context_lens.astype(np.int64)
    kv_per_token = 2 * case.Hkv * case.D * 2
    blocks = int(((ctx + case.page - 1) // case.page).sum())
    rows = case.B * case.Hq
    return int(kv_per_token * ctx.sum() + rows * case.D * 2 + rows * case.D * out_bytes + rows * 4
               + 4 * blocks + 4 * case.B)


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the kernel as it is now."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        fetch = float(kv["fetch_kib_per_dispatch"]) * float(kv.get("copy_scale_fetch", 1.0))
        write = float(kv["write_kib_per_dispatch"]) * float(kv.get("copy_scale_write", 1.0))
    except (KeyError, ValueError):
        return None
    return (fetch + write) * 1024.0


def append_algorithmic_bytes(case, inputs) -> int:
    """Bytes an append must move: each new token's K and V rows read and
    written, its q rows read and written, one table entry per token, the
    lengths and the row offsets."""
    T = int(inputs.new_start[-1]) if inputs.new_start is not None else int((case.context_lens > 0).sum())
    kv = 2 * case.Hkv * case.D * 2
    qb = case.Hq * case.D * 2 if inputs.q is not None else 0
    offsets = 4 * (case.B + 1) if inputs.new_start is not None else 0
    return int(T * (2 * kv + 2 * qb + 4) + 4 * case.B + offsets)


def prefill_algorithmic_flops(case, inputs) -> int:
    """Matrix flops the method needs: for every chunk row and query head,
    2 * 128 for q.k and 2 * 128 for p.v per visible key (p + 1 keys)."""
    total = 0
    for b in range(case.B):
        n = int(inputs.new_start[b + 1] - inputs.new_start[b])
        c = int(case.context_lens[b])
        first = c - n + 1                     # visible keys of the first row
        total += (first + c) * n // 2         # sum of p + 1 over the chunk
    return int(total * case.Hq * case.D * 4)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--op", default="decode", choices=["decode", "append", "prefill", "step"])
    ap.add_argument("--workload", default=None,
                    help="decode: c1 c2 c3 c4 c5 c3b (default c4); append: a1 a2 (default a2); "
                         "prefill: p1 p2 (default p1); step: s1 s2 (default s2)")
    ap.add_argument("--context", type=int, default=0,
                    help="decode: one request of this many tokens (a shuffled pool of exactly its pages, "
                         "N(0,1) bf16) instead of a named workload; for sweeps of the per-call fixed cost")
    ap.add_argument("--partition", type=int, default=0, help="split-K partition tokens (0 = planner)")
    ap.add_argument("--waves", type=int, default=0, help="wavefronts per workgroup, 4 or 16 (0 = planner)")
    ap.add_argument("--schedule", type=int, default=0, help="1 = split (0 = planner; split is the only one)")
    ap.add_argument("--rotate", type=int, default=0, help="distinct KV pool copies (0 = auto)")
    ap.add_argument("--v-offset", type=int, default=None, metavar="BYTES",
                    help="decode: place each V pool BYTES after the end of its K pool in one allocation "
                         "(default: separate allocations)")
    ap.add_argument("--graph", dest="graph", action="store_true", default=True,
                    help="replay one captured HIP graph per step (the default: the decode step of the "
                         "MOSS-TD article runs from captured graphs)")
    ap.add_argument("--eager", dest="graph", action="store_false", help="issue the 28 launches of a step eagerly")
    ap.add_argument("--configs", default="c3,c3b,c5",
                    help="decode, default workload only: further workloads timed the same way after c4 and "
                         "reported under \"configs\" (comma-separated; \"none\" to skip)")
    ap.add_argument("--no-other-ops", dest="other_ops", action="store_false",
                    help="decode, default workload only: skip timing prefill p1 and append a2 after the "
                         "decode workloads (reported under \"other_ops\")")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the traffic counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU sharding)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_decode_gqa_amd as hd
    from workloads import make_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        n = 1 << 28   # 2**28 float32 = 1 GiB read and 1 GiB written per copy
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            dst.copy_(src)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / 3
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": 4 * n,
                          "bytes_written_per_copy": 4 * n, "copies": 4,
                          "read_plus_write_GBps": round(8 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return 0
    hd.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.op == "append":
        return run_append(args, dev)
    if args.op == "prefill":
        return run_prefill(args, dev)
    if args.op == "step":
        return run_step(args, dev)
    named = False
    if args.context > 0:
        from workloads import make_case
        t0 = time.time()
        args.workload = f"b1_ctx{args.context}"
        case = make_case([args.context], seed=3, name=args.workload)
        t_gen = time.time() - t0
    else:
        named = args.workload is not None
        args.workload = args.workload or "c4"
        if args.workload not in DECODE_WORKLOADS:
            print(f"unknown decode workload {args.workload}", file=sys.stderr)
            return 2
        t0 = time.time()
        case = make_config(args.workload)
        t_gen = time.time() - t0
    m = measure_decode(case, args.workload, args, dev)
    out, m = m.pop("_out"), m
    result = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 KV pages, shuffled pools; no dataset)",
        "config": m["config"],
        "us_per_layer": m["us_per_layer"],
        "us_per_layer_p10_p50_p90": m["us_per_layer_p10_p50_p90"],
        "kv_tokens_per_s": m["kv_tokens_per_s"],
        "wall_s_timed": m["wall_s_timed"],
        "roofline": m["roofline"],
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        import oracle
        o_gpu = out.float().cpu().numpy().astype(np.float64)
        reps, t_cpu = 0, 0.0
        ref_out = None
        while reps < 50 and (t_cpu < 10.0 or reps == 0):
            c0 = time.perf_counter()
            ref_out, _ = oracle.run_case(case)
            t_cpu += time.perf_counter() - c0
            reps += 1
        t_layer = t_cpu / reps
        result["cpu_baseline"] = {
            "value": round(case.B / (LAYERS * t_layer), 4),
            "unit": "tokens/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "cpu_model": host_cpu_model(),
            "sample": f"fp64 oracle over all {case.B * case.Hq} (request, head) pairs of one layer call, "
                      f"{reps} run(s), {t_layer:.3f} s per layer, scaled to {LAYERS} layers per token",
            "parity_max_abs_err": float(np.abs(o_gpu - ref_out).max()),
        }
    del out, case
    torch.cuda.empty_cache()

    # the rest of the metric's 28k-64k range, each timed the same way
    extra = [] if args.context > 0 or named or args.configs == "none" else \
        [w for w in args.configs.split(",") if w and w != args.workload]
    if extra:
        result["configs"] = {}
    for w in extra:
        if w not in DECODE_WORKLOADS:
            print(f"unknown decode workload {w}", file=sys.stderr)
            return 2
        c = make_config(w)
        mw = measure_decode(c, w, args, dev)
        mw.pop("_out")
        r = mw["roofline"]
        result["configs"][w] = {
            "workload": c.name,
            "batch": c.B,
            "max_context": c.max_context_len,
            "tokens_per_s": mw["tokens_per_s"],
            "us_per_layer": mw["us_per_layer"],
            "us_per_layer_p10_p50_p90": mw["us_per_layer_p10_p50_p90"],
            "achieved_GBps": r["achieved"],
            "frac": r["frac"],
            "traffic": r["traffic"],
            "algorithmic_bytes_per_launch": r["algorithmic_bytes_per_launch"],
            "partition_tokens": mw["config"]["partition_tokens"],
            "kv_pool_copies": mw["config"]["kv_pool_copies"],
        }
        del c, mw
        torch.cuda.empty_cache()
    # the other entry points on their named workloads, timed the same way in
    # the same run: the last 4,096-token prefill chunk of a 28,672-token
    # prompt, and the append of such a chunk with RoPE
    if args.other_ops and not (args.context > 0 or named):
        result["other_ops"] = {}
        for key, fn, w in (("prefill_p1", run_prefill, "p1"), ("append_a2", run_append, "a2")):
            r = fn(args, dev, name=w, emit=False)
            rr = r["roofline"]
            result["other_ops"][key] = {
                "metric": r["metric"],
                "workload": r["config"]["workload"],
                "tokens_per_s": r["value"],
                "us_per_layer": r["us_per_layer"],
                "achieved": rr["achieved"],
                "unit": rr["unit"],
                "peak": rr["peak"],
                "bound": rr["bound"],
                "frac": rr["frac"],
                "traffic": rr["traffic"],
                "kernel": rr["kernel"],
            }
            del r
            torch.cuda.empty_cache()
    result["setup_s"] = round(t_gen, 2)
    print(json.dumps(result), flush=True)
    return 0


def measure_decode(case, workload: str, args, dev) -> dict:
    """Time `case` as bench's decode step does (28 calls per step over rotated
    pool copies, graph replay unless --eager) and return the figures; the
    last call's output tensor is under "_out"."""
    import numpy as np
    import torch

    import paged_kv_decode_gqa_amd as hd

    out_dtype = torch.float32 if case.out_dtype == "f32" else torch.bfloat16
    out_bytes = 4 if case.out_dtype == "f32" else 2
    alg_bytes = algorithmic_bytes(case, out_bytes)
    kv_bytes_call = 2 * case.Hkv * case.D * 2 * case.total_tokens

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    R = args.rotate or max(2, min(LAYERS, math.ceil(ROTATE_MIN_BYTES / max(1, kv_bytes_call))))
    q = bf(case.q)
    k0, v0 = bf(case.k_pool), bf(case.v_pool)
    if args.v_offset is None:
        pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
    else:
        pools = [shifted_pools(k0, v0, args.v_offset) for _ in range(R)]
        del k0, v0
    table = torch.from_numpy(case.block_table).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    params = hd.make_params(num_seqs=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                            num_pages=case.num_pages, max_blocks_per_seq=case.max_blocks,
                            max_context_len=case.max_context_len, scale=case.scale,
                            partition_tokens=args.partition, workgroup_waves=args.waves,
                            schedule=args.schedule,
                            out_dtype=hd.HIPDECODE_F32 if out_bytes == 4 else hd.HIPDECODE_BF16)
    st = hd.hipdecode_check_params(params)
    if st != 0:
        raise hd.HipDecodeError(st, "params")
    part = hd.hipdecode_partition_tokens(params)
    waves = hd.hipdecode_workgroup_waves(params)
    schedule = {1: "split"}[hd.hipdecode_schedule(params)]
    ws = torch.zeros(hd.hipdecode_workspace_bytes(params) // 4 + 4, dtype=torch.int32, device=dev)
    out = torch.empty((case.B, case.Hq, case.D), dtype=out_dtype, device=dev)
    lse = torch.empty((case.B, case.Hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    calls = [hd.PreparedCall(params, q, kp, vp, table, ctx, out, lse, ws) for kp, vp in pools]

    def one_step():
        # launches go to the current stream: the timed stream, or the capture stream
        for layer in range(LAYERS):
            calls[layer % R]()

    graph = None
    if args.graph:
        one_step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
    run = graph.replay if graph is not None else one_step

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    ev1.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1)
    call_s = ms * 1e-3 / (args.steps * LAYERS)
    achieved = alg_bytes / call_s / 1e9
    spread = per_step_spread(run, stream, args.steps)
    kernel = KERNEL_NAMES[schedule]
    traffic = read_traffic(kernel, workload)
    m = {
        "tokens_per_s": round(case.B * args.steps / (ms * 1e-3), 2),
        "ms_per_step": round(ms / args.steps, 4),
        "config": {
            "workload": case.name,
            "batch": case.B,
            "context_tokens_total": case.total_tokens,
            "max_context": case.max_context_len,
            "num_q_heads": case.Hq,
            "num_kv_heads": case.Hkv,
            "head_dim": case.D,
            "page_size": case.page,
            "layers_per_step": LAYERS,
            "partition_tokens": part,
            "workgroup_waves": waves,
            "schedule": schedule,
            "kv_pool_copies": R,
            "v_pool_offset": args.v_offset,
            "mode": "hipgraph" if graph is not None else "eager",
            "out_dtype": case.out_dtype,
        },
        "us_per_layer": round(call_s * 1e6, 3),
        "us_per_layer_p10_p50_p90": spread,
        "kv_tokens_per_s": round(case.total_tokens / call_s, 1),
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "algorithmic_bytes_per_launch": alg_bytes,
            "avg_launch_us": round(call_s * 1e6, 3),
        },
        "_out": out,
    }
    del graph, calls, pools, q, table, ctx, ws, lse
    return m


def run_append(args, dev, name=None, emit=True):
    """Time the append workload `name` (default a2); print its JSON line, or
    return the result without the CPU baseline when `emit` is false."""
    import numpy as np
    import torch

    import paged_kv_decode_gqa_amd as hd
    from workloads import APPEND_CONFIGS, make_append_config

    name = name or args.workload or "a2"
    if name not in APPEND_CONFIGS:
        print(f"unknown append workload {name}", file=sys.stderr)
        return 2
    t0 = time.time()
    case, inputs = make_append_config(name)
    alg_bytes = append_algorithmic_bytes(case, inputs)
    # distinct copies (inputs, table and pool each) so the calls stream from HBM
    R = args.rotate or max(2, min(LAYERS, math.ceil(ROTATE_MIN_BYTES / max(1, alg_bytes))))
    copies = [(case, inputs)] + [make_append_config(name, copy=i) for i in range(1, R)]
    t_gen = time.time() - t0

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    dev_copies = []
    for c, inp in copies:
        dev_copies.append(dict(q=bf(inp.q), k_new=bf(inp.k_new), v_new=bf(inp.v_new), new_start=i32(inp.new_start),
                               table=i32(c.block_table), ctx=i32(c.context_lens), k=bf(c.k_pool), v=bf(c.v_pool)))
    params = hd.make_append_params(num_seqs=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                                   num_pages=case.num_pages, max_blocks_per_seq=case.max_blocks,
                                   num_rows=inputs.rows, max_new_tokens=inputs.max_new_tokens,
                                   rope=hd.HIPDECODE_ROPE_HALF, rope_theta=inputs.theta)
    st = hd.hipdecode_check_append_params(params)
    if st != 0:
        raise hd.HipDecodeError(st, "append params")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    calls = [hd.PreparedAppend(params, d["q"], d["k_new"], d["v_new"], d["new_start"], d["table"], d["ctx"],
                               d["k"], d["v"]) for d in dev_copies]

    def one_step():
        for layer in range(LAYERS):
            calls[layer % R]()

    graph = None
    if args.graph:
        one_step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
    run = graph.replay if graph is not None else one_step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    ev1.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1)
    call_s = ms * 1e-3 / (args.steps * LAYERS)
    T = int(inputs.new_start[-1]) if inputs.new_start is not None else case.B
    achieved = alg_bytes / call_s / 1e9
    result = {
        "metric": APPEND_METRIC,
        "value": round(T / call_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 rows and pools; no dataset)",
        "config": {
            "workload": case.name,
            "batch": case.B,
            "new_tokens_per_call": T,
            "max_context": int(case.context_lens.max()),
            "num_q_heads": case.Hq,
            "num_kv_heads": case.Hkv,
            "head_dim": case.D,
            "page_size": case.page,
            "rope_theta": inputs.theta,
            "layers_per_step": LAYERS,
            "copies": R,
            "mode": "hipgraph" if graph is not None else "eager",
        },
        "us_per_layer": round(call_s * 1e6, 3),
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "kv_append_kernel",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": alg_bytes,
            "avg_launch_us": round(call_s * 1e6, 3),
        },
        "cpu_baseline": None,
    }
    traffic = read_traffic("kv_append_kernel", name)
    if traffic is not None:
        result["roofline"]["traffic"] = round(traffic)
    if not emit:
        return result
    if not args.no_cpu_baseline:
        import oracle
        reps, t_cpu = 0, 0.0
        while reps < 50 and (t_cpu < 10.0 or reps == 0):
            c0 = time.perf_counter()
            oracle.kv_append(inputs.k_new, inputs.v_new, case.block_table, case.context_lens, case.k_pool,
                             case.v_pool, new_start=inputs.new_start, q=inputs.q, rope=True, theta=inputs.theta)
            t_cpu += time.perf_counter() - c0
            reps += 1
        t_call = t_cpu / reps
        result["cpu_baseline"] = {
            "value": round(T / t_call, 1),
            "unit": "tokens/s",
            "cores": 1,
            "kind": "oracle",
            "cpu_model": host_cpu_model(),
            "sample": f"fp64 oracle append of the same {T} new tokens (copies of the pools included), "
                      f"{reps} run(s), {t_call * 1e3:.2f} ms per call",
        }
    result["setup_s"] = round(t_gen, 2)
    print(json.dumps(result), flush=True)
    return 0


STEP_WORKLOADS = {"s1": "c1", "s2": "c2"}   # decode shapes whose steps are launch-bound
STEP_METRIC = "decode-step tokens/s, graph-replayed fused append + attention over 28 layers"


def run_step(args, dev) -> int:
    import numpy as np
    import torch

    import paged_kv_decode_gqa_amd as hd
    from workloads import ROPE_THETA, make_append_inputs, make_config

    name = args.workload or "s2"
    if name not in STEP_WORKLOADS:
        print(f"unknown step workload {name}", file=sys.stderr)
        return 2
    t0 = time.time()
    case = make_config(STEP_WORKLOADS[name])
    rows = make_append_inputs(case, None, seed=99)
    t_gen = time.time() - t0
    B = case.B
    bucket = hd.hipdecode_step_bucket(B, B)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def pad(t, n):
        out = torch.zeros((n,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
        out[: t.shape[0]].copy_(t)
        return out

    k0, v0 = bf(case.k_pool), bf(case.v_pool)
    q0, kn, vn = bf(rows.q), bf(rows.k_new), bf(rows.v_new)
    layers = []
    for _ in range(LAYERS):          # every layer its own pools and rows
        layers.append(dict(k_pool=k0.clone(), v_pool=v0.clone(), q=pad(q0, bucket), k_new=pad(kn, bucket),
                           v_new=pad(vn, bucket),
                           out=torch.empty((bucket, case.Hq, case.D), dtype=torch.bfloat16, device=dev),
                           lse=torch.empty((bucket, case.Hq), dtype=torch.float32, device=dev)))
    table = pad(torch.from_numpy(case.block_table).to(dev), bucket)
    ctx_dev = pad(torch.from_numpy(case.context_lens).to(dev), bucket)
    ctx_host = case.context_lens.copy()
    runner = hd.StepRunner(layers, table, ctx_dev, max_seqs=B, num_pages=case.num_pages,
                           max_context_len=case.max_context_len, scale=case.scale, rope_theta=ROPE_THETA)
    # the same launches, issued eagerly
    aparams = hd.make_append_params(num_seqs=bucket, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                                    num_pages=case.num_pages, max_blocks_per_seq=case.max_blocks, num_rows=bucket,
                                    rope=hd.HIPDECODE_ROPE_HALF, rope_theta=ROPE_THETA)
    params = hd.make_params(num_seqs=bucket, num_q_heads=case.Hq, num_kv_heads=case.Hkv, num_pages=case.num_pages,
                            max_blocks_per_seq=case.max_blocks, max_context_len=case.max_context_len,
                            scale=case.scale)
    ws = torch.zeros(hd.hipdecode_workspace_bytes(params) // 4 + 4, dtype=torch.int32, device=dev)
    eager = []           # two launches per layer: append, then attention
    fused = []           # one fused launch per layer
    for d in layers:
        eager.append(hd.PreparedAppend(aparams, d["q"], d["k_new"], d["v_new"], None, table, ctx_dev, d["k_pool"],
                                       d["v_pool"]))
        eager.append(hd.PreparedCall(params, d["q"], d["k_pool"], d["v_pool"], table, ctx_dev, d["out"], d["lse"], ws))
        fused.append(hd.PreparedAttnAppend(params, ROPE_THETA, d["q"], d["k_new"], d["v_new"], d["k_pool"],
                                           d["v_pool"], table, ctx_dev, d["out"], d["lse"], ws))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def eager_step():
        for c in eager:
            c()

    def fused_step():
        for c in fused:
            c()

    ms_eager = timed(eager_step)
    ms_fused = timed(fused_step)
    ms_graph = timed(lambda: runner.step(ctx_host))
    runner.close()
    kv_bytes = 2 * case.Hkv * case.D * 2 * case.total_tokens * LAYERS
    achieved = kv_bytes / (ms_graph * 1e-3) / 1e9
    result = {
        "metric": STEP_METRIC,
        "value": round(B / (ms_graph * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_graph, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 rows and KV pages; no dataset)",
        "config": {
            "workload": f"{name}_{case.name}",
            "batch": B,
            "bucket": bucket,
            "layers_per_step": LAYERS,
            "context_tokens_total": case.total_tokens,
            "rope_theta": ROPE_THETA,
            "mode": "hip graph per bucket (step runner)",
        },
        "eager_ms_per_step": round(ms_eager, 4),
        "eager_fused_ms_per_step": round(ms_fused, 4),
        "speedup_vs_eager": round(ms_eager / ms_graph, 3),
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_decode_kernel + kv_append_kernel",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_step": kv_bytes,
        },
        "cpu_baseline": None,
        "setup_s": round(t_gen, 2),
    }
    print(json.dumps(result), flush=True)
    return 0


def run_prefill(args, dev, name=None, emit=True):
    """Time the prefill workload `name` (default p1); print its JSON line, or
    return the result without the CPU baseline when `emit` is false."""
    import numpy as np
    import torch

    import paged_kv_decode_gqa_amd as hd
    from workloads import PREFILL_CONFIGS, make_prefill_config

    name = name or args.workload or "p1"
    if name not in PREFILL_CONFIGS:
        print(f"unknown prefill workload {name}", file=sys.stderr)
        return 2
    t0 = time.time()
    case, inp = make_prefill_config(name)
    t_gen = time.time() - t0
    flops = prefill_algorithmic_flops(case, inp)
    kv_bytes = 2 * case.Hkv * case.D * 2 * case.total_tokens

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    R = args.rotate or max(2, min(LAYERS, math.ceil(ROTATE_MIN_BYTES / max(1, kv_bytes))))
    k0, v0 = bf(case.k_pool), bf(case.v_pool)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
    q = bf(inp.q)
    table = torch.from_numpy(case.block_table).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    ns = torch.from_numpy(inp.new_start).to(dev)
    out = torch.empty((inp.rows, case.Hq, case.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.rows, case.Hq), dtype=torch.float32, device=dev)
    params = hd.make_prefill_params(num_seqs=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                                    num_pages=case.num_pages, max_blocks_per_seq=case.max_blocks,
                                    num_rows=inp.rows, max_new_tokens=inp.max_new_tokens, scale=case.scale)
    st = hd.hipdecode_check_prefill_params(params)
    if st != 0:
        raise hd.HipDecodeError(st, "prefill params")
    calls = [hd.PreparedPrefill(params, q, kp, vp, ns, table, ctx, out, lse) for kp, vp in pools]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def one_step():
        for layer in range(LAYERS):
            calls[layer % R]()

    graph = None
    if args.graph:
        one_step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
    run = graph.replay if graph is not None else one_step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    ev1.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1)
    call_s = ms * 1e-3 / (args.steps * LAYERS)
    T = int(inp.new_start[-1])
    achieved = flops / call_s / 1e12
    result = {
        "metric": PREFILL_METRIC,
        "value": round(T / call_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q rows and KV pages, shuffled pools; no dataset)",
        "config": {
            "workload": case.name,
            "batch": case.B,
            "chunk_tokens": T,
            "context": int(case.context_lens.max()),
            "num_q_heads": case.Hq,
            "num_kv_heads": case.Hkv,
            "head_dim": case.D,
            "page_size": case.page,
            "layers_per_step": LAYERS,
            "kv_pool_copies": R,
            "mode": "hipgraph" if graph is not None else "eager",
        },
        "us_per_layer": round(call_s * 1e6, 3),
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "bound": "mfma",
            "kernel": "prefill_attn_kernel",
            "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": round(call_s * 1e6, 3),
        },
        "cpu_baseline": None,
    }
    traffic = read_traffic("prefill_attn_kernel", name)
    if traffic is not None:
        result["roofline"]["traffic"] = round(traffic)
    if not emit:
        return result
    if not args.no_cpu_baseline:
        import oracle
        rng = np.random.default_rng(0)
        rows = rng.integers(0, T, size=16)
        pairs = [(int(r), int(h)) for r in rows for h in range(case.Hq)]
        reps, t_cpu = 0, 0.0
        while reps < 50 and (t_cpu < 10.0 or reps == 0):
            c0 = time.perf_counter()
            oracle.prefill_attn_pairs(inp.q, case.k_pool, case.v_pool, case.block_table, case.context_lens,
                                      inp.new_start, case.scale, pairs)
            t_cpu += time.perf_counter() - c0
            reps += 1
        t_rows = t_cpu / reps
        result["cpu_baseline"] = {
            "value": round(len(rows) / t_rows, 2),
            "unit": "tokens/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "cpu_model": host_cpu_model(),
            "sample": f"fp64 oracle over 16 random chunk rows x all {case.Hq} heads, {reps} run(s), "
                      f"{t_rows:.3f} s per 16 rows",
        }
    result["setup_s"] = round(t_gen, 2)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
