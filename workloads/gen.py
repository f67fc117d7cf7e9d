"""Seeded synthetic workloads for one decode step of paged GQA attention.

Shapes follow the decoder of the audio-LLM speech recogniser on the pages
(FunASR vLLM guide, "Supported Models": a Qwen3-0.6B LLM; audio.cpp
"Fun-ASR-Nano Native Runtime Design", "Decoder And Prompt": 16 query heads and
8 KV heads) with head_dim 128 and 16-token pages, and the context lengths
follow the long-meeting workloads of the MOSS-TD article ("Benchmark results":
~12 s clips and ~38 min meetings; "Overview": recordings of up to ~90 min).
The datasets behind those numbers are private; these draws stand in for them.

Everything here is data preparation: normal draws, rounding to bfloat16 bit
patterns, page permutations and block tables.  No attention arithmetic.

Random streams.  Each tensor has its own ``numpy.random.default_rng`` stream
keyed by ``[seed, stream_id(, chunk)]`` so that the multi-GB pools can be drawn
chunk by chunk on several threads and still be reproducible bit for bit:

* stream 0 ("meta"): context lengths, then the page permutation, then the
  positions of the scaled ("peaky") keys, in that order;
* stream 1: q, one draw of shape [B, Hq, D];
* stream 2, chunk c: K pool pages [c*256, (c+1)*256);
* stream 3, chunk c: V pool pages, same chunking.

All values are float32 N(0, 1) draws rounded to bfloat16 with
round-to-nearest-even.  The whole pool is filled, unused pages included.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HQ = 16
HKV = 8
HEAD_DIM = 128
PAGE = 16
SCALE = 1.0 / math.sqrt(HEAD_DIM)
CHUNK_PAGES = 256
BF16_QNAN = 0x7FC0


# --------------------------------------------------------------------------
# bfloat16 bit patterns
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite values cannot carry out of 32 bits here: the largest finite
    # pattern 0xFF7FFFFF plus 0x8000 stays below 2**32.
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_QNAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads(threads: int | None) -> int:
    if threads:
        return threads
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return min(int(env), 16)
    return min(os.cpu_count() or 1, 16)


def _normal_pool_bits(seed: int, stream: int, n_pages: int, page_elems: int,
                      threads: int | None) -> np.ndarray:
    out = np.empty((n_pages, page_elems), dtype=np.uint16)
    n_chunks = (n_pages + CHUNK_PAGES - 1) // CHUNK_PAGES

    def work(c: int) -> None:
        lo = c * CHUNK_PAGES
        hi = min(n_pages, lo + CHUNK_PAGES)
        rng = np.random.default_rng([seed, stream, c])
        x = rng.standard_normal((hi - lo) * page_elems, dtype=np.float32)
        out[lo:hi] = f32_to_bf16_bits(x).reshape(hi - lo, page_elems)

    nt = _threads(threads)
    if nt == 1 or n_chunks == 1:
        for c in range(n_chunks):
            work(c)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


# --------------------------------------------------------------------------
# A case: everything one call of the path consumes
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Case:
    name: str
    q: np.ndarray             # uint16 [B, Hq, D]            bf16 bit patterns
    k_pool: np.ndarray        # uint16 [P, page, Hkv, D]     bf16 bit patterns
    v_pool: np.ndarray        # uint16 [P, page, Hkv, D]
    block_table: np.ndarray   # int32  [B, max_blocks]       -1 where unused
    context_lens: np.ndarray  # int32  [B]
    scale: float
    out_dtype: str            # "bf16" or "f32"
    seed: int
    notes: str = ""

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def Hq(self) -> int:
        return int(self.q.shape[1])

    @property
    def D(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def page(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def Hkv(self) -> int:
        return int(self.k_pool.shape[2])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.B else 0

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def used_pages(self) -> int:
        return int(sum((int(n) + self.page - 1) // self.page for n in self.context_lens))


def _build(name: str, ctx: list[int], rng_meta: np.random.Generator, *, seed: int,
           Hq: int, Hkv: int, D: int, page: int, pool_pages: int | None,
           max_blocks: int | None, out_dtype: str, shared_q_pairs: bool,
           peaky_frac: float, peaky_factor: float, poison: bool,
           shared_prefix_pages: int, threads: int | None, notes: str,
           scale: float | None) -> Case:
    B = len(ctx)
    ctx_arr = np.asarray(ctx, dtype=np.int32).reshape(B)
    need = [(int(n) + page - 1) // page for n in ctx_arr]
    total = int(sum(need))
    if pool_pages is None:
        pool_pages = max(total, 1)
    if pool_pages < total:
        raise ValueError(f"pool of {pool_pages} pages cannot hold {total} pages")
    if max_blocks is None:
        max_blocks = max(need) if need else 1
        max_blocks = max(max_blocks, 1)
    if max(need, default=0) > max_blocks:
        raise ValueError("max_blocks too small for the longest context")

    perm = rng_meta.permutation(pool_pages).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    if shared_prefix_pages and B > 1:
        k = shared_prefix_pages
        for b in range(1, B):
            kk = min(k, need[b], need[0])
            table[b, :kk] = table[0, :kk]

    peaky_pos: list[np.ndarray] = []
    if peaky_frac > 0.0:
        for b in range(B):
            n = int(ctx_arr[b])
            cnt = int(math.floor(peaky_frac * n))
            peaky_pos.append(np.sort(rng_meta.choice(n, size=cnt, replace=False)) if cnt else
                             np.zeros(0, dtype=np.int64))

    q = f32_to_bf16_bits(np.random.default_rng([seed, 1]).standard_normal((B, Hq, D), dtype=np.float32))
    if shared_q_pairs:
        q[1::2] = q[0::2][: q[1::2].shape[0]]

    page_elems = page * Hkv * D
    k_pool = _normal_pool_bits(seed, 2, pool_pages, page_elems, threads).reshape(pool_pages, page, Hkv, D)
    v_pool = _normal_pool_bits(seed, 3, pool_pages, page_elems, threads).reshape(pool_pages, page, Hkv, D)

    for b, pos in enumerate(peaky_pos):
        if pos.size == 0:
            continue
        pages = table[b, pos // page]
        slots = pos % page
        rows = bf16_bits_to_f32(k_pool[pages, slots]) * np.float32(peaky_factor)
        k_pool[pages, slots] = f32_to_bf16_bits(rows)

    if poison:
        used = np.zeros((pool_pages, page), dtype=bool)
        for b in range(B):
            n = int(ctx_arr[b])
            for j in range(need[b]):
                lo = j * page
                used[table[b, j], : min(page, n - lo)] = True
        k_pool[~used] = BF16_QNAN
        v_pool[~used] = BF16_QNAN

    return Case(name=name, q=q, k_pool=k_pool, v_pool=v_pool, block_table=table,
                context_lens=ctx_arr, scale=SCALE if scale is None else float(scale),
                out_dtype=out_dtype, seed=seed, notes=notes)


def make_case(ctx_lens, *, seed: int = 0, Hq: int = HQ, Hkv: int = HKV, D: int = HEAD_DIM,
              page: int = PAGE, pool_pages: int | None = None, max_blocks: int | None = None,
              out_dtype: str = "bf16", shared_q_pairs: bool = False, peaky_frac: float = 0.0,
              peaky_factor: float = 4.0, poison: bool = False, shared_prefix_pages: int = 0,
              threads: int | None = None, name: str = "custom", scale: float | None = None) -> Case:
    """A case with the given context lengths (one per request)."""
    rng_meta = np.random.default_rng([seed, 0])
    return _build(name, [int(n) for n in ctx_lens], rng_meta, seed=seed, Hq=Hq, Hkv=Hkv, D=D,
                  page=page, pool_pages=pool_pages, max_blocks=max_blocks, out_dtype=out_dtype,
                  shared_q_pairs=shared_q_pairs, peaky_frac=peaky_frac, peaky_factor=peaky_factor,
                  poison=poison, shared_prefix_pages=shared_prefix_pages, threads=threads,
                  notes="", scale=scale)


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------
def _c1(rng, seed, threads):
    return _build("c1_b1_ctx512", [512], rng, seed=seed, Hq=HQ, Hkv=HKV, D=HEAD_DIM, page=PAGE,
                  pool_pages=64, max_blocks=32, out_dtype="f32", shared_q_pairs=False,
                  peaky_frac=0.0, peaky_factor=4.0, poison=False, shared_prefix_pages=0,
                  threads=threads, scale=None,
                  notes="B=1, ctx 512, 32 pages drawn from a shuffled 64-page pool, fp32 out")


def _c2(rng, seed, threads):
    ctx = [int(x) for x in rng.integers(200, 421, size=16)]
    return _build("c2_b16_short_clips", ctx, rng, seed=seed, Hq=HQ, Hkv=HKV, D=HEAD_DIM, page=PAGE,
                  pool_pages=512, max_blocks=27, out_dtype="bf16", shared_q_pairs=False,
                  peaky_frac=0.0, peaky_factor=4.0, poison=False, shared_prefix_pages=0,
                  threads=threads, scale=None,
                  notes="B=16 short clips, ctx ~ U{200..420}, pages from one shuffled 512-page pool")


def _c3(rng, seed, threads):
    return _build("c3_b1_ctx28672_peaky", [28672], rng, seed=seed, Hq=HQ, Hkv=HKV, D=HEAD_DIM,
                  page=PAGE, pool_pages=2048, max_blocks=1792, out_dtype="bf16",
                  shared_q_pairs=False, peaky_frac=0.01, peaky_factor=4.0, poison=False,
                  shared_prefix_pages=0, threads=threads, scale=None,
                  notes="B=1 long meeting, ctx 28672 (~38 min), 1% of key positions x4")


def _c4(rng, seed, threads):
    return _build("c4_b16_ctx28672", [28672] * 16, rng, seed=seed, Hq=HQ, Hkv=HKV, D=HEAD_DIM,
                  page=PAGE, pool_pages=28672, max_blocks=1792, out_dtype="bf16",
                  shared_q_pairs=False, peaky_frac=0.0, peaky_factor=4.0, poison=False,
                  shared_prefix_pages=0, threads=threads, scale=None,
                  notes="B=16 long meetings, ctx 28672 each, the whole 28672-page pool shuffled")


def c5_context_lens(rng: np.random.Generator) -> list[int]:
    lo, hi = math.log(256.0), math.log(67500.0)
    u = rng.uniform(lo, hi, size=32)
    ctx = [min(67500, max(256, int(math.floor(math.exp(x))))) for x in u]
    ctx[0] = 67500
    return ctx


def _c5(rng, seed, threads):
    ctx = c5_context_lens(rng)
    return _build("c5_b32_mixed_cfg_pairs", ctx, rng, seed=seed, Hq=HQ, Hkv=HKV, D=HEAD_DIM,
                  page=PAGE, pool_pages=None, max_blocks=4219, out_dtype="bf16",
                  shared_q_pairs=True, peaky_frac=0.0, peaky_factor=4.0, poison=False,
                  shared_prefix_pages=0, threads=threads, scale=None,
                  notes="B=32 ragged, ctx log-uniform in [256, 67500] with request 0 at 67500; "
                        "requests (2i, 2i+1) share q (CFG pairs) and have distinct KV")


def _c3b(rng, seed, threads):
    return _build("c3b_b1_ctx65536", [65536], rng, seed=seed, Hq=HQ, Hkv=HKV, D=HEAD_DIM,
                  page=PAGE, pool_pages=4608, max_blocks=4096, out_dtype="bf16",
                  shared_q_pairs=False, peaky_frac=0.0, peaky_factor=4.0, poison=False,
                  shared_prefix_pages=0, threads=threads, scale=None,
                  notes="supplementary: B=1 at ctx 65536 (the 64k point of the metric)")


CONFIGS = {
    "c1": (1, _c1),
    "c2": (2, _c2),
    "c3": (3, _c3),
    "c4": (4, _c4),
    "c5": (5, _c5),
    "c3b": (6, _c3b),
}


def make_config(name: str, *, seed: int | None = None, threads: int | None = None) -> Case:
    """One of the named workloads; the default seed of config ``cN`` is N."""
    default_seed, fn = CONFIGS[name]
    s = default_seed if seed is None else int(seed)
    rng_meta = np.random.default_rng([s, 0])
    return fn(rng_meta, s, threads)


# --------------------------------------------------------------------------
# KV-cache append: new tokens' K/V (and q) rows
# --------------------------------------------------------------------------
# Streams of an append: 4 = k_new, 5 = v_new, 6 = q rows, 7 = the compact
# pool's page permutation.  RoPE theta 1e6 is the Qwen3 decoder's (audio.cpp
# "Fun-ASR-Nano Native Runtime Design", "Decoder And Prompt").
ROPE_THETA = 1e6


@dataclasses.dataclass
class AppendInputs:
    """New rows for an append into some case's pool: row r of k_new/v_new/q."""
    k_new: np.ndarray              # uint16 bf16 bits [T, Hkv, D]
    v_new: np.ndarray              # uint16 bf16 bits [T, Hkv, D]
    q: np.ndarray | None           # uint16 bf16 bits [T, Hq, D]
    new_start: np.ndarray | None   # int32 [B + 1]; None: one row per request
    max_new_tokens: int
    theta: float = ROPE_THETA

    @property
    def rows(self) -> int:
        return int(self.k_new.shape[0])


def make_append_inputs(case: Case, new_lens=None, *, seed: int = 0, with_q: bool = True,
                       extra_rows: int = 0, theta: float = ROPE_THETA) -> AppendInputs:
    """Rows for appending to ``case``: ``new_lens[b]`` tokens for request b
    (the last ones of its context), or one per request when ``new_lens`` is
    None.  ``extra_rows`` spare rows that no request names are added at the end."""
    B, Hkv, D, Hq = case.B, case.Hkv, case.D, case.Hq
    if new_lens is None:
        T = B
        new_start = None
        max_new = 1
    else:
        n = np.asarray(new_lens, dtype=np.int64).reshape(B)
        if np.any(n < 0) or np.any(n > case.context_lens):
            raise ValueError("new_lens must lie in [0, context_lens]")
        new_start = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        T = int(new_start[-1])
        max_new = int(n.max()) if B else 0
    T += int(extra_rows)

    def draw(stream, heads):
        x = np.random.default_rng([seed, stream]).standard_normal((T, heads, D), dtype=np.float32)
        return f32_to_bf16_bits(x)

    return AppendInputs(k_new=draw(4, Hkv), v_new=draw(5, Hkv), q=draw(6, Hq) if with_q else None,
                        new_start=new_start, max_new_tokens=max_new, theta=theta)


def make_append_case(ctx_lens, new_lens=None, *, seed: int = 0, Hq: int = HQ, Hkv: int = HKV,
                     D: int = HEAD_DIM, page: int = PAGE, extra_pages: int = 0,
                     name: str = "append") -> tuple[Case, AppendInputs]:
    """A compact case for appends alone: the pool holds only the pages the new
    tokens land in (plus ``extra_pages``), shuffled; table entries of earlier
    blocks are -1, since an append reads only the blocks it writes."""
    ctx = np.asarray([int(c) for c in ctx_lens], dtype=np.int32)
    B = ctx.shape[0]
    n = np.ones(B, dtype=np.int64) * (ctx > 0) if new_lens is None else np.asarray(new_lens, dtype=np.int64)
    first = [(int(c) - int(k)) // page for c, k in zip(ctx, n)]
    need = [((int(c) + page - 1) // page - f) if k > 0 else 0 for c, k, f in zip(ctx, n, first)]
    max_blocks = max(1, max(((int(c) + page - 1) // page for c in ctx), default=1))
    pool_pages = max(1, int(sum(need)) + int(extra_pages))
    perm = np.random.default_rng([seed, 7]).permutation(pool_pages).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, first[b]:first[b] + need[b]] = perm[off:off + need[b]]
        off += need[b]
    page_elems = page * Hkv * D
    k_pool = _normal_pool_bits(seed, 2, pool_pages, page_elems, None).reshape(pool_pages, page, Hkv, D)
    v_pool = _normal_pool_bits(seed, 3, pool_pages, page_elems, None).reshape(pool_pages, page, Hkv, D)
    q = f32_to_bf16_bits(np.random.default_rng([seed, 1]).standard_normal((B, Hq, D), dtype=np.float32))
    case = Case(name=name, q=q, k_pool=k_pool, v_pool=v_pool, block_table=table, context_lens=ctx,
                scale=SCALE, out_dtype="bf16", seed=seed,
                notes="compact pool: only the pages the appended tokens land in")
    inputs = make_append_inputs(case, None if new_lens is None else n, seed=seed)
    return case, inputs


# Named append workloads.  a1: the decode step of the 16 x 28672 batch, one
# new token per request.  a2: one 4096-token prefill chunk, the last of a
# 28672-token context (MOSS-TD article, "Chunked prefill for long audio").
APPEND_CONFIGS = {
    "a1": (11, [28672] * 16, None),
    "a2": (12, [28672], [4096]),
}


def make_append_config(name: str, *, copy: int = 0) -> tuple[Case, AppendInputs]:
    """A named append workload; ``copy`` draws an independent instance."""
    seed, ctx, new = APPEND_CONFIGS[name]
    seed = seed * 1000 + int(copy)
    case, inputs = make_append_case(ctx, new, seed=seed, name=f"{name}_{'decode' if new is None else 'chunk'}")
    return case, inputs


# --------------------------------------------------------------------------
# Chunked prefill: query rows of a chunk over a filled cache
# --------------------------------------------------------------------------
@dataclasses.dataclass
class PrefillInputs:
    """Chunk query rows for a case whose cache already holds the chunk's K/V."""
    q: np.ndarray               # uint16 bf16 bits [T, Hq, D]
    new_start: np.ndarray       # int32 [B + 1]
    max_new_tokens: int

    @property
    def rows(self) -> int:
        return int(self.q.shape[0])


def make_prefill_case(ctx_lens, new_lens, *, seed: int = 0, Hq: int = HQ, Hkv: int = HKV,
                      pool_pages: int | None = None, max_blocks: int | None = None, extra_rows: int = 0,
                      poison: bool = False, threads: int | None = None,
                      name: str = "prefill") -> tuple[Case, PrefillInputs]:
    """A full cache (``make_case``) and the query rows of one chunk per
    request: the last ``new_lens[b]`` tokens of request b's context.  The
    rows come from the append generator's q stream.  ``poison`` fills every
    slot no context covers with NaN."""
    case = make_case(ctx_lens, seed=seed, Hq=Hq, Hkv=Hkv, pool_pages=pool_pages, max_blocks=max_blocks,
                     poison=poison, threads=threads, name=name)
    rows = make_append_inputs(case, new_lens, seed=seed, extra_rows=extra_rows)
    return case, PrefillInputs(q=rows.q, new_start=rows.new_start, max_new_tokens=rows.max_new_tokens)


# Named prefill workloads (MOSS-TD article, "Chunked prefill for long audio":
# 4096-token query blocks).  p1: the last chunk of a 28672-token prompt, the
# heaviest; p2: the first chunk, a causal triangle.
PREFILL_CONFIGS = {
    "p1": (21, [28672], [4096]),
    "p2": (22, [4096], [4096]),
}


def make_prefill_config(name: str, *, threads: int | None = None) -> tuple[Case, PrefillInputs]:
    seed, ctx, new = PREFILL_CONFIGS[name]
    label = {"p1": "p1_last_chunk_of_28672", "p2": "p2_first_chunk_4096"}[name]
    return make_prefill_case(ctx, new, seed=seed, threads=threads, name=label)
