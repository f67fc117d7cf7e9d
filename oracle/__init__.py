"""ctypes front end of the fp64 paged-attention oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library and
its Python binding never do; a product path that reached this code would not be
a GPU result.

The arithmetic lives in C:

- ``paged_attn_oracle.c``: the plain definition out = softmax(scale * q K^T) V
  and lse = ln(sum exp(scale * q K^T)) over the tokens a request's block table
  names, in fp64;
- ``kv_append_oracle.c``: writing new tokens' K and V into their pages, with
  optional RoPE on K and q, rotated in fp64 and rounded once to bf16;
- ``prefill_attn_oracle.c``: chunked-prefill attention, each chunk row being
  the decode definition over the cache up to its own position.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB_CACHE: dict[str, ctypes.CDLL] = {}


class OracleShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
    ]


class OracleError(RuntimeError):
    pass


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if it is absent) the oracle library at ``path``."""
    path = path or _build.LIB
    if path in _LIB_CACHE:
        return _LIB_CACHE[path]
    if path == _build.LIB and not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    lib.oracle_validate.argtypes = [ctypes.POINTER(OracleShape), p, p]
    lib.oracle_validate.restype = ctypes.c_int
    lib.oracle_attend_one.argtypes = [ctypes.POINTER(OracleShape), p, p, p, p, p, ctypes.c_double,
                                      ctypes.c_int32, ctypes.c_int32, p, p]
    lib.oracle_attend_one.restype = ctypes.c_int
    lib.oracle_paged_attn.argtypes = [ctypes.POINTER(OracleShape), p, p, p, p, p, ctypes.c_double, p, p]
    lib.oracle_paged_attn.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_rope_f64.argtypes = [p, ctypes.c_int32, ctypes.c_double, ctypes.c_double]
    lib.oracle_rope_f64.restype = None
    lib.oracle_kv_append_validate.argtypes = [ctypes.POINTER(OracleShape), ctypes.c_int32, p, p, p]
    lib.oracle_kv_append_validate.restype = ctypes.c_int
    lib.oracle_kv_append.argtypes = [ctypes.POINTER(OracleShape), ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_double, p, p, p, p, p, p, p, p]
    lib.oracle_kv_append.restype = ctypes.c_int
    lib.oracle_prefill_validate.argtypes = [ctypes.POINTER(OracleShape), ctypes.c_int32, p, p, p]
    lib.oracle_prefill_validate.restype = ctypes.c_int
    lib.oracle_prefill_attn.argtypes = [ctypes.POINTER(OracleShape), ctypes.c_int32, p, p, p, p, p, p,
                                        ctypes.c_double, p, p]
    lib.oracle_prefill_attn.restype = ctypes.c_int
    lib.oracle_prefill_attn_pairs.argtypes = [ctypes.POINTER(OracleShape), ctypes.c_int32, p, p, p, p, p, p,
                                              ctypes.c_double, p, ctypes.c_int32, p, p]
    lib.oracle_prefill_attn_pairs.restype = ctypes.c_int
    _LIB_CACHE[path] = lib
    return lib


def _prep(q, k_pool, v_pool, block_table, context_lens):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_pool = np.ascontiguousarray(k_pool, dtype=np.uint16)
    v_pool = np.ascontiguousarray(v_pool, dtype=np.uint16)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    if q.ndim != 3 or k_pool.ndim != 4 or k_pool.shape != v_pool.shape:
        raise OracleError("q must be [B,Hq,D]; pools must be [P,page,Hkv,D] and equal in shape")
    B, Hq, D = q.shape
    P, page, Hkv, Dk = k_pool.shape
    if Dk != D or block_table.ndim != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise OracleError("inconsistent shapes")
    shape = OracleShape(B, Hq, Hkv, D, page, P, block_table.shape[1])
    return shape, q, k_pool, v_pool, block_table, context_lens


def paged_attn(q, k_pool, v_pool, block_table, context_lens, scale, *, lib: ctypes.CDLL | None = None):
    """fp64 (out [B,Hq,D], lse [B,Hq]) for every request and query head."""
    lib = lib or load()
    shape, q, k_pool, v_pool, block_table, context_lens = _prep(q, k_pool, v_pool, block_table, context_lens)
    out = np.zeros((shape.num_seqs, shape.num_q_heads, shape.head_dim), dtype=np.float64)
    lse = np.zeros((shape.num_seqs, shape.num_q_heads), dtype=np.float64)
    rc = lib.oracle_paged_attn(ctypes.byref(shape), q.ctypes.data, k_pool.ctypes.data, v_pool.ctypes.data,
                               block_table.ctypes.data, context_lens.ctypes.data, float(scale),
                               out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise OracleError(f"oracle_paged_attn returned {rc}")
    return out, lse


def run_case(case, *, lib: ctypes.CDLL | None = None):
    """Oracle over a ``workloads.Case`` (any object with the same fields)."""
    return paged_attn(case.q, case.k_pool, case.v_pool, case.block_table, case.context_lens,
                      case.scale, lib=lib)


def validate(q, k_pool, v_pool, block_table, context_lens, *, lib: ctypes.CDLL | None = None) -> int:
    lib = lib or load()
    shape, q, k_pool, v_pool, block_table, context_lens = _prep(q, k_pool, v_pool, block_table, context_lens)
    return int(lib.oracle_validate(ctypes.byref(shape), block_table.ctypes.data, context_lens.ctypes.data))


def max_threads(lib: ctypes.CDLL | None = None) -> int:
    return int((lib or load()).oracle_max_threads())


def round_bf16(x, *, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """Nearest-even bf16 bit patterns (uint16) of the float64 values ``x``."""
    lib = lib or load()
    flat = np.asarray(x, dtype=np.float64).ravel()
    out = np.fromiter((lib.oracle_round_bf16(float(v)) for v in flat), dtype=np.uint16, count=flat.size)
    return out.reshape(np.shape(x))


def rope_f64(x, pos, theta, *, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """RoPE of float64 head vectors ``x[..., D]`` at position ``pos`` (a copy)."""
    lib = lib or load()
    y = np.array(x, dtype=np.float64, copy=True)
    rows = y.reshape(-1, y.shape[-1])
    for r in rows:
        lib.oracle_rope_f64(r.ctypes.data, r.shape[0], float(pos), float(theta))
    return y


def _append_prep(k_new, v_new, block_table, context_lens, k_pool, new_start, q, num_q_heads):
    k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
    v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    if k_new.ndim != 3 or k_new.shape != v_new.shape or k_pool.ndim != 4:
        raise OracleError("k_new/v_new must be [T,Hkv,D] and equal; pools [P,page,Hkv,D]")
    T, Hkv, D = k_new.shape
    P, page, Hkv_p, D_p = k_pool.shape
    if (Hkv_p, D_p) != (Hkv, D) or block_table.ndim != 2 or context_lens.ndim != 1 \
            or block_table.shape[0] != context_lens.shape[0]:
        raise OracleError("inconsistent shapes")
    B = context_lens.shape[0]
    if q is not None:
        if q.ndim != 3 or q.shape[0] != T or q.shape[2] != D:
            raise OracleError("q must be [T,Hq,D]")
        num_q_heads = q.shape[1]
    shape = OracleShape(B, num_q_heads or Hkv, Hkv, D, page, P, block_table.shape[1])
    ns = None if new_start is None else np.ascontiguousarray(new_start, dtype=np.int32)
    if ns is not None and ns.shape != (B + 1,):
        raise OracleError("new_start must have num_seqs + 1 entries")
    return shape, T, k_new, v_new, block_table, context_lens, ns


def kv_append(k_new, v_new, block_table, context_lens, k_pool, v_pool, *, new_start=None, q=None,
              rope=False, theta=1e6, lib: ctypes.CDLL | None = None):
    """Append new tokens' K/V (bf16 bits) to copies of the pools.

    Returns ``(k_pool, v_pool, q)``: the updated copies, and q rotated (a copy)
    or ``None``.  ``new_start`` [B+1] gives each request's rows of ``k_new``;
    ``None`` means one row per request with a non-empty context.
    """
    lib = lib or load()
    k_out = np.array(k_pool, dtype=np.uint16, copy=True, order="C")
    v_out = np.array(v_pool, dtype=np.uint16, copy=True, order="C")
    q_out = None if q is None else np.array(q, dtype=np.uint16, copy=True, order="C")
    shape, T, k_new, v_new, table, ctx, ns = _append_prep(k_new, v_new, block_table, context_lens, k_out,
                                                          new_start, q_out, None)
    rc = lib.oracle_kv_append(ctypes.byref(shape), T, 1 if rope else 0, float(theta),
                              None if q_out is None else q_out.ctypes.data, k_new.ctypes.data,
                              v_new.ctypes.data, None if ns is None else ns.ctypes.data,
                              table.ctypes.data, ctx.ctypes.data, k_out.ctypes.data, v_out.ctypes.data)
    if rc != 0:
        raise OracleError(f"oracle_kv_append returned {rc}")
    return k_out, v_out, q_out


def kv_append_validate(k_new, block_table, context_lens, k_pool, *, new_start=None,
                       lib: ctypes.CDLL | None = None) -> int:
    lib = lib or load()
    k_new = np.asarray(k_new)
    shape, T, _, _, table, ctx, ns = _append_prep(k_new, k_new, block_table, context_lens, np.asarray(k_pool),
                                                  new_start, None, None)
    return int(lib.oracle_kv_append_validate(ctypes.byref(shape), T, None if ns is None else ns.ctypes.data,
                                             table.ctypes.data, ctx.ctypes.data))


def _prefill_prep(q, k_pool, v_pool, block_table, context_lens, new_start):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_pool = np.ascontiguousarray(k_pool, dtype=np.uint16)
    v_pool = np.ascontiguousarray(v_pool, dtype=np.uint16)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    new_start = np.ascontiguousarray(new_start, dtype=np.int32)
    if q.ndim != 3 or k_pool.ndim != 4 or k_pool.shape != v_pool.shape:
        raise OracleError("q must be [T,Hq,D]; pools must be [P,page,Hkv,D] and equal in shape")
    T, Hq, D = q.shape
    P, page, Hkv, Dk = k_pool.shape
    B = context_lens.shape[0]
    if Dk != D or block_table.ndim != 2 or block_table.shape[0] != B or new_start.shape != (B + 1,):
        raise OracleError("inconsistent shapes")
    shape = OracleShape(B, Hq, Hkv, D, page, P, block_table.shape[1])
    return shape, T, q, k_pool, v_pool, block_table, context_lens, new_start


def prefill_attn(q, k_pool, v_pool, block_table, context_lens, new_start, scale, *,
                 lib: ctypes.CDLL | None = None):
    """fp64 (out [T,Hq,D], lse [T,Hq]) of every chunk row; rows no request
    names are NaN."""
    lib = lib or load()
    shape, T, q, k_pool, v_pool, table, ctx, ns = _prefill_prep(q, k_pool, v_pool, block_table, context_lens,
                                                                new_start)
    out = np.full((T, shape.num_q_heads, shape.head_dim), np.nan, dtype=np.float64)
    lse = np.full((T, shape.num_q_heads), np.nan, dtype=np.float64)
    rc = lib.oracle_prefill_attn(ctypes.byref(shape), T, q.ctypes.data, k_pool.ctypes.data, v_pool.ctypes.data,
                                 ns.ctypes.data, table.ctypes.data, ctx.ctypes.data, float(scale),
                                 out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise OracleError(f"oracle_prefill_attn returned {rc}")
    return out, lse


def prefill_attn_pairs(q, k_pool, v_pool, block_table, context_lens, new_start, scale, pairs, *,
                       lib: ctypes.CDLL | None = None):
    """fp64 (out [n,D], lse [n]) for the (row, query head) pairs listed."""
    lib = lib or load()
    shape, T, q, k_pool, v_pool, table, ctx, ns = _prefill_prep(q, k_pool, v_pool, block_table, context_lens,
                                                                new_start)
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    n = pairs.shape[0]
    out = np.zeros((n, shape.head_dim), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    rc = lib.oracle_prefill_attn_pairs(ctypes.byref(shape), T, q.ctypes.data, k_pool.ctypes.data,
                                       v_pool.ctypes.data, ns.ctypes.data, table.ctypes.data, ctx.ctypes.data,
                                       float(scale), pairs.ctypes.data, n, out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise OracleError(f"oracle_prefill_attn_pairs returned {rc}")
    return out, lse


def prefill_validate(q, k_pool, block_table, context_lens, new_start, *, lib: ctypes.CDLL | None = None) -> int:
    lib = lib or load()
    shape, T, _, _, _, table, ctx, ns = _prefill_prep(q, k_pool, k_pool, block_table, context_lens, new_start)
    return int(lib.oracle_prefill_validate(ctypes.byref(shape), T, ns.ctypes.data, table.ctypes.data,
                                           ctx.ctypes.data))
