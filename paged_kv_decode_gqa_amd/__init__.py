"""Python binding of ``libhipdecode.so`` (the C ABI in ``include/hipdecode.h``).

Argument marshalling only: every step of the decode attention, the KV-cache
append and the chunked-prefill attention runs in the library's HIP kernels.  The functions carry the C names; tensors are PyTorch device
tensors and are passed as raw pointers on the current HIP stream.

If the library has not been built, importing works but every call raises
``RuntimeError``; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhipdecode.so")

HIPDECODE_OK = 0
HIPDECODE_ERR_NULL = 1
HIPDECODE_ERR_SHAPE = 2
HIPDECODE_ERR_UNSUPPORTED = 3
HIPDECODE_ERR_ALIGN = 4
HIPDECODE_ERR_WORKSPACE = 5
HIPDECODE_ERR_SCALE = 6
HIPDECODE_ERR_HIP = 7
HIPDECODE_BF16 = 0
HIPDECODE_F32 = 1
HIPDECODE_SCHEDULE_SPLIT = 1
HIPDECODE_ROPE_NONE = 0
HIPDECODE_ROPE_HALF = 1

EXPORTED = (
    "hipdecode_abi_version",
    "hipdecode_check_params",
    "hipdecode_partition_tokens",
    "hipdecode_workgroup_waves",
    "hipdecode_schedule",
    "hipdecode_workspace_bytes",
    "hipdecode_workspace_init",
    "hipdecode_paged_attn",
    "hipdecode_paged_attn_append",
    "hipdecode_check_append_params",
    "hipdecode_kv_append",
    "hipdecode_check_prefill_params",
    "hipdecode_prefill_attn",
    "hipdecode_step_bucket",
    "hipdecode_step_runner_create",
    "hipdecode_step_runner_step",
    "hipdecode_step_runner_destroy",
    "hipdecode_paged_attn_noalloc",
    "hipdecode_contract_violations",
    "hipdecode_status_string",
)

# Bits of hipdecode_contract_violations: device-side contents that broke the
# contract (the kernels clamped or skipped them; the results are unspecified).
HIPDECODE_VIOLATION_CONTEXT = 1
HIPDECODE_VIOLATION_PAGE = 2
HIPDECODE_VIOLATION_ROWS = 4
HIPDECODE_VIOLATION_VALUE = 8

# Bytes of the library's static scratch behind hipdecode_paged_attn_noalloc.
HIPDECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


class hipdecode_params(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_context_len", ctypes.c_int32),
        ("partition_tokens", ctypes.c_int32),
        ("workgroup_waves", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class hipdecode_append_params(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_rows", ctypes.c_int32),
        ("max_new_tokens", ctypes.c_int32),
        ("rope", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
    ]


class hipdecode_prefill_params(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_rows", ctypes.c_int32),
        ("max_new_tokens", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class hipdecode_step_config(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("max_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_context_len", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("rope_theta", ctypes.c_double),
    ]


class hipdecode_step_buffers(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.POINTER(ctypes.c_void_p)),
        ("v_pool", ctypes.POINTER(ctypes.c_void_p)),
        ("q", ctypes.POINTER(ctypes.c_void_p)),
        ("k_new", ctypes.POINTER(ctypes.c_void_p)),
        ("v_new", ctypes.POINTER(ctypes.c_void_p)),
        ("out", ctypes.POINTER(ctypes.c_void_p)),
        ("lse", ctypes.POINTER(ctypes.c_void_p)),
        ("block_table", ctypes.c_void_p),
        ("context_lens", ctypes.c_void_p),
    ]


class HipDecodeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({hipdecode_status_string(status)})")


_lib = None


def library() -> ctypes.CDLL:
    """The loaded HIP library; raises RuntimeError if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_decode_gqa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(hipdecode_params)
    vp = ctypes.c_void_p
    lib.hipdecode_abi_version.argtypes = []
    lib.hipdecode_abi_version.restype = ctypes.c_int
    lib.hipdecode_check_params.argtypes = [P]
    lib.hipdecode_check_params.restype = ctypes.c_int
    lib.hipdecode_partition_tokens.argtypes = [P]
    lib.hipdecode_partition_tokens.restype = ctypes.c_int32
    lib.hipdecode_workgroup_waves.argtypes = [P]
    lib.hipdecode_workgroup_waves.restype = ctypes.c_int32
    lib.hipdecode_schedule.argtypes = [P]
    lib.hipdecode_schedule.restype = ctypes.c_int32
    lib.hipdecode_workspace_bytes.argtypes = [P]
    lib.hipdecode_workspace_bytes.restype = ctypes.c_size_t
    lib.hipdecode_workspace_init.argtypes = [vp, ctypes.c_size_t, vp]
    lib.hipdecode_workspace_init.restype = ctypes.c_int
    lib.hipdecode_paged_attn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.hipdecode_paged_attn.restype = ctypes.c_int
    lib.hipdecode_paged_attn_append.argtypes = [P, ctypes.c_double, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                ctypes.c_size_t, vp]
    lib.hipdecode_paged_attn_append.restype = ctypes.c_int
    PA = ctypes.POINTER(hipdecode_append_params)
    lib.hipdecode_check_append_params.argtypes = [PA]
    lib.hipdecode_check_append_params.restype = ctypes.c_int
    lib.hipdecode_kv_append.argtypes = [PA, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hipdecode_kv_append.restype = ctypes.c_int
    PP = ctypes.POINTER(hipdecode_prefill_params)
    lib.hipdecode_check_prefill_params.argtypes = [PP]
    lib.hipdecode_check_prefill_params.restype = ctypes.c_int
    lib.hipdecode_prefill_attn.argtypes = [PP, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hipdecode_prefill_attn.restype = ctypes.c_int
    lib.hipdecode_step_bucket.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.hipdecode_step_bucket.restype = ctypes.c_int32
    lib.hipdecode_step_runner_create.argtypes = [ctypes.POINTER(hipdecode_step_config),
                                                 ctypes.POINTER(hipdecode_step_buffers), ctypes.POINTER(vp)]
    lib.hipdecode_step_runner_create.restype = ctypes.c_int
    lib.hipdecode_step_runner_step.argtypes = [vp, ctypes.c_int32, vp, vp]
    lib.hipdecode_step_runner_step.restype = ctypes.c_int
    lib.hipdecode_step_runner_destroy.argtypes = [vp]
    lib.hipdecode_step_runner_destroy.restype = ctypes.c_int
    lib.hipdecode_paged_attn_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hipdecode_paged_attn_noalloc.restype = ctypes.c_int
    lib.hipdecode_contract_violations.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    lib.hipdecode_contract_violations.restype = ctypes.c_int
    lib.hipdecode_status_string.argtypes = [ctypes.c_int]
    lib.hipdecode_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def make_params(*, num_seqs, num_q_heads, num_kv_heads, num_pages, max_blocks_per_seq,
                max_context_len, scale, head_dim=128, page_size=16, partition_tokens=0,
                workgroup_waves=0, schedule=0, out_dtype=HIPDECODE_BF16) -> hipdecode_params:
    return hipdecode_params(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim),
                            int(page_size), int(num_pages), int(max_blocks_per_seq),
                            int(max_context_len), int(partition_tokens), int(workgroup_waves),
                            int(schedule), int(out_dtype), float(scale))


def make_append_params(*, num_seqs, num_q_heads, num_kv_heads, num_pages, max_blocks_per_seq, num_rows,
                       max_new_tokens=1, rope=HIPDECODE_ROPE_NONE, rope_theta=1e6, head_dim=128,
                       page_size=16) -> hipdecode_append_params:
    return hipdecode_append_params(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim),
                                   int(page_size), int(num_pages), int(max_blocks_per_seq), int(num_rows),
                                   int(max_new_tokens), int(rope), float(rope_theta))


def make_prefill_params(*, num_seqs, num_q_heads, num_kv_heads, num_pages, max_blocks_per_seq, num_rows,
                        max_new_tokens, scale, head_dim=128, page_size=16,
                        out_dtype=HIPDECODE_BF16) -> hipdecode_prefill_params:
    return hipdecode_prefill_params(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim),
                                    int(page_size), int(num_pages), int(max_blocks_per_seq), int(num_rows),
                                    int(max_new_tokens), int(out_dtype), float(scale))


def hipdecode_abi_version() -> int:
    return int(library().hipdecode_abi_version())


def hipdecode_check_params(params: hipdecode_params | None) -> int:
    return int(library().hipdecode_check_params(ctypes.byref(params) if params is not None else None))


def hipdecode_partition_tokens(params: hipdecode_params) -> int:
    return int(library().hipdecode_partition_tokens(ctypes.byref(params)))


def hipdecode_workgroup_waves(params: hipdecode_params) -> int:
    return int(library().hipdecode_workgroup_waves(ctypes.byref(params)))


def hipdecode_schedule(params: hipdecode_params) -> int:
    return int(library().hipdecode_schedule(ctypes.byref(params)))


def hipdecode_workspace_bytes(params: hipdecode_params) -> int:
    return int(library().hipdecode_workspace_bytes(ctypes.byref(params)))


def hipdecode_status_string(status: int) -> str:
    return library().hipdecode_status_string(int(status)).decode()


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream) if hasattr(stream, "cuda_stream") else ctypes.c_void_p(stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def hipdecode_workspace_init(workspace, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size()
    st = library().hipdecode_workspace_init(_ptr(workspace), nbytes, _stream_handle(stream))
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_workspace_init")


def hipdecode_paged_attn(params: hipdecode_params, q, k_pool, v_pool, block_table, context_lens,
                         out, lse, workspace, stream=None) -> None:
    """Enqueue one call on ``stream`` (default: torch's current stream).

    Tensors must be contiguous device tensors laid out as ``include/hipdecode.h``
    states; ``lse`` may be None.  Raises HipDecodeError on a non-OK status."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("block_table", block_table),
                    ("context_lens", context_lens), ("out", out), ("lse", lse), ("workspace", workspace)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().hipdecode_paged_attn(ctypes.byref(params), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        _ptr(block_table), _ptr(context_lens), _ptr(out), _ptr(lse),
                                        _ptr(workspace), ws_bytes, _stream_handle(stream))
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_paged_attn")


def hipdecode_paged_attn_noalloc(params: hipdecode_params, q, k_pool, v_pool, block_table, context_lens,
                                 out, lse, stream=None) -> None:
    """Enqueue one allocation-free call (the library's static scratch stands
    in for the workspace).  Raises HipDecodeError on a non-OK status."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("block_table", block_table),
                    ("context_lens", context_lens), ("out", out), ("lse", lse)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    st = library().hipdecode_paged_attn_noalloc(ctypes.byref(params), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                                _ptr(block_table), _ptr(context_lens), _ptr(out), _ptr(lse),
                                                _stream_handle(stream))
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_paged_attn_noalloc")


def hipdecode_contract_violations() -> int:
    """Wait for the current device, return the HIPDECODE_VIOLATION_* bits the
    library's kernels set there since the last call, and clear them."""
    flags = ctypes.c_uint32(0)
    st = library().hipdecode_contract_violations(ctypes.byref(flags))
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_contract_violations")
    return int(flags.value)


class PreparedCall:
    """The marshalled argument list of one ``hipdecode_paged_attn`` call.

    Built once from tensors that stay alive (and in place) across calls, then
    invoked many times; each invocation enqueues the kernel on the current
    stream (or ``stream``) without re-marshalling the tensors."""

    def __init__(self, params, q, k_pool, v_pool, block_table, context_lens, out, lse, workspace):
        self._keep = (params, q, k_pool, v_pool, block_table, context_lens, out, lse, workspace)
        for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("block_table", block_table),
                        ("context_lens", context_lens), ("out", out), ("lse", lse), ("workspace", workspace)):
            if t is not None and not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        ws_bytes = workspace.numel() * workspace.element_size()
        self._args = (ctypes.byref(params), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                      _ptr(context_lens), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes)
        self._fn = library().hipdecode_paged_attn

    def __call__(self, stream=None) -> None:
        st = self._fn(*self._args, _stream_handle(stream))
        if st != HIPDECODE_OK:
            raise HipDecodeError(st, "hipdecode_paged_attn")


def _check_tensor(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_call_tensors(q, k_pool, v_pool, block_table, context_lens, rows, out, lse, out_dtype):
    """Host checks of what the C ABI cannot see: shapes, dtypes and devices of
    the tensors a convenience call passes, so that a mismatched buffer is a
    ValueError rather than a kernel writing past it."""
    import torch
    if q.dim() != 3 or k_pool.dim() != 4:
        raise ValueError("q must be [rows, Hq, 128] and k_pool [P, 16, Hkv, 128]")
    dev = q.device
    _, Hq, D = q.shape
    _check_tensor("v_pool", v_pool, k_pool.shape, torch.bfloat16, dev)
    _check_tensor("k_pool", k_pool, k_pool.shape, torch.bfloat16, dev)
    B = context_lens.shape[0] if context_lens.dim() == 1 else -1
    _check_tensor("context_lens", context_lens, (B,), torch.int32, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [{B}, max_blocks]")
    _check_tensor("block_table", block_table, block_table.shape, torch.int32, dev)
    if out is not None:
        _check_tensor("out", out, (rows, Hq, D), out_dtype, dev)
    if lse is not None:
        _check_tensor("lse", lse, (rows, Hq), torch.float32, dev)


def paged_attn(q, k_pool, v_pool, block_table, context_lens, scale, *, max_context_len,
               out_dtype=None, partition_tokens=0, workgroup_waves=0, schedule=0, out=None, lse=None,
               workspace=None):
    """Allocate outputs (and a zeroed workspace) as needed and run one call.

    q: bf16 [B,Hq,128]; k_pool, v_pool: bf16 [P,16,Hkv,128]; block_table: int32
    [B, max_blocks]; context_lens: int32 [B].  Returns (out, lse)."""
    import torch
    if q.dtype != torch.bfloat16 or k_pool.dtype != torch.bfloat16 or v_pool.dtype != torch.bfloat16:
        raise ValueError("q, k_pool and v_pool must be bfloat16")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_table and context_lens must be int32")
    B, Hq, D = q.shape
    P, page, Hkv, Dk = k_pool.shape
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    _check_call_tensors(q, k_pool, v_pool, block_table, context_lens, B, out, lse, out_dtype)
    code = HIPDECODE_F32 if out_dtype == torch.float32 else HIPDECODE_BF16
    params = make_params(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, num_pages=P,
                         max_blocks_per_seq=block_table.shape[1], max_context_len=max_context_len,
                         scale=scale, head_dim=D, page_size=page, partition_tokens=partition_tokens,
                         workgroup_waves=workgroup_waves, schedule=schedule, out_dtype=code)
    st = hipdecode_check_params(params)
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_check_params")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = hipdecode_workspace_bytes(params)
        workspace = torch.zeros(max(nbytes, 16) // 4 + 4, dtype=torch.int32, device=q.device)
    hipdecode_paged_attn(params, q, k_pool, v_pool, block_table, context_lens, out, lse, workspace)
    return out, lse


def hipdecode_check_append_params(params: hipdecode_append_params | None) -> int:
    return int(library().hipdecode_check_append_params(ctypes.byref(params) if params is not None else None))


def hipdecode_kv_append(params: hipdecode_append_params, q, k_new, v_new, new_start, block_table,
                        context_lens, k_pool, v_pool, stream=None) -> None:
    """Enqueue one append on ``stream`` (default: torch's current stream).

    ``q`` and ``new_start`` may be None.  Raises HipDecodeError on a non-OK
    status."""
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("new_start", new_start),
                    ("block_table", block_table), ("context_lens", context_lens), ("k_pool", k_pool),
                    ("v_pool", v_pool)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    st = library().hipdecode_kv_append(ctypes.byref(params), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(new_start),
                                       _ptr(block_table), _ptr(context_lens), _ptr(k_pool), _ptr(v_pool),
                                       _stream_handle(stream))
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_kv_append")


class PreparedAttnAppend:
    """The marshalled argument list of one ``hipdecode_paged_attn_append``
    call, invoked many times without re-marshalling."""

    def __init__(self, params, rope_theta, q, k_new, v_new, k_pool, v_pool, block_table, context_lens, out, lse,
                 workspace):
        self._keep = (params, q, k_new, v_new, k_pool, v_pool, block_table, context_lens, out, lse, workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
        self._args = (ctypes.byref(params), float(rope_theta), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                      _ptr(v_pool), _ptr(block_table), _ptr(context_lens), _ptr(out), _ptr(lse), _ptr(workspace),
                      ws_bytes)
        self._fn = library().hipdecode_paged_attn_append

    def __call__(self, stream=None) -> None:
        st = self._fn(*self._args, _stream_handle(stream))
        if st != HIPDECODE_OK:
            raise HipDecodeError(st, "hipdecode_paged_attn_append")


class PreparedAppend:
    """The marshalled argument list of one ``hipdecode_kv_append`` call,
    invoked many times on the current stream (or ``stream``) without
    re-marshalling; the tensors must stay alive and in place."""

    def __init__(self, params, q, k_new, v_new, new_start, block_table, context_lens, k_pool, v_pool):
        self._keep = (params, q, k_new, v_new, new_start, block_table, context_lens, k_pool, v_pool)
        for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("new_start", new_start),
                        ("block_table", block_table), ("context_lens", context_lens), ("k_pool", k_pool),
                        ("v_pool", v_pool)):
            if t is not None and not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        self._args = (ctypes.byref(params), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(new_start),
                      _ptr(block_table), _ptr(context_lens), _ptr(k_pool), _ptr(v_pool))
        self._fn = library().hipdecode_kv_append

    def __call__(self, stream=None) -> None:
        st = self._fn(*self._args, _stream_handle(stream))
        if st != HIPDECODE_OK:
            raise HipDecodeError(st, "hipdecode_kv_append")


def kv_append(k_new, v_new, block_table, context_lens, k_pool, v_pool, *, q=None, new_start=None,
              max_new_tokens=None, rope_theta=None):
    """Write new tokens' K/V into the pools in place (rotating K and ``q`` by
    RoPE when ``rope_theta`` is given).

    k_new, v_new: bf16 [T,Hkv,128]; q: bf16 [T,Hq,128] or None; new_start:
    int32 [B+1] or None (one row per request); block_table, context_lens and
    the pools as for ``paged_attn``.  ``max_new_tokens`` bounds any request's
    new tokens when ``new_start`` is given (default: T)."""
    import torch
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool), ("v_pool", v_pool), ("q", q)):
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    for name, t in (("block_table", block_table), ("context_lens", context_lens), ("new_start", new_start)):
        if t is not None and t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    T, Hkv, D = k_new.shape
    P, page, Hkv_p, D_p = k_pool.shape
    if (Hkv_p, D_p) != (Hkv, D) or v_new.shape != k_new.shape or v_pool.shape != k_pool.shape:
        raise ValueError("inconsistent K/V shapes")
    if q is not None and (q.dim() != 3 or q.shape[0] != T or q.shape[2] != D):
        raise ValueError("q must be [T, Hq, head_dim]")
    Hq = q.shape[1] if q is not None else Hkv
    B = context_lens.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [{B}, max_blocks]")
    if new_start is not None and new_start.shape != (B + 1,):
        raise ValueError("new_start must have num_seqs + 1 entries")
    if max_new_tokens is None:
        max_new_tokens = T if new_start is not None else 1
    params = make_append_params(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, num_pages=P,
                                max_blocks_per_seq=block_table.shape[1], num_rows=T,
                                max_new_tokens=max_new_tokens,
                                rope=HIPDECODE_ROPE_NONE if rope_theta is None else HIPDECODE_ROPE_HALF,
                                rope_theta=1e6 if rope_theta is None else rope_theta,
                                head_dim=D, page_size=page)
    hipdecode_kv_append(params, q, k_new, v_new, new_start, block_table, context_lens, k_pool, v_pool)


def hipdecode_check_prefill_params(params: hipdecode_prefill_params | None) -> int:
    return int(library().hipdecode_check_prefill_params(ctypes.byref(params) if params is not None else None))


def hipdecode_prefill_attn(params: hipdecode_prefill_params, q, k_pool, v_pool, new_start, block_table,
                           context_lens, out, lse, stream=None) -> None:
    """Enqueue one chunked-prefill attention call; ``lse`` may be None."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("new_start", new_start),
                    ("block_table", block_table), ("context_lens", context_lens), ("out", out), ("lse", lse)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    st = library().hipdecode_prefill_attn(ctypes.byref(params), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                          _ptr(new_start), _ptr(block_table), _ptr(context_lens), _ptr(out),
                                          _ptr(lse), _stream_handle(stream))
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_prefill_attn")


class PreparedPrefill:
    """The marshalled argument list of one ``hipdecode_prefill_attn`` call,
    invoked many times without re-marshalling; tensors must stay in place."""

    def __init__(self, params, q, k_pool, v_pool, new_start, block_table, context_lens, out, lse):
        self._keep = (params, q, k_pool, v_pool, new_start, block_table, context_lens, out, lse)
        self._args = (ctypes.byref(params), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(new_start),
                      _ptr(block_table), _ptr(context_lens), _ptr(out), _ptr(lse))
        self._fn = library().hipdecode_prefill_attn

    def __call__(self, stream=None) -> None:
        st = self._fn(*self._args, _stream_handle(stream))
        if st != HIPDECODE_OK:
            raise HipDecodeError(st, "hipdecode_prefill_attn")


def prefill_attn(q, k_pool, v_pool, block_table, context_lens, new_start, scale, *, max_new_tokens=None,
                 out_dtype=None, out=None, lse=None):
    """Chunked-prefill attention: q bf16 [T,Hq,128] (row new_start[b] + j is
    chunk token j of request b); returns (out [T,Hq,128], lse [T,Hq]).  Rows
    no request names are left as allocated (uninitialised unless ``out`` and
    ``lse`` are given)."""
    import torch
    if q.dtype != torch.bfloat16 or k_pool.dtype != torch.bfloat16 or v_pool.dtype != torch.bfloat16:
        raise ValueError("q, k_pool and v_pool must be bfloat16")
    for name, t in (("block_table", block_table), ("context_lens", context_lens), ("new_start", new_start)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    T, Hq, D = q.shape
    P, page, Hkv, Dk = k_pool.shape
    B = context_lens.shape[0]
    if new_start.shape != (B + 1,):
        raise ValueError("new_start must have num_seqs + 1 entries")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    _check_call_tensors(q, k_pool, v_pool, block_table, context_lens, T, out, lse, out_dtype)
    params = make_prefill_params(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, num_pages=P,
                                 max_blocks_per_seq=block_table.shape[1], num_rows=T,
                                 max_new_tokens=T if max_new_tokens is None else max_new_tokens, scale=scale,
                                 head_dim=D, page_size=page,
                                 out_dtype=HIPDECODE_F32 if out_dtype == torch.float32 else HIPDECODE_BF16)
    st = hipdecode_check_prefill_params(params)
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_check_prefill_params")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    hipdecode_prefill_attn(params, q, k_pool, v_pool, new_start, block_table, context_lens, out, lse)
    return out, lse


def hipdecode_step_bucket(max_seqs: int, num_seqs: int) -> int:
    return int(library().hipdecode_step_bucket(int(max_seqs), int(num_seqs)))


class StepRunner:
    """A ``hipdecode_step_runner``: per-layer append + attention, replayed as
    one captured graph per batch bucket.

    ``layers`` is a list of dicts of device tensors with keys k_pool, v_pool,
    q, k_new, v_new, out and (optionally) lse, shaped for ``bucket(max_seqs)``
    rows; ``block_table`` and ``context_lens`` are device int32 tensors of
    that many rows.  The tensors must stay alive and in place while the runner
    exists.  ``step(context_lens)`` takes a host sequence of ints."""

    def __init__(self, layers, block_table, context_lens, *, max_seqs, num_pages, max_context_len, scale,
                 rope_theta=0.0, out_dtype=HIPDECODE_BF16):
        import numpy as np
        import torch
        first = layers[0]
        L = len(layers)
        self._keep = (layers, block_table, context_lens)
        # host checks of what the C ABI cannot see: every layer's tensors
        # shaped for the largest bucket, on one device
        rows = hipdecode_step_bucket(int(max_seqs), int(max_seqs))
        if rows <= 0:
            raise ValueError("max_seqs must be at least 1")
        dev = first["q"].device
        Hq, D = first["q"].shape[1], first["q"].shape[2]
        Hkv = first["k_pool"].shape[2]
        out_torch = torch.float32 if out_dtype == HIPDECODE_F32 else torch.bfloat16
        for i, layer in enumerate(layers):
            _check_tensor(f"layers[{i}].k_pool", layer["k_pool"], (int(num_pages), 16, Hkv, D), torch.bfloat16, dev)
            _check_tensor(f"layers[{i}].v_pool", layer["v_pool"], (int(num_pages), 16, Hkv, D), torch.bfloat16, dev)
            _check_tensor(f"layers[{i}].q", layer["q"], (rows, Hq, D), torch.bfloat16, dev)
            _check_tensor(f"layers[{i}].k_new", layer["k_new"], (rows, Hkv, D), torch.bfloat16, dev)
            _check_tensor(f"layers[{i}].v_new", layer["v_new"], (rows, Hkv, D), torch.bfloat16, dev)
            _check_tensor(f"layers[{i}].out", layer["out"], (rows, Hq, D), out_torch, dev)
            if layer.get("lse") is not None:
                _check_tensor(f"layers[{i}].lse", layer["lse"], (rows, Hq), torch.float32, dev)
        if block_table.dim() != 2 or block_table.shape[0] != rows:
            raise ValueError(f"block_table must be [{rows}, max_blocks]")
        _check_tensor("block_table", block_table, block_table.shape, torch.int32, dev)
        _check_tensor("context_lens", context_lens, (rows,), torch.int32, dev)

        def ptrs(key):
            if any(layer.get(key) is None for layer in layers):
                return None
            for layer in layers:
                if not layer[key].is_contiguous():
                    raise ValueError(f"{key} must be contiguous")
            arr = (ctypes.c_void_p * L)(*[layer[key].data_ptr() for layer in layers])
            return arr

        self._arrays = {k: ptrs(k) for k in ("k_pool", "v_pool", "q", "k_new", "v_new", "out", "lse")}
        cast = ctypes.cast
        P = ctypes.POINTER(ctypes.c_void_p)
        self.buffers = hipdecode_step_buffers(
            *[cast(self._arrays[k], P) if self._arrays[k] is not None else None
              for k in ("k_pool", "v_pool", "q", "k_new", "v_new", "out", "lse")],
            block_table.data_ptr(), context_lens.data_ptr())
        self.config = hipdecode_step_config(L, int(max_seqs), first["q"].shape[1], first["k_pool"].shape[2],
                                            first["q"].shape[2], first["k_pool"].shape[1], int(num_pages),
                                            block_table.shape[1], int(max_context_len), int(out_dtype),
                                            float(scale), float(rope_theta))
        handle = ctypes.c_void_p()
        st = library().hipdecode_step_runner_create(ctypes.byref(self.config), ctypes.byref(self.buffers),
                                                    ctypes.byref(handle))
        if st != HIPDECODE_OK:
            raise HipDecodeError(st, "hipdecode_step_runner_create")
        self._handle = handle
        self._np = np

    def bucket(self, num_seqs: int) -> int:
        return hipdecode_step_bucket(self.config.max_seqs, num_seqs)

    def step(self, context_lens, stream=None) -> None:
        ctx = self._np.ascontiguousarray(context_lens, dtype=self._np.int32)
        st = library().hipdecode_step_runner_step(self._handle, int(ctx.shape[0]), ctx.ctypes.data,
                                                  _stream_handle(stream))
        if st != HIPDECODE_OK:
            raise HipDecodeError(st, "hipdecode_step_runner_step")

    def close(self) -> None:
        if getattr(self, "_handle", None):
            st = library().hipdecode_step_runner_destroy(self._handle)
            self._handle = None
            if st != HIPDECODE_OK:
                raise HipDecodeError(st, "hipdecode_step_runner_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def hipdecode_paged_attn_append(params: hipdecode_params, rope_theta, q, k_new, v_new, k_pool, v_pool, block_table,
                                context_lens, out, lse, workspace, stream=None) -> None:
    """Enqueue one fused append + attention call (q is not modified)."""
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool), ("v_pool", v_pool),
                    ("block_table", block_table), ("context_lens", context_lens), ("out", out), ("lse", lse),
                    ("workspace", workspace)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().hipdecode_paged_attn_append(ctypes.byref(params), float(rope_theta), _ptr(q), _ptr(k_new),
                                               _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                               _ptr(context_lens), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                               _stream_handle(stream))
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_paged_attn_append")


def paged_attn_append(q, k_new, v_new, k_pool, v_pool, block_table, context_lens, scale, *, max_context_len,
                      rope_theta=0.0, out_dtype=None, partition_tokens=0, workgroup_waves=0, out=None, lse=None,
                      workspace=None):
    """Append each request's new token (k_new/v_new [B,Hkv,128], RoPE when
    rope_theta > 0) and attend, in one launch; returns (out, lse)."""
    import torch
    B, Hq, D = q.shape
    P, page, Hkv, _ = k_pool.shape
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16")
    _check_call_tensors(q, k_pool, v_pool, block_table, context_lens, B, out, lse, out_dtype)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _check_tensor(name, t, (B, Hkv, D), torch.bfloat16, q.device)
    params = make_params(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, num_pages=P,
                         max_blocks_per_seq=block_table.shape[1], max_context_len=max_context_len, scale=scale,
                         head_dim=D, page_size=page, partition_tokens=partition_tokens,
                         workgroup_waves=workgroup_waves, schedule=HIPDECODE_SCHEDULE_SPLIT,
                         out_dtype=HIPDECODE_F32 if out_dtype == torch.float32 else HIPDECODE_BF16)
    st = hipdecode_check_params(params)
    if st != HIPDECODE_OK:
        raise HipDecodeError(st, "hipdecode_check_params")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = hipdecode_workspace_bytes(params)
        workspace = torch.zeros(max(nbytes, 16) // 4 + 4, dtype=torch.int32, device=q.device)
    hipdecode_paged_attn_append(params, rope_theta, q, k_new, v_new, k_pool, v_pool, block_table, context_lens, out,
                                lse, workspace)
    return out, lse
