"""Helpers for GPU parity tests: move a case to the device, run the HIP path,
compare with the oracle at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_decode_gqa_amd as hd

OUT_ATOL = 1e-2      # max |out - oracle| on bf16 (and fp32) outputs
BF16_REACH = 4.0     # below this magnitude the nearest bf16 is within 2^-7 of any value; from 4 to 8, 2^-6
LSE_RTOL = 1e-4      # |lse - oracle| <= 1e-4 * max(1, |oracle|)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


class DeviceCase:
    def __init__(self, case, device="cuda"):
        self.case = case
        self.q = bits_to_bf16(case.q, device)
        self.k = bits_to_bf16(case.k_pool, device)
        self.v = bits_to_bf16(case.v_pool, device)
        self.table = torch.from_numpy(case.block_table).to(device)
        self.ctx = torch.from_numpy(case.context_lens).to(device)
        self.out_dtype = torch.float32 if case.out_dtype == "f32" else torch.bfloat16


def run_hip(dc: DeviceCase, *, partition_tokens=0, workgroup_waves=0, schedule=0, max_context_len=None,
            workspace=None, out_dtype=None):
    c = dc.case
    mcl = c.max_context_len if max_context_len is None else max_context_len
    out, lse = hd.paged_attn(dc.q, dc.k, dc.v, dc.table, dc.ctx, c.scale, max_context_len=mcl,
                             out_dtype=out_dtype or dc.out_dtype, partition_tokens=partition_tokens,
                             workgroup_waves=workgroup_waves, schedule=schedule, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def compare(out, lse, ref_out, ref_lse, ctx=None, *, what=""):
    """Assert the stated tolerances and a rounding-level bound; return max errors."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert o.shape == ref_out.shape and l.shape == ref_lse.shape, what
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - ref_out)
    max_err = float(err.max()) if err.size else 0.0
    # 1e-2 binds where a bf16 result can meet it (|oracle| < 4); fp32 outputs everywhere
    bar = np.abs(ref_out) < BF16_REACH if out.dtype == torch.bfloat16 else np.ones(err.shape, dtype=bool)
    max_bar = float(err[bar].max()) if bar.any() else 0.0
    assert max_bar <= OUT_ATOL, f"{what}: max |out err| {max_bar} > {OUT_ATOL}"
    # rounding level: within one bf16 half-ulp of the exact value plus fp32 noise
    if out.dtype == torch.bfloat16:
        bound = np.abs(ref_out) * 2.0 ** -8 + 2e-5
    else:
        bound = np.abs(ref_out) * 1e-5 + 2e-5
    worst = float((err - bound).max()) if err.size else -1.0
    assert worst <= 0, f"{what}: error above rounding level by {worst}"
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), empty), f"{what}: -inf LSE rows differ"
    if empty.any():
        assert np.all(o[empty] == 0), f"{what}: empty context must give zeros"
    fin = ~empty
    lerr = np.abs(l[fin] - ref_lse[fin])
    lim = LSE_RTOL * np.maximum(1.0, np.abs(ref_lse[fin]))
    assert np.all(lerr <= lim), f"{what}: LSE err {float((lerr / lim).max())} x tolerance"
    return max_err, float((lerr / np.maximum(1.0, np.abs(ref_lse[fin]))).max()) if fin.any() else 0.0
