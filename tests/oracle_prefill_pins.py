"""Pins for the chunked-prefill oracle: checks against things other than the oracle.

Each ``pin_*`` function raises ``AssertionError`` when the oracle library it is
given disagrees with an independent fact:

* library routine: ``torch.nn.functional.scaled_dot_product_attention`` in
  float64 with an explicit mask, query row j of a chunk of n seeing the keys
  t <= c - n + j of its request's c cached tokens (MOSS-TD article, "Chunked
  prefill for long audio": the prompt is processed in query blocks over the
  cache), and ``torch.logsumexp`` over the same masked scores;
* the last row of every chunk sees the whole context, so it equals the
  decode-step oracle for that query;
* a chunk that is the whole context starts with a row that sees one token:
  out = v_0 exactly and lse = z_0;
* splitting a chunk into two smaller chunks, the second after the first has
  been cached, gives the same rows;
* closed form: when every key of a request is the same, the softmax is
  uniform over the visible keys, so chunk row j returns the mean of V over
  positions 0 .. p_j and its LSE is z + ln(p_j + 1), z being the one score;
* argument validation.

Dense keys and values are scattered into a shuffled pool by this file's own
code (``tests.oracle_pins.Dense``).  Run as a script (``python -m
tests.oracle_prefill_pins --lib PATH``) it executes every pin against the
library at PATH and exits non-zero on the first failure.
"""
from __future__ import annotations

import argparse
import math
import sys

import numpy as np

import oracle
from tests.oracle_pins import Dense, _bits, _close, _f64  # noqa: F401

SHAPES = [  # (Hq, Hkv, D, page, [(context, chunk) per request])
    (2, 1, 4, 4, [(9, 9)]),
    (4, 2, 16, 4, [(13, 5), (6, 2)]),
    (16, 8, 128, 16, [(48, 20), (1, 1), (33, 33)]),
    (6, 2, 8, 3, [(10, 4), (17, 17)]),
    (8, 8, 32, 16, [(40, 0), (16, 7)]),
]


def _case(rng, Hq, Hkv, D, page, reqs, extra_rows=0):
    ks = [_bits(rng, (c, Hkv, D)) for c, _ in reqs]
    vs = [_bits(rng, (c, Hkv, D)) for c, _ in reqs]
    n = [k for _, k in reqs]
    new_start = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    T = int(new_start[-1]) + extra_rows
    q_rows = _bits(rng, (T, Hq, D))
    dn = Dense(_bits(rng, (len(reqs), Hq, D)), ks, vs, page, rng)   # Dense's own q is not used here
    return dn, q_rows, new_start


def pin_sdpa_causal_library(lib):
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(301)
    for Hq, Hkv, D, page, reqs in SHAPES:
        dn, q, ns = _case(rng, Hq, Hkv, D, page, reqs, extra_rows=1)
        scale = 1.0 / math.sqrt(D) * 0.9
        out, lse = oracle.prefill_attn(q, dn.k_pool, dn.v_pool, dn.table, dn.ctx, ns, scale, lib=lib)
        G = Hq // Hkv
        for b, (c, n) in enumerate(reqs):
            if n == 0:
                continue
            rows = slice(int(ns[b]), int(ns[b + 1]))
            qb = torch.from_numpy(_f64(q[rows])).permute(1, 0, 2).unsqueeze(0)              # [1,Hq,n,D]
            kb = torch.from_numpy(_f64(dn.ks[b])).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
            vb = torch.from_numpy(_f64(dn.vs[b])).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
            pos = c - n + np.arange(n)
            mask = torch.from_numpy(np.arange(c)[None, :] <= pos[:, None])                  # [n, c]
            ref = F.scaled_dot_product_attention(qb, kb.contiguous(), vb.contiguous(), attn_mask=mask, scale=scale)
            _close(out[rows], ref[0].permute(1, 0, 2).numpy(), what=f"sdpa out {Hq, Hkv, D, page} b={b}")
            scores = torch.matmul(qb, kb.transpose(-1, -2).contiguous()) * scale
            scores = scores.masked_fill(~mask, -math.inf)
            ref_lse = torch.logsumexp(scores, dim=-1)[0].permute(1, 0)                      # [n, Hq]
            _close(lse[rows], ref_lse.numpy(), what=f"sdpa lse b={b}")
        extra = out[-1]
        assert np.isnan(extra).all(), "a row no request names must be left untouched"


def pin_last_row_is_decode(lib):
    rng = np.random.default_rng(302)
    dn, q, ns = _case(rng, 16, 8, 128, 16, [(70, 12), (33, 1), (16, 16)])
    out, lse = oracle.prefill_attn(q, dn.k_pool, dn.v_pool, dn.table, dn.ctx, ns, 0.1, lib=lib)
    last = ns[1:] - 1
    d_out, d_lse = oracle.paged_attn(q[last], dn.k_pool, dn.v_pool, dn.table, dn.ctx, 0.1, lib=lib)
    assert np.array_equal(out[last], d_out) and np.array_equal(lse[last], d_lse), \
        "the last row of a chunk must equal the decode step"


def pin_first_row_sees_one_token(lib):
    rng = np.random.default_rng(303)
    dn, q, ns = _case(rng, 4, 2, 16, 4, [(11, 11), (5, 5)])
    scale = 0.3
    out, lse = oracle.prefill_attn(q, dn.k_pool, dn.v_pool, dn.table, dn.ctx, ns, scale, lib=lib)
    for b in range(2):
        r = int(ns[b])
        for h in range(4):
            g = h // 2
            assert np.array_equal(out[r, h], _f64(dn.vs[b][0, g])), "first row must return v_0"
            z0 = scale * float(_f64(q[r, h]) @ _f64(dn.ks[b][0, g]))
            assert abs(lse[r, h] - z0) <= 1e-12 * max(1.0, abs(z0)), "first row LSE must be z_0"


def pin_rechunking(lib):
    rng = np.random.default_rng(304)
    Hq, Hkv, D, page = 8, 2, 32, 4
    c, n = 37, 19
    dn, q, ns = _case(rng, Hq, Hkv, D, page, [(c, n)])
    whole, whole_lse = oracle.prefill_attn(q, dn.k_pool, dn.v_pool, dn.table, dn.ctx, ns, 0.2, lib=lib)
    n1 = 8                         # first sub-chunk, with the context as it was then
    ctx1 = np.array([c - (n - n1)], dtype=np.int32)
    a, a_lse = oracle.prefill_attn(q[:n1], dn.k_pool, dn.v_pool, dn.table, ctx1, np.array([0, n1], np.int32),
                                   0.2, lib=lib)
    b, b_lse = oracle.prefill_attn(q[n1:n], dn.k_pool, dn.v_pool, dn.table, dn.ctx,
                                   np.array([0, n - n1], np.int32), 0.2, lib=lib)
    assert np.array_equal(np.concatenate([a, b]), whole[:n]) and \
        np.array_equal(np.concatenate([a_lse, b_lse]), whole_lse[:n]), "re-chunking changed the rows"


def pin_equal_keys_prefix_mean(lib):
    rng = np.random.default_rng(307)
    Hq, Hkv, D, page = 4, 2, 16, 4
    reqs = [(13, 13), (9, 4)]
    G = Hq // Hkv
    ks = [np.repeat(_bits(rng, (1, Hkv, D)), c, axis=0) for c, _ in reqs]   # one key row per request
    vs = [_bits(rng, (c, Hkv, D)) for c, _ in reqs]
    dn = Dense(_bits(rng, (len(reqs), Hq, D)), ks, vs, page, rng)
    ns = np.concatenate([[0], np.cumsum([n for _, n in reqs])]).astype(np.int32)
    q = _bits(rng, (int(ns[-1]), Hq, D))
    scale = 0.25
    out, lse = oracle.prefill_attn(q, dn.k_pool, dn.v_pool, dn.table, dn.ctx, ns, scale, lib=lib)
    for b, (c, n) in enumerate(reqs):
        for j in range(n):
            r, p = int(ns[b]) + j, c - n + j
            for h in range(Hq):
                g = h // G
                mean = _f64(vs[b][: p + 1, g]).mean(axis=0)
                assert np.allclose(out[r, h], mean, rtol=0.0, atol=1e-12), \
                    f"equal keys: row {r} head {h} must be the mean of V over positions 0..{p}"
                z = scale * float(_f64(q[r, h]) @ _f64(ks[b][0, g]))
                want = z + math.log(p + 1)
                assert abs(lse[r, h] - want) <= 1e-12 * max(1.0, abs(want)), f"equal keys: LSE of row {r} head {h}"


def pin_pairs_match_full(lib):
    rng = np.random.default_rng(305)
    dn, q, ns = _case(rng, 16, 8, 128, 16, [(50, 30), (20, 3)])
    out, lse = oracle.prefill_attn(q, dn.k_pool, dn.v_pool, dn.table, dn.ctx, ns, 0.1, lib=lib)
    pairs = [(0, 0), (29, 15), (31, 7), (32, 1), (10, 3)]
    po, pl = oracle.prefill_attn_pairs(q, dn.k_pool, dn.v_pool, dn.table, dn.ctx, ns, 0.1, pairs, lib=lib)
    for i, (r, h) in enumerate(pairs):
        assert np.array_equal(po[i], out[r, h]) and pl[i] == lse[r, h]


def pin_validation(lib):
    rng = np.random.default_rng(306)
    dn, q, ns = _case(rng, 4, 2, 16, 4, [(13, 5), (6, 2)])
    ok = oracle.prefill_validate(q, dn.k_pool, dn.table, dn.ctx, ns, lib=lib)
    assert ok == 0
    assert oracle.prefill_validate(q, dn.k_pool, dn.table, dn.ctx, np.array([0, 5, 9], np.int32), lib=lib) == 1
    assert oracle.prefill_validate(q, dn.k_pool, dn.table, dn.ctx, np.array([0, 14, 16], np.int32), lib=lib) == 1
    assert oracle.prefill_validate(q, dn.k_pool, dn.table, dn.ctx, np.array([3, 2, 4], np.int32), lib=lib) == 1
    bad = dn.table.copy()
    bad[0, 0] = dn.k_pool.shape[0]
    assert oracle.prefill_validate(q, dn.k_pool, bad, dn.ctx, ns, lib=lib) == 1
    try:
        oracle.prefill_attn_pairs(q, dn.k_pool, dn.v_pool, dn.table, dn.ctx, ns, 0.1, [(q.shape[0], 0)], lib=lib)
    except oracle.OracleError:
        pass
    else:
        raise AssertionError("a row outside the inputs must be refused")


PINS = [
    pin_sdpa_causal_library,
    pin_last_row_is_decode,
    pin_first_row_sees_one_token,
    pin_rechunking,
    pin_equal_keys_prefix_mean,
    pin_pairs_match_full,
    pin_validation,
]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--lib", default=None)
    args = ap.parse_args(argv)
    lib = oracle.load(args.lib)
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError as e:
            print(f"FAIL {pin.__name__}: {e}")
            return 1
        except oracle.OracleError as e:
            print(f"FAIL {pin.__name__}: oracle error {e}")
            return 1
        print(f"ok   {pin.__name__}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
