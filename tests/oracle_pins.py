"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle library it is
given disagrees with an independent fact:

* library routines: ``torch.nn.functional.scaled_dot_product_attention`` and
  ``torch.logsumexp`` in float64 on the CPU, with each KV head repeated for the
  query heads of its group (the grouping of the audio.cpp "Decoder And Prompt"
  section: 16 query heads over 8 KV heads);
* brute force with exact ``math.fsum`` sums on tiny inputs;
* closed forms: one cached token, all keys equal, a zero query, one dominant key;
* invariants: page relabelling, token order, affine maps of V, (c*q, scale/c),
  request independence, and the merge of two halves of a context by their LSEs;
* argument validation.

Tiny cases are built dense first, in logical token order, and then scattered
into a shuffled pool by code in this file, so no check reuses the oracle's own
block-table walk.

Run as a script (``python -m tests.oracle_pins --lib PATH``) it executes every
pin against the library at PATH and exits non-zero on the first failure; the
mutation test uses that to show planted mistakes are caught.
"""
from __future__ import annotations

import argparse
import math
import sys

import numpy as np

import oracle
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

TOL = 1e-12


# --------------------------------------------------------------------------
# dense -> paged construction (independent of the oracle's table walk)
# --------------------------------------------------------------------------
class Dense:
    """Per-request dense q/K/V in logical order, plus a paged layout of them."""

    def __init__(self, q, ks, vs, page, rng, extra_pages=3, table_width=None):
        # q: [B,Hq,D] bits; ks[b], vs[b]: [n_b, Hkv, D] bits
        self.q = q
        self.ks = ks
        self.vs = vs
        self.page = page
        B = q.shape[0]
        Hkv, D = (ks[0].shape[1], ks[0].shape[2]) if ks else (1, q.shape[2])
        need = [(k.shape[0] + page - 1) // page for k in ks]
        P = sum(need) + extra_pages
        width = table_width or max(1, max(need, default=1))
        perm = rng.permutation(P)
        # fill the pool with junk first; every used slot is overwritten below
        junk = f32_to_bf16_bits(rng.standard_normal((P, page, Hkv, D)).astype(np.float32) * 7)
        self.k_pool = junk.copy()
        self.v_pool = f32_to_bf16_bits(rng.standard_normal((P, page, Hkv, D)).astype(np.float32) * 7)
        self.table = np.full((B, width), -1, dtype=np.int32)
        nxt = 0
        for b in range(B):
            n = ks[b].shape[0]
            for j in range(need[b]):
                p = int(perm[nxt])
                nxt += 1
                self.table[b, j] = p
                lo, hi = j * page, min(n, (j + 1) * page)
                self.k_pool[p, : hi - lo] = ks[b][lo:hi]
                self.v_pool[p, : hi - lo] = vs[b][lo:hi]
        self.ctx = np.array([k.shape[0] for k in ks], dtype=np.int32)

    def run(self, lib, scale):
        return oracle.paged_attn(self.q, self.k_pool, self.v_pool, self.table, self.ctx, scale, lib=lib)


def _bits(rng, shape, mult=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * mult).astype(np.float32))


def _rand_dense(rng, B, Hq, Hkv, D, page, ctxs, mult=1.0, **kw):
    q = _bits(rng, (B, Hq, D), mult)
    ks = [_bits(rng, (n, Hkv, D), mult) for n in ctxs]
    vs = [_bits(rng, (n, Hkv, D)) for n in ctxs]
    return Dense(q, ks, vs, page, rng, **kw)


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(a - b))
    lim = tol * np.maximum(1.0, np.abs(b))
    bad = ~(err <= lim)
    assert not bad.any(), f"{what}: max err {np.nanmax(np.where(both_inf, 0, err))} (n_bad={int(bad.sum())})"


# --------------------------------------------------------------------------
# library-routine pins
# --------------------------------------------------------------------------
SHAPES = [  # (B, Hq, Hkv, D, page, ctxs)
    (1, 2, 1, 4, 4, [7]),
    (2, 4, 2, 16, 4, [13, 5]),
    (3, 16, 8, 128, 16, [48, 1, 33]),
    (2, 6, 2, 8, 3, [10, 17]),
    (2, 8, 8, 32, 16, [16, 40]),
    (1, 16, 4, 64, 8, [29]),
]


def pin_sdpa_library(lib):
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(101)
    for (B, Hq, Hkv, D, page, ctxs) in SHAPES:
        dn = _rand_dense(rng, B, Hq, Hkv, D, page, ctxs)
        scale = 1.0 / math.sqrt(D) * 1.25
        out, lse = dn.run(lib, scale)
        G = Hq // Hkv
        for b in range(B):
            qb = torch.from_numpy(_f64(dn.q[b])).reshape(1, Hq, 1, D)
            kb = torch.from_numpy(_f64(dn.ks[b])).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
            vb = torch.from_numpy(_f64(dn.vs[b])).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
            ref = F.scaled_dot_product_attention(qb, kb.contiguous(), vb.contiguous(), scale=scale)
            _close(out[b], ref.reshape(Hq, D).numpy(), what=f"sdpa out {B,Hq,Hkv,D,page} b={b}")
            scores = torch.matmul(qb, kb.transpose(-1, -2).contiguous()) * scale  # [1,Hq,1,n]
            ref_lse = torch.logsumexp(scores, dim=-1).reshape(Hq)
            _close(lse[b], ref_lse.numpy(), what=f"sdpa lse b={b}")


def pin_fsum_bruteforce(lib):
    """Exact-sum brute force on tiny inputs, in plain Python."""
    rng = np.random.default_rng(202)
    B, Hq, Hkv, D, page = 2, 4, 2, 4, 2
    dn = _rand_dense(rng, B, Hq, Hkv, D, page, [5, 9])
    scale = 0.37
    out, lse = dn.run(lib, scale)
    for b in range(B):
        n = int(dn.ctx[b])
        kf = _f64(dn.ks[b]).tolist()
        vf = _f64(dn.vs[b]).tolist()
        for h in range(Hq):
            g = h // (Hq // Hkv)
            qv = _f64(dn.q[b, h]).tolist()
            z = [scale * math.fsum(qv[d] * kf[t][g][d] for d in range(D)) for t in range(n)]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            l_ = math.fsum(w)
            for d in range(D):
                ref = math.fsum(w[t] * vf[t][g][d] for t in range(n)) / l_
                _close(out[b, h, d], ref, what="fsum out")
            _close(lse[b, h], m + math.log(l_), what="fsum lse")


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def pin_single_token(lib):
    rng = np.random.default_rng(303)
    dn = _rand_dense(rng, 3, 16, 8, 128, 16, [1, 1, 1])
    scale = 1 / math.sqrt(128)
    out, lse = dn.run(lib, scale)
    for b in range(3):
        for h in range(16):
            g = h // 2
            v0 = _f64(dn.vs[b][0, g])
            assert np.array_equal(out[b, h], v0), "ctx=1 must return v_0 exactly"
            z0 = scale * math.fsum(_f64(dn.q[b, h]) * _f64(dn.ks[b][0, g]))
            _close(lse[b, h], z0, tol=1e-14, what="ctx=1 lse = z_0")


def pin_equal_keys(lib):
    rng = np.random.default_rng(404)
    n, Hq, Hkv, D = 37, 4, 2, 16
    q = _bits(rng, (1, Hq, D))
    k1 = _bits(rng, (1, Hkv, D))
    ks = [np.repeat(k1, n, axis=0)]
    vs = [_bits(rng, (n, Hkv, D))]
    dn = Dense(q, ks, vs, 8, rng)
    scale = 0.2
    out, lse = dn.run(lib, scale)
    for h in range(Hq):
        g = h // 2
        _close(out[0, h], np.mean(_f64(vs[0][:, g]), axis=0), what="equal keys -> mean of V")
        z = scale * math.fsum(_f64(q[0, h]) * _f64(k1[0, g]))
        _close(lse[0, h], z + math.log(n), what="equal keys lse = z + ln n")


def pin_zero_query(lib):
    rng = np.random.default_rng(505)
    n, Hq, Hkv, D = 23, 4, 4, 8
    q = np.zeros((1, Hq, D), dtype=np.uint16)
    ks = [_bits(rng, (n, Hkv, D))]
    vs = [_bits(rng, (n, Hkv, D))]
    dn = Dense(q, ks, vs, 4, rng)
    out, lse = dn.run(lib, 0.5)
    for h in range(Hq):
        _close(out[0, h], np.mean(_f64(vs[0][:, h]), axis=0), what="q=0 -> mean of V")
        _close(lse[0, h], math.log(n), what="q=0 lse = ln n")


def pin_dominant_key(lib):
    """One key far ahead of the rest: out is that token's value row.

    The winning score is ~1000, so exp of an unshifted score would overflow."""
    rng = np.random.default_rng(606)
    n, Hq, Hkv, D = 19, 2, 1, 4
    q = f32_to_bf16_bits(np.full((1, Hq, D), 16.0, dtype=np.float32))
    kf = np.ones((n, Hkv, D), dtype=np.float32) * rng.choice([-1.0, 1.0], size=(n, Hkv, D)).astype(np.float32)
    j = 11
    kf[j] = 16.0
    ks = [f32_to_bf16_bits(kf)]
    vs = [_bits(rng, (n, Hkv, D))]
    dn = Dense(q, ks, vs, 4, rng)
    out, lse = dn.run(lib, 1.0)
    for h in range(Hq):
        assert np.all(np.isfinite(out[0, h])), "dominant key: non-finite output"
        _close(out[0, h], _f64(vs[0][j, 0]), tol=1e-13, what="dominant key -> v_j")
        _close(lse[0, h], 4 * 16.0 * 16.0, tol=1e-13, what="dominant key lse = z_j")


def pin_empty_context(lib):
    rng = np.random.default_rng(707)
    dn = _rand_dense(rng, 3, 4, 2, 8, 4, [0, 5, 0])
    out, lse = dn.run(lib, 0.3)
    assert np.all(out[0] == 0) and np.all(out[2] == 0), "ctx=0 must give a zero output"
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2])), "ctx=0 must give lse=-inf"
    assert np.all(np.isfinite(lse[1]))


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def pin_page_relabel(lib):
    """Moving pages to other pool rows (and fixing the table) changes nothing, bit for bit."""
    rng = np.random.default_rng(808)
    dn = _rand_dense(rng, 3, 16, 8, 128, 16, [40, 16, 77], extra_pages=5)
    out, lse = dn.run(lib, 0.088)
    P = dn.k_pool.shape[0]
    perm = rng.permutation(P)           # new row of old page p is perm[p]
    k2 = np.empty_like(dn.k_pool)
    v2 = np.empty_like(dn.v_pool)
    k2[perm] = dn.k_pool
    v2[perm] = dn.v_pool
    t2 = np.where(dn.table >= 0, perm[np.maximum(dn.table, 0)], -1).astype(np.int32)
    out2, lse2 = oracle.paged_attn(dn.q, k2, v2, t2, dn.ctx, 0.088, lib=lib)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2), "page relabelling changed the result"


def pin_token_order(lib):
    rng = np.random.default_rng(909)
    dn = _rand_dense(rng, 2, 4, 2, 16, 4, [21, 30])
    out, lse = dn.run(lib, 0.25)
    ks2, vs2 = [], []
    for b in range(2):
        p = rng.permutation(dn.ks[b].shape[0])
        ks2.append(dn.ks[b][p])
        vs2.append(dn.vs[b][p])
    dn2 = Dense(dn.q, ks2, vs2, 4, rng)
    out2, lse2 = dn2.run(lib, 0.25)
    _close(out2, out, what="token order: out")
    _close(lse2, lse, what="token order: lse")


def pin_affine_values(lib):
    """V -> 2V + 1 maps out -> 2 out + 1 (integer V keeps 2V+1 exact in bf16)."""
    rng = np.random.default_rng(1010)
    n, Hq, Hkv, D = 26, 4, 2, 8
    q = _bits(rng, (1, Hq, D))
    ks = [_bits(rng, (n, Hkv, D))]
    vi = rng.integers(-8, 9, size=(n, Hkv, D)).astype(np.float32)
    dn1 = Dense(q, ks, [f32_to_bf16_bits(vi)], 4, np.random.default_rng(1))
    dn2 = Dense(q, ks, [f32_to_bf16_bits(2 * vi + 1)], 4, np.random.default_rng(2))
    o1, l1 = dn1.run(lib, 0.3)
    o2, l2 = dn2.run(lib, 0.3)
    _close(o2, 2 * o1 + 1, what="affine V")
    _close(l2, l1, what="affine V leaves lse")


def pin_scale_query_tradeoff(lib):
    """(2q, scale/2) scores equal (q, scale)."""
    rng = np.random.default_rng(1111)
    dn = _rand_dense(rng, 2, 8, 4, 32, 8, [19, 44])
    o1, l1 = dn.run(lib, 0.2)
    q2 = f32_to_bf16_bits(_f64(dn.q).astype(np.float32) * 2)
    o2, l2 = oracle.paged_attn(q2, dn.k_pool, dn.v_pool, dn.table, dn.ctx, 0.1, lib=lib)
    _close(o2, o1, tol=1e-13, what="(2q, s/2) out")
    _close(l2, l1, tol=1e-13, what="(2q, s/2) lse")


def pin_split_merge(lib):
    """Attention over a context equals the LSE-weighted merge of its two halves.

    With (o1, L1) and (o2, L2) from disjoint halves, the whole gives
    L = logaddexp(L1, L2) and o = exp(L1 - L) o1 + exp(L2 - L) o2."""
    rng = np.random.default_rng(1212)
    page = 16
    n1_pages, n = 2, 45
    dn = _rand_dense(rng, 1, 16, 8, 128, page, [n])
    o, L = dn.run(lib, 0.09)
    o1, L1 = oracle.paged_attn(dn.q, dn.k_pool, dn.v_pool, dn.table,
                               np.array([n1_pages * page], np.int32), 0.09, lib=lib)
    t2 = np.full_like(dn.table, -1)
    rest = dn.table[0, n1_pages:]
    t2[0, : rest.shape[0]] = rest
    o2, L2 = oracle.paged_attn(dn.q, dn.k_pool, dn.v_pool, t2,
                               np.array([n - n1_pages * page], np.int32), 0.09, lib=lib)
    Lm = np.logaddexp(L1, L2)
    om = np.exp(L1 - Lm)[..., None] * o1 + np.exp(L2 - Lm)[..., None] * o2
    _close(Lm, L, what="merged lse")
    _close(om, o, what="merged out")


def pin_request_independence(lib):
    """A batch gives, bit for bit, what each request gives alone; a duplicated
    request gives identical rows; a CFG pair (same q, its own KV) does not."""
    rng = np.random.default_rng(1313)
    q = _bits(rng, (4, 16, 128))
    q[1] = q[0]              # CFG pair: shared query
    q[3] = q[2]              # exact duplicate below
    ks = [_bits(rng, (n, 8, 128)) for n in (33, 50, 18)]
    vs = [_bits(rng, (n, 8, 128)) for n in (33, 50, 18)]
    ks.append(ks[2].copy())
    vs.append(vs[2].copy())
    dn = Dense(q, ks, vs, 16, rng)
    out, lse = dn.run(lib, 0.088)
    for b in range(4):
        t = np.full((1, dn.table.shape[1]), -1, np.int32)
        t[0] = dn.table[b]
        ob, lb = oracle.paged_attn(dn.q[b:b + 1], dn.k_pool, dn.v_pool, t, dn.ctx[b:b + 1], 0.088, lib=lib)
        assert np.array_equal(ob[0], out[b]) and np.array_equal(lb[0], lse[b]), f"request {b} not independent"
    assert np.array_equal(out[2], out[3]) and np.array_equal(lse[2], lse[3]), "duplicate request differs"
    assert not np.allclose(out[0], out[1]), "CFG pair with distinct KV must differ"


def pin_validation(lib):
    rng = np.random.default_rng(1414)
    dn = _rand_dense(rng, 2, 4, 2, 8, 4, [9, 6])
    ok = oracle.validate(dn.q, dn.k_pool, dn.v_pool, dn.table, dn.ctx, lib=lib)
    assert ok == 0
    bad = dn.table.copy()
    bad[1, 0] = dn.k_pool.shape[0]
    assert oracle.validate(dn.q, dn.k_pool, dn.v_pool, bad, dn.ctx, lib=lib) != 0, "page index past pool"
    bad[1, 0] = -1
    assert oracle.validate(dn.q, dn.k_pool, dn.v_pool, bad, dn.ctx, lib=lib) != 0, "negative page index"
    long_ctx = np.array([9, dn.table.shape[1] * 4 + 1], np.int32)
    assert oracle.validate(dn.q, dn.k_pool, dn.v_pool, dn.table, long_ctx, lib=lib) != 0, "ctx past table"
    # entries past the used blocks are never looked at
    stale = dn.table.copy()
    stale[1, 2:] = 10 ** 6
    assert oracle.validate(dn.q, dn.k_pool, dn.v_pool, stale, dn.ctx, lib=lib) == 0


PINS = [
    pin_sdpa_library,
    pin_fsum_bruteforce,
    pin_single_token,
    pin_equal_keys,
    pin_zero_query,
    pin_dominant_key,
    pin_empty_context,
    pin_page_relabel,
    pin_token_order,
    pin_affine_values,
    pin_scale_query_tradeoff,
    pin_split_merge,
    pin_request_independence,
    pin_validation,
]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--lib", required=True)
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
