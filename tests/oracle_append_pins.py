"""Pins for the KV-append oracle: checks against things other than the oracle.

Each ``pin_*`` function raises ``AssertionError`` when the oracle library it is
given disagrees with an independent fact:

* rounding to bf16: the result is the nearest bf16 value (brute force over its
  neighbours, ties to even), agrees with the generators' float32 rounding on
  float32 inputs, and matches hand-worked values (ties, subnormals, overflow);
* RoPE (audio.cpp "Fun-ASR-Nano Native Runtime Design", "Decoder And Prompt":
  Qwen3 decoder, RoPE theta 1e6): the rotate-half rotation equals multiplying
  the complex numbers x[i] + i x[i + d/2] by exp(i p theta^(-2i/d)), closed
  forms at frequencies 1 and theta^(-1/2), norm preservation, the
  relative-position identity <R_m q, R_n k> = <R_(m-n) q, k>, and R_-p R_p = I;
* the append itself: every new token lands in the slot the test computes from
  the block table on its own, with V copied bit for bit, K and q rotated to the
  nearest bf16 of the exact rotation, and every other slot of the pools
  untouched; padding rows and empty chunks write nothing;
* argument validation.

Run as a script (``python -m tests.oracle_append_pins --lib PATH``) it executes
every pin against the library at PATH and exits non-zero on the first failure;
the mutation test uses that.
"""
from __future__ import annotations

import argparse
import math
import sys

import numpy as np

import oracle
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

THETA = 1e6


def _val(bits) -> np.ndarray:
    return bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def _round(lib, x):
    return oracle.round_bf16(x, lib=lib)


def _neighbours(bits: int) -> tuple[float, float]:
    """The bf16 values just below and just above the finite bf16 ``bits``."""
    v = float(_val([bits])[0])
    if bits & 0x7FFF == 0:                        # +-0: neighbours are +-min subnormal
        tiny = float(_val([0x0001])[0])
        return -tiny, tiny
    mag_up = (bits & 0x7FFF) + 1
    mag_dn = (bits & 0x7FFF) - 1
    up_mag = float(_val([mag_up])[0])             # 0x7F80 is infinity
    dn_mag = float(_val([mag_dn])[0])
    if v < 0:
        return -up_mag, -dn_mag
    return dn_mag, up_mag


def nearest_ok(bits: np.ndarray, exact: np.ndarray, slack: float = 0.0) -> np.ndarray:
    """True where ``bits`` is a nearest bf16 of ``exact`` (within ``slack``
    relative, for exact values only known to about that precision)."""
    vals = _val(bits)
    ok = np.empty(vals.shape, dtype=bool)
    for i, (b, v, x) in enumerate(zip(bits.ravel(), vals.ravel(), np.asarray(exact, np.float64).ravel())):
        lo, hi = _neighbours(int(b))
        d = abs(x - v)
        tol = slack * abs(x)
        ok.ravel()[i] = d <= abs(x - lo) + tol and d <= abs(x - hi) + tol
    return ok


# --------------------------------------------------------------------------
# rounding
# --------------------------------------------------------------------------
def pin_round_nearest_bruteforce(lib):
    rng = np.random.default_rng(101)
    xs = np.concatenate([
        rng.standard_normal(3000),
        rng.standard_normal(500) * 1e-39,              # binary32 subnormal range
        rng.standard_normal(500) * 1e-42,
        rng.standard_normal(300) * 3e38,               # near the top of the range
        np.ldexp(rng.uniform(1, 2, 500), rng.integers(-140, 128, 500)),
    ])
    got = _round(lib, xs)
    fin = np.abs(_val(got)) < math.inf
    ok = nearest_ok(got[fin], xs[fin])
    assert ok.all(), f"not nearest at {xs[fin][~ok][:5]}"
    # ties: exact midpoints between neighbours go to the even pattern
    base = f32_to_bf16_bits(rng.standard_normal(2000).astype(np.float32))
    base = base[(base & 0x7FFF) < 0x7F7F]
    lo = _val(base)
    up = _val((base + 1).astype(np.uint16))            # next magnitude, same sign
    mid = (lo + up) / 2                                  # exact in fp64
    got = _round(lib, mid)
    even = np.where(base % 2 == 0, base, (base + 1).astype(np.uint16))
    assert np.array_equal(got, even), "ties are not broken to even"


def pin_round_matches_float32_rounding(lib):
    rng = np.random.default_rng(102)
    f = np.concatenate([rng.standard_normal(5000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-39).astype(np.float32),
                        rng.uniform(-3e38, 3e38, 1000).astype(np.float32)])
    assert np.array_equal(_round(lib, f.astype(np.float64)), f32_to_bf16_bits(f))


def pin_round_worked_values(lib):
    cases = [
        (1.0, 0x3F80), (-1.0, 0xBF80), (0.0, 0x0000), (-0.0, 0x8000),
        (1.0 + 2.0 ** -8, 0x3F80),            # tie between 1 and 1 + 2^-7: even
        (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie between 1 + 2^-7 and 1 + 2^-6: even
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),
        (2.0 ** -133, 0x0001),                # smallest subnormal
        (2.0 ** -134, 0x0000),                # tie with zero: even
        (1.5 * 2.0 ** -134, 0x0001),
        (2.0 ** -126, 0x0080),                # smallest normal
        (float.fromhex("0x1.fep127"), 0x7F7F),  # largest finite
        (float.fromhex("0x1.ffp127"), 0x7F80),  # tie past the largest: even is infinity
        (math.inf, 0x7F80), (-math.inf, 0xFF80), (1e300, 0x7F80),
        (math.pi, 0x4049),
    ]
    for x, want in cases:
        got = int(_round(lib, [x])[0])
        assert got == want, f"round({x!r}) = {got:#06x}, want {want:#06x}"
    assert int(_round(lib, [math.nan])[0]) == 0x7FC0


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------
def _complex_rope(x: np.ndarray, pos: float, theta: float) -> np.ndarray:
    d = x.shape[-1]
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * pos * theta ** (-2.0 * np.arange(h) / d))
    return np.concatenate([z.real, z.imag], axis=-1)


def pin_rope_complex_form(lib):
    rng = np.random.default_rng(103)
    for d in (2, 8, 128):
        x = rng.standard_normal((6, d))
        for pos in (0, 1, 5, 17, 1000, 28671, 67499):
            got = oracle.rope_f64(x, pos, THETA, lib=lib)
            want = _complex_rope(x, pos, THETA)
            err = np.abs(got - want).max()
            assert err <= 1e-9, f"d={d} pos={pos}: {err}"
    x = rng.standard_normal((3, 64))
    assert np.abs(oracle.rope_f64(x, 300, 10000.0, lib=lib) - _complex_rope(x, 300, 10000.0)).max() <= 1e-10


def pin_rope_closed_forms(lib):
    d = 128
    for pos in (1.0, 5.0, 123.0):
        e0 = np.zeros(d)
        e0[0] = 1.0
        y = oracle.rope_f64(e0, pos, THETA, lib=lib)       # frequency theta^0 = 1
        assert abs(y[0] - math.cos(pos)) <= 1e-15 and abs(y[64] - math.sin(pos)) <= 1e-15, y[[0, 64]]
        assert np.count_nonzero(y) == 2
        e32 = np.zeros(d)
        e32[96] = 1.0                                      # second half of pair 32
        y = oracle.rope_f64(e32, 1000.0 * pos, THETA, lib=lib)   # frequency 1e6^(-1/2) = 1e-3
        assert abs(y[96] - math.cos(pos)) <= 1e-12 and abs(y[32] + math.sin(pos)) <= 1e-12, y[[32, 96]]
    x = np.random.default_rng(104).standard_normal(d)
    assert np.array_equal(oracle.rope_f64(x, 0.0, THETA, lib=lib), x), "position 0 must be the identity"


def pin_rope_invariants(lib):
    rng = np.random.default_rng(105)
    d = 128
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    for m, n in ((7, 3), (28671, 100), (67499, 67000), (5, 5), (2, 9)):
        lhs = oracle.rope_f64(q, m, THETA, lib=lib) @ oracle.rope_f64(k, n, THETA, lib=lib)
        rhs = oracle.rope_f64(q, m - n, THETA, lib=lib) @ k
        assert abs(lhs - rhs) <= 1e-8, f"relative position ({m},{n}): {lhs} vs {rhs}"
        y = oracle.rope_f64(q, m, THETA, lib=lib)
        pair_in = q[:64] ** 2 + q[64:] ** 2
        pair_out = y[:64] ** 2 + y[64:] ** 2
        assert np.abs(pair_in - pair_out).max() <= 1e-12, "pair norms must be preserved"
        back = oracle.rope_f64(y, -m, THETA, lib=lib)
        assert np.abs(back - q).max() <= 1e-10, "R(-p) R(p) must be the identity"


# --------------------------------------------------------------------------
# the append
# --------------------------------------------------------------------------
class AppendCase:
    """A small pool, table and new tokens, with slots computed by this file."""

    def __init__(self, rng, ctx, n_new, Hq=4, Hkv=2, D=16, page=4, extra_pages=4, new_start=True):
        B = len(ctx)
        self.ctx = np.asarray(ctx, dtype=np.int32)
        self.n = np.asarray(n_new, dtype=np.int64)
        need = [(c + page - 1) // page for c in ctx]
        P = sum(need) + extra_pages
        width = max(1, max(need))
        perm = rng.permutation(P)
        self.table = np.full((B, width), -1, dtype=np.int32)
        o = 0
        for b, k in enumerate(need):
            self.table[b, :k] = perm[o:o + k]
            o += k
        T = int(self.n.sum()) + 2                      # two spare rows nobody names
        self.k_pool = f32_to_bf16_bits(rng.standard_normal((P, page, Hkv, D)).astype(np.float32))
        self.v_pool = f32_to_bf16_bits(rng.standard_normal((P, page, Hkv, D)).astype(np.float32))
        self.k_new = f32_to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
        self.v_new = f32_to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
        self.q = f32_to_bf16_bits(rng.standard_normal((T, Hq, D)).astype(np.float32))
        self.page = page
        if new_start:
            self.new_start = np.concatenate([[0], np.cumsum(self.n)]).astype(np.int32)
        else:
            self.new_start = None

    def writes(self):
        """(row, page, slot, position) of every new token, from the table."""
        out = []
        for b, c in enumerate(self.ctx):
            start = int(self.new_start[b]) if self.new_start is not None else b
            n = int(self.n[b])
            for j in range(n):
                p = int(c) - n + j
                out.append((start + j, int(self.table[b, p // self.page]), p % self.page, p))
        return out


def _check_append(lib, case, rope):
    k, v, q = oracle.kv_append(case.k_new, case.v_new, case.table, case.ctx, case.k_pool, case.v_pool,
                               new_start=case.new_start, q=case.q, rope=rope, theta=THETA, lib=lib)
    touched = np.zeros(case.k_pool.shape[:2], dtype=bool)
    q_rows = set()
    for row, page, slot, pos in case.writes():
        touched[page, slot] = True
        assert np.array_equal(v[page, slot], case.v_new[row]), f"V row {row}"
        if rope:
            exact = _complex_rope(_val(case.k_new[row]), pos, THETA)
            assert nearest_ok(k[page, slot], exact, 1e-12).all(), f"K row {row} at {pos}"
            exact_q = _complex_rope(_val(case.q[row]), pos, THETA)
            assert nearest_ok(q[row], exact_q, 1e-12).all(), f"q row {row} at {pos}"
        else:
            assert np.array_equal(k[page, slot], case.k_new[row]), f"K row {row}"
        q_rows.add(row)
    assert np.array_equal(k[~touched], case.k_pool[~touched]), "K slots outside the append changed"
    assert np.array_equal(v[~touched], case.v_pool[~touched]), "V slots outside the append changed"
    others = [r for r in range(case.q.shape[0]) if r not in q_rows or not rope]
    assert np.array_equal(q[others], case.q[others]), "q rows that are not rotated changed"


def pin_append_decode_rows(lib):
    rng = np.random.default_rng(106)
    case = AppendCase(rng, ctx=[9, 1, 0, 4, 13], n_new=[1, 1, 0, 1, 1], new_start=False)
    for rope in (False, True):
        _check_append(lib, case, rope)


def pin_append_chunks(lib):
    rng = np.random.default_rng(107)
    # chunks that cross page boundaries, an empty chunk, a chunk that is the whole context
    case = AppendCase(rng, ctx=[11, 7, 20, 3, 0], n_new=[6, 0, 9, 3, 0])
    for rope in (False, True):
        _check_append(lib, case, rope)
    big = AppendCase(rng, ctx=[70000], n_new=[5], Hq=2, Hkv=1, D=128, page=16, extra_pages=1)
    _check_append(lib, big, True)


def pin_append_validation(lib):
    rng = np.random.default_rng(108)
    ok = AppendCase(rng, ctx=[9, 4], n_new=[2, 1])
    assert oracle.kv_append_validate(ok.k_new, ok.table, ok.ctx, ok.k_pool, new_start=ok.new_start, lib=lib) == 0
    bad_page = ok.table.copy()
    bad_page[0, 2] = ok.k_pool.shape[0]
    assert oracle.kv_append_validate(ok.k_new, bad_page, ok.ctx, ok.k_pool, new_start=ok.new_start, lib=lib) == 1
    too_many = np.array([0, 10, 11], dtype=np.int32)               # 10 new tokens, context 9
    assert oracle.kv_append_validate(ok.k_new, ok.table, ok.ctx, ok.k_pool, new_start=too_many, lib=lib) == 1
    past_rows = np.array([0, 2, ok.k_new.shape[0] + 1], dtype=np.int32)
    assert oracle.kv_append_validate(ok.k_new, ok.table, ok.ctx, ok.k_pool, new_start=past_rows, lib=lib) == 1
    shared = ok.table.copy()
    shared[1, 0] = shared[0, 2]                                    # both write slot 0 of one page
    ctx = np.array([9, 1], dtype=np.int32)
    assert oracle.kv_append_validate(ok.k_new, shared, ctx, ok.k_pool, new_start=ok.new_start, lib=lib) == 1
    long_ctx = np.array([9, ok.table.shape[1] * ok.page + 1], dtype=np.int32)
    assert oracle.kv_append_validate(ok.k_new, ok.table, long_ctx, ok.k_pool, new_start=ok.new_start, lib=lib) == 1
    try:
        oracle.kv_append(ok.k_new, ok.v_new, bad_page, ok.ctx, ok.k_pool, ok.v_pool, new_start=ok.new_start,
                         lib=lib)
    except oracle.OracleError:
        pass
    else:
        raise AssertionError("an out-of-pool page must be refused")


PINS = [
    pin_round_nearest_bruteforce,
    pin_round_matches_float32_rounding,
    pin_round_worked_values,
    pin_rope_complex_form,
    pin_rope_closed_forms,
    pin_rope_invariants,
    pin_append_decode_rows,
    pin_append_chunks,
    pin_append_validation,
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
