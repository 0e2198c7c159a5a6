"""Pins of the block-boundary gradient scaling oracle (oracle/blockscale.py) to what the pages
and exact arithmetic fix, independent of the oracle's own formulas:
  * the float-format values and the scale-quantise-unscale demo printed in
    "AIGC 基本功|混合精度与数值稳定性-AMP" §4 (tests/golden/amp_float_formats.txt);
  * every 16-bit code decoded from its sign/exponent/mantissa fields;
  * round-to-nearest-even chosen between the two neighbouring codes by exact distances;
  * exact rational arithmetic (fractions.Fraction) for the once-rounded float32 quotient
    and sum;
  * the fp16 relative error bound 2^-11 for a round trip through a power-of-two scale.
Planted mistakes in the oracle (MUTANTS) must each fail one of these checks.
"""
from __future__ import annotations

import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "amp_float_formats.txt")


def _rows():
    rows = []
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append(line.split())
    return rows


def _sig_equal(got, text):
    exp = float(text)
    if math.isinf(exp):
        return math.isinf(got) and (got > 0) == (exp > 0)
    if exp == 0.0:
        return got == 0.0
    digits = len(text.split("e")[0].replace("-", "").replace(".", "").lstrip("0")) or 1
    return abs(got - exp) <= 0.5 * 10 ** (math.floor(math.log10(abs(exp))) - digits + 1) * 1.0001


def _decode_fields(code: int, ebits: int, mbits: int) -> float:
    """Value of a binary floating-point code from its fields (IEEE layout)."""
    sign = -1.0 if code >> (ebits + mbits) else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    bias = (1 << (ebits - 1)) - 1
    if e == (1 << ebits) - 1:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(m, 1 - bias - mbits)
    return sign * math.ldexp((1 << mbits) + m, e - bias - mbits)


def _round_f32(x: Fraction) -> np.float32:
    """Nearest float32 to an exact rational, ties to even, chosen by exact comparison."""
    guess = np.float32(float(x))
    best = None
    for cand in (np.nextafter(guess, np.float32(-np.inf)), guess, np.nextafter(guess, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - x)
        even = (int(np.float32(cand).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, cand)
    return np.float32(best[1])


def _value16(impl, codes, dtype):
    if dtype == "f16":
        return np.asarray(codes, np.float16).astype(np.float64)
    return impl.bf16_bits_to_f64(codes)


# ------------------------------------------------------------------------------------------
# checks (each takes an implementation namespace so that planted mistakes can be run)
# ------------------------------------------------------------------------------------------
def check_printed_conversions(impl):
    """S = 1: entering a block is the plain 16-bit conversion, whose values §4 prints."""
    n = 0
    for kind, x, expect, *_ in _rows():
        if kind not in ("fp16", "bf16"):
            continue
        dt = "f16" if kind == "fp16" else "bf16"
        code = impl.block_grad_enter(np.array([float(x)], np.float32), 1.0, dt)
        got = float(_value16(impl, code, dt)[0])
        assert _sig_equal(got, expect), (kind, x, got, expect)
        n += 1
    assert n == 11


def check_printed_loss_scaling_demo(impl):
    """§4's demo: multiply by 1024, quantise to fp16, divide by 1024 (printed per input); and
    without the scale 1e-8 flushes to zero."""
    n = 0
    for kind, x, expect, *_ in _rows():
        if kind != "fp16x1024":
            continue
        g = impl.block_grad_enter(np.array([float(x)], np.float32), 1024.0, "f16")
        out, flag = impl.block_grad_exit(np.zeros(1, np.float32), g, 1024.0, "f16")
        assert not flag
        assert _sig_equal(float(out[0]), expect), (x, float(out[0]), expect)
        n += 1
    assert n == 5
    assert float(impl.block_grad_enter(np.array([1e-8], np.float32), 1.0, "f16")[0]) == 0.0


def check_all_codes_decode(impl):
    """Leaving a block with S = 1 and dx = 0 returns every finite 16-bit code's exact value
    (decoded from its fields) and 0 for inf and NaN codes, for fp16 and bf16."""
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dt, eb, mb in (("f16", 5, 10), ("bf16", 8, 7)):
        g = codes.view(np.float16) if dt == "f16" else codes
        out, flag = impl.block_grad_exit(np.zeros(codes.size, np.float32), g, 1.0, dt)
        assert flag
        want = np.array([_decode_fields(int(c), eb, mb) for c in codes])
        want = np.where(np.isfinite(want), want, 0.0)
        assert np.array_equal(out.astype(np.float64), want), dt
        finite = np.isfinite(np.array([_decode_fields(int(c), eb, mb) for c in codes[:1000]]))
        _, f2 = impl.block_grad_exit(np.zeros(int(finite.sum()), np.float32), g[:1000][finite], 1.0, dt)
        assert not f2


def check_bf16_round_to_nearest_even(impl, seed=21):
    """bf16 conversion picks the nearer of the two neighbouring codes by exact distance, the
    even code on a tie; overflow past the largest finite value goes to inf."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, 4000, dtype=np.uint64).astype(np.uint32)
    bits[:8] = [0x3F808000, 0x3F818000, 0x3F80C000, 0x3F807FFF, 0x7F7FFFFF, 0x7F7F7FFF, 0x00008000, 0x80018000]
    x = bits.view(np.float32)
    keep = np.isfinite(x)
    x, bits = x[keep], bits[keep]
    got = impl.f32_to_bf16_bits(x)
    for xv, b, c in zip(x, bits, got):
        sign = int(b) >> 31
        lo = (int(b) & 0x7FFFFFFF) >> 16                     # magnitude code, truncated
        ex = abs(Fraction(float(xv)))
        v0 = Fraction(_decode_fields(lo, 8, 7))
        v1 = _decode_fields(lo + 1, 8, 7)
        if math.isinf(v1):
            # past the largest finite bf16 (an odd code): RNE reaches inf from the halfway point
            want = lo + 1 if ex >= (v0 + Fraction(2) ** 128) / 2 else lo
        else:
            d0, d1 = ex - v0, Fraction(v1) - ex
            want = lo if d0 < d1 or (d0 == d1 and lo % 2 == 0) else lo + 1
        assert int(c) == ((sign << 15) | want), (hex(int(b)), hex(int(c)), hex((sign << 15) | want))


def check_exit_exact_rounding(impl, seed=22):
    """dx + fp32(g / S) with each operation rounded once to float32, checked in exact
    rational arithmetic, for scales that are not powers of two; non-finite g adds nothing."""
    rng = np.random.default_rng(seed)
    for dt in ("f16", "bf16"):
        for S in (3.0, 0.7, 1000.0, 12345.678):
            s32 = np.float32(S)
            dx = (rng.standard_normal(300) * 10.0 ** rng.uniform(-6, 0, 300)).astype(np.float32)
            v = (rng.standard_normal(300) * 10.0 ** rng.uniform(-3, 2, 300)).astype(np.float32)
            g = v.astype(np.float16) if dt == "f16" else impl.f32_to_bf16_bits(v)
            gv = _value16(impl, g, dt)
            if dt == "f16":
                g[5], g[9] = np.float16(np.inf), np.float16(np.nan)
            else:
                g[5], g[9] = 0x7F80, 0x7FC1
            gv = _value16(impl, g, dt)
            out, flag = impl.block_grad_exit(dx, g, float(s32), dt)
            assert flag
            for i in range(dx.size):
                if not np.isfinite(gv[i]):
                    assert out[i] == dx[i]
                    continue
                q = _round_f32(Fraction(float(gv[i])) / Fraction(float(s32)))
                want = _round_f32(Fraction(float(dx[i])) + Fraction(float(q)))
                assert out[i] == want, (dt, S, i, out[i], want)


def check_enter_exact_rounding(impl, seed=23):
    """to16(fp32(S * dx)): the exact product rounded to float32, then to the 16-bit format by
    nearest code (ties to even), checked against exact rationals."""
    rng = np.random.default_rng(seed)
    f16_codes = np.arange(0, 0x7C01, dtype=np.uint16)          # +0 .. +inf
    f16_vals = [Fraction(_decode_fields(int(c), 5, 10)) for c in f16_codes[:-1]]
    for S in (3.0, 1024.0, 0.3):
        s32 = np.float32(S)
        dx = (rng.standard_normal(200) * 10.0 ** rng.uniform(-9, 4, 200)).astype(np.float32)
        # products that land within float32 rounding of an fp16 tie (the midpoint of two
        # neighbouring fp16 values): their float32 rounding decides the tie
        c = rng.integers(0x0400, 0x7BFF, 200)
        mid = np.array([(_decode_fields(int(k), 5, 10) + _decode_fields(int(k) + 1, 5, 10)) / 2 for k in c])
        dx = np.concatenate([dx, (mid / float(s32)).astype(np.float32)])
        got = impl.block_grad_enter(dx, float(s32), "f16")
        for i in range(dx.size):
            p = _round_f32(Fraction(float(dx[i])) * Fraction(float(s32)))
            a = abs(Fraction(float(p)))
            # nearest fp16 magnitude code by bisection over the ordered codes
            lo, hi = 0, len(f16_vals) - 1
            while hi - lo > 1:
                mid = (lo + hi) // 2
                if f16_vals[mid] <= a:
                    lo = mid
                else:
                    hi = mid
            if a >= f16_vals[-1] + (Fraction(2) ** 16 - f16_vals[-1]) / 2:
                want = math.inf
            else:
                d0, d1 = a - f16_vals[lo], f16_vals[hi] - a
                k = lo if d0 < d1 or (d0 == d1 and lo % 2 == 0) else hi
                if a > f16_vals[-1]:
                    k = len(f16_vals) - 1
                want = float(f16_vals[k])
            want = math.copysign(want, float(p))
            assert float(got[i]) == want or (want == 0 and float(got[i]) == 0), (S, dx[i], float(got[i]), want)


def check_power_of_two_round_trip(impl, seed=24):
    """With S = 2^k keeping S*dx in fp16's normal range, a block's round trip loses at most
    fp16's relative rounding error 2^-11 (plus the float32 one)."""
    rng = np.random.default_rng(seed)
    x = (10.0 ** rng.uniform(-8, -2, 2000) * rng.choice([-1, 1], 2000)).astype(np.float32)
    for k in range(4, 26, 3):
        S = 2.0 ** k
        sx = np.abs(x.astype(np.float64)) * S
        ok = (sx >= 2.0 ** -14) & (sx <= 60000.0)
        g = impl.block_grad_enter(x[ok], S, "f16")
        out, flag = impl.block_grad_exit(np.zeros(int(ok.sum()), np.float32), g, S, "f16")
        assert not flag
        err = np.abs(out.astype(np.float64) - x[ok].astype(np.float64))
        assert (err <= (2.0 ** -11 + 2.0 ** -23) * np.abs(x[ok].astype(np.float64))).all(), k


ALL_CHECKS = (check_printed_conversions, check_printed_loss_scaling_demo, check_all_codes_decode,
              check_bf16_round_to_nearest_even, check_exit_exact_rounding, check_enter_exact_rounding,
              check_power_of_two_round_trip)


def _impl(**over):
    ns = types.SimpleNamespace(block_grad_enter=oracle.block_grad_enter,
                               block_grad_exit=oracle.block_grad_exit,
                               f32_to_bf16_bits=oracle.f32_to_bf16_bits,
                               bf16_bits_to_f64=oracle.bf16_bits_to_f64)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_blockscale_pin(check):
    check(_impl())


# ------------------------------------------------------------------------------------------
# planted mistakes
# ------------------------------------------------------------------------------------------
def _exit_multiplies(dx, g, scale, dtype="f16"):
    return oracle.block_grad_exit(dx, g, 1.0 / float(np.float32(scale)) if scale else scale, dtype)


def _exit_keeps_nan(dx, g, scale, dtype="f16"):
    out, flag = oracle.block_grad_exit(dx, g, scale, dtype)
    gv = np.asarray(g, np.float16).astype(np.float64) if dtype == "f16" else oracle.bf16_bits_to_f64(g)
    out = np.where(np.isnan(gv), np.float32(np.nan), out).astype(np.float32)
    return out, bool(np.isinf(gv).any())


def _enter_truncates(dx, scale, dtype="f16"):
    p = (np.float64(np.float32(scale)) * np.asarray(dx, np.float32).astype(np.float64)).astype(np.float32)
    if dtype == "f16":
        r = p.astype(np.float16)
        over = np.abs(r.astype(np.float64)) > np.abs(p.astype(np.float64))
        return np.where(over, np.nextafter(r, np.float16(0)), r).astype(np.float16)
    return (p.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_truncates(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _enter_no_f32_product(dx, scale, dtype="f16"):
    """Rounds the product straight from float64 (skips the float32 rounding) and scales by
    the float64 scale rather than its float32 value."""
    p = float(scale) * np.asarray(dx, np.float32).astype(np.float64)
    return p.astype(np.float16) if dtype == "f16" else oracle.f32_to_bf16_bits(p.astype(np.float32))


def _exit_adds_in_f64(dx, g, scale, dtype="f16"):
    """Skips the float32 rounding of the quotient."""
    gv = np.asarray(g, np.float16).astype(np.float64) if dtype == "f16" else oracle.bf16_bits_to_f64(g)
    fin = np.isfinite(gv)
    q = np.where(fin, gv, 0.0) / np.float64(np.float32(scale))
    return (np.asarray(dx, np.float32).astype(np.float64) + q).astype(np.float32), bool((~fin).any())


MUTANTS = {
    "exit_multiplies_by_scale": dict(block_grad_exit=_exit_multiplies),
    "exit_keeps_nan": dict(block_grad_exit=_exit_keeps_nan),
    "enter_truncates": dict(block_grad_enter=_enter_truncates),
    "bf16_truncates": dict(f32_to_bf16_bits=_bf16_truncates),
    "enter_skips_f32_product": dict(block_grad_enter=_enter_no_f32_product),
    "exit_unrounded_quotient": dict(block_grad_exit=_exit_adds_in_f64),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_blockscale_pins_catch_mutant(name):
    impl = _impl(**MUTANTS[name])
    caught = []
    for check in ALL_CHECKS:
        try:
            check(impl)
        except AssertionError:
            caught.append(check.__name__)
        except Exception:
            caught.append(check.__name__ + " (error)")
    assert caught, f"no pin caught mutant {name}"
