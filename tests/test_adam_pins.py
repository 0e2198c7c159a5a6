"""Pins of the optimizer oracle (oracle/adam.py) to facts other than itself:
  * the printed Adam run of "AIGC 基本功|数据并行与 ZeRO 显存切分" §4.2
    (tests/golden/zero_adam_first_step.txt);
  * textbook closed forms of Adam: the bias-corrected first step, a constant gradient, a
    gradient that stops, decoupled weight decay with no gradient;
  * clipping: the clipped norm is min(N, C); with eps = 0 and no decay a clipped first step
    moves the parameters exactly as an unclipped one;
  * brute-force element loops for the global norm;
  * the ue8m8 storage format decoded from its exponent and fraction fields for every code,
    and rounded to the nearest code by exact rational distance (ties to even);
  * planted mistakes in copies of the update, each caught by one of the pins.
"""
import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "zero_adam_first_step.txt")


def _golden():
    d = {}
    with open(GOLDEN) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            vals = [float(x) for x in t[1:]]
            d[t[0]] = vals if len(vals) > 1 else vals[0]
    return d


# ------------------------------------------------------------------------------------------
# checks, each taking an object with adam_update (the oracle module or a mutant)
# ------------------------------------------------------------------------------------------
def check_printed_first_step(impl):
    g = _golden()
    hp = oracle.AdamHyper(lr=g["lr"], beta1=g["beta1"], beta2=g["beta2"], eps=g["eps"])
    params = np.array(g["params"])
    # the page's per-rank gradients, averaged as its all-reduce does
    local = [[((k + 1) * (i + 2) - 3) / 100.0 for i in range(len(params))] for k in range(4)]
    avg = np.mean(np.array(local), axis=0)
    assert np.allclose(avg, g["averaged_gradient"], rtol=0, atol=1e-15)
    th, m1, m2 = impl.adam_update(params, np.zeros(8), np.zeros(8), avg, 1, hp)
    half = 0.5 * 10.0 ** (-int(g["printed_decimals"]))
    assert np.abs(th - np.array(g["updated_params"])).max() <= half, th
    # ZeRO-2's path: each rank updates its 2-parameter shard with its own moments; the
    # gathered result is the full update (the page prints max_abs_diff = 0)
    shard = [impl.adam_update(params[2 * k:2 * k + 2], np.zeros(2), np.zeros(2), avg[2 * k:2 * k + 2], 1, hp)[0]
             for k in range(4)]
    assert np.array_equal(np.concatenate(shard), th)
    assert m1.size + m2.size == g["moment_scalars_full"]
    assert shard[0].size * 2 == g["moment_scalars_shard"]


def check_first_step_closed_form(impl, seed=1):
    """m1_hat = g and m2_hat = g^2 at t = 1, so the step is lr g / (|g| + eps)."""
    rng = np.random.default_rng(seed)
    th0 = rng.standard_normal(64)
    g = rng.standard_normal(64) * np.exp(rng.uniform(-20, 2, 64))
    hp = oracle.AdamHyper(lr=3e-3, beta1=0.85, beta2=0.97, eps=1e-6)
    th, m1, m2 = impl.adam_update(th0, np.zeros(64), np.zeros(64), g, 1, hp)
    want = th0 - 3e-3 * g / (np.abs(g) + 1e-6)
    assert np.abs(th - want).max() <= 1e-15
    assert np.allclose(m1, 0.15 * g, rtol=1e-15, atol=0) and np.allclose(m2, 0.03 * g * g, rtol=1e-14, atol=0)


def check_constant_gradient(impl, seed=2):
    """A constant gradient keeps m1_hat = g and m2_hat = g^2 at every t (exact bias
    correction), so every step moves theta by lr g / (|g| + eps)."""
    rng = np.random.default_rng(seed)
    th = rng.standard_normal(32)
    th0 = th.copy()
    g = rng.standard_normal(32)
    m1, m2 = np.zeros(32), np.zeros(32)
    hp = oracle.AdamHyper(lr=1e-2, beta1=0.9, beta2=0.96, eps=1e-8)
    T = 12
    for t in range(1, T + 1):
        th, m1, m2 = impl.adam_update(th, m1, m2, g, t, hp)
    want = th0 - T * 1e-2 * g / (np.abs(g) + 1e-8)
    assert np.abs(th - want).max() <= 1e-12


def check_gradient_stops(impl, seed=3):
    """g at step 1, zero afterwards: m1_t = beta1^(t-1) (1 - beta1) g and
    m2_t = beta2^(t-1) (1 - beta2) g^2, so step t moves theta by
    lr m1_t / (1 - beta1^t) / (sqrt(m2_t / (1 - beta2^t)) + eps)."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(16)
    b1, b2, lr, eps = 0.8, 0.95, 5e-3, 1e-7
    hp = oracle.AdamHyper(lr=lr, beta1=b1, beta2=b2, eps=eps)
    th = rng.standard_normal(16)
    want = th.copy()
    m1, m2 = np.zeros(16), np.zeros(16)
    for t in range(1, 9):
        gt = g if t == 1 else np.zeros(16)
        th, m1, m2 = impl.adam_update(th, m1, m2, gt, t, hp)
        a1 = b1 ** (t - 1) * (1 - b1) * g
        a2 = b2 ** (t - 1) * (1 - b2) * g * g
        want = want - lr * (a1 / (1 - b1 ** t)) / (np.sqrt(a2 / (1 - b2 ** t)) + eps)
        assert np.abs(th - want).max() <= 1e-13, t


def check_decoupled_decay(impl, seed=4):
    """No gradient: both moments stay 0, so only the decoupled decay acts:
    theta_t = theta_0 (1 - lr wd)^t."""
    rng = np.random.default_rng(seed)
    th0 = rng.standard_normal(10)
    th = th0.copy()
    m1, m2 = np.zeros(10), np.zeros(10)
    hp = oracle.AdamHyper(lr=0.01, weight_decay=0.1)
    for t in range(1, 6):
        th, m1, m2 = impl.adam_update(th, m1, m2, np.zeros(10), t, hp)
    assert np.abs(th - th0 * (1 - 0.001) ** 5).max() <= 1e-15


def check_clip_invariance(impl, seed=5):
    """With eps = 0 and no decay, a first step moves theta by lr sign(g) whatever positive
    factor scales g: the clipped and the unclipped step agree."""
    rng = np.random.default_rng(seed)
    th0 = rng.standard_normal(20)
    g = rng.standard_normal(20) * 10
    hp = oracle.AdamHyper(lr=1e-3, eps=0.0)
    c = oracle.clip_factor(float(np.linalg.norm(g)), 1.0)
    a = impl.adam_update(th0, np.zeros(20), np.zeros(20), g, 1, hp)[0]
    b = impl.adam_update(th0, np.zeros(20), np.zeros(20), c * g, 1, hp)[0]
    assert c < 0.1 and np.abs(a - b).max() <= 1e-15
    assert np.abs(a - (th0 - 1e-3 * np.sign(g))).max() <= 1e-15


ALL_CHECKS = [check_printed_first_step, check_first_step_closed_form, check_constant_gradient,
              check_gradient_stops, check_decoupled_decay, check_clip_invariance]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_adam_pin(check):
    check(oracle)


# ------------------------------------------------------------------------------------------
# clipping and the global norm
# ------------------------------------------------------------------------------------------
def test_global_norm_brute_force_and_clip():
    rng = np.random.default_rng(6)
    grads = [rng.standard_normal((3, 5)), rng.standard_normal(7) * 1e-3, np.zeros(4)]
    total = 0.0
    for g in grads:
        for v in np.asarray(g).ravel():
            total += float(v) * float(v)
    assert abs(oracle.global_norm(grads) - math.sqrt(total)) <= 1e-15 * math.sqrt(total)
    for C in (0.5, 2.0, 1e9):
        n = oracle.global_norm(grads)
        c = oracle.clip_factor(n, C)
        assert 0 < c <= 1
        assert abs(oracle.global_norm([c * np.asarray(g) for g in grads]) - min(n, C)) <= 1e-14 * n
    assert oracle.clip_factor(5.0, 0.0) == 1.0 and oracle.clip_factor(5.0, -1.0) == 1.0
    assert oracle.clip_factor(0.0, 1.0) == 1.0


def test_group_step_skip_and_order():
    """A skipped step leaves every state and t untouched; an applied one increments t, clips
    every gradient by one global factor and stores each value in its format."""
    rng = np.random.default_rng(7)
    states = [oracle.AdamState(oracle.store_param(rng.standard_normal((4, 8)) * 0.05, "f16"),
                               np.zeros((4, 8)), np.zeros((4, 8))),
              oracle.AdamState(rng.standard_normal(6), np.zeros(6), np.zeros(6), "f32", "f32", "f32")]
    grads = [rng.standard_normal((4, 8)), rng.standard_normal(6) * 3]
    hp = oracle.AdamHyper(lr=1e-2, weight_decay=0.01)
    same, t, n, c = oracle.adam_group_step(states, grads, 7, True, hp, n_mats=1, max_norm=1.0)
    assert t == 7 and n is None and c is None
    for a, b in zip(same, states):
        assert np.array_equal(a.theta, b.theta) and np.array_equal(a.m1, b.m1) and np.array_equal(a.m2, b.m2)
    new, t, n, c = oracle.adam_group_step(states, grads, 7, False, hp, hp_pass=oracle.AdamHyper(lr=1e-2),
                                          n_mats=1, max_norm=1.0)
    assert t == 8
    assert abs(n - math.sqrt(sum(float(np.sum(g ** 2)) for g in grads))) <= 1e-12 * n
    assert abs(c - 1.0 / n) <= 1e-15
    th, m1, m2 = oracle.adam_update(states[0].theta, 0, 0, c * grads[0], 8, hp)
    assert np.array_equal(new[0].theta, oracle.store_param(th, "f16"))
    assert np.array_equal(new[0].m1, oracle.store_param(m1, "bf16"))
    assert np.array_equal(new[0].m2, oracle.store_param(m2, "ue8m8"))
    th, m1, m2 = oracle.adam_update(states[1].theta, 0, 0, c * grads[1], 8, oracle.AdamHyper(lr=1e-2))
    assert np.array_equal(new[1].theta, th.astype(np.float32).astype(np.float64))


# ------------------------------------------------------------------------------------------
# the ue8m8 second-moment format
# ------------------------------------------------------------------------------------------
def _ue8m8_value(code: int) -> Fraction:
    e, f = code >> 8, code & 0xFF
    if e == 0:
        return Fraction(f, 256) * Fraction(1, 2 ** 126)
    return (1 + Fraction(f, 256)) * (Fraction(2) ** (e - 127))


def test_ue8m8_decodes_every_code_from_its_fields():
    codes = np.arange(0xFF00, dtype=np.uint32).astype(np.uint16)
    vals = oracle.ue8m8_decode(codes)
    assert np.all(np.diff(vals) > 0)
    for c in list(range(0, 600)) + list(range(0x3F00, 0x4100)) + list(range(0xFE00, 0xFF00)):
        assert Fraction(float(vals[c])) == _ue8m8_value(c), hex(c)
    assert np.isposinf(oracle.ue8m8_decode(np.array([0xFF00], np.uint16)))[0]
    assert np.array_equal(oracle.ue8m8_encode(vals.astype(np.float32)), codes)


def test_ue8m8_rounds_to_the_nearest_code():
    rng = np.random.default_rng(8)
    x = np.abs(rng.standard_normal(4000).astype(np.float32)) * np.exp2(rng.integers(-140, 120, 4000)).astype(np.float32)
    x = x[np.isfinite(x)]
    codes = oracle.ue8m8_encode(x)
    for xi, ci in zip(x[:1500], codes[:1500]):
        v = Fraction(float(xi))
        got = _ue8m8_value(int(ci))
        for nb in (int(ci) - 1, int(ci) + 1):
            if 0 <= nb < 0xFF00:
                alt = _ue8m8_value(nb)
                assert abs(v - got) <= abs(v - alt), (xi, ci, nb)
                if abs(v - got) == abs(v - alt):
                    assert int(ci) % 2 == 0
    # exact midpoints between neighbouring codes go to the even one
    for c in (0x3F80, 0x3F81, 0x0001, 0x0100, 0x7000, 0x7001):
        mid = (_ue8m8_value(c) + _ue8m8_value(c + 1)) / 2
        xm = np.array([float(mid)], dtype=np.float32)
        assert Fraction(float(xm[0])) == mid
        assert int(oracle.ue8m8_encode(xm)[0]) == (c if c % 2 == 0 else c + 1)
    # overflow: at or beyond the halfway point above the largest code -> infinity code
    top = _ue8m8_value(0xFEFF)
    half = top + (Fraction(2) ** 128 - top) / 2
    assert int(oracle.ue8m8_encode(np.array([float(half)], np.float32))[0]) == 0xFF00
    below = np.nextafter(np.float32(float(half)), np.float32(0))
    assert int(oracle.ue8m8_encode(np.array([below], np.float32))[0]) == 0xFEFF
    assert int(oracle.ue8m8_encode(np.array([np.inf], np.float32))[0]) == 0xFF00
    assert int(oracle.ue8m8_encode(np.array([-0.0], np.float32))[0]) == 0
    with pytest.raises(ValueError):
        oracle.ue8m8_encode(np.array([-1.0], np.float32))


def test_store_param_goes_through_float32():
    """The 16-bit decision is taken on the float32 value: a float64 value just above a bf16
    midpoint whose float32 rounding lands on the midpoint rounds to even."""
    mid = 1.0 + 2.0 ** -8                       # halfway between bf16 1 and 1 + 2^-7
    x = mid + 2.0 ** -40                        # float32(x) == mid
    assert oracle.store_param(np.array([x]), "bf16")[0] == 1.0
    assert oracle.store_param(np.array([mid + 2.0 ** -20]), "bf16")[0] == 1.0 + 2.0 ** -7


# ------------------------------------------------------------------------------------------
# planted mistakes
# ------------------------------------------------------------------------------------------
def _mutant(kind):
    def adam_update(theta, m1, m2, g, t, hp):
        theta = np.asarray(theta, dtype=np.float64)
        g = np.asarray(g, dtype=np.float64)
        b1, b2 = hp.beta1, hp.beta2
        if kind == "swapped_betas":
            b1, b2 = b2, b1
        gg = g + hp.weight_decay * theta if kind == "coupled_decay" else g
        m1 = b1 * np.asarray(m1, dtype=np.float64) + (1 - b1) * gg
        m2 = b2 * np.asarray(m2, dtype=np.float64) + (1 - b2) * gg * gg
        c1 = 1.0 if kind == "no_bias_correction" else 1 - b1 ** t
        c2 = 1.0 if kind == "no_bias_correction" else 1 - b2 ** t
        if kind == "bias_correction_at_t_minus_1":
            c1, c2 = 1 - b1 ** max(t - 1, 1), 1 - b2 ** max(t - 1, 1)
        den = (m2 / c2) if kind == "no_sqrt" else np.sqrt(m2 / c2)
        step = (m1 / c1) / (den + hp.eps)
        if kind != "coupled_decay":
            step = step + hp.weight_decay * theta
        sign = -1.0 if kind == "ascent" else 1.0
        return theta - sign * hp.lr * step, m1, m2
    return types.SimpleNamespace(adam_update=adam_update)


MUTANTS = ["swapped_betas", "coupled_decay", "no_bias_correction", "bias_correction_at_t_minus_1",
           "no_sqrt", "ascent"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_adam_pins_catch_mutant(kind):
    impl = _mutant(kind)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(impl)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin caught {kind}"


def test_unmodified_mutant_passes():
    impl = _mutant("none")
    for check in ALL_CHECKS:
        check(impl)
