"""The oracle, pinned to facts other than itself (CPU only)."""
import math
import os
import types

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_tiny_workload_against_svd():
    """256x128 N(0,1) at rank 4: 1 and 20 subspace iterations versus numpy's SVD, plus the
    exact rank-4 matrix recovered to round-off in one step."""
    w = wl.workload(1)
    spec = w.matrices[0]
    G = wl.gradient_np(w, spec, 0)
    Q0 = wl.initial_q_np(w, spec)
    errs = pins.check_svd_bounds(oracle, G, Q0)
    assert 0.0 < errs[1] < 0.2          # one iteration is not yet converged
    M = wl.exact_rank_np(256, 128, 4, seed=wl.step_seed(1, 0))
    st = oracle.step_matrix(M, 1.0, np.zeros_like(M), Q0)
    assert np.linalg.norm(st.E_next) / np.linalg.norm(M) <= 1e-12


def test_mgs_matches_cgs2_when_well_conditioned():
    rng = np.random.default_rng(21)
    P = rng.standard_normal((200, 12))
    assert np.abs(oracle.modified_gram_schmidt(P) - oracle.gram_schmidt(P)).max() <= 1e-13


def test_zero_and_dependent_columns():
    P = np.zeros((5, 3))
    assert np.array_equal(oracle.gram_schmidt(P), np.zeros((5, 3)))
    P = np.array([[1.0, 2.0, 0.0], [0.0, 0.0, 1.0], [0.0, 0.0, 0.0]])
    out = oracle.gram_schmidt(P)
    assert np.array_equal(out[:, 1], np.zeros(3))        # exactly dependent column -> 0
    assert np.allclose(out[:, [0, 2]], [[1, 0], [0, 1], [0, 0]])
    # M == 0: every factor and the error buffer stay zero.
    st = oracle.step_matrix(np.zeros((4, 3)), 1.0, np.zeros((4, 3)), np.ones((3, 2)))
    assert not st.P.any() and not st.D.any() and not st.E_next.any() and not st.Q_next.any()


# --------------------------------------------------------------------------------------
# dtype pins: the printed conversions of the AMP article
# --------------------------------------------------------------------------------------
def _golden_formats():
    rows = []
    with open(os.path.join(pins.GOLDEN, "amp_float_formats.txt")) as f:
        for line in f:
            t = line.split()
            if t and not t[0].startswith("#"):
                rows.append(t)
    return rows


def _sig_equal(got, text):
    exp = float(text)
    if math.isinf(exp):
        return math.isinf(got) and (got > 0) == (exp > 0)
    if exp == 0.0:
        return got == 0.0
    digits = len(text.split("e")[0].replace("-", "").replace(".", "").lstrip("0")) or 1
    return abs(got - exp) <= 0.5 * 10 ** (math.floor(math.log10(abs(exp))) - digits + 1) * 1.0001


def test_amp_printed_conversions():
    rows = _golden_formats()
    n = 0
    for kind, x, expect, *_ in rows:
        if kind == "fp16":
            got = float(wl.to_fp16(float(x)))
        elif kind == "bf16":
            got = float(wl.to_bf16_f32(np.float32(float(x))).reshape(-1)[0])
        elif kind == "fp16x1024":
            got = float(wl.to_fp16(float(x) * 1024.0)) / 1024.0
        else:
            continue
        assert _sig_equal(got, expect), (kind, x, got, expect)
        n += 1
    assert n == 16


def test_amp_format_constants():
    consts = {t[1]: t[2] for t in _golden_formats() if t[0] == "const"}
    fi16 = np.finfo(np.float16)
    assert _sig_equal(float(fi16.tiny), consts["fp16_min_normal"])
    assert _sig_equal(2.0 ** -24, consts["fp16_min_subnormal"])
    assert float(wl.to_fp16(2.0 ** -24)) == 2.0 ** -24
    assert _sig_equal(float(fi16.max), consts["fp16_max_finite"])
    assert _sig_equal(float(fi16.eps), consts["fp16_epsilon"])
    bmax = float(wl.bf16_bits_to_f32(np.array([0x7F7F], dtype=np.uint16))[0])
    assert _sig_equal(bmax, consts["bf16_max_finite"])
    assert _sig_equal(float(wl.bf16_bits_to_f32(np.array([0x0080], dtype=np.uint16))[0]),
                      consts["bf16_min_normal"])
    assert _sig_equal(2.0 ** -7, consts["bf16_epsilon"])
    assert _sig_equal(2.0 ** -23, consts["fp32_epsilon"])


def test_fp16_rounding_thresholds():
    """Round-to-nearest-even keeps subnormals: |x| <= 2^-25 goes to zero, anything larger
    reaches the smallest subnormal 2^-24; past the top of the range the result is inf."""
    assert float(wl.to_fp16(2.0 ** -25)) == 0.0
    assert float(wl.to_fp16(-(2.0 ** -25))) == 0.0
    assert float(wl.to_fp16(2.0 ** -25 * (1 + 2 ** -20))) == 2.0 ** -24
    assert float(wl.to_fp16(65504.0)) == 65504.0
    assert math.isinf(float(wl.to_fp16(65520.0)))
    assert float(wl.to_fp16(65519.0)) == 65504.0


def test_bf16_specials():
    x = np.array([np.inf, -np.inf, np.nan, 3.4e38, 1.0, -0.0], dtype=np.float32)
    back = wl.bf16_bits_to_f32(wl.to_bf16_bits(x))
    assert np.isposinf(back[0]) and np.isneginf(back[1]) and np.isnan(back[2])
    assert np.isposinf(back[3])                  # rounds past the largest bf16
    assert back[4] == 1.0 and back[5] == 0.0 and np.signbit(back[5])


# --------------------------------------------------------------------------------------
# the pins catch planted mistakes (mutants of the oracle, on the CPU)
# --------------------------------------------------------------------------------------
def _mutant(**overrides):
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in oracle.__all__})

    def step_matrix(G, s, E, Q):
        G, E, Q = oracle.as_f64(G), oracle.as_f64(E), oracle.as_f64(Q)
        M = overrides.get("M", lambda G, s, E: s * G + E)(G, float(s), E)
        P_raw = M @ Q
        P = ns.gram_schmidt(P_raw)
        Qn = overrides.get("Qn", lambda M, P: M.T @ P)(M, P)
        D = overrides.get("D", lambda P, Qn: P @ Qn.T)(P, Qn)
        En = overrides.get("En", lambda M, D: M - D)(M, D)
        return oracle.MatrixStep(M, P_raw, P, Qn, D, En)

    ns.step_matrix = step_matrix
    if "gram_schmidt" in overrides:
        ns.gram_schmidt = overrides["gram_schmidt"]

    def subspace_iteration(M, Q0, iters):
        Q = oracle.as_f64(Q0)
        for _ in range(iters):
            P = ns.gram_schmidt(oracle.as_f64(M) @ Q)
            Q = overrides.get("Qn", lambda M, P: M.T @ P)(oracle.as_f64(M), P)
        return P, Q, overrides.get("D", lambda P, Qn: P @ Qn.T)(P, Q)

    ns.subspace_iteration = subspace_iteration
    return ns


def _gs_no_normalise(P):
    P = oracle.as_f64(P)
    out = np.zeros_like(P)
    for j in range(P.shape[1]):
        v = P[:, j] - out[:, :j] @ (out[:, :j].T @ P[:, j])
        out[:, j] = v
    return out


def _gs_wrong_index(P):
    P = oracle.as_f64(P)
    out = np.zeros_like(P)
    for j in range(P.shape[1]):
        v = P[:, j].copy()
        prev = out[:, :max(j - 1, 0)]               # skips the previous column
        v = v - prev @ (prev.T @ v)
        n = np.linalg.norm(v)
        out[:, j] = v / n if n > 0 else 0
    return out


MUTANTS = {
    "drops_scale": dict(M=lambda G, s, E: G + E),
    "drops_error_buffer": dict(M=lambda G, s, E: s * G),
    "scales_error_buffer": dict(M=lambda G, s, E: s * (G + E)),
    "error_sign": dict(En=lambda M, D: M + D),
    "transposed_decompress": dict(D=lambda P, Qn: Qn @ P.T),
    "q_not_transposed": dict(Qn=lambda M, P: M @ P if M.shape[0] == M.shape[1] else M[:, :P.shape[0]] @ P),
    "gs_no_normalise": dict(gram_schmidt=_gs_no_normalise),
    "gs_skips_column": dict(gram_schmidt=_gs_wrong_index),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    impl = _mutant(**MUTANTS[name])
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(impl)
        except AssertionError:
            caught.append(check.__name__)
        except Exception:
            caught.append(check.__name__ + " (error)")
    assert caught, f"no pin caught mutant {name}"


def test_unmodified_mutant_passes():
    impl = _mutant()
    for check in pins.ALL_CHECKS:
        check(impl)


# ------------------------------------------------------------------------------------------
# data-parallel step (factor all-reduces), pinned to the single-GPU step it must reduce to
# ------------------------------------------------------------------------------------------
def test_data_parallel_identical_ranks_is_the_single_step():
    """k ranks holding the same gradient and error buffer: the averaged factors equal each
    rank's own, so the group step must be exactly the single-GPU step."""
    rng = np.random.default_rng(901)
    G = rng.standard_normal((40, 24))
    E = rng.standard_normal((40, 24)) * 0.1
    Q = rng.standard_normal((24, 5))
    one = oracle.step_matrix(G, 0.5, E, Q)
    dp = oracle.step_data_parallel([G] * 3, [E] * 3, Q, 0.5)
    for a, b in ((dp.P, one.P), (dp.Q_next, one.Q_next), (dp.D, one.D)):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())
    for e in dp.E_next:
        assert np.abs(e - one.E_next).max() <= 1e-12 * max(1.0, np.abs(one.E_next).max())


def test_data_parallel_mean_error_is_the_step_of_the_mean():
    """Every product in the step is linear in M, so with the factors averaged across ranks the
    decompressed gradient is the single step of the mean M, and the ranks' error buffers
    average to that step's error buffer. Averaging P after orthonormalisation, or D instead of
    Q, breaks this."""
    rng = np.random.default_rng(902)
    Gs = [rng.standard_normal((36, 20)) for _ in range(3)]
    Es = [rng.standard_normal((36, 20)) * 0.2 for _ in range(3)]
    Q = rng.standard_normal((20, 4))
    dp = oracle.step_data_parallel(Gs, Es, Q, 1.0)
    Mbar = sum(G + E for G, E in zip(Gs, Es)) / 3
    one = oracle.step_matrix(Mbar, 1.0, np.zeros_like(Mbar), Q)
    assert np.abs(dp.D - one.D).max() <= 1e-12 * np.abs(one.D).max()
    assert np.abs(sum(dp.E_next) / 3 - one.E_next).max() <= 1e-12 * np.abs(one.E_next).max()
    for G, E, En in zip(Gs, Es, dp.E_next):
        assert np.abs(G + E - dp.D - En).max() == 0.0


# ------------------------------------------------------------------------------------------
# the Householder route of the orthonormalisation, pinned to the definition of the factor
# ------------------------------------------------------------------------------------------
def test_thin_qr_factor_meets_its_definition():
    """thin_qr_factor(P) must be THE thin-QR factor with a positive R diagonal: orthonormal
    columns, R = F^T P upper triangular with a positive diagonal, and F R = P. These properties
    fix F uniquely for full-rank P, so it must also equal the (separately pinned) CGS2 column
    loop; a dependent panel is rejected instead of completed arbitrarily."""
    rng = np.random.default_rng(31)
    for m, r, cond in ((50, 9, 1.0), (400, 40, 1e3), (64, 64, 30.0)):
        U, _ = np.linalg.qr(rng.standard_normal((m, r)))
        V, _ = np.linalg.qr(rng.standard_normal((r, r)))
        P = (U * np.geomspace(1.0, 1.0 / cond, r)) @ V.T * 3.0
        F = oracle.thin_qr_factor(P)
        R = F.T @ P
        assert np.abs(F.T @ F - np.eye(r)).max() <= 1e-13
        assert np.abs(np.tril(R, -1)).max() <= 1e-13 * np.abs(R).max() * cond
        assert np.diag(R).min() > 0
        assert np.abs(F @ np.triu(R) - P).max() <= 1e-13 * np.abs(P).max()
        assert np.abs(F - oracle.gram_schmidt(P)).max() <= 1e-13 * cond
    Pdep = rng.standard_normal((30, 4))
    Pdep[:, 3] = Pdep[:, 0] - 2.0 * Pdep[:, 1]
    with pytest.raises(ValueError):
        oracle.thin_qr_factor(Pdep)


def test_step_matrix_routes_agree():
    """The step with the Householder route equals the step with the column loop (full rank)."""
    rng = np.random.default_rng(32)
    G = rng.standard_normal((120, 56))
    E = rng.standard_normal((120, 56)) * 0.3
    Q = rng.standard_normal((56, 12))
    a = oracle.step_matrix(G, 0.25, E, Q)
    b = oracle.step_matrix(G, 0.25, E, Q, oracle.thin_qr_factor)
    for x, y in ((a.P, b.P), (a.Q_next, b.Q_next), (a.D, b.D), (a.E_next, b.E_next)):
        assert np.abs(x - y).max() <= 1e-12 * max(1.0, np.abs(y).max())
