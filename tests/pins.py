"""Checks that pin the oracle to facts other than itself.

Each check takes an implementation object exposing `step_matrix`, `gram_schmidt`,
`subspace_iteration` and `step_group` (the oracle module, or a deliberately broken copy of it
in the mutation test) and raises AssertionError when the implementation disagrees with:
  * hand-derived worked examples (tests/golden/),
  * LAPACK's Householder QR with its signs normalised (a different algorithm that yields the
    same thin-QR factor),
  * numpy's SVD (Eckart-Young bound and the truncated SVD),
  * closed forms: exact recovery of a rank-r matrix, the projection identities of the step,
  * brute-force element-by-element finiteness,
  * exact power-of-two scale invariance and permutation invariance.
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------------------
# fixture parsing
# --------------------------------------------------------------------------------------
def _mat(text):
    return np.array([[float(v) for v in row.split(",")] for row in text.split(";")])


def _col(text, div):
    v = np.array([float(x) for x in text.split(";")])
    return (v / math.sqrt(float(div)))[:, None]


def load_step_cases():
    cases = []
    with open(os.path.join(GOLDEN, "step_worked_r1.txt")) as f:
        for line in f:
            if not line.startswith("case "):
                continue
            tok = line.split()
            d = {"name": tok[1]}
            i = 2
            while i < len(tok):
                key = tok[i]
                if key in ("P", "Qn"):
                    d[key] = _col(tok[i + 1], tok[i + 2][1:])
                    i += 3
                elif key == "s":
                    d[key] = float(tok[i + 1])
                    i += 2
                elif key == "Q":
                    d[key] = np.array([float(x) for x in tok[i + 1].split(";")])[:, None]
                    i += 2
                else:
                    d[key] = _mat(tok[i + 1])
                    i += 2
            cases.append(d)
    return cases


def load_gs_case():
    P, Q, R = [], [], []
    scale = None
    with open(os.path.join(GOLDEN, "gs_worked_3x2.txt")) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            vals = [float(x) for x in t[1:]]
            if t[0] == "P":
                P.append(vals)
            elif t[0] == "Q":
                Q.append(vals)
            elif t[0] == "R":
                R.append(vals)
            elif t[0] == "QCOLSCALE":
                scale = np.sqrt(np.array(vals))
    Q = np.array(Q) / scale[None, :]
    R = np.array(R)
    R[1, 1] = math.sqrt(R[1, 1])
    return np.array(P), Q, R


# --------------------------------------------------------------------------------------
# checks
# --------------------------------------------------------------------------------------
def householder_qfactor(P):
    """LAPACK Householder thin QR with the signs fixed so that diag(R) >= 0."""
    q, r = np.linalg.qr(np.asarray(P, dtype=np.float64))
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def check_gs_worked_example(impl):
    P, Q, R = load_gs_case()
    got = impl.gram_schmidt(P)
    assert np.allclose(got, Q, rtol=0, atol=1e-14), (got, Q)
    assert np.allclose(got.T @ P, R, rtol=0, atol=1e-13)


def check_gs_vs_householder(impl, seed=11):
    rng = np.random.default_rng(seed)
    for m, r, cond in ((40, 7, 1.0), (300, 16, 1e3), (513, 33, 30.0), (64, 64, 10.0)):
        U, _ = np.linalg.qr(rng.standard_normal((m, r)))
        V, _ = np.linalg.qr(rng.standard_normal((r, r)))
        sv = np.geomspace(1.0, 1.0 / cond, r)
        P = (U * sv) @ V.T * 7.0
        got = impl.gram_schmidt(P)
        ref = householder_qfactor(P)
        err = np.abs(got - ref).max()
        assert err <= 1e-13 * max(1.0, cond), (m, r, cond, err)
        orth = np.abs(got.T @ got - np.eye(r)).max()
        assert orth <= 1e-13, (m, r, cond, orth)


def check_step_worked_examples(impl):
    for c in load_step_cases():
        st = impl.step_matrix(c["G"], c["s"], c["E"], c["Q"])
        for key, got in (("P", st.P), ("Qn", st.Q_next), ("D", st.D), ("En", st.E_next)):
            assert got.shape == c[key].shape, (c["name"], key, got.shape)
            assert np.allclose(got, c[key], rtol=0, atol=1e-14), (c["name"], key, got, c[key])


def check_exact_rank_recovery(impl, seed=1001):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((256, 4))
    B = rng.standard_normal((4, 128))
    M = A @ B
    Q0 = rng.standard_normal((128, 4))
    st = impl.step_matrix(M, 1.0, np.zeros_like(M), Q0)
    rel = np.linalg.norm(st.E_next) / np.linalg.norm(M)
    assert rel <= 1e-12, rel
    # Non-square the other way round and with a non-zero error buffer carried in.
    A = rng.standard_normal((90, 3))
    B = rng.standard_normal((3, 200))
    E = A @ B * 0.25
    G = A @ B * 1.5
    st = impl.step_matrix(G, 0.5, E, rng.standard_normal((200, 3)))
    M = 0.5 * G + E
    assert np.linalg.norm(st.E_next) / np.linalg.norm(M) <= 1e-12


def check_projection_identities(impl, seed=5):
    rng = np.random.default_rng(seed)
    m, n, r = 120, 75, 9
    G = rng.standard_normal((m, n)) * np.exp(rng.uniform(-4, 0, size=(m, 1)))
    E = rng.standard_normal((m, n)) * 0.1
    Q = rng.standard_normal((n, r))
    st = impl.step_matrix(G, 0.75, E, Q)
    M = 0.75 * G + E
    nM = np.linalg.norm(M)
    # E_new is orthogonal to span(P); D is the projection of M onto span(P).
    assert np.abs(st.P.T @ st.E_next).max() <= 1e-12 * nM
    assert np.abs(st.D - st.P @ (st.P.T @ M)).max() <= 1e-12 * nM
    assert np.abs(st.D + st.E_next - M).max() <= 1e-13 * np.abs(M).max()
    # span(P) is span(M Q): the residual of M Q after projecting onto P vanishes.
    MQ = M @ Q
    assert np.abs(MQ - st.P @ (st.P.T @ MQ)).max() <= 1e-11 * np.abs(MQ).max()
    # P has orthonormal columns and the triangular factor has a positive diagonal.
    assert np.abs(st.P.T @ st.P - np.eye(r)).max() <= 1e-13
    R = st.P.T @ MQ
    assert np.all(np.diag(R) > 0)
    assert np.abs(np.tril(R, -1)).max() <= 1e-11 * np.abs(R).max()


def check_svd_bounds(impl, G, Q0):
    """Subspace iteration on the tiny 256x128 workload against numpy's SVD."""
    M = np.asarray(G, dtype=np.float64)
    sv = np.linalg.svd(M, compute_uv=False)
    r = Q0.shape[1]
    floor = math.sqrt(float(np.sum(sv[r:] ** 2)))
    errs = {}
    for iters in (1, 20):
        _, _, D = impl.subspace_iteration(M, Q0, iters)
        err = float(np.linalg.norm(M - D))
        assert err >= floor * (1 - 1e-12), (iters, err, floor)
        errs[iters] = err / floor - 1.0
    assert errs[20] <= errs[1]
    assert errs[20] <= 5e-3, errs
    return errs


def check_designed_spectrum(impl, seed=77):
    """sigma_4 / sigma_5 = 2: 20 iterations reach the truncated SVD to round-off."""
    rng = np.random.default_rng(seed)
    m, n, r = 256, 128, 4
    U, _ = np.linalg.qr(rng.standard_normal((m, n)))
    V, _ = np.linalg.qr(rng.standard_normal((n, n)))
    sv = np.concatenate([[10.0, 8.0, 6.0, 4.0], 2.0 * np.geomspace(1.0, 0.01, n - 4)])
    M = (U * sv) @ V.T
    Mr = (U[:, :r] * sv[:r]) @ V[:, :r].T
    _, _, D = impl.subspace_iteration(M, rng.standard_normal((n, r)), 20)
    assert np.linalg.norm(D - Mr) / np.linalg.norm(Mr) <= 1e-10
    floor = math.sqrt(float(np.sum(sv[r:] ** 2)))
    assert abs(np.linalg.norm(M - D) / floor - 1.0) <= 1e-12


def check_nonfinite_bruteforce(impl, seed=3):
    rng = np.random.default_rng(seed)
    shapes = ((3, 2), (2, 5))
    base_g = [rng.standard_normal(s) for s in shapes]
    base_e = [rng.standard_normal(s) for s in shapes]
    qs = [rng.standard_normal((s[1], 1)) for s in shapes]
    scales = np.array([1.0, 0.5])
    blocks = [0, 1]
    bad_values = (math.inf, -math.inf, math.nan)
    for which in ("G", "E"):
        for mi, s in enumerate(shapes):
            for i in range(s[0]):
                for j in range(s[1]):
                    val = bad_values[(i + j + mi) % 3]
                    gs = [g.copy() for g in base_g]
                    es = [e.copy() for e in base_e]
                    (gs if which == "G" else es)[mi][i, j] = val
                    out = impl.step_group(gs, es, qs, blocks, scales)
                    expect = []
                    for g, e in zip(gs, es):
                        bad = False
                        for x in list(g.ravel()) + list(e.ravel()):
                            bad = bad or not math.isfinite(float(x))
                        expect.append(bad)
                    assert out.flags == expect, (which, mi, i, j, out.flags)
                    assert out.skip
    out = impl.step_group(base_g, base_e, qs, blocks, scales)
    assert out.flags == [False, False] and not out.skip


def check_skip_semantics(impl, seed=4):
    rng = np.random.default_rng(seed)
    gs = [rng.standard_normal((6, 4)), rng.standard_normal((5, 7))]
    es = [rng.standard_normal((6, 4)), rng.standard_normal((5, 7))]
    qs = [rng.standard_normal((4, 2)), rng.standard_normal((7, 2))]
    blocks = [0, 0]
    ok = impl.step_group(gs, es, qs, blocks, np.array([1.0]), [np.ones(5)])
    assert not ok.skip and ok.D is not None
    cases = [
        ("grad", dict(grads=[gs[0], np.where(np.arange(35).reshape(5, 7) == 3, np.nan, gs[1])])),
        ("pass", dict(passthrough=[np.array([0.0, math.inf])])),
        ("scale", dict(scales=np.array([math.nan]))),
    ]
    for name, kw in cases:
        args = dict(grads=gs, errs=es, qs=qs, blocks=blocks, scales=np.array([1.0]),
                    passthrough=[np.ones(5)])
        args.update(kw)
        out = impl.step_group(**args)
        assert out.skip, name
        assert out.D is None
        for e in out.E_next:
            assert np.all(e == 0.0)
        for q_new, q_old in zip(out.Q_next, qs):
            assert np.array_equal(q_new, q_old)
    assert impl.step_group(gs, es, qs, blocks, np.array([1.0]),
                           [np.array([math.inf])]).passthrough_flags == [True]


def check_scale_invariance(impl, seed=6):
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((50, 30))
    E = rng.standard_normal((50, 30)) * 0.3
    Q = rng.standard_normal((30, 5))
    a = impl.step_matrix(G, 0.75, E, Q)
    for k in (-20, 7):
        f = 2.0 ** k
        b = impl.step_matrix(G * f, 0.75, E * f, Q)
        assert np.array_equal(a.P, b.P), k
        assert np.array_equal(a.D * f, b.D), k
        assert np.array_equal(a.E_next * f, b.E_next), k
        assert np.array_equal(a.Q_next * f, b.Q_next), k


def check_permutation_invariance(impl, seed=8):
    rng = np.random.default_rng(seed)
    shapes = ((9, 4), (3, 11), (7, 7))
    gs = [rng.standard_normal(s) for s in shapes]
    es = [rng.standard_normal(s) * 0.1 for s in shapes]
    qs = [rng.standard_normal((s[1], 2)) for s in shapes]
    blocks = [0, 1, 1]
    scales = np.array([1.0, 0.25])
    a = impl.step_group(gs, es, qs, blocks, scales)
    perm = [2, 0, 1]
    b = impl.step_group([gs[i] for i in perm], [es[i] for i in perm], [qs[i] for i in perm],
                        [blocks[i] for i in perm], scales)
    for k, i in enumerate(perm):
        assert np.array_equal(a.D[i], b.D[k])
        assert np.array_equal(a.E_next[i], b.E_next[k])
        assert np.array_equal(a.Q_next[i], b.Q_next[k])


ALL_CHECKS = (
    check_gs_worked_example, check_gs_vs_householder, check_step_worked_examples,
    check_exact_rank_recovery, check_projection_identities, check_designed_spectrum,
    check_nonfinite_bruteforce, check_skip_semantics, check_scale_invariance,
    check_permutation_invariance,
)
