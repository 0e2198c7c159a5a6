"""Plain float64 CPU PowerSGD step: the oracle the HIP path is checked against.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg, never by the product path. Nothing here is shared with the HIP library.

Sources (cited by page title and section):
  [card] "Zero-Shot Text-to-Image Generation — 中文验证版" (ai-papers.xuzou.cn reading card of
         the DALL·E paper), sections 瓶颈, 方法适配 and 证据.
  [ko]   Korean summary of the same paper (only-wanna.tistory.com), sections
         "Mixed-Precision Training" and "Distributed Optimization".

What the pages fix:
  * gradients are averaged by all-reducing low-rank factors instead of full gradient matrices
    ([card] 方法适配; [ko] Distributed Optimization: the P·Q factorisation);
  * each GPU compresses its own parameter shard at rank 112 ([card] 方法适配, 证据);
  * an error buffer carries what the factors miss, finite-value checks guard the step, and the
    decompressed gradient is formed with 32-bit products ([card] 证据);
  * non-finite values from mixed-precision backprop are one of the few occasions on which the
    error buffer is zeroed ([ko] Distributed Optimization), and a non-finite step skips the
    update ([card] 方法适配);
  * gains, biases, embeddings and unembeddings are not compressed and stay 32-bit
    ([card] 方法适配; [ko] Distributed Optimization).

Readings taken where the pages are silent:
  * The iteration is one warm-started power (subspace) iteration per step:
        M  = s_b * G + E
        P  = M @ Q
        P  = orthonormalise(P)        (Gram-Schmidt)
        Qn = M.T @ P                  (next warm start)
        D  = P @ Qn.T                 (decompressed gradient)
        En = M - D                    (new error buffer)
  * Orthonormalisation is classical Gram-Schmidt with one re-orthogonalisation sweep (CGS2).
    Its result is the thin-QR factor with a positive R diagonal, so any stable variant gives
    the same P. A column whose residual norm is exactly zero (or non-finite) is set to zero.
  * s_b is the multiplier that turns a stored per-resblock-scaled gradient back into true
    units ([ko] Mixed-Precision Training: scale at block start, unscale at block end).
  * A matrix's flag is set when any element of G or E is non-finite. The step is skipped when
    any matrix flag, any pass-through tensor element or any scale is non-finite. On a skipped
    step every error buffer becomes zero, Q is kept, and no decompressed gradient is produced.

Parity pins (tests/test_oracle_pins.py): Householder QR with a sign fix, hand-derived worked
examples (tests/golden/), the Eckart-Young bound and the truncated SVD, exact recovery of rank-r
matrices, projection identities, brute-force finiteness, scale and permutation invariance.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "as_f64", "gram_schmidt", "modified_gram_schmidt", "nonfinite", "MatrixStep",
    "thin_qr_factor", "step_matrix", "GroupStep", "step_group", "subspace_iteration",
    "DataParallelStep", "step_data_parallel",
]


def as_f64(x) -> np.ndarray:
    """Widen to float64. Exact for float16, float32 (and bf16 values held as float32)."""
    return np.asarray(x, dtype=np.float64)


def gram_schmidt(P, sweeps: int = 2) -> np.ndarray:
    """Classical Gram-Schmidt over the columns of P, with `sweeps` projection sweeps per
    column (2 = CGS2, the re-orthogonalised variant).

    Column j: v = p_j; repeat `sweeps` times { h = Qprev^T v; v = v - Qprev h }; then
    q_j = v / ||v||, or q_j = 0 when ||v|| is zero or not finite.
    """
    P = as_f64(P)
    m, r = P.shape
    out = np.zeros((m, r))
    for j in range(r):
        v = P[:, j].copy()
        prev = out[:, :j]
        for _ in range(sweeps):
            h = prev.T @ v
            v = v - prev @ h
        nrm = float(np.sqrt(v @ v))
        if nrm > 0.0 and np.isfinite(nrm):
            out[:, j] = v / nrm
    return out


def modified_gram_schmidt(P) -> np.ndarray:
    """Modified Gram-Schmidt (each new column is swept against the updated trailing columns).
    Used as an independent cross-check of gram_schmidt on well-conditioned inputs."""
    V = as_f64(P).copy()
    m, r = V.shape
    out = np.zeros((m, r))
    for i in range(r):
        nrm = float(np.sqrt(V[:, i] @ V[:, i]))
        if nrm > 0.0 and np.isfinite(nrm):
            out[:, i] = V[:, i] / nrm
        for j in range(i + 1, r):
            V[:, j] = V[:, j] - (out[:, i] @ V[:, j]) * out[:, i]
    return out


def thin_qr_factor(P) -> np.ndarray:
    """The thin-QR factor of P with a positive R diagonal, from LAPACK's Householder QR with
    the column signs fixed. For P of full column rank this is the same matrix gram_schmidt
    defines (that factor is unique); it is the route for panels too long for the column loop
    to finish in seconds (thousands of rows at ranks in the hundreds). It has no rule for
    dependent columns, so a rank-deficient P is rejected."""
    P = as_f64(P)
    Qf, R = np.linalg.qr(P)
    d = np.diag(R)
    if not np.all(np.isfinite(d)) or np.any(np.abs(d) <= 1e-13 * max(1.0, np.abs(d).max())):
        raise ValueError("thin_qr_factor needs a panel of full column rank; use gram_schmidt")
    return Qf * np.sign(d)[None, :]


def nonfinite(x) -> bool:
    """True when any element of x is +-inf or NaN."""
    return not bool(np.isfinite(as_f64(x)).all())


@dataclasses.dataclass
class MatrixStep:
    M: np.ndarray        # s*G + E
    P_raw: np.ndarray    # M @ Q before orthonormalisation
    P: np.ndarray        # orthonormal factor
    Q_next: np.ndarray   # M^T @ P
    D: np.ndarray        # P @ Q_next^T
    E_next: np.ndarray   # M - D


def step_matrix(G, s: float, E, Q, orthonormalise=None) -> MatrixStep:
    """One PowerSGD step on one gradient matrix (all arithmetic in float64).
    orthonormalise: gram_schmidt (the default) or thin_qr_factor (full-rank panels only)."""
    G, E, Q = as_f64(G), as_f64(E), as_f64(Q)
    M = float(s) * G + E
    P_raw = M @ Q
    P = (orthonormalise or gram_schmidt)(P_raw)
    Q_next = M.T @ P
    D = P @ Q_next.T
    return MatrixStep(M, P_raw, P, Q_next, D, M - D)


@dataclasses.dataclass
class GroupStep:
    flags: List[bool]                    # per matrix: G or E holds a non-finite value
    passthrough_flags: List[bool]        # per pass-through tensor
    scale_flag: bool                     # any scale non-finite
    skip: bool
    E_next: List[np.ndarray]             # zeros on a skipped step
    Q_next: List[np.ndarray]             # unchanged on a skipped step
    D: Optional[List[np.ndarray]]        # None on a skipped step
    P: Optional[List[np.ndarray]]        # None on a skipped step


def step_group(grads: Sequence, errs: Sequence, qs: Sequence, blocks: Sequence[int],
               scales, passthrough: Sequence = ()) -> GroupStep:
    """One step over a group of gradient matrices sharing one skip decision.

    grads/errs/qs: per-matrix G (m x n), E (m x n), Q (n x r); blocks: index into `scales`
    for each matrix; passthrough: uncompressed 32-bit tensors, which only take part in the
    finite check (their reduction is the identity on one GPU).
    """
    scales = as_f64(scales)
    flags = [nonfinite(g) or nonfinite(e) for g, e in zip(grads, errs)]
    pflags = [nonfinite(t) for t in passthrough]
    sflag = nonfinite(scales)
    skip = any(flags) or any(pflags) or sflag
    if skip:
        return GroupStep(flags, pflags, sflag, True,
                         [np.zeros(as_f64(e).shape) for e in errs],
                         [as_f64(q).copy() for q in qs], None, None)
    E_next, Q_next, D, P = [], [], [], []
    for g, e, q, b in zip(grads, errs, qs, blocks):
        st = step_matrix(g, scales[b], e, q)
        E_next.append(st.E_next)
        Q_next.append(st.Q_next)
        D.append(st.D)
        P.append(st.P)
    return GroupStep(flags, pflags, sflag, False, E_next, Q_next, D, P)


@dataclasses.dataclass
class DataParallelStep:
    P: np.ndarray              # orthonormal factor, the same on every rank
    Q_next: np.ndarray         # mean over ranks of M_i^T P
    D: np.ndarray              # P @ Q_next.T, the same on every rank
    E_next: List[np.ndarray]   # per rank: M_i - D


def step_data_parallel(grads: Sequence, errs: Sequence, Q, s: float = 1.0) -> DataParallelStep:
    """One step of one matrix across a data-parallel group of k ranks (float64).

    The pages replace the all-reduce of the gradients by an all-reduce of the low-rank factors
    ([card] 方法适配, 证据). They do not say where the mean is taken; the plainest order that
    keeps P identical on every rank is read here: the raw factors M_i Q are averaged before
    orthonormalisation, the products M_i^T P after it, and each rank keeps its own error
    buffer E_i = M_i - P Q_next^T.
    """
    Ms = [float(s) * as_f64(g) + as_f64(e) for g, e in zip(grads, errs)]
    Q = as_f64(Q)
    k = len(Ms)
    P = gram_schmidt(sum(M @ Q for M in Ms) / k)
    Qn = sum(M.T @ P for M in Ms) / k
    D = P @ Qn.T
    return DataParallelStep(P, Qn, D, [M - D for M in Ms])


def subspace_iteration(M, Q0, iters: int):
    """`iters` rounds of P = orthonormalise(M @ Q); Q = M^T @ P on a fixed M (no error
    feedback). Returns (P, Q, D = P @ Q^T)."""
    M = as_f64(M)
    Q = as_f64(Q0)
    P = None
    for _ in range(iters):
        P = gram_schmidt(M @ Q)
        Q = M.T @ P
    return P, Q, P @ Q.T

