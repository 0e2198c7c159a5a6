"""Full-size parity: the 64-resblock d_model=3968 per-GPU shard (256 matrices, 1.51e9
gradient elements) in the launch configuration bench.py times.

The oracle cannot afford every matrix, so sampled matrices (one of each shape, spread over the
depth) are compared one by one; the non-finite flags are checked for all 256 matrices.
Inputs are generated on the device from seeds (workloads.gradient_torch) and copied to the host
for the oracle before the step runs.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_helpers import REL_TOL, ORTH_TOL, log, orth_err, rel

pytestmark = pytest.mark.gpu

SAMPLES = (0, 4 * 17 + 1, 4 * 40 + 2, 4 * 63 + 3)   # rb0.qkv, rb17.attn_out, rb40.mlp_in, rb63.mlp_out


def _build(config, write_out=True):
    import torch
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    w = wl.workload(config)
    dev = torch.device("cuda", 0)
    grads = [wl.gradient_torch(w, s, 0, dev) for s in w.matrices]
    q0 = [wl.initial_q_torch(w, s, dev) for s in w.matrices]
    scale = torch.tensor(wl.scales_np(w), device=dev)
    group = PowerSGDGroup(grads, [s.block for s in w.matrices], scale, w.rank, q0, None, write_out)
    torch.cuda.synchronize()
    return w, grads, group


def _host_flags(grads):
    return np.array([0 if bool(np.isfinite(g.cpu().numpy()).all()) else 1 for g in grads], np.uint8)


def test_full_shard_sampled_against_oracle():
    import torch
    w, grads, group = _build(3)
    scales = wl.scales_np(w)
    pt = [torch.from_numpy(wl.passthrough_np(3, w.n_blocks)).cuda().reshape(-1)]
    E_or = {i: np.zeros((w.matrices[i].m, w.matrices[i].n)) for i in SAMPLES}
    Q_or = {i: group.q[i].cpu().numpy().astype(np.float64) for i in SAMPLES}
    for step in range(3):
        if step:
            for s, g in zip(w.matrices, grads):
                wl.gradient_torch(w, s, step, g.device, out=g)
        G = {i: grads[i].float().cpu().numpy() for i in SAMPLES}
        expect_flags = _host_flags(grads)
        log(f"full shard step {step}: 256 matrices, r=112")
        skip = group.step(pt, host=True)
        torch.cuda.synchronize()
        assert skip == 0
        assert np.array_equal(group.flags.cpu().numpy(), expect_flags)
        for i in SAMPLES:
            s = w.matrices[i]
            st = oracle.step_matrix(G[i], float(scales[s.block]), E_or[i], Q_or[i])
            D = group.out[i].cpu().numpy()
            E = group.err[i].cpu().numpy()
            P = group.p[i].cpu().numpy()
            Q = group.q[i].cpu().numpy()
            r = dict(D=rel(D, st.D), E=rel(E, st.E_next), Q=rel(Q, st.Q_next), P=rel(P, st.P),
                     orth=orth_err(P))
            log(f"  {s.name}: " + " ".join(f"{k}={v:.2e}" for k, v in r.items()))
            for k in ("D", "E", "Q", "P"):
                assert r[k] <= REL_TOL, (step, s.name, k, r[k])
            assert r["orth"] <= ORTH_TOL
            E_or[i], Q_or[i] = st.E_next, st.Q_next
    group.close()


def _device_flags(grads):
    """Brute-force finiteness of every gradient matrix, on the device (torch's isfinite)."""
    import torch
    return np.array([0 if bool(torch.isfinite(g).all()) else 1 for g in grads], np.uint8)


def test_full_underflow_shard_200_steps():
    """Rank 80, Student-t(3) gradients near fp16 underflow over all 64 resblocks: 200 warm steps,
    each non-finite with probability 0.01 (workloads.injection_schedule: seeded, at least two
    forced, the injected value cycling +inf, -inf, NaN into one random element of one random
    matrix), then step 200 with a NaN in a pass-through tensor and step 201 with an inf scale.
    Every step: flags (256 matrices) and skip bit-exact against torch's isfinite on the inputs;
    skipped steps zero every error buffer and keep q. On the steps before, at and after each
    event the injected matrix (or, for the pass-through and scale events, one matrix of each
    shape) is checked against the oracle's step from the state the GPU carried into that step
    (one-step protocol: warm-started error feedback amplifies rounding differences over 200
    steps, so free-running trajectories cannot be compared this far)."""
    import torch
    w, grads, group = _build(4, write_out=True)
    scales = wl.scales_np(w)
    pt = torch.from_numpy(wl.passthrough_np(4, w.n_blocks)).cuda().reshape(-1)
    events = wl.injection_schedule(w, 200)
    sched = {e.step: e for e in events}
    steps = max(sched) + 1
    assert steps == 202 and sched[200].kind == "passthrough" and sched[201].kind == "scale"
    assert sum(e.kind == "grad" for e in events) >= 2
    checked = set()
    for t in sched:
        checked.update({t - 1, t, t + 1})
    log(f"underflow shard: {steps} steps, events at {sorted(sched)}")
    n_skip = 0
    for step in range(steps):
        for s, g in zip(w.matrices, grads):
            wl.gradient_torch(w, s, step, g.device, out=g)
        ev = sched.get(step)
        ptx = pt
        if ev and ev.kind == "grad":
            grads[ev.matrix][ev.row, ev.col] = ev.value
        if ev and ev.kind == "passthrough":
            ptx = pt.clone()
            ptx[ev.row] = ev.value
        if ev and ev.kind == "scale":
            group.scale[ev.block] = ev.value
        sample = []
        if step in checked:
            near = [e for e in (sched.get(step), sched.get(step - 1), sched.get(step + 1)) if e]
            sample = sorted({e.matrix for e in near if e.kind == "grad"}
                            | ({0, 69, 162, 255} if any(e.kind != "grad" for e in near) else set()))
            host = {i: (grads[i].float().cpu().numpy(), group.err[i].cpu().numpy(), group.q[i].cpu().numpy()) for i in sample}
        expect_flags = _device_flags(grads)
        expect_skip = int(expect_flags.any() or not bool(torch.isfinite(ptx).all())
                          or not bool(torch.isfinite(group.scale).all()))
        q_before = {i: group.q[i].clone() for i in (sample or [0])}
        skip = group.step([ptx], host=True)
        torch.cuda.synchronize()
        assert np.array_equal(group.flags.cpu().numpy(), expect_flags), step
        assert skip == expect_skip, step
        if ev:
            assert skip == 1, (step, ev)
        n_skip += skip
        if skip:
            for e in group.err:
                assert float(e.abs().max()) == 0.0
            for i, qb in q_before.items():
                assert torch.equal(qb, group.q[i])
        elif sample:
            for i in sample:
                G, E, Q = host[i]
                st = oracle.step_matrix(G, float(group.scale[w.matrices[i].block]), E, Q)
                P = group.p[i].cpu().numpy()
                r = dict(D=rel(group.out[i].cpu().numpy(), st.D), E=rel(group.err[i].cpu().numpy(), st.E_next),
                         Q=rel(group.q[i].cpu().numpy(), st.Q_next), orth=orth_err(P))
                log(f"  step {step} {w.matrices[i].name}: " + " ".join(f"{k}={v:.2e}" for k, v in r.items()))
                for k in ("D", "E", "Q"):
                    assert r[k] <= REL_TOL, (step, w.matrices[i].name, k, r[k])
                assert r["orth"] <= ORTH_TOL
        if ev and ev.kind == "scale":
            group.scale[ev.block] = float(scales[ev.block])
    assert n_skip == len(sched)
    group.close()


def test_unsharded_rank896():
    """The unsharded resblock (3968x11904, 3968x3968, 3968x15872, 15872x3968 bf16, planted rank-64
    component at 10x energy) at rank 896 over 5 warm-started steps. Every matrix is compared
    with its own free-running float64 oracle chain at every step (D, E, q_next and P within the
    relative Frobenius tolerance, P orthonormal). The panels have full column rank, so the
    oracle orthonormalises them with LAPACK's Householder QR (sign-fixed thin-QR factor), which
    finishes in seconds where the column loop takes minutes. The properties that hold at any
    size are checked as well: E + D = M element by element and P^T E = 0."""
    import torch
    w, grads, group = _build(5)
    E_or = [np.zeros((s.m, s.n)) for s in w.matrices]
    Q_or = [q.cpu().numpy().astype(np.float64) for q in group.q]
    for step in range(5):
        if step:
            for s, g in zip(w.matrices, grads):
                wl.gradient_torch(w, s, step, g.device, out=g)
        Gs = [g.float().cpu().numpy() for g in grads]
        Es = [e.cpu().numpy() for e in group.err]
        log(f"unsharded rank 896 step {step}")
        skip = group.step([], host=True)
        torch.cuda.synchronize()
        assert skip == 0
        for i, s in enumerate(w.matrices):
            P = group.p[i].cpu().numpy().astype(np.float64)
            E = group.err[i].cpu().numpy().astype(np.float64)
            D = group.out[i].cpu().numpy().astype(np.float64)
            Q = group.q[i].cpu().numpy().astype(np.float64)
            M = Gs[i].astype(np.float64) + Es[i]
            ident = float(np.abs(E + D - M).max() / np.abs(M).max())
            pe = float(np.linalg.norm(P.T @ E) / np.linalg.norm(E))
            del M
            st = oracle.step_matrix(Gs[i], 1.0, E_or[i], Q_or[i], oracle.thin_qr_factor)
            r_ = dict(D=rel(D, st.D), E=rel(E, st.E_next), Q=rel(Q, st.Q_next), P=rel(P, st.P),
                      orth=orth_err(P), ident=ident, PtE=pe)
            log(f"  {s.name}: " + " ".join(f"{k}={v:.2e}" for k, v in r_.items()))
            for k in ("D", "E", "Q", "P"):
                assert r_[k] <= REL_TOL, (step, s.name, k, r_[k])
            assert r_["orth"] <= ORTH_TOL
            assert ident <= 2.0 ** -20
            assert pe <= REL_TOL
            E_or[i], Q_or[i] = st.E_next, st.Q_next
            del st, P, E, D, Q
    group.close()


@pytest.mark.parametrize("rank", [112, 256])
def test_largest_matrix_at_the_buffer_limit(rank):
    """One fp16 gradient matrix whose error buffer and decompressed output come within 3% of the
    2 GiB buffer-range limit (16000 x 32760: 2.097e9 bytes of fp32), at rank 112 (the streaming
    products) and rank 256 (M split once, the GEMM path, and the blocked factorisation), one
    step from a seeded error buffer and warm start, against the float64 oracle: D, E, q_next
    and P within the relative Frobenius tolerance, P orthonormal, E + D = M. Every byte offset
    of the kernels stays below 2^32 here; a 32-bit overflow in any of them would show."""
    import torch
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    m, n = 16000, 32760
    assert m * n * 4 < 2 ** 31 and m * n * 4 > 0.97 * 2 ** 31
    rng = np.random.default_rng(9_600_000 + rank)
    dev = torch.device("cuda", 0)
    x = rng.standard_normal((m, n), dtype=np.float32)
    x *= np.exp(rng.uniform(-3.0, 0.0, size=(m, 1))).astype(np.float32)
    G16 = x.astype(np.float16)
    del x
    E0 = (rng.standard_normal((m, n), dtype=np.float32) * np.float32(0.05))
    Q0 = rng.standard_normal((n, rank), dtype=np.float32)
    log(f"largest matrix {m}x{n} rank {rank}: inputs generated")
    g = torch.from_numpy(G16).to(dev)
    e = torch.from_numpy(E0).to(dev)
    group = PowerSGDGroup([g], [0], torch.ones(1, device=dev), rank, [torch.from_numpy(Q0)], [e])
    skip = group.step([], host=True)
    torch.cuda.synchronize()
    assert skip == 0
    P = group.p[0].cpu().numpy().astype(np.float64)
    E = group.err[0].cpu().numpy()
    D = group.out[0].cpu().numpy()
    Q = group.q[0].cpu().numpy().astype(np.float64)
    group.close()
    del g, e, group
    torch.cuda.empty_cache()
    log("  GPU step done; oracle step")
    G = G16.astype(np.float32)
    del G16
    st = oracle.step_matrix(G, 1.0, E0, Q0, oracle.thin_qr_factor)
    r_ = dict(D=rel(D, st.D), E=rel(E, st.E_next), Q=rel(Q, st.Q_next), P=rel(P, st.P), orth=orth_err(P))
    log(f"  rank {rank}: " + " ".join(f"{k}={v:.2e}" for k, v in r_.items()))
    for k in ("D", "E", "Q", "P"):
        assert r_[k] <= REL_TOL, (rank, k, r_[k])
    assert r_["orth"] <= ORTH_TOL
    del st
    # E + D = M, row block by row block (M in fp64 would take another 4 GB at once)
    worst, mmax = 0.0, 0.0
    for r0 in range(0, m, 2000):
        M = G[r0:r0 + 2000].astype(np.float64) + E0[r0:r0 + 2000]
        worst = max(worst, float(np.abs(E[r0:r0 + 2000].astype(np.float64) + D[r0:r0 + 2000] - M).max()))
        mmax = max(mmax, float(np.abs(M).max()))
    assert worst <= 2.0 ** -20 * mmax, (worst, mmax)
