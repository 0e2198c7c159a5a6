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
    """Rank 80, Student-t(3) gradients near fp16 underflow over all 64 resblocks, 200 warm steps.
    Each step is non-finite with probability 0.01 (seeded; two forced), the injected value
    cycling +inf, -inf, NaN into one random element of one random matrix; one extra step has a
    NaN in a pass-through tensor and one an inf scale. Every step: flags (256 matrices) and skip
    bit-exact; skipped steps zero every error buffer and keep q. On the steps before, at and
    after each injection the injected matrix (or, for the pass-through and scale events, one of
    each shape) is checked against the oracle's step from the GPU's own E and q (one-step
    protocol)."""
    import torch
    w, grads, group = _build(4, write_out=True)
    scales = wl.scales_np(w)
    pt = torch.from_numpy(wl.passthrough_np(4, w.n_blocks)).cuda().reshape(-1)
    rng = np.random.default_rng(4_000_200)
    steps = 200
    inject = [t for t in range(steps) if rng.random() < 0.01]
    for forced in (50, 120):
        if len(inject) < 2 and forced not in inject:
            inject.append(forced)
    values = (np.inf, -np.inf, np.nan)
    sched = {t: ("grad", int(rng.integers(len(w.matrices))), k) for k, t in enumerate(sorted(inject))}
    sched[150] = ("pass", 0, 0)
    sched[170] = ("scale", 13, 0)
    checked = set()
    for t in sched:
        checked.update({t - 1, t, t + 1})
    log(f"underflow shard: 200 steps, events at {sorted(sched)}")
    n_skip = 0
    for step in range(steps):
        for s, g in zip(w.matrices, grads):
            wl.gradient_torch(w, s, step, g.device, out=g)
        ev = sched.get(step)
        ptx = pt
        if ev and ev[0] == "grad":
            s = w.matrices[ev[1]]
            r, c = int(rng.integers(s.m)), int(rng.integers(s.n))
            grads[ev[1]][r, c] = float(values[ev[2] % 3])
        if ev and ev[0] == "pass":
            ptx = pt.clone()
            ptx[int(rng.integers(ptx.numel()))] = float("nan")
        if ev and ev[0] == "scale":
            group.scale[ev[1]] = float("inf")
        sample = []
        if step in checked:
            near = [e for e in (sched.get(step), sched.get(step - 1), sched.get(step + 1)) if e]
            sample = sorted({e[1] for e in near if e[0] == "grad"} | ({0, 69, 162, 255} if any(e[0] != "grad" for e in near) else set()))
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
        if ev and ev[0] == "scale":
            group.scale[ev[1]] = float(scales[ev[1]])
    assert n_skip == len(sched)
    group.close()


def test_unsharded_rank896():
    """The unsharded resblock (3968x11904, 3968x3968, 3968x15872, 15872x3968 bf16, planted rank-64
    component at 10x energy) at rank 896 over 5 warm-started steps. The 3968x3968 matrix is
    compared with the oracle at every step; for all four matrices the properties that hold at
    any size are checked: orthonormal P, E + D = M element by element, P^T E = 0, q_next =
    M^T P on sampled columns."""
    import torch
    w, grads, group = _build(5)
    r = w.rank
    PROJ = 1
    E_or = np.zeros((w.matrices[PROJ].m, w.matrices[PROJ].n))
    Q_or = group.q[PROJ].cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(5)
    for step in range(5):
        if step:
            for s, g in zip(w.matrices, grads):
                wl.gradient_torch(w, s, step, g.device, out=g)
        Gs = [g.float().cpu().numpy().astype(np.float64) for g in grads]
        Es = [e.cpu().numpy().astype(np.float64) for e in group.err]
        log(f"unsharded rank 896 step {step}")
        skip = group.step([], host=True)
        torch.cuda.synchronize()
        assert skip == 0
        for i, s in enumerate(w.matrices):
            M = Gs[i] + Es[i]
            P = group.p[i].cpu().numpy().astype(np.float64)
            E = group.err[i].cpu().numpy().astype(np.float64)
            D = group.out[i].cpu().numpy().astype(np.float64)
            Q = group.q[i].cpu().numpy().astype(np.float64)
            oe = orth_err(P)
            ident = float(np.abs(E + D - M).max() / np.abs(M).max())
            pe = float(np.linalg.norm(P.T @ E) / np.linalg.norm(E))
            cols = rng.choice(r, size=8, replace=False)
            qs = rel(Q[:, cols], M.T @ P[:, cols])
            log(f"  {s.name}: orth={oe:.2e} |E+D-M|/|M|max={ident:.2e} |P^T E|/|E|={pe:.2e} q_next={qs:.2e}")
            assert oe <= ORTH_TOL
            assert ident <= 2.0 ** -20
            assert pe <= REL_TOL
            assert qs <= REL_TOL
        st = oracle.step_matrix(Gs[PROJ], 1.0, E_or, Q_or)
        r_ = dict(D=rel(group.out[PROJ].cpu().numpy(), st.D), E=rel(group.err[PROJ].cpu().numpy(), st.E_next),
                  Q=rel(group.q[PROJ].cpu().numpy(), st.Q_next), P=rel(group.p[PROJ].cpu().numpy(), st.P))
        log("  oracle proj: " + " ".join(f"{k}={v:.2e}" for k, v in r_.items()))
        for k in ("D", "E", "Q", "P"):
            assert r_[k] <= REL_TOL, (step, k, r_[k])
        E_or, Q_or = st.E_next, st.Q_next
    group.close()
