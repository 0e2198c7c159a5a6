"""The optimizer step through the C ABI (psgd_adam_prepare, psgd_decompress_adam,
psgd_adam_update) against the float64 oracle (oracle/adam.py).

Two protocols:
  * exact inputs: matrices whose G and E are zero have D = 0 exactly on both sides, and the
    pass-through tensors take seeded fp32 gradients directly, so the oracle sees exactly the
    GPU's inputs (seeded parameters, moment codes and step count, fresh for every case). The global norm, the
    clipping factor, the step count and every fp32 value then agree to a few float32 units;
    each 16-bit stored code is the oracle's or (at a rounding midpoint within float32 error) a
    neighbour, in at most 1e-3 of the elements;
  * free-running: a one-resblock shard (fp16 gradients, rank 112) and small groups (rank 160
    with bf16 gradients and an in-place matrix; fp32 gradients) take steps with clipping and
    weight decay; the oracle runs its own PowerSGD step (float64) and its own optimizer step
    from the same seeded state. Both moments must agree within the relative Frobenius
    tolerance of the compression (2e-3): their differences come from the decompressed
    gradients, which agree to that bound. So must the applied parameter update, over the
    elements where Adam's step is well conditioned in the gradient (sqrt(m2_hat) > 100 eps);
    where sqrt(m2_hat) is near eps the step depends on digits of D far inside the tolerance,
    and there it is only required to be a valid step (at most 3 lr).
Both protocols end with a skipped step: nothing changes, the step count included, and the
error buffers are zero.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_helpers import REL_TOL, log, rel

pytestmark = pytest.mark.gpu

HP = oracle.AdamHyper(lr=2e-3, beta1=0.9, beta2=0.96, eps=1e-8, weight_decay=0.05)
HP_PASS = oracle.AdamHyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def _f32(hp):
    """The hyperparameters as the ABI holds them (float32), for the oracle."""
    return oracle.AdamHyper(*[float(np.float32(v)) for v in (hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)])


def _decode(t, fmt):
    """Stored values as float64: floating tensors exactly, 16-bit code tensors by format."""
    import torch
    if t.dtype in (torch.float16, torch.bfloat16, torch.float32):
        return t.float().cpu().numpy().astype(np.float64)
    bits = t.cpu().view(torch.int16).numpy().view(np.uint16)
    if fmt == "bf16":
        return oracle.bf16_bits_to_f64(bits)
    return oracle.ue8m8_decode(bits)


def _codes_close(got, want, fmt, what, frac=1e-3):
    """Stored values equal, or neighbouring codes in at most `frac` of the elements."""
    diff = got != want
    if not diff.any():
        return 0.0
    g, w = got[diff], want[diff]
    if fmt == "f16":
        step = np.abs(np.spacing(np.maximum(np.abs(g), np.abs(w)).astype(np.float16)).astype(np.float64))
    elif fmt == "bf16":
        step = np.exp2(np.floor(np.log2(np.maximum(np.abs(g), np.abs(w)))) - 7)
    else:
        step = np.exp2(np.floor(np.log2(np.maximum(np.abs(g), np.abs(w)))) - 8)
    assert np.all(np.abs(g - w) <= step * (1 + 1e-12)), (what, "codes further apart than one step")
    f = float(diff.mean())
    assert f <= frac, (what, f)
    return f


def _update_errors(th, th_prev, st, st_prev, t, hp):
    """Relative Frobenius error of the applied parameter update where the oracle's update is
    well conditioned in the gradient, and the largest update elsewhere (in units of lr).

    Adam's step m1_hat / (sqrt(m2_hat) + eps) is ill conditioned where sqrt(m2_hat) is near
    eps: there a gradient difference far inside the compression tolerance (1e-6 of ||D||)
    moves the step by a large fraction (g / (|g| + eps) at t = 1). Those elements hold no
    unique answer at this tolerance; their updates are only required to be valid steps,
    |step| <= 3 lr. Everywhere sqrt(m2_hat) > 100 eps the update is compared."""
    dg = th - th_prev
    do = st.theta - st_prev.theta
    m2_hat = st.m2 / (1.0 - hp.beta2 ** t)
    ok = np.sqrt(m2_hat) > 100.0 * hp.eps
    err = rel(dg[ok], do[ok]) if ok.any() else 0.0
    rest = float(np.abs(dg[~ok] + hp.lr * hp.weight_decay * th_prev[~ok]).max() / hp.lr) if (~ok).any() else 0.0
    return err, rest, float((~ok).mean())


def _seed_state(shape, seed, param_dtype):
    import torch
    rng = wl.matrix_rng(seed, 0)
    th = rng.standard_normal(shape) * 0.02
    m1 = rng.standard_normal(shape) * 1e-3
    m2 = (rng.standard_normal(shape) * 1e-3) ** 2
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[param_dtype]
    th_t = torch.from_numpy(th.astype(np.float32)).to(tdt).cuda()
    m1_t = torch.from_numpy(oracle.f32_to_bf16_bits(m1.astype(np.float32)).view(np.int16)).cuda()
    m2_t = torch.from_numpy(oracle.ue8m8_encode(m2.astype(np.float32)).view(np.int16)).cuda()
    return th_t, m1_t, m2_t


def _oracle_states(params, m1s, m2s, param_dtype, pass_state):
    st = [oracle.AdamState(_decode(p, param_dtype), _decode(a, "bf16"), _decode(b, "ue8m8"), param_dtype)
          for p, a, b in zip(params, m1s, m2s)]
    for p, a, b, _ in pass_state:
        st.append(oracle.AdamState(_decode(p, "f32"), _decode(a, "f32"), _decode(b, "f32"), "f32", "f32", "f32"))
    return st


def _pass_tensors(seed, sizes, step):
    import torch
    out = []
    for k, n in enumerate(sizes):
        rng = wl.matrix_rng(seed + 17, k)
        p = torch.from_numpy((rng.standard_normal(n) * 0.1).astype(np.float32)).cuda()
        a = torch.from_numpy((rng.standard_normal(n) * 1e-2).astype(np.float32)).cuda()
        b = torch.from_numpy(((rng.standard_normal(n) * 1e-2) ** 2).astype(np.float32)).cuda()
        g = torch.empty(n, dtype=torch.float32, device="cuda")
        out.append([p, a, b, g])
    return out


def _set_pass_grads(pts, seed, step):
    import torch
    for k, t in enumerate(pts):
        rng = wl.matrix_rng(seed + 1000 * (step + 1), k)
        t[3].copy_(torch.from_numpy((rng.standard_normal(t[3].numel()) * (0.5 + k)).astype(np.float32)))


@pytest.mark.parametrize("param_dtype", ["f16", "bf16", "f32"])
def test_exact_inputs_against_oracle(param_dtype):
    """D = 0 matrices plus pass-through tensors: every input of the optimizer is known exactly.
    Each case starts from freshly seeded parameters, moment codes, gradients and step count
    (so no stored value carries an earlier rounding decision into the next comparison); the
    cases alternate clipping on and off, and one carries a NaN pass-through gradient."""
    import torch
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    shapes = [(300, 264), (129, 520)]
    rank = 16
    seed = 9_100_000 + {"f16": 1, "bf16": 2, "f32": 3}[param_dtype]
    grads = [torch.zeros(s, dtype=torch.float16, device="cuda") for s in shapes]
    q0 = [torch.from_numpy(wl.matrix_rng(seed, 50 + i).standard_normal((s[1], rank)).astype(np.float32))
          for i, s in enumerate(shapes)]
    scale = torch.ones(1, dtype=torch.float32, device="cuda")
    group = PowerSGDGroup(grads, [0, 0], scale, rank, q0, None, False)
    st = [_seed_state(s, seed + i, param_dtype) for i, s in enumerate(shapes)]
    params, m1s, m2s = [x[0] for x in st], [x[1] for x in st], [x[2] for x in st]
    group.attach_adam(params, m1s, m2s)
    pts = _pass_tensors(seed, [2 * 3968, 1000, 13], 0)
    for case, (t0, max_norm, skip_now) in enumerate(((0, 5.0, False), (1, 0.0, False), (6, 5.0, False),
                                                    (6, 5.0, True), (99, 1e9, False))):
        cs = seed + 100 * (case + 1)
        for i, s in enumerate(shapes):
            fresh = _seed_state(s, cs + i, param_dtype)
            for dst, src in zip((params[i], m1s[i], m2s[i]), fresh):
                dst.copy_(src)
        for k, p in enumerate(_pass_tensors(cs, [t[3].numel() for t in pts], 0)):
            for dst, src in zip(pts[k][:3], p[:3]):
                dst.copy_(src)
        _set_pass_grads(pts, cs, case)
        if skip_now:
            pts[1][3][7] = float("nan")
        group.adam_step.fill_(t0)
        ost = _oracle_states(params, m1s, m2s, param_dtype, pts)
        before = [(p.clone(), a.clone(), b.clone()) for p, a, b in zip(params, m1s, m2s)]
        before_pass = [[x.clone() for x in p[:3]] for p in pts]
        log(f"adam exact inputs {param_dtype} case {case}: t {t0} -> {t0 + (0 if skip_now else 1)}, "
            f"max_norm {max_norm}, skip {skip_now}")
        skip = group.step_adam(HP, pts, HP_PASS, max_norm, host=True)
        torch.cuda.synchronize()
        assert skip == int(skip_now)
        gr = [np.zeros(s) for s in shapes] + [p[3].cpu().numpy().astype(np.float64) for p in pts]
        ost, t_new, n_or, c_or = oracle.adam_group_step(ost, gr, t0, skip_now, _f32(HP), _f32(HP_PASS),
                                                        n_mats=len(shapes), max_norm=max_norm)
        assert int(group.adam_step.item()) == t_new
        if skip_now:
            for (p0, a0, b0), p, a, b in zip(before, params, m1s, m2s):
                assert torch.equal(p0, p) and torch.equal(a0, a) and torch.equal(b0, b)
            for b4, p in zip(before_pass, pts):
                for x0, x in zip(b4, p[:3]):
                    assert torch.equal(x0, x)
            for e in group.err:
                assert float(e.abs().max()) == 0.0
            continue
        nrm = group.adam_norm.cpu().numpy().astype(np.float64)
        assert abs(nrm[0] - n_or) <= 2e-7 * n_or, (nrm[0], n_or)
        assert abs(nrm[1] - c_or) <= 2e-7 * c_or, (nrm[1], c_or)
        for i in range(len(shapes)):
            th = _decode(params[i], param_dtype)
            if param_dtype == "f32":
                err = np.abs(th - ost[i].theta).max()
                tol = 4e-7 * np.abs(ost[i].theta).max() + 1e-5 * HP.lr
                assert err <= tol, (i, "theta", err, tol)
                f1 = float((th != ost[i].theta).mean())
            else:
                f1 = _codes_close(th, ost[i].theta, param_dtype, ("theta", i))
            f2 = _codes_close(_decode(m1s[i], "bf16"), ost[i].m1, "bf16", ("m1", i))
            f3 = _codes_close(_decode(m2s[i], "ue8m8"), ost[i].m2, "ue8m8", ("m2", i))
            log(f"  matrix {i}: stored values differing theta {f1:.1e} m1 {f2:.1e} m2 {f3:.1e}")
        for k, p in enumerate(pts):
            o = ost[len(shapes) + k]
            for name, got, want in (("theta", p[0], o.theta), ("m1", p[1], o.m1), ("m2", p[2], o.m2)):
                g = got.cpu().numpy().astype(np.float64)
                tol = 4e-7 * np.abs(want).max() + (1e-5 * HP_PASS.lr if name == "theta" else 0.0)
                assert np.abs(g - want).max() <= tol, (k, name, np.abs(g - want).max(), tol)
    group.close()


def test_free_running_shard_against_oracle():
    """One resblock shard (fp16 gradients and parameters, rank 112), three optimizer steps with
    clipping active and weight decay, then a skipped step."""
    import torch
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    w = wl.workload(2)
    seed = 9_200_000
    grads = [torch.from_numpy(wl.gradient_np(w, s, 0)).cuda() for s in w.matrices]
    q0 = [wl.initial_q_np(w, s) for s in w.matrices]
    scale = torch.ones(1, dtype=torch.float32, device="cuda")
    group = PowerSGDGroup(grads, [0] * 4, scale, w.rank, [torch.from_numpy(q) for q in q0], None, False)
    params = []
    for i, s in enumerate(w.matrices):
        rng = wl.matrix_rng(seed, i)
        params.append(torch.from_numpy((rng.standard_normal((s.m, s.n)) * 0.02).astype(np.float16)).cuda())
    m1s = [torch.zeros((s.m, s.n), dtype=torch.int16, device="cuda") for s in w.matrices]
    m2s = [torch.zeros((s.m, s.n), dtype=torch.int16, device="cuda") for s in w.matrices]
    group.attach_adam(params, m1s, m2s)
    pts = _pass_tensors(seed, [2 * 3968], 0)
    ost = _oracle_states(params, m1s, m2s, "f16", pts)
    E_or = [np.zeros((s.m, s.n)) for s in w.matrices]
    Q_or = [q.astype(np.float64) for q in q0]
    t = 0
    max_norm = 20.0
    for step in range(4):
        skip_now = step == 3
        if step:
            for s, g in zip(w.matrices, grads):
                g.copy_(torch.from_numpy(wl.gradient_np(w, s, step)))
        if skip_now:
            grads[2][5, 9] = float("inf")
        _set_pass_grads(pts, seed, step)
        G = [g.float().cpu().numpy() for g in grads]
        th_before = [_decode(p, "f16") for p in params]
        log(f"adam free-running shard step {step}")
        skip = group.step_adam(HP, pts, HP_PASS, max_norm, host=True)
        torch.cuda.synchronize()
        assert skip == int(skip_now)
        gs = oracle.step_group(G, E_or, Q_or, [0] * 4, np.ones(1, np.float32),
                               [p[3].cpu().numpy() for p in pts])
        assert gs.skip == skip_now
        gr = (gs.D if not skip_now else [None] * 4) + [p[3].cpu().numpy().astype(np.float64) for p in pts]
        prev = [oracle.AdamState(s.theta.copy(), s.m1.copy(), s.m2.copy(), s.param_fmt, s.m1_fmt, s.m2_fmt)
                for s in ost]
        ost, t, n_or, c_or = oracle.adam_group_step(ost, gr, t, skip_now, _f32(HP), _f32(HP_PASS),
                                                    n_mats=4, max_norm=max_norm)
        E_or, Q_or = gs.E_next, gs.Q_next
        assert int(group.adam_step.item()) == t
        if skip_now:
            for i in range(4):
                assert np.array_equal(_decode(params[i], "f16"), th_before[i])
            for e in group.err:
                assert float(e.abs().max()) == 0.0
            break
        nrm = group.adam_norm.cpu().numpy().astype(np.float64)
        assert c_or < 1.0, "the step was meant to clip"
        assert abs(nrm[0] - n_or) <= REL_TOL * n_or and abs(nrm[1] - c_or) <= REL_TOL * c_or, (nrm, n_or, c_or)
        worst = {}
        for i, s in enumerate(w.matrices):
            th = _decode(params[i], "f16")
            du, rest, frac = _update_errors(th, th_before[i], ost[i], prev[i], t, _f32(HP))
            r = dict(dtheta=du, m1=rel(_decode(m1s[i], "bf16"), ost[i].m1), m2=rel(_decode(m2s[i], "ue8m8"), ost[i].m2),
                     ill_conditioned=frac, theta_values_differing=float((th != ost[i].theta).mean()))
            for k, v in r.items():
                worst[k] = max(worst.get(k, 0.0), v)
            for k in ("dtheta", "m1", "m2"):
                assert r[k] <= REL_TOL, (step, s.name, k, r[k])
            assert rest <= 3.0, (step, s.name, "update outside the valid range", rest)
        o = ost[4]
        for name, got, want in (("theta", pts[0][0], o.theta), ("m1", pts[0][1], o.m1), ("m2", pts[0][2], o.m2)):
            assert rel(got.cpu().numpy(), want) <= REL_TOL, (step, "pass-through", name)
        log(f"  norm {nrm[0]:.6g} (oracle {n_or:.6g}) clip {nrm[1]:.4g}: "
            + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    group.close()


def _free_running(shapes, gdt, pdt, rank, steps, seed, inplace=(), max_norm=5.0):
    """A small group with optimizer state, `steps` steps against the oracle (free-running), the
    last one skipped through an inf gradient element; returns the group's step counters."""
    import torch
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    grads_np = lambda step: [wl.matrix_rng(seed + step, i).standard_normal(s) *  # noqa: E731
                             np.exp(wl.matrix_rng(seed, 100 + i).uniform(np.log(1e-3), 0.0, size=(s[0], 1)))
                             for i, s in enumerate(shapes)]
    def dev(x):
        t = torch.from_numpy(x.astype(np.float32)).cuda()
        return t.to(tdt[gdt])
    g0 = [dev(x) for x in grads_np(0)]
    scale = torch.tensor([1.0, 0.5], dtype=torch.float32, device="cuda")
    blocks = [i % 2 for i in range(len(shapes))]
    q0 = [wl.matrix_rng(seed, 200 + i).standard_normal((s[1], rank)).astype(np.float32) for i, s in enumerate(shapes)]
    err = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    grads = [None if i in inplace else g0[i] for i in range(len(shapes))]
    for i in inplace:                                   # the error buffer already holds s_b G
        err[i].copy_(g0[i].float() * float(scale[blocks[i]]))
    group = PowerSGDGroup(grads, blocks, scale, rank, [torch.from_numpy(q) for q in q0], err, False)
    params = [torch.from_numpy((wl.matrix_rng(seed, 300 + i).standard_normal(s) * 0.02).astype(np.float32))
              .to(tdt[pdt]).cuda() for i, s in enumerate(shapes)]
    m1s = [torch.zeros(s, dtype=torch.int16, device="cuda") for s in shapes]
    m2s = [torch.zeros(s, dtype=torch.int16, device="cuda") for s in shapes]
    group.attach_adam(params, m1s, m2s)
    ost = _oracle_states(params, m1s, m2s, pdt, [])
    E_or = [np.zeros(s) for s in shapes]
    Q_or = [q.astype(np.float64) for q in q0]
    t = 0
    for step in range(steps):
        skip_now = step == steps - 1
        G = [dev(x) for x in grads_np(step)]
        if skip_now:
            G[0][1, 1] = float("inf")
        Gf = [g.float().cpu().numpy() for g in G]
        for i in range(len(shapes)):
            if i in inplace:
                if step:
                    group.err[i].add_(G[i].float() * float(scale[blocks[i]]))
            else:
                grads[i].copy_(G[i])
        Eo = [np.zeros(s) if i in inplace else E_or[i] for i, s in enumerate(shapes)]
        Go = [(E_or[i] + Gf[i] * float(scale[blocks[i]])) if (i in inplace and step) else
              (Gf[i] * float(scale[blocks[i]]) if i in inplace else Gf[i]) for i in range(len(shapes))]
        sc = np.array([1.0 if i in inplace else float(scale[blocks[i]]) for i in range(len(shapes))])
        th_before = [_decode(p, pdt) for p in params]
        log(f"adam {gdt} grads, {pdt} params, rank {rank}, in-place {sorted(inplace)}: step {step}")
        skip = group.step_adam(HP, [], None, max_norm, host=True)
        torch.cuda.synchronize()
        assert skip == int(skip_now)
        # per-matrix multipliers: the in-place matrices carry M already (multiplier 1, E = 0)
        gs = oracle.step_group(Go, Eo, Q_or, list(range(len(shapes))), sc)
        assert gs.skip == skip_now
        prev = [oracle.AdamState(s.theta.copy(), s.m1.copy(), s.m2.copy(), s.param_fmt) for s in ost]
        ost, t, n_or, c_or = oracle.adam_group_step(ost, gs.D if not skip_now else [None] * len(shapes), t,
                                                    skip_now, _f32(HP), n_mats=len(shapes), max_norm=max_norm)
        E_or, Q_or = gs.E_next, gs.Q_next
        assert int(group.adam_step.item()) == t
        if skip_now:
            for i in range(len(shapes)):
                assert np.array_equal(_decode(params[i], pdt), th_before[i])
            break
        nrm = group.adam_norm.cpu().numpy().astype(np.float64)
        assert abs(nrm[0] - n_or) <= REL_TOL * n_or and abs(nrm[1] - c_or) <= REL_TOL * c_or, (nrm, n_or, c_or)
        for i in range(len(shapes)):
            th = _decode(params[i], pdt)
            du, rest, frac = _update_errors(th, th_before[i], ost[i], prev[i], t, _f32(HP))
            r = dict(dtheta=du, m1=rel(_decode(m1s[i], "bf16"), ost[i].m1), m2=rel(_decode(m2s[i], "ue8m8"), ost[i].m2))
            log(f"  matrix {i}: " + " ".join(f"{k}={v:.2e}" for k, v in r.items())
                + f" ill-conditioned {frac:.1e} (largest step there {rest:.2f} lr)")
            for k, v in r.items():
                assert v <= REL_TOL, (step, i, k, v)
            assert rest <= 3.0, (step, i, "update outside the valid range", rest)
    group.reset_errors()                                 # not a step: the counters stay
    counts = group.counters()
    for e in group.err:
        assert float(e.abs().max()) == 0.0
    group.close()
    return counts


def test_large_rank_bf16_with_inplace_matrix():
    """Rank 160 (the split-once GEMM path and the blocked factorisation), bf16 gradients and
    parameters, one in-place matrix; three steps, the last skipped; step counters (3, 1)."""
    counts = _free_running([(600, 512), (257, 768), (320, 264)], "bf16", "bf16", 160, 3, 9_300_000,
                           inplace=(2,))
    assert counts == (3, 1), counts


def test_fp32_gradients_fp16_params_counters_and_reset():
    """fp32 gradients, fp16 parameters, rank 24; the step counters count every decompression
    and its skips, and psgd_reset_errors is not counted."""
    import torch
    counts = _free_running([(130, 96), (64, 200)], "f32", "f16", 24, 4, 9_400_000)
    assert counts == (4, 1), counts


def test_optimizer_arguments_rejected():
    """Bad optimizer calls return PSGD_EINVAL / PSGD_EDTYPE before anything is launched: calls
    before an attachment, unknown or mismatched parameter formats, hyperparameters outside
    their ranges (beta = 1, negative or infinite lr, NaN eps), missing device words; the
    optimizer state and the step count are untouched."""
    import torch
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    from rank_gradient_compression_powersgd_amd import binding as B
    dev = torch.device("cuda", 0)
    shape, rank = (64, 96), 8
    rng = np.random.default_rng(9_500_000)
    g = torch.from_numpy(wl.to_fp16(rng.standard_normal(shape))).to(dev)
    q0 = [torch.from_numpy(rng.standard_normal((shape[1], rank)).astype(np.float32))]
    scale = torch.ones(1, dtype=torch.float32, device=dev)
    group = PowerSGDGroup([g], [0], scale, rank, q0)
    step = torch.zeros(1, dtype=torch.int32, device=dev)
    norm = torch.zeros(2, dtype=torch.float32, device=dev)
    try:
        with pytest.raises(B.PsgdError) as ei:        # nothing attached yet
            B.psgd_adam_prepare(group.ctx, group.plan, [], 1.0, group.skip, step, norm)
        assert ei.value.status == B.PSGD_EINVAL and "attach" in str(ei.value)
        with pytest.raises(B.PsgdError) as ei:
            B.psgd_decompress_adam(group.ctx, group.plan, scale, group.skip, step, norm, HP)
        assert ei.value.status == B.PSGD_EINVAL
        param = torch.zeros(shape, dtype=torch.float16, device=dev)
        m1 = torch.zeros(shape, dtype=torch.int16, device=dev)
        m2 = torch.zeros(shape, dtype=torch.int16, device=dev)
        opt = [B.make_adam_matrix(param, m1, m2)]
        with pytest.raises(B.PsgdError) as ei:        # unknown parameter format
            B.psgd_adam_attach(group.ctx, group.plan, opt, 9)
        assert ei.value.status == B.PSGD_EDTYPE
        with pytest.raises(B.PsgdError):              # moments of another shape
            B.make_adam_matrix(param, m1[:, :64], m2)
        group.attach_adam([param], [m1], [m2])
        group.compress()
        group.check_finite()
        for bad in (oracle.AdamHyper(beta1=1.0), oracle.AdamHyper(beta2=-0.1), oracle.AdamHyper(lr=-1e-3),
                    oracle.AdamHyper(lr=float("inf")), oracle.AdamHyper(eps=float("nan")),
                    oracle.AdamHyper(weight_decay=float("inf"))):
            with pytest.raises(B.PsgdError) as ei:
                B.psgd_decompress_adam(group.ctx, group.plan, scale, group.skip, group.adam_step,
                                       group.adam_norm, bad)
            assert ei.value.status == B.PSGD_EINVAL, bad
            with pytest.raises(B.PsgdError) as ei:
                B.psgd_adam_update(group.ctx, [], group.skip, group.adam_step, group.adam_norm, bad)
            assert ei.value.status == B.PSGD_EINVAL, bad
        with pytest.raises(B.PsgdError) as ei:        # no device step word
            B.psgd_adam_prepare(group.ctx, group.plan, [], 1.0, group.skip, None, group.adam_norm)
        assert ei.value.status == B.PSGD_EINVAL
        torch.cuda.synchronize()
        assert int(group.adam_step.item()) == 0
        assert int(param.abs().max().item()) == 0 and int(m1.abs().max()) == 0 and int(m2.abs().max()) == 0
    finally:
        group.close()


@pytest.mark.parametrize("seed", range(8))
def test_random_configuration_with_optimizer(seed):
    """Seeded random groups with the fused optimizer: rank on both sides of the 128-column chunk
    (odd ranks among them), one to three ragged matrices, gradient and parameter dtypes, and
    an in-place matrix or none; three steps against the oracle, the last skipped."""
    rng = np.random.default_rng(9_500_000 + seed)
    rank = int(rng.choice([5, 24, 64, 112, 129, 200]))
    shapes = [(int(rng.integers(rank, rank + 400)), 8 * int(rng.integers((rank + 7) // 8, (rank + 7) // 8 + 60)))
              for _ in range(int(rng.integers(1, 4)))]
    gdt = str(rng.choice(["f16", "bf16", "f32"]))
    pdt = str(rng.choice(["f16", "bf16", "f32"]))
    inplace = (int(rng.integers(0, len(shapes))),) if rng.random() < 0.4 else ()
    counts = _free_running(shapes, gdt, pdt, rank, 3, 9_600_000 + 1000 * seed, inplace=inplace)
    assert counts == (3, 1), counts
