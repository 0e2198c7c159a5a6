"""GPU parity: the HIP path through the C ABI against the float64 oracle on the same inputs.

Every input is seeded and synthetic (workloads/). The oracle never sees a value produced by
the HIP path: it starts from the same generated state and evolves its own state.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_helpers import Case, compare_step, log, orth_err, rel, REL_TOL, ORTH_TOL

pytestmark = pytest.mark.gpu


def _shard_case(config, n_blocks, err_warm=False, write_out=True, rank=None):
    w = wl.workload(config, n_blocks) if config in (3, 4) else wl.workload(config)
    specs = w.matrices
    r = rank or w.rank
    q0 = [wl.initial_q_np(w, s, r) for s in specs]
    err0 = [wl.warm_error_np(w, s) for s in specs] if err_warm else None
    case = Case([(s.m, s.n) for s in specs], [s.block for s in specs], w.dtype, r,
                wl.scales_np(w), q0, err0, write_out)
    return w, specs, case


# ------------------------------------------------------------------------------------------
# tiny 256x128 fp32 workload at rank 4
# ------------------------------------------------------------------------------------------
def test_tiny_single_step_and_exact_rank():
    w = wl.workload(1)
    spec = w.matrices[0]
    G = wl.gradient_np(w, spec, 0)
    Q0 = wl.initial_q_np(w, spec)
    log("tiny 256x128 fp32 r=4: one step")
    case = Case([(256, 128)], [0], "f32", 4, np.ones(1, np.float32), [Q0])
    case.set_grads([G])
    assert case.gpu_step() == 0
    compare_step(case.fetch(), case.oracle_step(), "tiny step 0")
    case.close()

    log("tiny exact rank-4 matrix recovered in one step")
    M = wl.exact_rank_np(256, 128, 4, seed=wl.step_seed(1, 0)).astype(np.float32)
    case = Case([(256, 128)], [0], "f32", 4, np.ones(1, np.float32), [Q0])
    case.set_grads([M])
    case.gpu_step()
    res = case.fetch()
    st = case.oracle_step()
    compare_step(res, st, "exact rank 4", exact_rank=True)
    assert np.linalg.norm(res["E"][0]) / np.linalg.norm(M) <= 1e-5
    case.close()


def test_tiny_subspace_iteration_against_svd():
    """Error buffer reset to zero before every step: the steps are subspace iterations on a
    fixed matrix. After 1 and 20 iterations the error is bounded below by Eckart-Young and the
    20-iteration excess is at most 5e-3; both match the oracle's iterations."""
    import torch
    w = wl.workload(1)
    spec = w.matrices[0]
    G = wl.gradient_np(w, spec, 0)
    Q0 = wl.initial_q_np(w, spec)
    M = G.astype(np.float64)
    sv = np.linalg.svd(M, compute_uv=False)
    floor = math.sqrt(float(np.sum(sv[4:] ** 2)))
    case = Case([(256, 128)], [0], "f32", 4, np.ones(1, np.float32), [Q0])
    case.set_grads([G])
    for it in range(1, 21):
        case.group.err[0].zero_()
        case.gpu_step()
        if it in (1, 20):
            D = case.fetch()["D"][0]
            _, _, Dor = oracle.subspace_iteration(M, Q0, it)
            err = float(np.linalg.norm(M - D))
            log(f"  iters={it}: |M-D|/floor - 1 = {err / floor - 1:.3e}, rel to oracle {rel(D, Dor):.2e}")
            assert err >= floor * (1 - 1e-6)
            assert rel(D, Dor) <= REL_TOL
            if it == 20:
                assert err / floor - 1 <= 5e-3
    case.close()


# ------------------------------------------------------------------------------------------
# one resblock shard (fp16, rank 112)
# ------------------------------------------------------------------------------------------
def test_shard_cold_start_one_step():
    w, specs, case = _shard_case(2, None)
    log("resblock shard fp16 r=112, E0 = 0, one step")
    case.set_grads([wl.gradient_np(w, s, 0) for s in specs])
    assert case.gpu_step() == 0
    res = case.fetch()
    assert not res["flags"].any()
    compare_step(res, case.oracle_step(), "shard cold")
    case.close()


def test_shard_warm_state_one_step():
    w, specs, case = _shard_case(2, None, err_warm=True)
    log("resblock shard fp16 r=112, generated warm E0, one step")
    case.set_grads([wl.gradient_np(w, s, 3) for s in specs])
    case.gpu_step()
    compare_step(case.fetch(), case.oracle_step(), "shard warm")
    case.close()


def test_shard_free_running_ten_steps():
    w, specs, case = _shard_case(2, None)
    log("resblock shard fp16 r=112, 10 warm-started steps, independent trajectories")
    for t in range(10):
        case.set_grads([wl.gradient_np(w, s, t) for s in specs])
        case.gpu_step()
        compare_step(case.fetch(), case.oracle_step(), f"shard step {t}")
    case.close()


def test_shard_without_output_buffer():
    w, specs, case = _shard_case(2, None, write_out=False)
    case.set_grads([wl.gradient_np(w, s, 0) for s in specs])
    case.gpu_step()
    res = case.fetch()
    st = case.oracle_step()
    for i in range(len(specs)):
        assert rel(res["E"][i], st.E_next[i]) <= REL_TOL
    case.close()


# ------------------------------------------------------------------------------------------
# ragged shapes, padded leading dimensions, other ranks and dtypes
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,rank", [("f16", 20), ("bf16", 37), ("f32", 128), ("f16", 1)])
def test_ragged_shapes(dtype, rank):
    shapes = [(1000, 200), (37, 1048), (513, 264), (300, 128), (129, 136)]
    shapes = [(m, n) for m, n in shapes if min(m, n) >= rank]
    rng = np.random.default_rng(7000 + rank)
    blocks = [i % 2 for i in range(len(shapes))]
    scales = np.array([1.0, 0.3125], np.float32)
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    err0 = [(rng.standard_normal((m, n)) * 0.05).astype(np.float32) for m, n in shapes]
    log(f"ragged {dtype} r={rank} shapes={shapes}, ld padded by 24")
    case = Case(shapes, blocks, dtype, rank, scales, q0, err0, ld_pad=24)
    for t in range(3):
        gs = []
        for m, n in shapes:
            x = rng.standard_normal((m, n)) * np.exp(rng.uniform(-3, 0, size=(m, 1)))
            gs.append(wl.to_bf16_bits(x) if dtype == "bf16" else
                      (wl.to_fp16(x) if dtype == "f16" else x.astype(np.float32)))
        case.set_grads(gs)
        case.gpu_step()
        compare_step(case.fetch(), case.oracle_step(), f"ragged step {t}", check_p=rank > 1)
    # padding columns between n and ld are never touched
    for gte in case.group.err:
        base = gte.as_strided((gte.shape[0], gte.shape[1] + 24), gte.stride())
        assert float(base[:, gte.shape[1]:].abs().max()) == 0.0
    case.close()


@pytest.mark.parametrize("rank,shapes", [
    (1, [(1, 8), (1, 64), (7, 8), (33, 16), (40, 24)]),
    (8, [(8, 8), (9, 8), (8, 4096), (17, 24), (40, 24)]),
], ids=["r1", "r8"])
def test_degenerate_shapes_and_a_zero_matrix(rank, shapes):
    """Shapes at the edges of the tiles: one-row matrices, fewer rows than one MFMA tile, the
    narrowest n (8), r = m = n (P square and orthogonal, D = M, E at round-off), and a matrix
    whose G and E stay zero (every column of P dependent: P, D, E and q_next zero), three
    warm-started steps in one group against the oracle."""
    rng = np.random.default_rng(7300 + rank)
    blocks = [0] * len(shapes)
    scales = np.array([1.0], np.float32)
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    err0 = [(rng.standard_normal((m, n)) * 0.05).astype(np.float32) for m, n in shapes]
    err0[-1][:] = 0.0                                    # the zero matrix
    log(f"degenerate shapes r={rank}: {shapes}")
    case = Case(shapes, blocks, "f16", rank, scales, q0, err0)
    for t in range(3):
        gs = [wl.to_fp16(rng.standard_normal((m, n))) for m, n in shapes]
        gs[-1] = np.zeros(shapes[-1], np.float16)
        case.set_grads(gs)
        assert case.gpu_step() == 0
        res = case.fetch()
        compare_step(res, case.oracle_step(), f"degenerate r={rank} step {t}")
        for key in ("P", "D", "E", "Qn"):
            assert float(np.abs(res[key][-1]).max()) == 0.0, (t, key)
    case.close()


# ------------------------------------------------------------------------------------------
# the flag reports non-finite G or E only: a finite M whose product overflows sets none
# ------------------------------------------------------------------------------------------
def test_product_overflow_is_not_a_flag():
    import torch
    log("flag: overflowing product of a finite M")
    m, n, rank = 128, 64, 4
    q0 = [np.full((n, rank), 2.0, np.float32)]
    err0 = [np.zeros((m, n), np.float32)]
    err0[0][5, :] = 3.0e38             # finite; the row's product with q exceeds fp32
    case = Case([(m, n)], [0], "f32", rank, np.ones(1, np.float32), q0, err0)
    case.set_grads([np.zeros((m, n), np.float32)])
    case.group.compress()
    torch.cuda.synchronize()
    assert case.group.flags.cpu().numpy().tolist() == [0]
    case.group.err[0][7, 3] = float("nan")
    case.group.compress()
    torch.cuda.synchronize()
    assert case.group.flags.cpu().numpy().tolist() == [1]
    case.close()


# ------------------------------------------------------------------------------------------
# non-finite values: flags and skip bit-exact, error buffers zeroed, q kept
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("rank,shapes", [(16, [(300, 256), (64, 512), (200, 104)]),
                                         (160, [(300, 256), (200, 512), (200, 176)])],
                         ids=["r16", "r160"])
def test_nonfinite_flags_skip_and_zeroing(rank, shapes):
    """Each non-finite event flags exactly its matrix (or only skips, for a pass-through NaN or a
    non-finite scale), the step is skipped, E is zeroed and q and out are kept; rank 160 takes
    the path where M is split once and the flag comes from that split."""
    import torch
    rng = np.random.default_rng(99)
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    err0 = [(rng.standard_normal((m, n)) * 0.1).astype(np.float32) for m, n in shapes]
    scales = np.array([1.0, 0.5], np.float32)
    case = Case(shapes, [0, 1, 1], "f16", rank, scales, q0, err0)
    base = [wl.to_fp16(rng.standard_normal((m, n))) for m, n in shapes]

    # clean step first
    case.set_grads(base)
    assert case.gpu_step(passthrough=[np.ones(10)]) == 0
    compare_step(case.fetch(), case.oracle_step([np.ones(10)]), "clean")

    events = [
        ("grad +inf", dict(grad=(1, 5, 7, np.inf))),
        ("grad nan", dict(grad=(2, 199, 103, np.nan))),
        ("grad -inf", dict(grad=(0, 0, 0, -np.inf))),
        # the only nonzero factor of this column is gone: inf * 0 in the product must still flag
        ("grad +inf on a zero row of q", dict(grad=(0, 9, 17, np.inf), zero_q_row=(0, 17))),
        ("err nan", dict(err=(1, 63, 511, np.nan))),
        ("pass nan", dict(passthrough=np.array([0.0, np.nan, 1.0]))),
        ("scale inf", dict(scale=(1, np.inf))),
    ]
    for name, ev in events:
        log(f"  inject {name}")
        gs = [g.copy() for g in base]
        if "grad" in ev:
            i, r, c, v = ev["grad"]
            gs[i][r, c] = v
        case.set_grads(gs)
        if "err" in ev:
            i, r, c, v = ev["err"]
            case.group.err[i][r, c] = float(v)
        if "scale" in ev:
            b, v = ev["scale"]
            case.group.scale[b] = float(v)
        if "zero_q_row" in ev:
            i, qr = ev["zero_q_row"]
            case.group.q[i][qr, :] = 0.0
            case.Q_or[i] = case.Q_or[i].copy()
            case.Q_or[i][qr, :] = 0.0
        q_before = [q.clone() for q in case.group.q]
        out_before = [o.clone() for o in case.group.out]
        pt = [ev["passthrough"]] if "passthrough" in ev else [np.ones(10)]
        skip = case.gpu_step(passthrough=pt)
        res = case.fetch()
        expect_flags = np.zeros(len(shapes), np.uint8)
        if "grad" in ev:
            expect_flags[ev["grad"][0]] = 1
        if "err" in ev:
            expect_flags[ev["err"][0]] = 1
        assert np.array_equal(res["flags"], expect_flags), (name, res["flags"])
        assert skip == 1, name
        assert int(case.group.skip.item()) == 1
        for e in res["E"]:
            assert np.all(e == 0.0), name
        for qb, qa in zip(q_before, case.group.q):
            assert torch.equal(qb, qa), name
        for ob, oa in zip(out_before, case.group.out):
            assert torch.equal(ob, oa), name
        if "scale" in ev:
            case.group.scale[ev["scale"][0]] = float(scales[ev["scale"][0]])
        # oracle agrees on the decision and zeroing
        Es = [np.asarray(e, np.float64) for e in case.E_or]
        if "err" in ev:
            i, r, c, v = ev["err"]
            Es[i] = Es[i].copy()
            Es[i][r, c] = v
        sc = scales.copy()
        if "scale" in ev:
            sc[ev["scale"][0]] = ev["scale"][1]
        st = oracle.step_group(case.cur_grads, Es, case.Q_or, case.blocks, sc, pt)
        assert st.skip and [bool(f) for f in res["flags"]] == st.flags
        case.E_or = st.E_next
        case.Q_or = st.Q_next

    # recovery: a clean step after the skips, from zeroed error buffers and the kept q
    case.set_grads(base)
    assert case.gpu_step(passthrough=[np.ones(10)]) == 0
    compare_step(case.fetch(), case.oracle_step([np.ones(10)]), "after skips")
    case.close()


# ------------------------------------------------------------------------------------------
# near-underflow heavy-tailed workload at rank 80 (2 resblocks)
# ------------------------------------------------------------------------------------------
def test_underflow_workload_two_resblocks():
    w, specs, case = _shard_case(4, 2)
    log("Student-t(3) near fp16 underflow, r=80, 2 resblocks, 3 steps")
    for t in range(3):
        case.set_grads([wl.gradient_np(w, s, t) for s in specs])
        assert case.gpu_step() == 0
        compare_step(case.fetch(), case.oracle_step(), f"underflow step {t}")
    case.close()


# ------------------------------------------------------------------------------------------
# determinism: the same inputs give bitwise identical outputs
# ------------------------------------------------------------------------------------------
def test_bitwise_deterministic():
    import torch
    w, specs, _ = _shard_case(2, None)
    outs = []
    for rep in range(2):
        w, specs, case = _shard_case(2, None, err_warm=True)
        case.set_grads([wl.gradient_np(w, s, 1) for s in specs])
        case.gpu_step()
        outs.append(case.fetch())
        case.close()
    for k in ("E", "Q", "P", "D"):
        for a, b in zip(outs[0][k], outs[1][k]):
            assert np.array_equal(a, b), k


# ------------------------------------------------------------------------------------------
# argument validation
# ------------------------------------------------------------------------------------------
def test_invalid_arguments_rejected():
    import torch
    from rank_gradient_compression_powersgd_amd import binding as B
    ctx = B.psgd_create(0, 8)
    try:
        g = torch.zeros((64, 60), dtype=torch.float16, device="cuda")   # n not a multiple of 8
        e = torch.zeros((64, 60), dtype=torch.float32, device="cuda")
        q = torch.zeros((60, 8), device="cuda")
        p = torch.zeros((64, 8), device="cuda")
        with pytest.raises(B.PsgdError) as ei:
            B.psgd_plan_create(ctx, [B.make_matrix(g, e, q, q.clone(), p, 0)], B.PSGD_F16, 1)
        assert ei.value.status == B.PSGD_EINVAL and "multiple of 8" in str(ei.value)
        g = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
        e = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
        q = torch.zeros((64, 8), device="cuda")
        with pytest.raises(B.PsgdError):   # block outside the scale array
            B.psgd_plan_create(ctx, [B.make_matrix(g, e, q, q.clone(), p, 3)], B.PSGD_F16, 2)
        with pytest.raises(B.PsgdError):   # unknown dtype
            B.psgd_plan_create(ctx, [B.make_matrix(g, e, q, q.clone(), p, 0)], 9, 1)
        with pytest.raises(B.PsgdError) as ei:   # empty group
            B.psgd_plan_create(ctx, [], B.PSGD_F16, 1)
        assert ei.value.status == B.PSGD_EINVAL
        small = torch.zeros((6, 64), dtype=torch.float16, device="cuda")   # rank 8 > m = 6
        with pytest.raises(B.PsgdError) as ei:
            B.psgd_plan_create(ctx, [B.make_matrix(small, torch.zeros((6, 64), device="cuda"), q, q.clone(),
                                                   torch.zeros((6, 8), device="cuda"), 0)], B.PSGD_F16, 1)
        assert "exceeds" in str(ei.value)
        wide = torch.zeros((64, 72), dtype=torch.float32, device="cuda")  # E view with ld 72, offset 2 floats
        with pytest.raises(B.PsgdError) as ei:
            B.psgd_plan_create(ctx, [B.make_matrix(g, wide[:, 2:66], q, q.clone(), p, 0)], B.PSGD_F16, 1)
        assert "aligned" in str(ei.value)
    finally:
        B.psgd_destroy(ctx)
    with pytest.raises(B.PsgdError):
        B.psgd_create(0, 0)
    with pytest.raises(B.PsgdError):
        B.psgd_create(0, 1025)


# ------------------------------------------------------------------------------------------
# ranks above 128: M split once, the two products as GEMMs, blocked orthonormalisation
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,rank", [("f16", 200), ("bf16", 260), ("f32", 136), ("f16", 1024), ("bf16", 201)])
def test_large_rank_ragged(dtype, rank):
    """Ranks above 128 with ragged shapes, every gradient dtype; rank 1024 is the largest the
    library takes (eight 128-column blocks), and the odd rank 201 leaves factor rows that are not
    whole 16-byte units."""
    shapes = [(1000, 1536), (700, 520), (300, 264)] if rank <= 300 else [(1100, 1032), (1030, 1088)]
    rng = np.random.default_rng(8000 + rank)
    blocks = [0, 1, 0][:len(shapes)]
    scales = np.array([1.0, 0.75], np.float32)
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    err0 = [(rng.standard_normal((m, n)) * 0.05).astype(np.float32) for m, n in shapes]
    log(f"large rank {dtype} r={rank} shapes={shapes}")
    case = Case(shapes, blocks, dtype, rank, scales, q0, err0)
    for t in range(3):
        gs = []
        for m, n in shapes:
            x = rng.standard_normal((m, n)) * np.exp(rng.uniform(-3, 0, size=(m, 1)))
            gs.append(wl.to_bf16_bits(x) if dtype == "bf16" else
                      x.astype(np.float32) if dtype == "f32" else wl.to_fp16(x))
        case.set_grads(gs)
        assert case.gpu_step() == 0
        compare_step(case.fetch(), case.oracle_step(), f"large rank step {t}")
    case.close()


def test_large_rank_many_matrices():
    """Rank 144 (a full 128-column block and a ragged 16-column one) over 24 matrices of mixed
    shapes: the block factorisation's per-step work lists, its diagonal blocks and the GEMM
    lists all carry many matrices at once."""
    rank = 144
    rng = np.random.default_rng(8144)
    shapes = [(int(rng.integers(150, 700)), 8 * int(rng.integers(19, 90))) for _ in range(24)]
    blocks = [i % 3 for i in range(len(shapes))]
    scales = np.array([1.0, 0.5, 2.0], np.float32)
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    err0 = [(rng.standard_normal((m, n)) * 0.05).astype(np.float32) for m, n in shapes]
    log(f"large rank, {len(shapes)} matrices, r={rank}")
    case = Case(shapes, blocks, "f16", rank, scales, q0, err0)
    for t in range(2):
        gs = [wl.to_fp16(rng.standard_normal((m, n)) * np.exp(rng.uniform(-3, 0, size=(m, 1))))
              for m, n in shapes]
        case.set_grads(gs)
        assert case.gpu_step() == 0
        compare_step(case.fetch(), case.oracle_step(), f"many matrices step {t}")
    case.close()


@pytest.mark.parametrize("rank,true_rank", [(100, 60), (200, 150)])
def test_rank_deficient_second_pass(rank, true_rank):
    """rank(M) < r: one step recovers M (E vanishes relative to M). The surplus columns of M q
    are rounding noise, which leaves the Gram form ill-conditioned, so the orthonormalisation
    takes its second pass; P must come out orthonormal. Which completion fills the surplus
    columns is rounding-dependent on both sides, so D and E are compared, not P."""
    m, n = 600, 512
    M = wl.exact_rank_np(m, n, true_rank, seed=4242).astype(np.float32)
    rng = np.random.default_rng(4243)
    q0 = [rng.standard_normal((n, rank)).astype(np.float32)]
    case = Case([(m, n)], [0], "f32", rank, np.ones(1, np.float32), q0)
    case.set_grads([M])
    assert case.gpu_step() == 0
    res = case.fetch()
    compare_step(res, case.oracle_step(), f"rank-{true_rank} matrix at r={rank}", exact_rank=True,
                 check_p=False)
    log(f"  |E|/|M| {np.linalg.norm(res['E'][0]) / np.linalg.norm(M):.2e}")
    assert np.linalg.norm(res["E"][0]) / np.linalg.norm(M) <= 1e-4
    case.close()


# ------------------------------------------------------------------------------------------
# in-place matrices: backprop has accumulated s_b G into the error buffer (grad NULL)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("rank", [24, 200])
def test_inplace_matrices_match_oracle_and_skip(rank):
    """Two of three matrices in-place (err holds M, no gradient read); the third as usual. The
    oracle sees the in-place matrices as G = 0, E = M. Then a non-finite element planted in an
    in-place error buffer flags that matrix and skips the step (every error buffer zeroed)."""
    import torch
    shapes = [(513, 264), (300, 1048), (640, 512)]
    rng = np.random.default_rng(31)
    scales = np.array([0.75], np.float32)
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    Ms = [(rng.standard_normal((m, n)) * 0.3).astype(np.float32) for m, n in shapes]
    G2 = wl.to_fp16(rng.standard_normal(shapes[2]))
    E2 = (rng.standard_normal(shapes[2]) * 0.05).astype(np.float32)
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    dev = torch.device("cuda", 0)
    err = [torch.from_numpy(x).to(dev) for x in (Ms[0], Ms[1], E2)]
    grads = [None, None, torch.from_numpy(G2).to(dev)]
    group = PowerSGDGroup(grads, [0, 0, 0], torch.from_numpy(scales).to(dev), rank,
                          [torch.from_numpy(q) for q in q0], err, True)
    skip = group.step([], host=True)
    torch.cuda.synchronize()
    assert skip == 0
    st = oracle.step_group([np.zeros(shapes[0], np.float32), np.zeros(shapes[1], np.float32),
                            G2.astype(np.float32)], [Ms[0], Ms[1], E2], q0, [0, 0, 0], scales)
    res = dict(E=[e.cpu().numpy() for e in group.err], Q=[q.cpu().numpy() for q in group.q],
               P=[p.cpu().numpy() for p in group.p], D=[o.cpu().numpy() for o in group.out],
               flags=group.flags.cpu().numpy())
    assert not res["flags"].any()
    compare_step(res, st, "in-place step")
    group.err[1][7, 11] = float("nan")
    skip = group.step([], host=True)
    torch.cuda.synchronize()
    assert skip == 1
    assert list(group.flags.cpu().numpy()) == [0, 1, 0]
    for e in group.err:
        assert float(e.abs().max()) == 0.0
    group.close()


def test_reset_errors_restart_from_checkpoint():
    """psgd_reset_errors after two steps: every error buffer becomes exactly zero over m x n
    (the padding columns of a strided buffer, q and the D buffers are untouched), and the next
    step matches the oracle started from E = 0 with the warm starts the run had reached."""
    import torch
    shapes = [(640, 264), (300, 1048), (1029, 512)]
    rank = 40
    rng = np.random.default_rng(47)
    scales = np.array([1.0, 0.5], np.float32)
    blocks = [0, 1, 1]
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    dev = torch.device("cuda", 0)
    # the second error buffer is a view into a wider allocation (8 padding columns per row)
    wide = torch.full((shapes[1][0], shapes[1][1] + 8), 7.0, dtype=torch.float32, device=dev)
    err = [torch.zeros(shapes[0], dtype=torch.float32, device=dev), wide[:, :shapes[1][1]],
           torch.zeros(shapes[2], dtype=torch.float32, device=dev)]
    err[1].zero_()
    Gs = [[wl.to_fp16(rng.standard_normal(sh)) for sh in shapes] for _ in range(3)]
    grads = [torch.from_numpy(g).to(dev) for g in Gs[0]]
    group = PowerSGDGroup(grads, blocks, torch.from_numpy(scales).to(dev), rank,
                          [torch.from_numpy(q) for q in q0], err, True)
    for t in range(2):
        for i in range(3):
            group.grads[i].copy_(torch.from_numpy(Gs[t][i]))
        assert group.step([], host=True) == 0
    torch.cuda.synchronize()
    assert all(float(e.abs().max()) > 0 for e in group.err)
    q_before = [q.clone() for q in group.q]
    out_before = [o.clone() for o in group.out]
    group.reset_errors()
    torch.cuda.synchronize()
    for e in group.err:
        assert float(e.abs().max()) == 0.0
    assert float(wide[:, shapes[1][1]:].sub(7.0).abs().max()) == 0.0
    for a, b in zip(group.q, q_before):
        assert torch.equal(a, b)
    for a, b in zip(group.out, out_before):
        assert torch.equal(a, b)
    for i in range(3):
        group.grads[i].copy_(torch.from_numpy(Gs[2][i]))
    assert group.step([], host=True) == 0
    torch.cuda.synchronize()
    st = oracle.step_group([g.astype(np.float32) for g in Gs[2]],
                           [np.zeros(sh, np.float32) for sh in shapes],
                           [q.cpu().numpy() for q in q_before], blocks, scales)
    res = dict(E=[e.cpu().numpy() for e in group.err], Q=[q.cpu().numpy() for q in group.q],
               P=[p.cpu().numpy() for p in group.p], D=[o.cpu().numpy() for o in group.out],
               flags=group.flags.cpu().numpy())
    compare_step(res, st, "step after reset")
    assert float(wide[:, shapes[1][1]:].sub(7.0).abs().max()) == 0.0
    group.close()


# ------------------------------------------------------------------------------------------
# data-parallel split calls: two ranks simulated on one GPU, factors averaged between calls
# ------------------------------------------------------------------------------------------
def _dev_copy(dst: int, src: int, nbytes: int):
    import ctypes
    lib = ctypes.CDLL("libamdhip64.so.7")
    lib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    assert lib.hipMemcpy(dst, src, nbytes, 3) == 0       # device to device


def _simulated_data_parallel(rank, shapes, n_ranks, rng, dtype="f16"):
    """psgd_compress_p -> mean of the factor buffers -> psgd_orthogonalize -> psgd_compress_q ->
    mean of q_next -> psgd_refresh_q -> check -> decompress, for n_ranks ranks holding
    different gradients of the same matrices (one plan each on one GPU, torch doing the means),
    against the oracle's data-parallel step: P and D identical on every rank, each rank's own
    E."""
    import torch
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    from rank_gradient_compression_powersgd_amd import binding as B
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    scale = torch.tensor([0.5], device="cuda")
    ranks = []
    for k in range(n_ranks):
        x = [rng.standard_normal(sh) for sh in shapes]
        gs = [wl.to_fp16(v) if dtype == "f16" else v.astype(np.float32) for v in x]
        es = [(rng.standard_normal(sh) * 0.05).astype(np.float32) for sh in shapes]
        grp = PowerSGDGroup([torch.from_numpy(g).cuda() for g in gs], [0] * len(shapes), scale, rank,
                            [torch.from_numpy(q) for q in q0],
                            [torch.from_numpy(e).cuda() for e in es], True)
        ranks.append((grp, gs, es))
    for grp, _, _ in ranks:
        B.psgd_compress_p(grp.ctx, grp.plan, grp.scale, grp.flags)
    bufs = [B.psgd_factor_buffer(grp.plan) for grp, _, _ in ranks]
    count = bufs[0][1]
    torch.cuda.synchronize()
    f = [torch.empty(count, device="cuda") for _ in ranks]
    for t, (ptr, cnt, _) in zip(f, bufs):
        assert cnt == count
        _dev_copy(t.data_ptr(), ptr, 4 * count)
    mean = sum(f) / n_ranks
    torch.cuda.synchronize()
    for ptr, _, _ in bufs:
        _dev_copy(ptr, mean.data_ptr(), 4 * count)
    for grp, _, _ in ranks:
        B.psgd_orthogonalize(grp.ctx, grp.plan)
        B.psgd_compress_q(grp.ctx, grp.plan, grp.scale)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        qm = sum(grp.q_next[i] for grp, _, _ in ranks) / n_ranks
        for grp, _, _ in ranks:
            grp.q_next[i].copy_(qm)
    torch.cuda.synchronize()
    for grp, _, _ in ranks:
        B.psgd_refresh_q(grp.ctx, grp.plan)
        assert grp.check_finite([], host=True) == 0
        grp.decompress_update()
    torch.cuda.synchronize()
    for i, sh in enumerate(shapes):
        st = oracle.step_data_parallel([ranks[k][1][i].astype(np.float32) for k in range(n_ranks)],
                                       [ranks[k][2][i] for k in range(n_ranks)], q0[i], 0.5)
        P = [grp.p[i].cpu().numpy() for grp, _, _ in ranks]
        D = [grp.out[i].cpu().numpy() for grp, _, _ in ranks]
        for k in range(1, n_ranks):
            assert np.array_equal(P[0], P[k]) and np.array_equal(D[0], D[k])
        r = dict(P=rel(P[0], st.P), D=rel(D[0], st.D), Q=rel(ranks[0][0].q[i].cpu().numpy(), st.Q_next),
                 orth=orth_err(P[0]))
        for k in range(n_ranks):
            r[f"E{k}"] = rel(ranks[k][0].err[i].cpu().numpy(), st.E_next[k])
        log(f"  matrix {i} {sh}: " + " ".join(f"{k}={v:.2e}" for k, v in r.items()))
        for k, v in r.items():
            if k != "orth":
                assert v <= REL_TOL, (i, k, v)
        assert r["orth"] <= ORTH_TOL
    for grp, _, _ in ranks:
        grp.close()


@pytest.mark.parametrize("rank", [16, 160])
def test_split_calls_two_simulated_ranks(rank):
    """Two simulated ranks of a data-parallel group on one GPU, against the oracle's
    data-parallel step (the split calls with the means taken between them)."""
    _simulated_data_parallel(rank, [(520, 264), (300, 512)], 2, np.random.default_rng(77))


@pytest.mark.parametrize("seed", range(6))
def test_split_calls_random_simulated_groups(seed):
    """Seeded random data-parallel groups: two to four simulated ranks, a rank on either side of
    the 128-column chunk, ragged shapes, fp16 or fp32 gradients."""
    rng = np.random.default_rng(7_900_000 + seed)
    rank = int(rng.choice([7, 48, 112, 144, 200]))
    shapes = [(int(rng.integers(rank, rank + 500)), 8 * int(rng.integers((rank + 7) // 8, (rank + 7) // 8 + 70)))
              for _ in range(int(rng.integers(1, 3)))]
    n_ranks = int(rng.integers(2, 5))
    dtype = str(rng.choice(["f16", "f32"]))
    log(f"simulated group {seed}: {n_ranks} ranks, rank {rank}, {dtype}, shapes {shapes}")
    _simulated_data_parallel(rank, shapes, n_ranks, rng, dtype)


@pytest.mark.parametrize("rank", [None, 160])
def test_split_calls_equal_the_fused_call(rank):
    """On one GPU the exchanges are the identity: the split calls must give bit-identical
    results to psgd_compress. Above rank 128 the fused call forms M^T on a second stream while
    the split calls run everything on one, so this also checks that fork and join."""
    import torch
    from rank_gradient_compression_powersgd_amd import binding as B
    outs = []
    for split in (False, True):
        w, specs, case = _shard_case(2, None, err_warm=True, rank=rank)
        case.set_grads([wl.gradient_np(w, s, 2) for s in specs])
        g = case.group
        if split:
            B.psgd_compress_p(g.ctx, g.plan, g.scale, g.flags)
            B.psgd_orthogonalize(g.ctx, g.plan)
            B.psgd_compress_q(g.ctx, g.plan, g.scale)
            B.psgd_refresh_q(g.ctx, g.plan)
        else:
            g.compress()
        g.check_finite([], host=True)
        g.decompress_update()
        torch.cuda.synchronize()
        outs.append(case.fetch())
        case.close()
    for k in ("E", "Q", "P", "D"):
        for a, b in zip(outs[0][k], outs[1][k]):
            assert np.array_equal(a, b), k
