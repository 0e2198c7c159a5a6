"""The allocation-free step (psgd_step_noalloc) against the plan-based step it mirrors
(psgd_plan_create, then psgd_compress, psgd_check_finite and psgd_decompress_update), through
the C ABI. Both paths run the same kernels over the same descriptors and work lists, so every
output must agree bit for bit (stronger than the parity tolerance). Two calls in a row share
the static scratch array, the second on a smaller group; a group too large for the array is
rejected before anything is launched.
"""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

RANK = 112


def _state(shapes, seed, rank=RANK):
    import torch
    g, e, q = [], [], []
    for i, (m, n) in enumerate(shapes):
        rng = wl.matrix_rng(seed, i)
        x = rng.standard_normal((m, n)) * np.exp(rng.uniform(np.log(1e-4), 0.0, size=(m, 1)))
        g.append(torch.from_numpy(wl.to_fp16(x)).cuda())
        e.append(torch.from_numpy((rng.standard_normal((m, n)) * 0.05).astype(np.float32)).cuda())
        q.append(torch.from_numpy(rng.standard_normal((n, rank)).astype(np.float32)).cuda())
    return g, e, q


class _Bufs:
    """One copy of a group's state and outputs, described to the ABI."""

    def __init__(self, grads, errs, qs, blocks, rank=RANK):
        import torch
        from rank_gradient_compression_powersgd_amd import binding as B
        self.err = [x.clone() for x in errs]
        self.q = [x.clone() for x in qs]
        self.q_next = [torch.empty_like(x) for x in qs]
        self.p = [torch.empty((x.shape[0], rank), dtype=torch.float32, device="cuda") for x in grads]
        self.out = [torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in grads]
        self.flags = torch.full((len(grads),), 7, dtype=torch.uint8, device="cuda")
        self.skip = torch.full((1,), 5, dtype=torch.int32, device="cuda")
        self.mats = [B.make_matrix(g, e, q, qn, p, b, o) for g, e, q, qn, p, b, o in
                     zip(grads, self.err, self.q, self.q_next, self.p, blocks, self.out)]


def _equal_bits(a, b):
    import torch
    if a.dtype in (torch.float32, torch.int32):
        return bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))
    return bool(torch.equal(a, b))


def _run_both(ctx, shapes, blocks, seed, inject=None, rank=RANK):
    import torch
    from rank_gradient_compression_powersgd_amd import binding as B
    grads, errs, qs = _state(shapes, seed, rank)
    if inject is not None:
        grads[inject][1, 2] = float("nan")
    scale = torch.tensor([1.0, 0.5, 0.25], dtype=torch.float32, device="cuda")
    pt = torch.from_numpy(wl.passthrough_np(2, 3, seed % 1000)).cuda().reshape(-1)
    ref = _Bufs(grads, errs, qs, blocks, rank)
    new = _Bufs(grads, errs, qs, blocks, rank)
    plan = B.psgd_plan_create(ctx, ref.mats, B.PSGD_F16, 3)
    B.psgd_compress(ctx, plan, scale, ref.flags)
    B.psgd_check_finite(ctx, plan, ref.flags, [pt], scale, ref.skip)
    B.psgd_decompress_update(ctx, plan, scale, ref.skip)
    B.psgd_step_noalloc(ctx, new.mats, B.PSGD_F16, scale, new.flags, new.skip, [pt])
    torch.cuda.synchronize()
    B.psgd_plan_destroy(plan)
    want_skip = 1 if inject is not None else 0
    assert int(ref.skip.item()) == want_skip and int(new.skip.item()) == want_skip
    assert _equal_bits(ref.flags, new.flags)
    for i in range(len(shapes)):
        pairs = [("E", ref.err[i], new.err[i]), ("q", ref.q[i], new.q[i])]
        if not want_skip:
            pairs += [("q_next", ref.q_next[i], new.q_next[i]), ("P", ref.p[i], new.p[i]),
                      ("D", ref.out[i], new.out[i])]
        for name, a, b in pairs:
            assert _equal_bits(a, b), (shapes[i], name, float((a - b).abs().max()))
    return ref, new


def test_noalloc_step_matches_the_plan_step_twice_then_smaller():
    from rank_gradient_compression_powersgd_amd import binding as B
    ctx = B.psgd_create(0, RANK)
    try:
        big = [(3968, 1488), (496, 3968), (3968, 1984), (1984, 3968)]   # one resblock shard
        log("no-alloc step: one resblock shard (4 matrices), rank 112")
        _run_both(ctx, big, [0, 1, 2, 0], 8_100_001)
        small = [(700, 264), (333, 1024)]
        log("no-alloc step: smaller group after it (2 matrices)")
        _run_both(ctx, small, [2, 1], 8_100_002)
        log("no-alloc step: smaller group with a NaN gradient (skip path)")
        _run_both(ctx, small, [2, 1], 8_100_003, inject=1)
        log("no-alloc step: the shard again after the smaller groups")
        _run_both(ctx, big, [0, 1, 2, 0], 8_100_004)
    finally:
        B.psgd_destroy(ctx)


def test_noalloc_step_large_rank_matches_the_plan_step():
    """Rank 160: the split-once GEMM path (M split into the scratch array, the balanced
    GEMM lists) and the blocked factorisation, twice in a row, the second group smaller."""
    from rank_gradient_compression_powersgd_amd import binding as B
    ctx = B.psgd_create(0, 160)
    try:
        log("no-alloc step: rank 160, three matrices")
        _run_both(ctx, [(600, 512), (257, 768), (320, 264)], [0, 1, 2], 8_100_011, rank=160)
        log("no-alloc step: rank 160, one matrix after it")
        _run_both(ctx, [(200, 776)], [1], 8_100_012, rank=160)
    finally:
        B.psgd_destroy(ctx)


def test_noalloc_step_rejects_a_group_beyond_the_scratch_array():
    import torch
    from rank_gradient_compression_powersgd_amd import binding as B
    ctx = B.psgd_create(0, RANK)
    try:
        m, n = 32768, 128          # m x 112 factors alone exceed the 32 MiB array
        g = torch.zeros((m, n), dtype=torch.float16, device="cuda")
        bufs = _Bufs([g], [torch.zeros((m, n), dtype=torch.float32, device="cuda")],
                     [torch.zeros((n, RANK), dtype=torch.float32, device="cuda")], [0])
        scale = torch.ones(1, dtype=torch.float32, device="cuda")
        log("no-alloc step: oversized group must be rejected")
        with pytest.raises(B.PsgdError) as ei:
            B.psgd_step_noalloc(ctx, bufs.mats, B.PSGD_F16, scale, bufs.flags, bufs.skip)
        assert ei.value.status == B.PSGD_EINVAL and "allocation-free" in str(ei.value)
        torch.cuda.synchronize()
        assert int(bufs.skip.item()) == 5            # nothing was launched
        assert int(bufs.flags[0].item()) == 7
    finally:
        B.psgd_destroy(ctx)


@pytest.mark.parametrize("rank", [80, 129])
def test_noalloc_step_over_random_groups_in_a_row(rank):
    """Ten seeded random groups in a row on one context (one to three ragged matrices, blocks
    and a NaN-gradient skip step drawn per group), each against the plan path bit for bit: the
    scratch array is re-laid out for every group and must hold no state from the one before."""
    from rank_gradient_compression_powersgd_amd import binding as B
    rng = np.random.default_rng(8_200_000 + rank)
    ctx = B.psgd_create(0, rank)
    try:
        for k in range(10):
            shapes = [(int(rng.integers(rank, rank + 600)), 8 * int(rng.integers((rank + 7) // 8, (rank + 7) // 8 + 90)))
                      for _ in range(int(rng.integers(1, 4)))]
            blocks = [int(b) for b in rng.integers(0, 3, len(shapes))]
            inject = int(rng.integers(0, len(shapes))) if k % 4 == 3 else None
            log(f"no-alloc step, rank {rank}, group {k}: {shapes}, blocks {blocks}, NaN in {inject}")
            _run_both(ctx, shapes, blocks, 8_300_000 + 100 * rank + k, inject=inject, rank=rank)
    finally:
        B.psgd_destroy(ctx)
