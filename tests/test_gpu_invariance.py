"""Bit-exact invariances of the HIP path, run through the C ABI.

Two properties the method fixes and that any correct implementation without hidden state keeps
exactly, in floating point as well, as long as nothing under- or overflows:

  * scale equivariance: multiplying G and E by 2^k multiplies M = s G + E by 2^k exactly, so
    the orthonormal factor P = orth(M Q) is unchanged and Q' = M^T P, D = P Q'^T and
    E' = M - D are multiplied by 2^k; every rounding of the step commutes with a power-of-two
    factor, so the GPU results must agree bit for bit;
  * permutation invariance: the matrices of a group are independent units, so the order in
    which a group lists them may not change any matrix's results (the flags move with the
    matrices).

Each case runs three warm-started steps (E != 0 and q != q0 from the second step on) on both
the rank <= 128 path (streaming products) and the rank > 128 path (split-once GEMMs and the
blocked factorisation).
"""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, rank, shapes): the one-resblock shard shapes at rank 112, and ragged shapes at
    # ranks that take the large-rank path
    ("f16", 112, [(3968, 1488), (496, 3968), (3968, 1984), (1984, 3968)]),
    ("bf16", 80, [(1000, 520), (333, 1024), (2047, 264)]),
    ("f16", 160, [(1000, 768), (520, 1024), (700, 704)]),
    ("bf16", 256, [(777, 1024), (1536, 512)]),
]


def _grads(dtype, shapes, seed, step):
    import torch
    out = []
    for i, (m, n) in enumerate(shapes):
        rng = wl.matrix_rng(seed + step, i)
        x = rng.standard_normal((m, n)) * np.exp(rng.uniform(np.log(1e-3), 0.0, size=(m, 1)))
        if dtype == "f16":
            out.append(torch.from_numpy(wl.to_fp16(x)).cuda())
        else:
            bits = wl.to_bf16_bits(x)
            out.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())
    return out


def _group(grads, blocks, scale, rank, q0):
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    return PowerSGDGroup(grads, blocks, scale, rank, q0, None, True)


def _same_bits(a, b):
    import torch
    return bool(torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32)))


@pytest.mark.parametrize("dtype,rank,shapes", CASES, ids=[f"{c[0]}-r{c[1]}" for c in CASES])
def test_power_of_two_scale_equivariance_bit_exact(dtype, rank, shapes):
    import torch
    k = 5                                    # G, E x 32: no fp16 overflow (|G| < 8 here)
    f = float(2 ** k)
    seed = 7_100_000 + rank
    blocks = [i % 2 for i in range(len(shapes))]
    scale = torch.tensor([1.0, 0.375], dtype=torch.float32, device="cuda")
    rng = wl.matrix_rng(seed, 999)
    q0 = [torch.from_numpy(rng.standard_normal((n, rank)).astype(np.float32)) for _, n in shapes]
    ga = _grads(dtype, shapes, seed, 0)
    gb = [(g.float() * f).to(g.dtype) for g in ga]
    for a, b in zip(ga, gb):
        assert torch.equal((b.float() / f), a.float()), "the scaled gradient is not exact"
    A = _group(ga, blocks, scale, rank, q0)
    B = _group(gb, blocks, scale, rank, q0)
    for step in range(3):
        if step:
            for a, b, new in zip(ga, gb, _grads(dtype, shapes, seed, step)):
                a.copy_(new)
                b.copy_((new.float() * f).to(new.dtype))
        log(f"scale equivariance {dtype} r={rank} step {step}: G, E x 2^{k}")
        sa = A.step([], host=True)
        sb = B.step([], host=True)
        torch.cuda.synchronize()
        assert sa == 0 and sb == 0
        for i in range(len(shapes)):
            assert _same_bits(A.p[i], B.p[i]), (step, i, "P")
            for name, xa, xb in (("D", A.out[i], B.out[i]), ("E", A.err[i], B.err[i]),
                                 ("q", A.q[i], B.q[i])):
                assert _same_bits(xa * f, xb), (step, i, name,
                                                float((xa * f - xb).abs().max()))
    A.close()
    B.close()


@pytest.mark.parametrize("dtype,rank,shapes", CASES, ids=[f"{c[0]}-r{c[1]}" for c in CASES])
def test_group_permutation_invariance_bit_exact(dtype, rank, shapes):
    import torch
    seed = 7_200_000 + rank
    nm = len(shapes)
    blocks = [i % 3 for i in range(nm)]
    scale = torch.tensor([1.0, 0.5, 0.1875], dtype=torch.float32, device="cuda")
    rng = wl.matrix_rng(seed, 999)
    q0 = [torch.from_numpy(rng.standard_normal((n, rank)).astype(np.float32)) for _, n in shapes]
    perm = list(reversed(range(nm)))
    perm = perm[1:] + perm[:1]
    ga = _grads(dtype, shapes, seed, 0)
    gb = [ga[j].clone() for j in perm]
    A = _group(ga, blocks, scale, rank, q0)
    B = _group(gb, [blocks[j] for j in perm], scale, rank, [q0[j] for j in perm])
    for step in range(3):
        if step:
            new = _grads(dtype, shapes, seed, step)
            if step == 2:
                new[perm[0]][3, 5] = float("inf")      # a flagged, skipped step
            for i in range(nm):
                ga[i].copy_(new[i])
                gb[i].copy_(new[perm[i]])
        log(f"permutation invariance {dtype} r={rank} step {step}: order {perm}")
        sa = A.step([], host=True)
        sb = B.step([], host=True)
        torch.cuda.synchronize()
        assert sa == sb == (1 if step == 2 else 0)
        fa, fb = A.flags.cpu().numpy(), B.flags.cpu().numpy()
        assert np.array_equal(fa[perm], fb), (step, fa, fb)
        for i in range(nm):
            j = perm[i]
            pairs = [("E", A.err[j], B.err[i]), ("q", A.q[j], B.q[i])]
            if not sa:
                pairs += [("P", A.p[j], B.p[i]), ("D", A.out[j], B.out[i])]
            for name, xa, xb in pairs:
                assert _same_bits(xa, xb), (step, i, name)
    A.close()
    B.close()


def test_two_groups_on_two_streams_match_one_stream_bit_exact():
    """Two groups (rank 112, the streaming path, and rank 160, the split-once GEMM path), each
    on its own context and plan, stepped three times with their launches on two non-default
    streams at once: every result must equal that of the same groups stepped one after the
    other on one stream, bit for bit. The library keeps no state across plans that concurrent
    steps could share."""
    import torch
    cfgs = [("f16", 112, [(1000, 1024), (512, 768)]), ("bf16", 160, [(900, 512), (400, 640)])]
    scale = torch.tensor([1.0, 0.5], dtype=torch.float32, device="cuda")

    def build(dtype, rank, shapes, seed):
        rng = wl.matrix_rng(seed, 999)
        q0 = [torch.from_numpy(rng.standard_normal((n, rank)).astype(np.float32)) for _, n in shapes]
        grads = _grads(dtype, shapes, seed, 0)
        return _group(grads, [i % 2 for i in range(len(shapes))], scale, rank, q0), grads

    def run(concurrent):
        groups = [build(dt, r, sh, 7_300_000 + r) for dt, r, sh in cfgs]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()] if concurrent else [None, None]
        for step in range(3):
            if step:
                for (grp, grads), (dt, r, sh) in zip(groups, cfgs):
                    for g, new in zip(grads, _grads(dt, sh, 7_300_000 + r, step)):
                        g.copy_(new)
            torch.cuda.synchronize()
            for (grp, _), s in zip(groups, streams):
                grp.step([], host=False, stream=s)
            torch.cuda.synchronize()
        out = [dict(p=[t.clone() for t in grp.p], q=[t.clone() for t in grp.q],
                    e=[t.clone() for t in grp.err], d=[t.clone() for t in grp.out],
                    skip=int(grp.skip.item())) for grp, _ in groups]
        for grp, _ in groups:
            grp.close()
        return out

    log("two groups, one stream")
    ref = run(False)
    log("two groups, two streams at once")
    got = run(True)
    for k, (a, b) in enumerate(zip(ref, got)):
        assert a["skip"] == 0 and b["skip"] == 0
        for name in ("p", "q", "e", "d"):
            for i, (x, y) in enumerate(zip(a[name], b[name])):
                assert _same_bits(x, y), (cfgs[k][1], name, i)
