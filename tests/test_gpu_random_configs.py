"""Seeded random configurations of the whole step, HIP path against the float64 oracle.

Each seed draws a rank (both sides of the 128-column chunk boundary, odd ranks among them), one
to three matrices of ragged shapes (m >= rank, n a multiple of 8 and >= rank), a gradient
dtype, a padded leading dimension for G and E, and two per-resblock scales. Two steps run from
a random warm start and a small random error buffer, each compared with the oracle at the
acceptance of the other parity tests. The draws are fixed by the seed, so a failure names a
reproducible configuration.
"""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_helpers import Case, compare_step, log

pytestmark = pytest.mark.gpu

RANKS = [1, 3, 16, 37, 64, 100, 112, 128, 129, 150, 200, 255, 300]


def _config(seed: int):
    rng = np.random.default_rng(7_700_000 + seed)
    rank = int(rng.choice(RANKS))
    shapes = []
    for _ in range(int(rng.integers(1, 4))):
        m = int(rng.integers(rank, rank + 700))
        n = 8 * int(rng.integers((rank + 7) // 8, (rank + 7) // 8 + 110))
        shapes.append((m, n))
    dtype = str(rng.choice(["f16", "bf16", "f32"]))
    ld_pad = int(rng.choice([0, 0, 8, 24]))
    blocks = [int(b) for b in rng.integers(0, 2, len(shapes))]
    scales = rng.uniform(0.5, 2.0, 2).astype(np.float32)
    return rng, rank, shapes, dtype, ld_pad, blocks, scales


@pytest.mark.parametrize("seed", range(40))
def test_random_configuration(seed):
    rng, rank, shapes, dtype, ld_pad, blocks, scales = _config(seed)
    log(f"random config {seed}: rank {rank}, {dtype}, shapes {shapes}, ld pad {ld_pad}, blocks {blocks}")
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    err0 = [(rng.standard_normal((m, n)) * 0.05).astype(np.float32) for m, n in shapes]
    case = Case(shapes, blocks, dtype, rank, scales, q0, err0, ld_pad=ld_pad)
    try:
        for t in range(2):
            gs = []
            for m, n in shapes:
                x = rng.standard_normal((m, n)) * np.exp(rng.uniform(-3.0, 0.0, size=(m, 1)))
                gs.append(wl.to_bf16_bits(x) if dtype == "bf16" else
                          x.astype(np.float32) if dtype == "f32" else wl.to_fp16(x))
            case.set_grads(gs)
            assert case.gpu_step() == 0
            compare_step(case.fetch(), case.oracle_step(), f"random config {seed} step {t}")
    finally:
        case.close()
