"""Seeded synthetic gradient workloads with the shapes of a DALL·E 12B per-GPU shard.

Nothing here computes any part of the PowerSGD step. The module only draws random numbers,
fixes shapes and converts dtypes. Both the float64 oracle and the HIP path receive the same bits
from it.

Shapes. The DALL·E transformer has 64 resblocks and d_model = 3968
("Zero-Shot Text-to-Image Generation — 中文验证版" reading card, section 计算设置). Parameters
are sharded over the 8 GPUs of a machine, and each GPU compresses its own shard at rank 112
(same card, section 方法适配). One resblock's per-GPU shard is therefore qkv 3968x1488,
attn-out 496x3968, mlp-in 3968x1984 and mlp-out 1984x3968.

Rounding. fp16 and bf16 values come from round-to-nearest-even with subnormals kept. The
printed conversions in "AIGC 基本功|混合精度与数值稳定性-AMP" (§3.1 and §4) pin this behaviour;
see tests/golden/amp_float_formats.txt.

Seeds. Step t of workload c uses seed 1000*c + t. Each matrix draws from its own stream,
SeedSequence([seed, matrix_index]), so any one matrix can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------------------
# shapes
# --------------------------------------------------------------------------------------
D_MODEL = 3968
N_RESBLOCKS = 64
SHARDS = 8

# (name, m, n) of one resblock's per-GPU shard, d_model split 8 ways.
SHARD_SHAPES: Tuple[Tuple[str, int, int], ...] = (
    ("qkv", D_MODEL, 3 * D_MODEL // SHARDS),          # 3968 x 1488
    ("attn_out", D_MODEL // SHARDS, D_MODEL),         # 496 x 3968
    ("mlp_in", D_MODEL, 4 * D_MODEL // SHARDS),       # 3968 x 1984
    ("mlp_out", 4 * D_MODEL // SHARDS, D_MODEL),        # 1984 x 3968
)
# Unsharded resblock matrices (one GPU holding a whole resblock).
FULL_SHAPES: Tuple[Tuple[str, int, int], ...] = (
    ("qkv", D_MODEL, 3 * D_MODEL),        # 3968 x 11904
    ("proj", D_MODEL, D_MODEL),           # 3968 x 3968
    ("mlp_in", D_MODEL, 4 * D_MODEL),     # 3968 x 15872
    ("mlp_out", 4 * D_MODEL, D_MODEL),    # 15872 x 3968
)

RANK_PER_GPU = 112          # total rank 896 over 8 shards
RANK_EARLIER_TABLE = 80     # total rank 640 over 8 shards
RANK_UNSHARDED = 896


def resblock_scale(k: int) -> float:
    """Per-resblock gradient multiplier used by the multi-resblock workloads: 2**(-k/8).

    Returned as the float32 value the device array holds.
    """
    return float(np.float32(2.0 ** (-k / 8.0)))


# --------------------------------------------------------------------------------------
# dtype conversion (round-to-nearest-even, subnormals kept)
# --------------------------------------------------------------------------------------
def to_fp16(x) -> np.ndarray:
    """float64 -> IEEE binary16 in one round-to-nearest-even step; overflow gives +-inf."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16)


def to_bf16_bits(x) -> np.ndarray:
    """float -> bfloat16 bit patterns (uint16), round-to-nearest-even on the float32 value.

    NaN stays NaN (quiet bit forced), +-inf stays +-inf, finite values that round past the
    largest bfloat16 become +-inf.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32)


def to_bf16_f32(x) -> np.ndarray:
    """float -> nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(to_bf16_bits(x))


# --------------------------------------------------------------------------------------
# matrix descriptions
# --------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class MatrixSpec:
    name: str
    m: int
    n: int
    block: int          # index into the per-resblock scale array
    index: int          # position in the group (seeds its random stream)


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    config: int
    dtype: str          # "f16", "bf16" or "f32"
    rank: int
    n_blocks: int
    matrices: Tuple[MatrixSpec, ...]
    description: str

    @property
    def numel(self) -> int:
        return sum(s.m * s.n for s in self.matrices)

    @property
    def grad_bytes(self) -> int:
        return self.numel * {"f16": 2, "bf16": 2, "f32": 4}[self.dtype]


def _group(shapes, n_blocks) -> Tuple[MatrixSpec, ...]:
    out: List[MatrixSpec] = []
    for b in range(n_blocks):
        for name, m, n in shapes:
            out.append(MatrixSpec(f"rb{b}.{name}", m, n, b, len(out)))
    return tuple(out)


def workload(config: int, n_blocks: Optional[int] = None) -> WorkloadSpec:
    """The five synthetic workloads. n_blocks trims configs 3 and 4 to fewer resblocks."""
    if config == 1:
        return WorkloadSpec(1, "f32", 4, 1, (MatrixSpec("tiny", 256, 128, 0, 0),),
                            "one 256x128 fp32 N(0,1) matrix, rank 4")
    if config == 2:
        return WorkloadSpec(2, "f16", RANK_PER_GPU, 1, _group(SHARD_SHAPES, 1),
                            "one resblock per-GPU shard, fp16, per-row log-uniform scale, rank 112")
    if config == 3:
        nb = N_RESBLOCKS if n_blocks is None else n_blocks
        return WorkloadSpec(3, "f16", RANK_PER_GPU, nb, _group(SHARD_SHAPES, nb),
                            f"{nb}-resblock per-GPU shard, fp16, scales 2^(-k/8), rank 112")
    if config == 4:
        nb = N_RESBLOCKS if n_blocks is None else n_blocks
        return WorkloadSpec(4, "f16", RANK_EARLIER_TABLE, nb, _group(SHARD_SHAPES, nb),
                            f"{nb}-resblock shard, Student-t(3) near fp16 underflow, rank 80")
    if config == 5:
        return WorkloadSpec(5, "bf16", RANK_UNSHARDED, 1, _group(FULL_SHAPES, 1),
                            "unsharded resblock, bf16, planted rank-64 component, rank 896")
    raise ValueError(f"unknown workload {config}")


def step_seed(config: int, step: int) -> int:
    return 1000 * config + step


def matrix_rng(seed: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index])))


# --------------------------------------------------------------------------------------
# numpy generators (CPU; small and medium sizes)
# --------------------------------------------------------------------------------------
def row_scales(config: int, spec: MatrixSpec) -> np.ndarray:
    """Per-row magnitudes, drawn once per matrix and fixed across steps (float64, shape m)."""
    rng = matrix_rng(10_000_000 + config, spec.index)
    if config in (2, 3):
        return np.exp(rng.uniform(math.log(1e-4), 0.0, size=spec.m))
    if config == 4:
        return np.exp(rng.uniform(math.log(1e-8), math.log(1e-6), size=spec.m))
    return np.ones(spec.m)


def planted_factors(spec: MatrixSpec, rank: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Fixed rank-64 component L = A @ B for the unsharded workload, scaled so that
    ||L||_F^2 = 10 * m * n. Returned as float64 factors (A m x 64, B 64 x n)."""
    rng = matrix_rng(20_000_000, spec.index)
    A = rng.standard_normal((spec.m, rank))
    B = rng.standard_normal((rank, spec.n))
    nrm2 = float(np.linalg.norm(A @ B) ** 2)
    c = math.sqrt(10.0 * spec.m * spec.n / nrm2)
    return A * c, B


def gradient_np(wl: WorkloadSpec, spec: MatrixSpec, step: int):
    """Stored gradient of one matrix at one step, as the device dtype.

    Returns a numpy array: float16 for "f16", uint16 bf16 bit patterns for "bf16",
    float32 for "f32".
    """
    rng = matrix_rng(step_seed(wl.config, step), spec.index)
    if wl.config == 1:
        return rng.standard_normal((spec.m, spec.n)).astype(np.float32)
    if wl.config in (2, 3):
        g = rng.standard_normal((spec.m, spec.n)) * row_scales(wl.config, spec)[:, None]
        return to_fp16(g)
    if wl.config == 4:
        t = rng.standard_t(3, size=(spec.m, spec.n)) * row_scales(4, spec)[:, None]
        s = resblock_scale(spec.block)
        return to_fp16(t / s)
    if wl.config == 5:
        A, B = planted_factors(spec)
        g = rng.standard_normal((spec.m, spec.n)) + A @ B
        return to_bf16_bits(g)
    raise ValueError(wl.config)


def grad_as_f32(wl: WorkloadSpec, g: np.ndarray) -> np.ndarray:
    """Exact float32 view of a stored gradient (bf16 bits are widened)."""
    if wl.dtype == "bf16":
        return bf16_bits_to_f32(g)
    return np.asarray(g, dtype=np.float32)


def initial_q_np(wl: WorkloadSpec, spec: MatrixSpec, rank: Optional[int] = None) -> np.ndarray:
    """Step-0 warm start Q0 ~ N(0,1), n x r float32."""
    r = wl.rank if rank is None else rank
    rng = matrix_rng(30_000_000 + wl.config, spec.index)
    return rng.standard_normal((spec.n, r)).astype(np.float32)


def warm_error_np(wl: WorkloadSpec, spec: MatrixSpec, scale: float = 0.1) -> np.ndarray:
    """A synthetic non-zero error-buffer state (float32, m x n) for single-step tests that start
    from a warm state: N(0,1) times the workload's per-row magnitude times `scale`."""
    rng = matrix_rng(40_000_000 + wl.config, spec.index)
    rs = row_scales(wl.config, spec)
    return (rng.standard_normal((spec.m, spec.n)) * rs[:, None] * scale).astype(np.float32)


def exact_rank_np(m: int, n: int, rank: int, seed: int) -> np.ndarray:
    """A @ B with A m x rank, B rank x n ~ N(0,1): an exact rank-`rank` matrix (float64)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((m, rank)) @ rng.standard_normal((rank, n))


def passthrough_np(config: int, n_blocks: int, step: int = 0) -> np.ndarray:
    """Gains and biases, n_blocks x 2 x d_model float32 ~ N(0,1) * 1e-3."""
    rng = matrix_rng(50_000_000 + step_seed(config, step), 0)
    return (rng.standard_normal((n_blocks, 2, D_MODEL)) * 1e-3).astype(np.float32)


def scales_np(wl: WorkloadSpec) -> np.ndarray:
    if wl.config in (3, 4):
        return np.array([resblock_scale(k) for k in range(wl.n_blocks)], dtype=np.float32)
    return np.ones(wl.n_blocks, dtype=np.float32)


# --------------------------------------------------------------------------------------
# non-finite injection schedule for the underflow workload
# --------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Injection:
    step: int
    kind: str           # "grad", "passthrough" or "scale"
    value: float        # +inf, -inf or nan
    matrix: int = -1    # for "grad"
    row: int = 0
    col: int = 0
    block: int = 0      # for "scale"


def injection_schedule(wl: WorkloadSpec, n_steps: int = 200, p: float = 0.01,
                       min_events: int = 2) -> List[Injection]:
    """Steps that carry a non-finite value: Bernoulli(p) per step from the seed, at least
    `min_events` forced, cycling +inf, -inf, nan into one random element of one random matrix.
    Two extra steps follow the run: a NaN in a pass-through tensor and an inf scale."""
    rng = matrix_rng(60_000_000 + wl.config, 0)
    hit = rng.random(n_steps) < p
    forced = rng.choice(n_steps, size=min_events, replace=False)
    for t in forced:
        if hit.sum() >= min_events:
            break
        hit[t] = True
    values = (math.inf, -math.inf, math.nan)
    out: List[Injection] = []
    for k, t in enumerate(np.nonzero(hit)[0]):
        mi = int(rng.integers(len(wl.matrices)))
        spec = wl.matrices[mi]
        out.append(Injection(int(t), "grad", values[k % 3], mi,
                             int(rng.integers(spec.m)), int(rng.integers(spec.n))))
    out.append(Injection(n_steps, "passthrough", math.nan, row=int(rng.integers(2 * D_MODEL))))
    out.append(Injection(n_steps + 1, "scale", math.inf, block=int(rng.integers(wl.n_blocks))))
    return out


# --------------------------------------------------------------------------------------
# torch generators (device; the full-size workloads)
# --------------------------------------------------------------------------------------
def _torch_gen(device, seed: int, index: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + index * 7_919 + 12345) % (2 ** 63 - 1))
    return g


def row_scales_torch(config: int, spec: MatrixSpec, device):
    import torch
    g = _torch_gen(device, 10_000_000 + config, spec.index)
    u = torch.rand(spec.m, 1, generator=g, device=device, dtype=torch.float32)
    if config in (2, 3):
        lo, hi = math.log(1e-4), 0.0
    elif config == 4:
        lo, hi = math.log(1e-8), math.log(1e-6)
    else:
        return torch.ones(spec.m, 1, device=device)
    return torch.exp(lo + (hi - lo) * u)


def gradient_torch(wl: WorkloadSpec, spec: MatrixSpec, step: int, device, out=None,
                   rowscale=None):
    """Device-side generator for the full-size workloads (same recipe as gradient_np, drawn
    from torch's generator instead of numpy's, so the values differ from gradient_np)."""
    import torch
    g = _torch_gen(device, step_seed(wl.config, step), spec.index)
    rs = rowscale if rowscale is not None else row_scales_torch(wl.config, spec, device)
    if wl.config in (2, 3):
        x = torch.randn(spec.m, spec.n, generator=g, device=device, dtype=torch.float32)
        x.mul_(rs)
        dt = torch.float16
    elif wl.config == 4:
        # Student-t(3) = Z / sqrt(chi2_3 / 3)
        z = torch.randn(spec.m, spec.n, generator=g, device=device, dtype=torch.float32)
        c = torch.randn(3, spec.m, spec.n, generator=g, device=device, dtype=torch.float32)
        chi = c.square_().sum(0).div_(3.0).sqrt_()
        x = z.div_(chi).mul_(rs).div_(resblock_scale(spec.block))
        dt = torch.float16
    elif wl.config == 5:
        x = torch.randn(spec.m, spec.n, generator=g, device=device, dtype=torch.float32)
        A, B = planted_torch(spec, device)
        x.add_(A @ B)
        dt = torch.bfloat16
    else:
        x = torch.randn(spec.m, spec.n, generator=g, device=device, dtype=torch.float32)
        dt = torch.float32
    if out is None:
        return x.to(dt)
    out.copy_(x)
    return out


def initial_q_torch(wl: WorkloadSpec, spec: MatrixSpec, device, rank: Optional[int] = None):
    import torch
    r = wl.rank if rank is None else rank
    g = _torch_gen(device, 30_000_000 + wl.config, spec.index)
    return torch.randn(spec.n, r, generator=g, device=device, dtype=torch.float32)


def planted_torch(spec: MatrixSpec, device, rank: int = 64):
    """Rank-64 planted component for the unsharded workload on device (float32 factors)."""
    import torch
    g = _torch_gen(device, 20_000_000, spec.index)
    A = torch.randn(spec.m, rank, generator=g, device=device, dtype=torch.float32)
    B = torch.randn(rank, spec.n, generator=g, device=device, dtype=torch.float32)
    nrm2 = float((A @ B).double().square().sum())
    A.mul_(math.sqrt(10.0 * spec.m * spec.n / nrm2))
    return A, B


__all__ = [n for n in dir() if not n.startswith("_")]
