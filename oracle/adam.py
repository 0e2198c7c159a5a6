"""The optimizer step that consumes the decompressed gradient: the CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (cited by page title and section):
  [card] "Zero-Shot Text-to-Image Generation — 中文验证版", section 方法适配: most Adam moments
         are kept in a custom 16-bit format, and the update comes with gradient clipping and
         a rule that skips updates carrying non-finite values.
  [ko]   Korean summary of the same paper, section "Mixed-Precision Training": most
         parameters and Adam moments are stored in 16 bits; gains, biases, embeddings,
         unembeddings, their gradients and their Adam moments stay 32-bit.
  [amp]  "AIGC 基本功|混合精度与数值稳定性-AMP", §6.1: one AdamW update on the unscaled gradient
         with first and second moments; §6.2: the order of a mixed-precision step (unscale,
         non-finite check, global norm over every gradient, clipping, optimizer step); §4:
         clipping happens after unscaling, with threshold C on the global norm.
  [zero] "AIGC 基本功|数据并行与 ZeRO 显存切分", §4.2: a printed first Adam step (learning rate
         1e-3, betas 0.9 and 0.999, eps 1e-8) with its averaged gradient and its updated
         parameters, which pins adam_update (tests/golden/zero_adam_first_step.txt).

The step (all arithmetic in float64; g is the decompressed gradient D of a compressed matrix,
or the gradient of a 32-bit pass-through tensor):
    skip                         -> nothing changes, the step count t included
    t      <- t + 1
    N      =  sqrt(sum of g^2 over every gradient of the step)       (global norm)
    c      =  min(1, C / N)  (c = 1 when C <= 0 or N = 0)            (clipping factor)
    g'     =  c g
    m1     <- beta1 m1 + (1 - beta1) g'
    m2     <- beta2 m2 + (1 - beta2) g'^2
    theta  <- theta - lr ( (m1 / (1 - beta1^t)) / (sqrt(m2 / (1 - beta2^t)) + eps)
                           + wd theta )                              (decoupled decay, AdamW)
The update uses the new moments before they are stored; each stored value is then rounded to
its storage format.

Readings taken where the pages are silent:
  * The "custom 16-bit format" is not defined by the pages. Their concern is underflow: late
    resblocks' gradients fall below fp16's 5-bit exponent range ([card] 瓶颈), and the second
    moment holds squares of those gradients (1e-16 for a gradient of 1e-8). So both moments
    keep float32's 8-bit exponent. The first moment is bfloat16 (sign, 8 exponent bits, 7
    fraction bits). The second moment is never negative, so its format drops the sign and
    keeps 8 fraction bits: code = bits 30..15 of the float32 value ("ue8m8"), value = code
    << 15 as a float32 pattern. Both round to nearest, ties to even.
  * Parameters of compressed matrices are 16-bit (fp16 here, the gradients' format; bf16 and
    fp32 are accepted too); pass-through tensors keep fp32 parameters and moments ([ko]).
  * Where floating point decides a 16-bit code, the decision is taken from the float32 value,
    as the kernels take it: the float64 result is rounded to float32 first, then to the
    storage format.
  * Clipping covers every gradient the step updates: the decompressed gradients and the
    pass-through gradients together.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from .blockscale import bf16_bits_to_f64, f32_to_bf16_bits

__all__ = [
    "AdamHyper", "ue8m8_encode", "ue8m8_decode", "store_param", "adam_update",
    "global_norm", "clip_factor", "AdamState", "adam_group_step",
]


@dataclasses.dataclass(frozen=True)
class AdamHyper:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0


# ------------------------------------------------------------------------------------------
# storage formats
# ------------------------------------------------------------------------------------------
def ue8m8_decode(code) -> np.ndarray:
    """Exact value of ue8m8 codes: the code is bits 30..15 of a non-negative float32."""
    u = np.asarray(code, dtype=np.uint16).astype(np.uint32) << 15
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def ue8m8_encode(x) -> np.ndarray:
    """Nearest ue8m8 code of non-negative float32 values, ties to the even code. The two
    candidates are the code that truncates x and the next one up; their exact values decide.
    Values at or beyond the halfway point above the largest finite code become the infinity
    code 0xFF00."""
    x32 = np.asarray(x, dtype=np.float32)
    if np.any(np.signbit(x32) & (x32 != 0)) or np.isnan(x32).any():
        raise ValueError("ue8m8 holds non-negative numbers only")
    x32 = np.abs(x32)                                 # -0 -> +0
    lo = (x32.view(np.uint32) >> 15).astype(np.int64)
    hi = lo + 1
    vx = x32.astype(np.float64)
    vlo = ue8m8_decode(lo.astype(np.uint16))
    # the code after the largest finite one stands for 2^128, where the exponent overflows
    vhi = np.where(hi >= 0xFF00, 2.0 ** 128, ue8m8_decode(np.minimum(hi, 0xFEFF).astype(np.uint16)))
    dlo, dhi = vx - vlo, vhi - vx
    with np.errstate(invalid="ignore"):
        pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    out = np.where(pick_hi, hi, lo)
    out = np.where(np.isinf(x32), 0xFF00, out)
    return np.minimum(out, 0xFF00).astype(np.uint16)


def store_param(x64, fmt: str) -> np.ndarray:
    """Round float64 values to a storage format through float32; returns the stored values as
    float64 (exactly representable in `fmt`)."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if fmt == "f32":
        return x32.astype(np.float64)
    if fmt == "f16":
        with np.errstate(over="ignore"):
            return x32.astype(np.float16).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(f32_to_bf16_bits(x32))
    if fmt == "ue8m8":
        return ue8m8_decode(ue8m8_encode(x32))
    raise ValueError(fmt)


# ------------------------------------------------------------------------------------------
# the update
# ------------------------------------------------------------------------------------------
def adam_update(theta, m1, m2, g, t: int, hp: AdamHyper):
    """One AdamW update at step t (t >= 1) in float64, nothing rounded. Returns the new
    (theta, m1, m2)."""
    theta = np.asarray(theta, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    b1, b2 = float(hp.beta1), float(hp.beta2)
    m1 = b1 * np.asarray(m1, dtype=np.float64) + (1.0 - b1) * g
    m2 = b2 * np.asarray(m2, dtype=np.float64) + (1.0 - b2) * g * g
    m1_hat = m1 / (1.0 - b1 ** t)
    m2_hat = m2 / (1.0 - b2 ** t)
    step = m1_hat / (np.sqrt(m2_hat) + float(hp.eps)) + float(hp.weight_decay) * theta
    return theta - float(hp.lr) * step, m1, m2


def global_norm(grads: Sequence) -> float:
    """Euclidean norm over every element of every gradient."""
    return float(np.sqrt(sum(float(np.sum(np.asarray(g, dtype=np.float64) ** 2)) for g in grads)))


def clip_factor(norm: float, max_norm: float) -> float:
    """min(1, C / N); 1 when clipping is off (C <= 0) or the gradient is zero."""
    if max_norm <= 0.0 or norm <= 0.0 or norm <= max_norm:
        return 1.0
    return float(max_norm) / norm


@dataclasses.dataclass
class AdamState:
    """Stored optimizer state of one tensor: values as float64, exactly representable in
    their formats (param_fmt for theta; m1_fmt and m2_fmt for the moments)."""
    theta: np.ndarray
    m1: np.ndarray
    m2: np.ndarray
    param_fmt: str = "f16"
    m1_fmt: str = "bf16"
    m2_fmt: str = "ue8m8"


def adam_group_step(states: Sequence[AdamState], grads: Sequence, t: int, skip: bool,
                    hp_mats: AdamHyper, hp_pass: Optional[AdamHyper] = None,
                    n_mats: Optional[int] = None, max_norm: float = 0.0):
    """One optimizer step over a group: states[:n_mats] are compressed matrices (updated with
    hp_mats), the rest pass-through tensors (hp_pass, default hp_mats); grads holds the
    decompressed gradients D of the matrices, then the pass-through gradients.
    Returns (new states, new t, global norm, clipping factor); a skipped step returns the
    states unchanged (new objects), t unchanged, and norm and factor as None."""
    n_mats = len(states) if n_mats is None else n_mats
    hp_pass = hp_pass or hp_mats
    if skip:
        return [dataclasses.replace(s) for s in states], t, None, None
    t = t + 1
    norm = global_norm(grads)
    c = clip_factor(norm, max_norm)
    out: List[AdamState] = []
    for k, (s, g) in enumerate(zip(states, grads)):
        hp = hp_mats if k < n_mats else hp_pass
        th, m1, m2 = adam_update(s.theta, s.m1, s.m2, c * np.asarray(g, dtype=np.float64), t, hp)
        out.append(AdamState(store_param(th, s.param_fmt), store_param(m1, s.m1_fmt),
                             store_param(m2, s.m2_fmt), s.param_fmt, s.m1_fmt, s.m2_fmt))
    return out, t, norm, c
