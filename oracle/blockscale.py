"""Per-resblock gradient scaling at the block boundaries of backprop: the CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (cited by page title and section):
  [ko]   Korean summary of "Zero-Shot Text-to-Image Generation" (only-wanna.tistory.com),
         section "Mixed-Precision Training": every resblock scales the gradient by its own
         factor when backprop enters it and unscales it when backprop leaves it, and Inf/NaN
         values are replaced by 0 there so that they do not spread to other blocks.
  [card] "Zero-Shot Text-to-Image Generation — 中文验证版", section 方法适配: each resblock
         has its own gradient scale factor.
  [amp]  "AIGC 基本功|混合精度与数值稳定性-AMP" (jefxiong.cn), §3.1 and §4: the 16-bit formats
         and the scale-quantise-unscale demo that pins these functions.

Readings taken where the pages are silent:
  * The gradient travelling between blocks (the residual-stream gradient) is float32 in true
    units; inside block b it is 16-bit and multiplied by S_b. Unscaling back to 16 bits in
    true units would bring back the underflow the scaling avoids, so leaving a block divides
    by S_b in float32 and adds the result to the float32 residual-stream gradient.
  * Entering: out = to16(fp32(S_b * dx)): the product is rounded to float32, then converted to
    fp16 or bf16 with round-to-nearest-even (subnormals kept, overflow to inf).
  * Leaving: dx += fp32(g / S_b) for every finite element g of the block's 16-bit output, and
    += 0 where g is inf or NaN. The division and the addition are float32 operations, each
    rounded once. The boundary flag is set when any g was non-finite (it reports which block
    overflowed, for the caller's choice of the next S_b; the pages give no rule for that).
  * The parameter gradients the block produces are scaled by S_b as well; the compression
    step's per-resblock multiplier s_b is 1 / S_b.

The float64 evaluation below is exact up to the float32 roundings it names: a product of two
float32 values is exact in float64, and a quotient or sum rounded first to float64 and then to
float32 equals the once-rounded float32 result (53 >= 2 * 24 + 2 bits).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

__all__ = ["f32_to_bf16_bits", "bf16_bits_to_f64", "block_grad_enter", "block_grad_exit"]


def f32_to_bf16_bits(x) -> np.ndarray:
    """bfloat16 code of float32 values, round to nearest, ties to even on the upper 16 bits;
    NaN stays NaN (quiet), inf stays inf."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    exp_all_ones = (b & 0x7F800000) == 0x7F800000
    is_nan = exp_all_ones & ((b & 0x007FFFFF) != 0)
    lsb = (b >> 16) & 1
    rounded = ((b + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan_code = ((b >> 16) | 0x0040) & 0xFFFF
    return np.where(is_nan, nan_code, rounded).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 codes (the upper half of a float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def _to16(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return x32.astype(np.float16)                   # IEEE RNE, subnormals, overflow to inf
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def _from16(g, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return np.asarray(g, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(g)
    raise ValueError(dtype)


def block_grad_enter(dx, scale: float, dtype: str = "f16") -> np.ndarray:
    """16-bit input of a block's backward pass: to16(fp32(S_b * dx)).
    Returns float16 values for "f16" and uint16 bfloat16 codes for "bf16"."""
    s = np.float64(np.float32(scale))
    prod = (s * np.asarray(dx, dtype=np.float32).astype(np.float64)).astype(np.float32)
    return _to16(prod, dtype)


def block_grad_exit(dx, g, scale: float, dtype: str = "f16") -> Tuple[np.ndarray, bool]:
    """Leave a block: dx + fp32(g / S_b) over the finite elements of the block's 16-bit output
    g (non-finite elements add 0). Returns (new float32 dx, whether any g was non-finite)."""
    gv = _from16(g, dtype)
    finite = np.isfinite(gv)
    s = np.float64(np.float32(scale))
    q = np.where(finite, gv, 0.0) / s
    q32 = q.astype(np.float32).astype(np.float64)
    out = (np.asarray(dx, dtype=np.float32).astype(np.float64) + q32).astype(np.float32)
    return out, bool((~finite).any())
