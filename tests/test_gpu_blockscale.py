"""GPU parity of the block-boundary gradient scaling (psgd_block_grad_enter / _exit) against
the float64 oracle (oracle/blockscale.py): bit-exact on every element, NaN positions compared
as NaN (the method fixes no NaN payload), flags exact. Sizes run from empty and ragged up to
one sequence of activations per GPU (1280 tokens x d_model 3968)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

TOKENS_X_DMODEL = 1280 * 3968          # 256 text + 1024 image tokens, d_model 3968


def _ctx():
    import rank_gradient_compression_powersgd_amd as psgd
    return psgd, psgd.psgd_create(0, 1)


def _codes16(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_codes(x, dt) -> np.ndarray:
    return x.view(np.uint16) if dt == "f16" else x


def _inputs(n, seed):
    rng = np.random.default_rng(seed)
    dx = (rng.standard_normal(n) * 10.0 ** rng.uniform(-9, 0, n)).astype(np.float32)
    if n > 16:
        idx = rng.choice(n, 6, replace=False)
        dx[idx[:2]] = np.inf
        dx[idx[2]] = -np.inf
        dx[idx[3:5]] = np.nan
        dx[idx[5]] = 0.0
    return dx


def _same_bits_or_nan(got_bits: np.ndarray, want_bits: np.ndarray, isnan_got, isnan_want, what):
    assert np.array_equal(isnan_got, isnan_want), (what, "NaN positions differ")
    keep = ~isnan_want
    bad = np.nonzero(got_bits[keep] != want_bits[keep])[0]
    assert bad.size == 0, (what, int(bad.size), bad[:5])


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("n,S", [(0, 1024.0), (1, 3.0), (7, 0.7), (8, 2.0 ** 20), (1000003, 3.0),
                                 (TOKENS_X_DMODEL, 2.0 ** 16), (TOKENS_X_DMODEL, 12345.678)])
def test_enter_then_exit_bit_exact(dt, n, S):
    import torch
    psgd, ctx = _ctx()
    dev = torch.device("cuda", 0)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    seed = 500 + n % 1000 + int(S) % 97
    log(f"block scaling {dt} n={n} S={S} seed={seed}")
    dx = _inputs(n, seed)
    s32 = np.float32(S)
    scale = torch.tensor([s32], device=dev)
    dx_d = torch.from_numpy(dx).to(dev)
    out = torch.empty(n, dtype=tdt, device=dev)
    psgd.psgd_block_grad_enter(ctx, dx_d, scale, out)
    torch.cuda.synchronize()
    want = _oracle_codes(oracle.block_grad_enter(dx, float(s32), dt), dt)
    got = _codes16(out)
    if dt == "f16":
        nan_g, nan_w = np.isnan(got.view(np.float16)), np.isnan(want.view(np.float16))
    else:
        nan_g, nan_w = np.isnan(oracle.bf16_bits_to_f64(got)), np.isnan(oracle.bf16_bits_to_f64(want))
    _same_bits_or_nan(got, want, nan_g, nan_w, "enter")

    # leaving the block: the block's output is stood in for by the entering codes (they hold
    # inf, NaN, zeros and subnormals), added onto a fresh fp32 residual gradient
    rng = np.random.default_rng(seed + 1)
    res = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    res_d = torch.from_numpy(res).to(dev)
    flag = torch.zeros(1, dtype=torch.uint8, device=dev)
    psgd.psgd_block_grad_exit(ctx, res_d, out, scale, flag)
    torch.cuda.synchronize()
    g_or = want.view(np.float16) if dt == "f16" else want
    want_dx, want_flag = oracle.block_grad_exit(res, g_or, float(s32), dt)
    got_dx = res_d.cpu().numpy()
    _same_bits_or_nan(got_dx.view(np.uint32), want_dx.view(np.uint32), np.isnan(got_dx), np.isnan(want_dx), "exit")
    assert bool(flag.item()) == want_flag
    assert not np.isnan(got_dx).any()           # non-finite block outputs never reach dx
    psgd.psgd_destroy(ctx)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_exit_flag_semantics(dt):
    """The flag is set by a non-finite value in the main part or in the n % 8 tail, and a later
    call with finite values leaves it set (several boundaries can share one flag)."""
    import torch
    psgd, ctx = _ctx()
    dev = torch.device("cuda", 0)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    n = 4099                                     # 512 groups of 8 and a tail of 3
    scale = torch.tensor([np.float32(4.0)], device=dev)
    for pos in (None, 17, n - 1):
        g = torch.randn(n, device=dev).to(tdt)
        if pos is not None:
            g[pos] = float("inf")
        dx = torch.zeros(n, dtype=torch.float32, device=dev)
        flag = torch.zeros(1, dtype=torch.uint8, device=dev)
        psgd.psgd_block_grad_exit(ctx, dx, g, scale, flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == (0 if pos is None else 1), pos
        if pos is not None:
            assert float(dx[pos]) == 0.0
            psgd.psgd_block_grad_exit(ctx, dx, torch.ones(n, dtype=tdt, device=dev), scale, flag)
            torch.cuda.synchronize()
            assert int(flag.item()) == 1
    # flag may be omitted
    psgd.psgd_block_grad_exit(ctx, torch.zeros(8, device=dev), torch.ones(8, dtype=tdt, device=dev), scale, None)
    torch.cuda.synchronize()
    psgd.psgd_destroy(ctx)


def test_scaling_rescues_underflow():
    """Gradients of 1e-8 flush to zero in fp16 (printed in the AMP page's §4 demo); entering
    the block with S_b = 2^16 keeps them, and leaving it restores them within fp16's 2^-11."""
    import torch
    psgd, ctx = _ctx()
    dev = torch.device("cuda", 0)
    x = torch.full((4096,), 1e-8, dtype=torch.float32, device=dev)
    out = torch.empty(4096, dtype=torch.float16, device=dev)
    psgd.psgd_block_grad_enter(ctx, x, torch.tensor([1.0], device=dev), out)
    torch.cuda.synchronize()
    assert float(out.float().abs().max()) == 0.0
    scale = torch.tensor([2.0 ** 16], device=dev)
    psgd.psgd_block_grad_enter(ctx, x, scale, out)
    back = torch.zeros(4096, dtype=torch.float32, device=dev)
    psgd.psgd_block_grad_exit(ctx, back, out, scale, None)
    torch.cuda.synchronize()
    err = (back.double() - 1e-8).abs().max().item()
    assert err <= 2.0 ** -11 * 1e-8 + 1e-16, err
    psgd.psgd_destroy(ctx)


def test_block_arguments_rejected():
    import torch
    psgd, ctx = _ctx()
    lib = psgd.load_library()
    dev = torch.device("cuda", 0)
    dx = torch.zeros(64, dtype=torch.float32, device=dev)
    out = torch.zeros(64, dtype=torch.float16, device=dev)
    scale = torch.ones(1, device=dev)
    vp = ctypes.c_void_p
    s = int(torch.cuda.current_stream().cuda_stream)
    # misaligned dx (4 bytes past a 16-byte boundary)
    assert lib.psgd_block_grad_enter(ctx, vp(dx.data_ptr() + 4), 8, vp(scale.data_ptr()),
                                     vp(out.data_ptr()), psgd.PSGD_F16, vp(s)) == 1
    # fp32 is not a block gradient type
    assert lib.psgd_block_grad_enter(ctx, vp(dx.data_ptr()), 8, vp(scale.data_ptr()),
                                     vp(out.data_ptr()), psgd.PSGD_F32, vp(s)) == 2
    assert lib.psgd_block_grad_exit(ctx, vp(dx.data_ptr()), None, 8, vp(scale.data_ptr()),
                                    psgd.PSGD_F16, None, vp(s)) == 1
    assert lib.psgd_block_grad_exit(ctx, vp(dx.data_ptr()), vp(out.data_ptr()), -1, vp(scale.data_ptr()),
                                    psgd.PSGD_F16, None, vp(s)) == 1
    # the fused boundary: misaligned out, missing second scale, fp32
    assert lib.psgd_block_grad_exit_enter(ctx, vp(dx.data_ptr()), vp(out.data_ptr()), 8, vp(scale.data_ptr()),
                                          vp(scale.data_ptr()), vp(out.data_ptr() + 2), psgd.PSGD_F16, None, vp(s)) == 1
    assert lib.psgd_block_grad_exit_enter(ctx, vp(dx.data_ptr()), vp(out.data_ptr()), 8, vp(scale.data_ptr()),
                                          None, vp(out.data_ptr()), psgd.PSGD_F16, None, vp(s)) == 1
    assert lib.psgd_block_grad_exit_enter(ctx, vp(dx.data_ptr()), vp(out.data_ptr()), 8, vp(scale.data_ptr()),
                                          vp(scale.data_ptr()), vp(out.data_ptr()), psgd.PSGD_F32, None, vp(s)) == 2
    # n = 0 is a no-op even with NULL pointers
    assert lib.psgd_block_grad_exit(ctx, None, None, 0, None, psgd.PSGD_BF16, None, vp(s)) == 0
    assert lib.psgd_block_grad_exit_enter(ctx, None, None, 0, None, None, None, psgd.PSGD_F16, None, vp(s)) == 0
    torch.cuda.synchronize()
    psgd.psgd_destroy(ctx)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("n", [1, 7, 1000003, TOKENS_X_DMODEL])
def test_exit_enter_fused(dt, n):
    """The boundary between block b and block b - 1 in one pass equals leaving block b and
    entering block b - 1 as two calls: against the oracle (bit for bit, NaN positions as NaN)
    and against the two library calls."""
    import torch
    psgd, ctx = _ctx()
    dev = torch.device("cuda", 0)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    seed = 900 + n % 1000
    log(f"block boundary fused {dt} n={n} seed={seed}")
    rng = np.random.default_rng(seed)
    s_exit, s_enter = np.float32(4096.0), np.float32(2896.309)
    dx0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    g_src = _inputs(n, seed + 1) * np.float32(1e4)
    g_codes = oracle.block_grad_enter(g_src, 1.0, dt)      # the block's 16-bit output (Inf/NaN kept)
    g_t = torch.from_numpy(g_codes.view(np.int16) if dt == "f16" else g_codes.view(np.int16)).to(dev).view(tdt)
    se, sn = torch.tensor([s_exit], device=dev), torch.tensor([s_enter], device=dev)
    dx = torch.from_numpy(dx0).to(dev)
    out = torch.empty(n, dtype=tdt, device=dev)
    flag = torch.zeros(1, dtype=torch.uint8, device=dev)
    psgd.psgd_block_grad_exit_enter(ctx, dx, g_t, se, sn, out, flag)
    # the same through the two calls
    dx2 = torch.from_numpy(dx0).to(dev)
    out2 = torch.empty(n, dtype=tdt, device=dev)
    flag2 = torch.zeros(1, dtype=torch.uint8, device=dev)
    psgd.psgd_block_grad_exit(ctx, dx2, g_t, se, flag2)
    psgd.psgd_block_grad_enter(ctx, dx2, sn, out2)
    torch.cuda.synchronize()
    want_dx, want_flag = oracle.block_grad_exit(dx0, g_codes, float(s_exit), dt)
    want_out = _oracle_codes(oracle.block_grad_enter(want_dx, float(s_enter), dt), dt)
    got_dx, got_out = dx.cpu().numpy(), _codes16(out)
    _same_bits_or_nan(got_dx.view(np.uint32), want_dx.view(np.uint32), np.isnan(got_dx), np.isnan(want_dx), "dx")
    if dt == "f16":
        nan_g, nan_w = np.isnan(got_out.view(np.float16)), np.isnan(want_out.view(np.float16))
    else:
        nan_g, nan_w = np.isnan(oracle.bf16_bits_to_f64(got_out)), np.isnan(oracle.bf16_bits_to_f64(want_out))
    _same_bits_or_nan(got_out, want_out, nan_g, nan_w, "out")
    assert bool(flag.item()) == want_flag == bool(flag2.item())
    assert np.array_equal(got_dx.view(np.uint32), dx2.cpu().numpy().view(np.uint32))
    assert np.array_equal(got_out, _codes16(out2))
    psgd.psgd_destroy(ctx)
