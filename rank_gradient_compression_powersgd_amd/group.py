"""One group of gradient matrices compressed together, over torch device tensors.

Holds the context, the plan and the per-step device words (flags, skip), and calls the three
entry points in order. All compute happens in libpsgd.so.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

from . import binding as B


class PowerSGDGroup:
    """State of a group: per matrix G (caller-filled each step), E, Q, Q_next, P, optional D.

    grads: list of 2-D device tensors (fp16, bf16 or fp32, all the same dtype, unit row stride);
           an entry None makes that matrix in-place (its err tensor, which must then be given,
           already holds M = s_b G + E)
    blocks: per matrix index into `scale`
    scale: device fp32 tensor of per-resblock multipliers
    q0: list of n x r fp32 initial warm starts (copied)
    err: optional list of m x n fp32 device tensors used in place as the error buffers
         (unit row stride; default: new zero buffers)
    write_out: allocate D buffers and have the decompression write them
    """

    def __init__(self, grads: Sequence, blocks: Sequence[int], scale, rank: int, q0: Sequence,
                 err: Optional[Sequence] = None, write_out: bool = True, device: int = 0):
        import torch
        self.torch = torch
        self.rank = rank
        self.grads = list(grads)
        self.blocks = list(blocks)
        self.scale = scale
        if err is None and any(g is None for g in self.grads):
            raise ValueError("in-place matrices (grad None) need their err tensors")
        dev = (self.grads[0] if self.grads[0] is not None else err[0]).device
        self.err = ([torch.zeros(g.shape, dtype=torch.float32, device=dev) for g in self.grads]
                    if err is None else list(err))
        shapes = [tuple(e.shape) for e in self.err]
        self.q = [q.to(device=dev, dtype=torch.float32).contiguous().clone() for q in q0]
        self.q_next = [torch.empty_like(q) for q in self.q]
        self.p = [torch.empty((sh[0], rank), dtype=torch.float32, device=dev) for sh in shapes]
        self.out = [torch.empty(sh, dtype=torch.float32, device=dev) if write_out else None
                    for sh in shapes]
        self.flags = torch.zeros(len(self.grads), dtype=torch.uint8, device=dev)
        self.skip = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ctx = B.psgd_create(device, rank)
        mats = [B.make_matrix(g, e, q, qn, p, b, o) for g, e, q, qn, p, b, o in
                zip(self.grads, self.err, self.q, self.q_next, self.p, self.blocks, self.out)]
        given = [g for g in self.grads if g is not None]
        self.plan = B.psgd_plan_create(self.ctx, mats,
                                       B.dtype_code(given[0].dtype) if given else B.PSGD_F32,
                                       int(scale.numel()))

    def compress(self, stream=None):
        B.psgd_compress(self.ctx, self.plan, self.scale, self.flags, stream)

    def check_finite(self, passthrough: Sequence = (), host: bool = False, stream=None):
        return B.psgd_check_finite(self.ctx, self.plan, self.flags, passthrough, self.scale,
                                   self.skip, host, stream)

    def decompress_update(self, stream=None):
        B.psgd_decompress_update(self.ctx, self.plan, self.scale, self.skip, stream)

    def counters(self):
        """(steps decompressed, steps skipped): the plan's device counters, copied to the host
        after a device synchronisation."""
        import ctypes
        self.torch.cuda.synchronize()
        addr = B.psgd_plan_counters(self.plan)
        out = (ctypes.c_int64 * 2)()
        hip = ctypes.CDLL("libamdhip64.so.7")
        hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        err = hip.hipMemcpy(ctypes.addressof(out), addr, 16, 2)          # device to host
        if err != 0:
            raise RuntimeError(f"hipMemcpy of the step counters failed ({err})")
        return int(out[0]), int(out[1])

    def reset_errors(self, stream=None):
        """E = 0 for every matrix: resuming from a checkpoint, which holds no error buffers."""
        B.psgd_reset_errors(self.ctx, self.plan, stream)

    # ---- optimizer ---------------------------------------------------------------------
    def attach_adam(self, params: Sequence, m1: Sequence, m2: Sequence):
        """Attach per-matrix optimizer state (caller-owned device tensors, updated in place):
        params m x n (fp16, bf16 or fp32), m1 and m2 m x n 16-bit codes (bf16 and ue8m8)."""
        torch = self.torch
        self.params, self.m1, self.m2 = list(params), list(m1), list(m2)
        opt = [B.make_adam_matrix(p, a, b) for p, a, b in zip(self.params, self.m1, self.m2)]
        B.psgd_adam_attach(self.ctx, self.plan, opt, B.dtype_code(self.params[0].dtype))
        dev = self.flags.device
        self.adam_step = torch.zeros(1, dtype=torch.int32, device=dev)
        self.adam_norm = torch.zeros(2, dtype=torch.float32, device=dev)

    def step_adam(self, hp, passthrough: Sequence = (), hp_pass=None, max_norm: float = 0.0,
                  host: bool = False, stream=None):
        """One step with the optimizer: compress, finite check, global norm and clipping,
        decompression fused with the matrices' Adam update, fp32 Adam on the pass-through
        tensors. passthrough: (param, m1, m2, grad) fp32 tensors; their gradients take part in
        the finite check and the global norm."""
        self.compress(stream)
        grads = [t[3] for t in passthrough]
        s = self.check_finite(grads, host, stream)
        ts = [B.make_adam_tensor(*t) for t in passthrough]
        B.psgd_adam_prepare(self.ctx, self.plan, ts, max_norm, self.skip, self.adam_step, self.adam_norm, stream)
        B.psgd_decompress_adam(self.ctx, self.plan, self.scale, self.skip, self.adam_step, self.adam_norm, hp,
                               stream)
        if ts:
            B.psgd_adam_update(self.ctx, ts, self.skip, self.adam_step, self.adam_norm, hp_pass or hp, stream)
        return s

    def step(self, passthrough: Sequence = (), host: bool = False, stream=None):
        self.compress(stream)
        s = self.check_finite(passthrough, host, stream)
        self.decompress_update(stream)
        return s

    def close(self):
        if getattr(self, "plan", None):
            B.psgd_plan_destroy(self.plan)
            self.plan = None
        if getattr(self, "ctx", None):
            B.psgd_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
