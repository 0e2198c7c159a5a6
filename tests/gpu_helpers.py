"""Shared machinery of the GPU parity tests: run the HIP path through the C ABI and the oracle
on the same inputs, and compare.

Acceptance, per matrix: relative Frobenius error of D and of E at most 2e-3 against the oracle,
and max |P^T P - I| at most 1e-4 over the non-zero columns of P. Flags and skip decisions must
be bit-exact.
"""
from __future__ import annotations

import sys
from typing import List, Optional, Sequence

import numpy as np

import oracle
import workloads as wl

REL_TOL = 2e-3
ORTH_TOL = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def orth_err(P) -> float:
    P = np.asarray(P, dtype=np.float64)
    keep = np.linalg.norm(P, axis=0) > 0
    P = P[:, keep]
    return float(np.abs(P.T @ P - np.eye(P.shape[1])).max()) if P.shape[1] else 0.0


def torch_dtype(code: str):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[code]


def to_device_grad(g_np: np.ndarray, dtype: str, ld: Optional[int] = None):
    """numpy gradient (float16 / bf16 bits / float32) -> device tensor of the same bits, with
    an optional padded leading dimension."""
    import torch
    m, n = g_np.shape
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(g_np).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(g_np))
    if ld is None or ld == n:
        return t.cuda()
    buf = torch.zeros((m, ld), dtype=t.dtype, device="cuda")
    buf[:, :n] = t.cuda()
    return buf[:, :n]


def grad_f32_from_device(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy() if t.dtype != torch.float32 else t.cpu().numpy()


class Case:
    """A group run on the GPU next to the oracle.

    mats: list of (m, n, block); grads_at(step) -> list of numpy gradients (device dtype).
    free_running: the oracle keeps its own state (float64) from the generated initial state.
    """

    def __init__(self, shapes, blocks, dtype: str, rank: int, scales: np.ndarray, q0, err0=None,
                 write_out=True, ld_pad: int = 0):
        import torch
        from rank_gradient_compression_powersgd_amd import PowerSGDGroup
        self.shapes = shapes
        self.dtype = dtype
        self.rank = rank
        self.scales_np = np.asarray(scales, dtype=np.float32)
        self.scale = torch.from_numpy(self.scales_np).cuda()
        self.ld_pad = ld_pad
        self.grads = []
        for (m, n) in shapes:
            ld = n + ld_pad if ld_pad else None
            if dtype == "bf16":
                z = np.zeros((m, n), dtype=np.uint16)
            else:
                z = np.zeros((m, n), dtype=np.float16 if dtype == "f16" else np.float32)
            self.grads.append(to_device_grad(z, dtype, ld))
        self.blocks = list(blocks)
        err_t = []
        for k, (m, n) in enumerate(shapes):
            buf = torch.zeros((m, n + ld_pad), dtype=torch.float32, device="cuda")[:, :n]
            if err0 is not None:
                buf.copy_(torch.from_numpy(np.asarray(err0[k], np.float32)).cuda())
            err_t.append(buf)
        q_t = [torch.from_numpy(np.asarray(q, np.float32)) for q in q0]
        self.group = PowerSGDGroup(self.grads, blocks, self.scale, rank, q_t, err_t, write_out)
        self.E_or = [np.zeros(sh) if err0 is None else np.asarray(err0[k], np.float64)
                     for k, sh in enumerate(shapes)]
        self.Q_or = [np.asarray(q, np.float64) for q in q0]

    def set_grads(self, grads_np: Sequence[np.ndarray]):
        import torch
        for dst, g in zip(self.grads, grads_np):
            if self.dtype == "bf16":
                src = torch.from_numpy(np.ascontiguousarray(g).view(np.int16)).view(torch.bfloat16)
            else:
                src = torch.from_numpy(np.ascontiguousarray(g))
            dst.copy_(src.cuda())
        self.cur_grads = [wl.bf16_bits_to_f32(g) if self.dtype == "bf16" else
                          np.asarray(g, dtype=np.float32) for g in grads_np]

    def gpu_step(self, passthrough=()):
        import torch
        skip = self.group.step([torch.from_numpy(np.asarray(p, np.float32)).cuda() for p in passthrough],
                               host=True)
        torch.cuda.synchronize()
        return skip

    def fetch(self):
        g = self.group
        return dict(
            E=[e.cpu().numpy() for e in g.err],
            Q=[q.cpu().numpy() for q in g.q],
            Qn=[q.cpu().numpy() for q in g.q_next],
            P=[p.cpu().numpy() for p in g.p],
            D=[o.cpu().numpy() if o is not None else None for o in g.out],
            flags=g.flags.cpu().numpy().copy(),
        )

    def oracle_step(self, passthrough=()):
        st = oracle.step_group(self.cur_grads, self.E_or, self.Q_or, self.blocks,
                               self.scales_np, passthrough)
        self.E_or = st.E_next
        self.Q_or = st.Q_next
        return st

    def close(self):
        self.group.close()


def compare_step(res, st, what="", exact_rank: bool = False, check_p: bool = True):
    """Assert one step's GPU results against the oracle's GroupStep."""
    worst = {}
    for i in range(len(res["E"])):
        rD = rel(res["D"][i], st.D[i]) if res["D"][i] is not None else 0.0
        nm = float(np.linalg.norm(st.D[i] + st.E_next[i]))       # ||M||
        if nm == 0.0:
            # M = 0: E must be exactly zero (no relative measure exists)
            rE = float(np.linalg.norm(res["E"][i]))
        elif exact_rank or np.linalg.norm(st.E_next[i]) <= 1e-8 * nm:
            # M lies in span(P) (rank(M) <= r): the oracle's E is round-off, so E is measured
            # against ||M|| instead of against itself
            rE = float(np.linalg.norm(res["E"][i] - st.E_next[i]) / nm)
        else:
            rE = rel(res["E"][i], st.E_next[i])
        rQ = rel(res["Q"][i], st.Q_next[i])
        rP = rel(res["P"][i], st.P[i])
        oe = orth_err(res["P"][i])
        for k, v in (("D", rD), ("E", rE), ("Q", rQ), ("P", rP), ("orth", oe)):
            worst[k] = max(worst.get(k, 0.0), v)
        assert rD <= REL_TOL, (what, i, "D", rD)
        assert rE <= REL_TOL, (what, i, "E", rE)
        assert rQ <= REL_TOL, (what, i, "q_next", rQ)
        if check_p:
            assert rP <= REL_TOL, (what, i, "P", rP)
        assert oe <= ORTH_TOL, (what, i, "orth", oe)
    log(f"  {what}: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    return worst
