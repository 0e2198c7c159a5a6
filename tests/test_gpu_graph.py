"""The whole step (compress, finite check without host copy, decompress/update) captured once in
a HIP graph and replayed: every replay must equal, bit for bit, the same step run eagerly on an
identical group. New gradients are written into the captured input buffers by ordinary eager
copies between replays, with a device synchronisation after each replay."""
from __future__ import annotations

import numpy as np
import pytest

import workloads as wl
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rank", [16, 160, 37, 255])
def test_step_graph_replays_match_eager(rank):
    import torch
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    dev = torch.device("cuda", 0)
    shapes = [(520, 264), (300, 512), (1000, 1032)]
    rng = np.random.default_rng(5150 + rank)
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    e0 = [(rng.standard_normal(sh) * 0.05).astype(np.float32) for sh in shapes]
    grads = [[wl.to_fp16(rng.standard_normal(sh)) for sh in shapes] for _ in range(4)]
    gains = torch.from_numpy((rng.standard_normal(2 * 3968) * 1e-3).astype(np.float32)).to(dev)
    scale = torch.tensor([0.5, 2.0], device=dev)
    blocks = [0, 1, 1]

    def group():
        g = PowerSGDGroup([torch.from_numpy(grads[0][i]).to(dev) for i in range(len(shapes))], blocks,
                          scale, rank, [torch.from_numpy(q) for q in q0],
                          [torch.from_numpy(e).to(dev) for e in e0], True)
        return g

    # every kernel of the step launched once outside the capture (code objects load lazily)
    warm = group()
    warm.step([gains], host=True)
    warm.close()
    eager, cap = group(), group()
    torch.cuda.synchronize()
    log(f"graph capture, rank {rank}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        cap.compress()
        cap.check_finite([gains])
        cap.decompress_update()
    torch.cuda.synchronize()
    # capturing ran nothing: the captured group still holds its initial state
    assert np.array_equal(cap.err[0].cpu().numpy(), e0[0])

    for t in range(len(grads)):
        for i in range(len(shapes)):
            src = torch.from_numpy(grads[t][i]).to(dev)
            eager.grads[i].copy_(src)
            cap.grads[i].copy_(src)
        assert eager.step([gains], host=True) == 0
        graph.replay()
        torch.cuda.synchronize()
        assert int(cap.skip.item()) == 0
        for name in ("err", "q", "p", "out"):
            for a, b in zip(getattr(eager, name), getattr(cap, name)):
                assert torch.equal(a, b), (t, name)
        assert torch.equal(eager.flags, cap.flags)
    # a non-finite gradient through the graph: the captured skip path zeroes every error buffer
    for i in range(len(shapes)):
        eager.grads[i].copy_(torch.from_numpy(grads[0][i]).to(dev))
        cap.grads[i].copy_(eager.grads[i])
    eager.grads[1][3, 5] = float("inf")
    cap.grads[1][3, 5] = float("inf")
    q_before = [q.clone() for q in cap.q]
    assert eager.step([gains], host=True) == 1
    graph.replay()
    torch.cuda.synchronize()
    assert int(cap.skip.item()) == 1
    for e in cap.err:
        assert float(e.abs().max()) == 0.0
    for a, b in zip(cap.q, q_before):
        assert torch.equal(a, b)
    eager.close()
    cap.close()


def test_step_with_optimizer_graph_replays_match_eager():
    """The step with the optimizer (compress, finite check, global norm and clip, decompression
    fused with the matrices' Adam update, fp32 Adam on a pass-through tensor) captured once and
    replayed three times with new gradients: parameters, moments, step count, norm, error
    buffers and warm starts equal the eager run bit for bit after every replay."""
    import torch
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    from rank_gradient_compression_powersgd_amd.binding import psgd_adam_hparams
    dev = torch.device("cuda", 0)
    rank = 24
    shapes = [(520, 264), (300, 512)]
    rng = np.random.default_rng(5170)
    q0 = [rng.standard_normal((n, rank)).astype(np.float32) for _, n in shapes]
    grads = [[wl.to_fp16(rng.standard_normal(sh)) for sh in shapes] for _ in range(3)]
    pgrads = [(rng.standard_normal(4096) * 1e-2).astype(np.float32) for _ in range(3)]
    th0 = [wl.to_fp16(rng.standard_normal(sh) * 0.02) for sh in shapes]
    hp = psgd_adam_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    scale = torch.tensor([1.0], device=dev)

    def group():
        g = PowerSGDGroup([torch.from_numpy(grads[0][i]).to(dev) for i in range(len(shapes))], [0, 0],
                          scale, rank, [torch.from_numpy(q) for q in q0])
        g.attach_adam([torch.from_numpy(t).to(dev) for t in th0],
                      [torch.zeros(sh, dtype=torch.int16, device=dev) for sh in shapes],
                      [torch.zeros(sh, dtype=torch.int16, device=dev) for sh in shapes])
        g.pass_state = (torch.full((4096,), 0.5, device=dev), torch.zeros(4096, device=dev),
                        torch.zeros(4096, device=dev), torch.from_numpy(pgrads[0]).to(dev))
        return g

    warm = group()
    warm.step_adam(hp, [warm.pass_state], max_norm=1.0)
    torch.cuda.synchronize()
    warm.close()
    eager, cap = group(), group()
    torch.cuda.synchronize()
    log("graph capture of the step with the optimizer")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        cap.step_adam(hp, [cap.pass_state], max_norm=1.0)
    torch.cuda.synchronize()
    assert int(cap.adam_step.item()) == 0             # capturing ran nothing
    for t in range(3):
        for i in range(len(shapes)):
            src = torch.from_numpy(grads[t][i]).to(dev)
            eager.grads[i].copy_(src)
            cap.grads[i].copy_(src)
        eager.pass_state[3].copy_(torch.from_numpy(pgrads[t]).to(dev))
        cap.pass_state[3].copy_(eager.pass_state[3])
        eager.step_adam(hp, [eager.pass_state], max_norm=1.0)
        graph.replay()
        torch.cuda.synchronize()
        assert int(cap.adam_step.item()) == t + 1 == int(eager.adam_step.item())
        assert torch.equal(eager.adam_norm, cap.adam_norm), t
        for name in ("params", "m1", "m2", "err", "q"):
            for a, b in zip(getattr(eager, name), getattr(cap, name)):
                assert torch.equal(a, b), (t, name)
        for a, b in zip(eager.pass_state[:3], cap.pass_state[:3]):
            assert torch.equal(a, b), (t, "pass-through")
    eager.close()
    cap.close()
