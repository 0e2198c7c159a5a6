"""Host logic of the seeded workload generators (no GPU)."""
import math

import numpy as np

import workloads as wl


def test_injection_schedule_layout():
    """The underflow workload's schedule: Bernoulli(0.01) gradient events inside the 200 steps
    (at least two), cycling +inf, -inf, NaN, each on a valid element of a valid matrix; then a
    NaN pass-through element at step 200 and an inf scale at step 201."""
    w = wl.workload(4)
    ev = wl.injection_schedule(w, 200)
    grad = [e for e in ev if e.kind == "grad"]
    assert len(grad) >= 2
    assert all(0 <= e.step < 200 for e in grad)
    assert [e.step for e in grad] == sorted({e.step for e in grad})
    for k, e in enumerate(grad):
        want = (math.inf, -math.inf, math.nan)[k % 3]
        assert (math.isnan(want) and math.isnan(e.value)) or e.value == want
        spec = w.matrices[e.matrix]
        assert 0 <= e.row < spec.m and 0 <= e.col < spec.n
    assert ev[-2].step == 200 and ev[-2].kind == "passthrough" and math.isnan(ev[-2].value)
    assert 0 <= ev[-2].row < 2 * wl.D_MODEL * w.n_blocks
    assert ev[-1].step == 201 and ev[-1].kind == "scale" and ev[-1].value == math.inf
    assert 0 <= ev[-1].block < w.n_blocks
    assert wl.injection_schedule(w, 200) == ev           # seeded


def test_injection_schedule_forces_events():
    """With p = 0 every event comes from the forced draws, which must all be distinct steps."""
    w = wl.workload(4)
    for n in (3, 10, 200):
        ev = [e for e in wl.injection_schedule(w, n, p=0.0, min_events=3) if e.kind == "grad"]
        assert len(ev) == 3 and len({e.step for e in ev}) == 3
    ev = [e for e in wl.injection_schedule(w, 50, p=1.0, min_events=2) if e.kind == "grad"]
    assert len(ev) == 50
