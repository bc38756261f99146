"""GPU: the step captured in a HIP graph replays exactly like the step run eagerly.

The step enqueues only kernels, event records and event waits (the internal
lane stream is forked from and joined back into the caller's stream; counters
are cleared by a kernel, never by a memset), so it can be captured.  Each test
captures one step on one copy of a state, then replays the graph several times
while the same step runs eagerly on an identical copy, with other eager work
and synchronisations between the replays, and requires every replay to leave
both copies bit for bit equal.
"""

import numpy as np
import pytest

import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _state(w, seed):
    st = wl.make_state(w, seed)
    nm = len(w.matrices)
    ema = wl.make_independent_ema(w, seed + 1)
    return {
        "P": [gu.dev(p) for p in st["params"][:nm]],
        "G": [gu.dev(g) for g in wl.make_grads(w, seed, 0)],
        "M": [gu.dev(m) for m in st["moms"]],
        "E": [gu.dev(e) for e in ema[:nm]],
        "XP": [gu.dev(p) for p in st["params"][nm:]],
        "XE": [gu.dev(e) for e in ema[nm:]],
    }


def _same(a, b, keys):
    for key in keys:
        for i, (x, y) in enumerate(zip(a[key], b[key])):
            hx, hy = np.ascontiguousarray(gu.host(x)), np.ascontiguousarray(gu.host(y))
            if not np.array_equal(hx.view(np.uint32), hy.view(np.uint32)):
                return f"{key}[{i}]"
    return None


@pytest.mark.parametrize("entry,workload,schedule", [
    ("prepared", 1, "phases"),
    ("prepared_ema", 2, "phases"),
    ("prepared", 2, "chain"),
    ("static", 1, "phases"),
])
def test_captured_step_replays_like_eager(entry, workload, schedule):
    import torch
    import muon_optimizer_step_amd as ms
    w = wl.workload(workload)
    coeffs = wl.coeff_table(w, 5).tolist()
    decay = w.ema_decay if w.ema_decay is not None else 0.99
    kw = dict(lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay, coeffs=coeffs, ema_decay=decay)
    keys = ["P", "M", "E"] + (["XE"] if entry == "prepared_ema" else [])
    prev = ms.set_ns_schedule(ms.MUON_NS_SCHEDULE_CHAIN if schedule == "chain" else ms.MUON_NS_SCHEDULE_PHASES)
    try:
        a, b = _state(w, 5), _state(w, 5)

        def caller(st):
            if entry == "static":
                return lambda: ms.muon_step_static(st["P"], st["G"], st["M"], emas=st["E"], **kw)
            extra = dict(extra_emas=st["XE"], extra_params=st["XP"]) if entry == "prepared_ema" else {}
            step = ms.PreparedMuonStep(st["P"], st["G"], st["M"], emas=st["E"], **extra)
            return lambda: step(**kw)

        run_a, run_b = caller(a), caller(b)
        # first calls outside the capture: lane streams, kernel attributes, schedules
        run_a()
        run_b()
        torch.cuda.synchronize()
        gu.say(f"[graph] {entry}, workload {workload}, {schedule}: capturing one step")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_a()
        torch.cuda.synchronize()
        assert _same(a, b, keys) is None, "capturing must not run the step"
        for r in range(4):
            g.replay()
            run_b()
            # the program's own eager work between replays
            junk = torch.randn(1 << 20, device="cuda")
            float(junk.mul_(2.0).sum())
            torch.cuda.synchronize()
            diff = _same(a, b, keys)
            gu.say(f"[graph] replay {r}: {'equal' if diff is None else 'differs at ' + diff}")
            assert diff is None, f"replay {r}: {diff} differs from the eager step"
    finally:
        ms.set_ns_schedule(prev)
