"""GPU: muon_step_ema, the Muon step with the other parameters' EMA in the same call.

Its results must be bit for bit those of muon_step followed by ema_update on
the other tensors (both schedules, with and without update outputs), and the
other tensors' EMA must match the float64 oracle's EMA to 1e-6.
"""

import numpy as np
import pytest

import oracle.muon as om
import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint32), np.ascontiguousarray(b).view(np.uint32))


def _state(w, seed):
    st = wl.make_state(w, seed)
    nm = len(w.matrices)
    ema = wl.make_independent_ema(w, seed + 1)   # no element trivially equal to its parameter
    return {
        "P": [gu.dev(p) for p in st["params"][:nm]],
        "G": [gu.dev(g) for g in wl.make_grads(w, seed, 0)],
        "M": [gu.dev(m) for m in st["moms"]],
        "E": [gu.dev(e) for e in ema[:nm]],
        "XP": [gu.dev(p) for p in st["params"][nm:]],
        "XE": [gu.dev(e) for e in ema[nm:]],
    }


@pytest.mark.parametrize("schedule", ["phases", "chain"])
@pytest.mark.parametrize("with_out", [False, True])
def test_step_ema_equals_step_then_ema_update(schedule, with_out):
    import torch
    import muon_optimizer_step_amd as ms
    w = wl.workload(2)
    decay = w.ema_decay
    coeffs = wl.coeff_table(w, 7).tolist()
    prev = ms.set_ns_schedule(ms.MUON_NS_SCHEDULE_CHAIN if schedule == "chain" else ms.MUON_NS_SCHEDULE_PHASES)
    try:
        gu.say(f"[step_ema] {schedule}, update outputs {with_out}")
        a, b = _state(w, 7), _state(w, 7)
        oa = [torch.empty_like(p) for p in a["P"]] if with_out else None
        ob = [torch.empty_like(p) for p in b["P"]] if with_out else None
        kw = dict(lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay, coeffs=coeffs, ema_decay=decay)
        ms.muon_step(a["P"], a["G"], a["M"], update_outs=oa, emas=a["E"], **kw)
        ms.ema_update(a["XE"], a["XP"], decay)
        ms.muon_step(b["P"], b["G"], b["M"], update_outs=ob, emas=b["E"], extra_emas=b["XE"], extra_params=b["XP"],
                     **kw)
        torch.cuda.synchronize()
        for key in ("P", "M", "E", "XE"):
            for i, (x, y) in enumerate(zip(a[key], b[key])):
                assert _bits_equal(gu.host(x), gu.host(y)), (key, i)
        if with_out:
            for i, (x, y) in enumerate(zip(oa, ob)):
                assert _bits_equal(gu.host(x), gu.host(y)), ("O", i)
        # the other tensors' EMA against the oracle (the parameters are not touched by the step)
        worst = 0.0
        st = wl.make_state(w, 7)
        ema = wl.make_independent_ema(w, 8)
        nm = len(w.matrices)
        for e_in, p_in, e_gpu in zip(ema[nm:], st["params"][nm:], b["XE"]):
            want = om.ema_update(e_in, p_in, gu.f32(decay))
            worst = max(worst, gu.rel_max(gu.host(e_gpu), want))
        gu.say(f"[step_ema] {len(b['XE'])} other tensors, worst EMA error {worst:.2e}")
        assert worst <= gu.ELEM_TOL
    finally:
        ms.set_ns_schedule(prev)


def test_prepared_step_with_extra_ema_and_empty_list():
    import torch
    import muon_optimizer_step_amd as ms
    w = wl.workload(1)
    coeffs = wl.coeff_table(w, 3).tolist()
    a, b = _state(w, 3), _state(w, 3)
    extra_p = [gu.dev(np.random.default_rng(5).standard_normal(1000).astype(np.float32)) for _ in range(3)]
    extra_a = [gu.dev(np.random.default_rng(6 + i).standard_normal(1000).astype(np.float32)) for i in range(3)]
    extra_b = [t.clone() for t in extra_a]
    kw = dict(lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay, coeffs=coeffs, ema_decay=0.99)
    step = ms.PreparedMuonStep(b["P"], b["G"], b["M"], emas=b["E"], extra_emas=extra_b, extra_params=extra_p)
    for _ in range(2):
        ms.muon_step(a["P"], a["G"], a["M"], emas=a["E"], **kw)
        ms.ema_update(extra_a, extra_p, 0.99)
        step(**kw)
    torch.cuda.synchronize()
    for x, y in zip(a["P"] + a["M"] + a["E"] + extra_a, b["P"] + b["M"] + b["E"] + extra_b):
        assert _bits_equal(gu.host(x), gu.host(y))
    # an empty extra list is muon_step itself
    c = _state(w, 3)
    ms.muon_step(c["P"], c["G"], c["M"], emas=c["E"], extra_emas=[], extra_params=[], **kw)
    d = _state(w, 3)
    ms.muon_step(d["P"], d["G"], d["M"], emas=d["E"], **kw)
    torch.cuda.synchronize()
    for x, y in zip(c["P"] + c["E"], d["P"] + d["E"]):
        assert _bits_equal(gu.host(x), gu.host(y))


def test_prepared_ema_equals_ema_update():
    import torch
    import muon_optimizer_step_amd as ms
    rng = np.random.default_rng(21)
    sizes = [1, 5, 4096, 4097, 123457, 300000]
    p_h = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    e_h = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    P = [gu.dev(x) for x in p_h]
    A = [gu.dev(x) for x in e_h]
    B = [gu.dev(x) for x in e_h]
    prepared = ms.PreparedEma(B, P)
    for decay in (0.9965, 0.5):
        ms.ema_update(A, P, decay)
        prepared(decay)
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(A, B)):
        assert _bits_equal(gu.host(x), gu.host(y)), i
    # and against the oracle, two updates in a row
    for i, (e0, p0) in enumerate(zip(e_h, p_h)):
        want = om.ema_update(om.ema_update(e0, p0, gu.f32(0.9965)), p0, gu.f32(0.5))
        assert gu.rel_max(gu.host(B[i]), want) <= gu.ELEM_TOL, i
