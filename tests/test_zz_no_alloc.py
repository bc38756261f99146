"""muon_step_static (the allocation-free entry point) against muon_step.

Two calls in a row through the C ABI, the second with fewer and smaller
matrices, each compared element by element with muon_step on a caller
workspace (the same kernels: bit-identical), and with the float64 oracle to the
parity bar.  Also: a call that needs more than the static workspace is rejected
before anything is enqueued.
"""

import numpy as np
import pytest

import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _inputs(shapes, seed):
    rng = np.random.default_rng(seed)
    mats = [(0.02 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    grads = [(1e-3 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    moms = [(1e-3 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    emas = [(0.02 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    return mats, grads, moms, emas


def _run(entry, mats, grads, moms, emas, coeffs):
    import torch
    import muon_optimizer_step_amd as ms
    P = [gu.dev(x) for x in mats]
    G = [gu.dev(x) for x in grads]
    M = [gu.dev(x) for x in moms]
    E = [gu.dev(x) for x in emas]
    O = [torch.full_like(p, float("nan")) for p in P]
    fn = ms.muon_step_static if entry == "static" else ms.muon_step
    fn(P, G, M, lr=0.022, momentum=0.99, weight_decay=0.105, coeffs=coeffs, update_outs=O, emas=E,
       ema_decay=0.9965)
    torch.cuda.synchronize()
    return [gu.host(t) for t in P + M + O + E]


@pytest.mark.parametrize("schedule", ["phases", "chain"])
def test_static_workspace_matches_caller_workspace(schedule):
    import muon_optimizer_step_amd as ms
    prev = ms.set_ns_schedule(ms.MUON_NS_SCHEDULE_CHAIN if schedule == "chain" else ms.MUON_NS_SCHEDULE_PHASES)
    try:
        coeffs = [list(wl.STANDARD_TRIPLE)] * 5
        # one layer of the 512-wide model (with a compensated 96-wide matrix), then a smaller set
        calls = [[(512, 512), (256, 512), (256, 512), (512, 512), (2048, 512), (512, 2048), (96, 200)],
                 [(300, 200), (512, 384), (64, 64)]]
        for k, shapes in enumerate(calls):
            assert ms.workspace_size(shapes) <= ms._lib.MUON_STATIC_WORKSPACE_BYTES
            mats, grads, moms, emas = _inputs(shapes, 100 + k)
            gu.say(f"[no-alloc] {schedule} call {k}: {len(shapes)} matrices")
            got = _run("static", mats, grads, moms, emas, coeffs)
            want = _run("workspace", mats, grads, moms, emas, coeffs)
            for a, b in zip(got, want):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
            n = len(shapes)
            w_gpu, m_gpu, o_gpu, e_gpu = got[:n], got[n:2 * n], got[2 * n:3 * n], got[3 * n:]
            gu.check_fused_ema(emas, w_gpu, e_gpu, 0.9965, label="static")
            for i, (r, c) in enumerate(shapes):
                tol = gu.NS_TOL_BF16 if min(r, c) >= 192 else gu.NS_TOL_BF16X3
                gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.022, momentum=0.99,
                                wd=0.105, coeffs=coeffs, nesterov=True, row_norm=True, ns_tol=tol,
                                label=f"static {r}x{c}")
    finally:
        ms.set_ns_schedule(prev)


def test_static_workspace_rejects_what_does_not_fit():
    import torch
    import muon_optimizer_step_amd as ms
    shapes = [(2048, 512)] * 30
    assert ms.workspace_size(shapes) > ms._lib.MUON_STATIC_WORKSPACE_BYTES
    P = [torch.zeros(s, device="cuda") for s in shapes]
    before = [p.clone() for p in P]
    with pytest.raises(ms.MuonError) as ei:
        ms.muon_step_static(P, [p.clone() for p in P], [p.clone() for p in P], lr=0.1, momentum=0.9,
                            weight_decay=0.0, coeffs=[[3.4445, -4.775, 2.0315]])
    assert ei.value.code == ms._lib.MUON_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(P, before))
