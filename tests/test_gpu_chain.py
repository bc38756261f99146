"""GPU parity of the persistent Newton-Schulz chain (MUON_NS_SCHEDULE_CHAIN).

The chain runs every NS iteration of the base-precision bf16 matrices in one
launch, each matrix bound to one XCD, tiles taken in dependency order.  It must
meet the same bars as the per-phase schedule: O within 2e-2 relative Frobenius
of the float64 oracle for every matrix, M', W' (given O) and E' (given W')
within 1e-6, deterministic and independent of the workspace contents.  Mixed
calls (compensated groups below a short side of 192 beside chain groups) run
both schedules in one step.
"""

import numpy as np
import pytest

import workloads as wl
from tests import gpu_util as gu
from tests.test_gpu_parity import _check_ema, _run_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def chain_schedule():
    import muon_optimizer_step_amd as ms
    prev = ms.set_ns_schedule(ms.MUON_NS_SCHEDULE_CHAIN)
    yield
    ms.set_ns_schedule(prev)


def test_chain_one_layer():
    _run_workload(1, wl.PRIMARY_SEED)


def test_chain_full_model_512d_with_ema():
    w, st, w_gpu = _run_workload(2, wl.PRIMARY_SEED)
    _check_ema(w, st, w_gpu, w.ema_decay)


def test_chain_full_model_1024d():
    _run_workload(3, wl.PRIMARY_SEED)


def test_chain_deterministic_and_workspace_contents_do_not_matter():
    import torch
    import muon_optimizer_step_amd as ms
    w = wl.workload(2)
    st = wl.make_state(w, 11)
    grads = wl.make_grads(w, 11, 0)
    nm = len(w.matrices)
    shapes = [(r, c) for _, r, c in w.matrices]
    nbytes = ms.workspace_size(shapes)
    std = [list(wl.STANDARD_TRIPLE)] * 5
    outs = []
    for fill in (0, 0xFF, 0x7F):   # zeros, NaN patterns, large finite values
        gu.say(f"[chain] workspace fill {fill:#x}")
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        P = [gu.dev(p) for p in st["params"][:nm]]
        M = [gu.dev(m) for m in st["moms"]]
        O = [torch.empty_like(p) for p in P]
        E = [gu.dev(e) for e in wl.make_independent_ema(w, 12)[:nm]]
        ms.muon_step(P, [gu.dev(g) for g in grads], M, lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay,
                     coeffs=std, update_outs=O, emas=E, ema_decay=0.9965, workspace=ws)
        torch.cuda.synchronize()
        outs.append([gu.host(t) for t in P + M + O + E])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("triple", [(0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (1.0, 0.0, 0.0), (0.5, -0.25, 0.125)])
def test_chain_single_iteration_mixed_with_compensated_groups(triple):
    """One iteration that isolates one product, wide / tall / square chain shapes beside compensated ones."""
    shapes = [(256, 256), (200, 520), (700, 300), (64, 96), (384, 1000), (130, 129), (1024, 192)]
    rng = np.random.default_rng(7)
    mats = [(0.02 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    grads = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    moms = [(0.1 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    gu.say(f"[chain] one iteration {triple}")
    w_gpu, m_gpu, o_gpu, _ = gu.gpu_step(mats, grads, moms, lr=0.02, momentum=0.9, wd=0.0, coeffs=[list(triple)])
    for i, (r, c) in enumerate(shapes):
        gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.02, momentum=0.9, wd=0.0,
                        coeffs=[list(triple)], nesterov=True, row_norm=True, ns_tol=gu.NS_TOL_BF16,
                        label=f"{r}x{c} {triple}")


@pytest.mark.parametrize("table", [
    [(16.0, 0.0, 0.0), (0.0, 0.0, 2.0 ** -16)],
    [(2.0 ** -20, 0.0, 0.0), (0.0, 0.0, 2.0 ** 80)],
])
def test_chain_tables_that_rescale_x(table):
    shapes = [(256, 512), (512, 256), (384, 384)]
    rng = np.random.default_rng(11)
    mats = [(0.02 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    grads = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    moms = [(0.1 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    gu.say(f"[chain] rescaling table {table}")
    w_gpu, m_gpu, o_gpu, _ = gu.gpu_step(mats, grads, moms, lr=0.02, momentum=0.9, wd=0.0, coeffs=table)
    for i, (r, c) in enumerate(shapes):
        gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.02, momentum=0.9, wd=0.0,
                        coeffs=np.asarray(table), nesterov=True, row_norm=True, ns_tol=gu.NS_TOL_BF16,
                        label=f"{r}x{c}")
