"""GPU parity: the HIP library against the float64 oracle on the same seeded inputs.

Layered checks per matrix: the momentum buffer M' (fp32, 1e-6 relative max
norm), the orthogonalised update O against the oracle run from the same inputs
(relative Frobenius 2e-2 for bf16 NS, 1e-4 for fp32 NS), the weight W' against
the oracle's apply step fed the GPU's O (1e-6), and the EMA against the oracle
EMA fed the GPU's W' (1e-6).  Full-size workloads run in the same launch
configuration as bench.py, and the oracle recomputes O for every matrix of
every workload (all 66 at full size, every step of the 10-step run), so a slip
confined to one slot of a shape group cannot pass.  Each run prints the worst
NS error per stored shape.
"""

import numpy as np
import pytest

import oracle.muon as om
import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _worst_per_shape(errs, names):
    """{stored-shape name: worst O error} from per-matrix errors (names like 'l3.up')."""
    worst = {}
    for nm, e in zip(names, errs):
        key = nm.split(".", 1)[-1]
        worst[key] = max(worst.get(key, 0.0), e)
    return worst


def _run_workload(cfg, seed):
    w = wl.workload(cfg)
    gu.say(f"[parity] workload {cfg} ({w.name}) seed {seed}")
    st = wl.make_state(w, seed)
    coeffs = wl.coeff_table(w, seed)
    nm = len(w.matrices)
    mats, moms = st["params"][:nm], st["moms"]
    grads = wl.make_grads(w, seed, 0)
    # workloads without an EMA still run the fused EMA at the pages' decay
    decay = w.ema_decay if w.ema_decay is not None else 0.9965
    e_in = wl.make_independent_ema(w, seed + 1)[:nm]
    w_gpu, m_gpu, o_gpu, e_gpu = gu.gpu_step(mats, grads, moms, lr=w.lr, momentum=w.momentum, wd=w.weight_decay,
                                             coeffs=coeffs.tolist(), nesterov=w.nesterov, row_norm=w.row_norm,
                                             ns_precision=w.ns_precision, emas=e_in, ema_decay=decay)
    e_worst = gu.check_fused_ema(e_in, w_gpu, e_gpu, decay, label=w.name)
    tol = gu.NS_TOL_BF16 if w.ns_precision == 0 else gu.NS_TOL_FP32
    errs = []
    for i in range(nm):
        errs.append(gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=w.lr,
                                    momentum=w.momentum, wd=w.weight_decay, coeffs=coeffs, nesterov=w.nesterov,
                                    row_norm=w.row_norm, ns_tol=tol, label=w.matrices[i][0]))
    worst = _worst_per_shape(errs, [m[0] for m in w.matrices])
    gu.say(f"[parity] workload {cfg} seed {seed}, all {nm} matrices, worst NS error per shape: " +
           ", ".join(f"{k}={v:.2e}" for k, v in worst.items()) + f"; fused EMA worst {e_worst:.2e}")
    return w, st, w_gpu


def test_single_matrix_fp32_ns():
    _run_workload(0, wl.PRIMARY_SEED)


@pytest.mark.parametrize("seed", [wl.PRIMARY_SEED, *wl.ROBUST_SEEDS])
def test_one_layer_bf16(seed):
    _run_workload(1, seed)


def _check_ema(w, st, w_gpu, decay):
    import torch
    import muon_optimizer_step_amd as ms
    nm = len(w.matrices)
    post = list(w_gpu) + st["params"][nm:]
    ema0 = wl.make_independent_ema(w, 7)
    E = [gu.dev(e) for e in ema0]
    P = [gu.dev(p) for p in post]
    ms.ema_update(E, P, decay)
    torch.cuda.synchronize()
    worst = 0.0
    for i, (e0, p, e) in enumerate(zip(ema0, post, E)):
        err = gu.rel_max(gu.host(e), om.ema_update(e0, p, gu.f32(decay)))
        worst = max(worst, err)
        assert err <= gu.ELEM_TOL, f"EMA tensor {i}: {err:.3e}"
    gu.say(f"[parity] EMA over {len(E)} tensors, worst rel err {worst:.2e}")


def test_full_model_512d_with_ema():
    w, st, w_gpu = _run_workload(2, wl.PRIMARY_SEED)
    _check_ema(w, st, w_gpu, w.ema_decay)


@pytest.mark.parametrize("seed", wl.ROBUST_SEEDS)
def test_full_model_512d_robustness_seeds(seed):
    """The bench workload on the other seeds, every matrix's NS output checked."""
    _run_workload(2, seed)


def test_full_model_1024d_with_ema():
    w, st, w_gpu = _run_workload(3, wl.PRIMARY_SEED)
    _check_ema(w, st, w_gpu, w.ema_decay)


def test_structured_gradients_ten_steps():
    """Rank-8 + noise gradients, drawn 4-step table, momentum and EMA carried over 10 steps.

    The matrices' EMA advances inside the step, the other tensors' in ema_update.

    Each step is checked layer by layer against the oracle fed the GPU's state
    from the step before (the momentum chain is exact fp32; the NS error of
    every one of the 66 matrices is re-measured at every step).  The drift of
    W after ten steps relative to a pure-oracle run of all 66 matrices is
    reported and bounded too.
    """
    import torch
    import muon_optimizer_step_amd as ms
    w = wl.workload(4)
    seed = wl.PRIMARY_SEED
    st = wl.make_state(w, seed)
    coeffs = wl.coeff_table(w, seed)
    nm = len(w.matrices)
    names = [m[0] for m in w.matrices]
    P = [gu.dev(p) for p in st["params"]]
    M = [gu.dev(m) for m in st["moms"]]
    E = [gu.dev(e) for e in st["ema"]]
    O = [torch.empty_like(p) for p in P[:nm]]
    ref_w = [st["params"][i].astype(np.float64) for i in range(nm)]
    ref_m = [st["moms"][i].astype(np.float64) for i in range(nm)]
    for step in range(w.steps):
        gu.say(f"[parity] structured step {step}")
        grads = wl.make_grads(w, seed, step)
        w_in = [gu.host(p) for p in P[:nm]]
        m_in = [gu.host(m) for m in M]
        e_in = [gu.host(e) for e in E]
        G = [gu.dev(g) for g in grads]
        ms.muon_step(P[:nm], G, M, lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay,
                     coeffs=coeffs.tolist(), nesterov=True, row_norm=True, update_outs=O,
                     emas=E[:nm], ema_decay=w.ema_decay)
        ms.ema_update(E[nm:], P[nm:], w.ema_decay)
        torch.cuda.synchronize()
        w_out = [gu.host(p) for p in P[:nm]]
        errs = []
        for i in range(nm):
            errs.append(gu.check_layers(w_in[i], grads[i], m_in[i], w_out[i], gu.host(M[i]), gu.host(O[i]),
                                        lr=w.lr, momentum=w.momentum, wd=w.weight_decay, coeffs=coeffs,
                                        nesterov=True, row_norm=True, ns_tol=gu.NS_TOL_BF16,
                                        label=f"step {step} {names[i]}"))
        post = w_out + [gu.host(p) for p in P[nm:]]
        for i, e in enumerate(E):
            err = gu.rel_max(gu.host(e), om.ema_update(e_in[i], post[i], gu.f32(w.ema_decay)))
            assert err <= gu.ELEM_TOL, f"step {step} EMA tensor {i}: {err:.3e}"
        for i in range(nm):  # independent pure-oracle trajectory for the drift
            ref_w[i], ref_m[i], _ = om.muon_step_matrix(
                ref_w[i], grads[i], ref_m[i], lr=gu.f32(w.lr), mu=gu.f32(w.momentum), nesterov=True,
                wd=gu.f32(w.weight_decay), row_norm=True, coeffs=coeffs.astype(np.float64))
        worst = _worst_per_shape(errs, names)
        gu.say(f"[parity] structured step {step}, all {nm} matrices, worst NS error per shape: " +
               ", ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    drift = max(gu.rel_frob(gu.host(P[i]) - st["params"][i], ref_w[i] - st["params"][i]) for i in range(nm))
    gu.say(f"[parity] structured: relative drift of the 10-step weight change vs oracle, worst of {nm}: {drift:.2e}")
    assert drift <= gu.NS_TOL_BF16


def test_compensated_mode_one_layer():
    """MUON_NS_BF16X3: hi/lo compensation in every product, ~1e-4 of float64."""
    w = wl.workload(1)
    st = wl.make_state(w, wl.PRIMARY_SEED)
    grads = wl.make_grads(w, wl.PRIMARY_SEED, 0)
    coeffs = wl.coeff_table(w, wl.PRIMARY_SEED)
    mats, moms = st["params"], st["moms"]
    w_gpu, m_gpu, o_gpu, _ = gu.gpu_step(mats, grads, moms, lr=w.lr, momentum=w.momentum, wd=w.weight_decay,
                                         coeffs=coeffs.tolist(), ns_precision=2)
    errs = []
    for i in range(len(mats)):
        errs.append(gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=w.lr,
                                    momentum=w.momentum, wd=w.weight_decay, coeffs=coeffs, nesterov=True,
                                    row_norm=True, ns_tol=gu.NS_TOL_BF16X3, label=w.matrices[i][0]))
    gu.say(f"[parity] compensated one layer: worst NS err {max(errs):.2e}")


@pytest.mark.parametrize("ns_precision", [0, 1, 2])
@pytest.mark.parametrize("nesterov,row_norm", [(True, True), (False, False), (True, False)])
def test_ragged_shapes(ns_precision, nesterov, row_norm):
    """Odd shapes (wide, tall, square, 1-row, 1-col) leave ragged tails in every tiling."""
    shapes = wl.small_ragged_matrices()
    rng = np.random.default_rng(99)
    mats = [(0.02 * rng.standard_normal((r, c))).astype(np.float32) for _, r, c in shapes]
    grads = [rng.standard_normal((r, c)).astype(np.float32) for _, r, c in shapes]
    moms = [(0.5 * rng.standard_normal((r, c))).astype(np.float32) for _, r, c in shapes]
    coeffs = wl.coeff_table(wl.workload(4), 5).tolist()
    # every other matrix carries an EMA shadow (vector and scalar, row and column epilogues)
    emas = [rng.standard_normal((r, c)).astype(np.float32) if i % 2 == 0 else None
            for i, (_, r, c) in enumerate(shapes)]
    gu.say(f"[parity] ragged shapes prec={ns_precision} nesterov={nesterov} row_norm={row_norm}")
    w_gpu, m_gpu, o_gpu, e_gpu = gu.gpu_step(mats, grads, moms, lr=0.05, momentum=0.9, wd=0.1, coeffs=coeffs,
                                             nesterov=nesterov, row_norm=row_norm, ns_precision=ns_precision,
                                             emas=emas, ema_decay=0.9)
    gu.check_fused_ema(emas, w_gpu, e_gpu, 0.9, label="ragged")
    tol = {0: gu.NS_TOL_BF16, 1: gu.NS_TOL_FP32, 2: gu.NS_TOL_BF16X3}[ns_precision]
    for i, (nm, r, c) in enumerate(shapes):
        gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.05, momentum=0.9, wd=0.1,
                        coeffs=coeffs, nesterov=nesterov, row_norm=row_norm, ns_tol=tol, label=f"{nm} {r}x{c}")


@pytest.mark.parametrize("ns_precision,tol", [(1, 1e-5), (0, gu.NS_TOL_BF16), (2, gu.NS_TOL_BF16X3)])
@pytest.mark.parametrize("triple", [(0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (1.0, 0.0, 0.0), (0.5, -0.25, 0.125)])
def test_single_iteration_isolates_each_product(ns_precision, tol, triple):
    """One NS iteration whose coefficients isolate one product: (0, 1, 0) gives X Xt X (the Gram and the
    update), (0, 0, 1) gives (X Xt)^2 X (the square), (1, 0, 0) gives X back (the a X term through the
    hi + lo planes).  Wide, tall and square shapes over several tiles with ragged tails, on both sides of
    the compensation threshold (short side 192), against the float64 oracle's product."""
    shapes = [(256, 256), (200, 520), (700, 300), (64, 96), (384, 1000), (130, 129)]
    rng = np.random.default_rng(7)
    mats = [(0.02 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    grads = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    moms = [(0.1 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    coeffs = [list(triple)]
    gu.say(f"[parity] one iteration {triple} prec={ns_precision}")
    w_gpu, m_gpu, o_gpu, _ = gu.gpu_step(mats, grads, moms, lr=0.02, momentum=0.9, wd=0.0, coeffs=coeffs,
                                         ns_precision=ns_precision)
    for i, (r, c) in enumerate(shapes):
        gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.02, momentum=0.9, wd=0.0,
                        coeffs=coeffs, nesterov=True, row_norm=True, ns_tol=tol, label=f"{r}x{c} {triple}")


@pytest.mark.parametrize("ns_precision,tol", [(1, 1e-5), (0, gu.NS_TOL_BF16), (2, gu.NS_TOL_BF16X3)])
@pytest.mark.parametrize("table", [
    [(16.0, 0.0, 0.0), (0.0, 0.0, 2.0 ** -16)],                    # X grows 16x, then the square alone
    [(4.0, 0.0, 0.0), (4.0, 0.0, 0.0), (0.0, 0.0, 2.0 ** -16)],    # the same in two steps
    [(1.0 / 16.0, 0.0, 0.0), (0.0, 0.0, 2.0 ** 16)],                # X shrinks 16x first
    [(2.0 ** 20, 0.0, 0.0), (0.0, 0.0, 2.0 ** -80)],                # far outside the unit range, both ways
    [(2.0 ** -20, 0.0, 0.0), (0.0, 0.0, 2.0 ** 80)],
])
def test_tables_that_rescale_x(ns_precision, tol, table):
    """Coefficient tables that scale X up or down before an iteration whose output is the square alone
    ((X Xt)^2 X): the square's low-order products must follow |A| wherever the table takes it, not
    assume the singular values stay near 1."""
    shapes = [(256, 512), (512, 256), (384, 384)]
    rng = np.random.default_rng(11)
    mats = [(0.02 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    grads = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    moms = [(0.1 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    gu.say(f"[parity] rescaling table {table} prec={ns_precision}")
    w_gpu, m_gpu, o_gpu, _ = gu.gpu_step(mats, grads, moms, lr=0.02, momentum=0.9, wd=0.0, coeffs=table,
                                         ns_precision=ns_precision)
    for i, (r, c) in enumerate(shapes):
        gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.02, momentum=0.9, wd=0.0,
                        coeffs=np.asarray(table), nesterov=True, row_norm=True, ns_tol=tol, label=f"{r}x{c}")
