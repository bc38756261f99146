"""GPU parity of adamw_step (the non-matrix parameters) against the float64 AdamW oracle.

Per tensor, on the same float32 inputs: the updated parameter, both moments
and (where given) the EMA shadow, each within 1e-6 relative max-norm of the
oracle; the EMA is checked against the oracle EMA fed the GPU's parameter, as
for the Muon matrices.
"""

import numpy as np
import pytest

import oracle.adamw as oa
import oracle.muon as om
import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HP = wl.ADAMW_HPARAMS


def _run(params, grads, ms1, ms2, emas, *, lr, beta1, beta2, eps, wd, step, decay, label=""):
    """One adamw_step on uploaded copies; checks every tensor; returns the device tensors."""
    import torch
    import muon_optimizer_step_amd as ms
    P = [gu.dev(p) for p in params]
    G = [gu.dev(g) for g in grads]
    M = [gu.dev(m) for m in ms1]
    V = [gu.dev(v) for v in ms2]
    E = [gu.dev(e) if e is not None else None for e in emas] if emas is not None else None
    ms.adamw_step(P, G, M, V, lr=lr, betas=(beta1, beta2), eps=eps, weight_decay=wd, step=step, emas=E,
                  ema_decay=decay)
    torch.cuda.synchronize()
    f = gu.f32
    worst = 0.0
    for i in range(len(params)):
        p_ref, m_ref, v_ref = oa.adamw_update(params[i], grads[i], ms1[i], ms2[i], lr=f(lr), beta1=f(beta1),
                                              beta2=f(beta2), eps=f(eps), wd=f(wd), step=step)
        p_gpu = gu.host(P[i])
        for got, want, what in ((p_gpu, p_ref, "param"), (gu.host(M[i]), m_ref, "exp_avg"),
                                (gu.host(V[i]), v_ref, "exp_avg_sq")):
            err = gu.rel_max(got, want)
            worst = max(worst, err)
            assert err <= gu.ELEM_TOL, f"{label} tensor {i} {what}: rel err {err:.3e}"
        if E is not None and E[i] is not None:
            err = gu.rel_max(gu.host(E[i]), om.ema_update(emas[i], p_gpu, f(decay)))
            worst = max(worst, err)
            assert err <= gu.ELEM_TOL, f"{label} tensor {i} ema: rel err {err:.3e}"
    gu.say(f"[adamw] {label}: {len(params)} tensors, worst rel err {worst:.2e}")
    return P, M, V, E


def test_model_extras_with_fused_ema():
    """The 121 non-matrix tensors of the 11-layer 512-wide model (2,681,948 elements)."""
    w = wl.workload(2)
    nm = len(w.matrices)
    st = wl.make_state(w, wl.PRIMARY_SEED)
    ad = wl.make_adamw_state(w, wl.PRIMARY_SEED)
    emas = wl.make_independent_ema(w, 5)[nm:]
    _run(st["params"][nm:], ad["grads"], ad["exp_avg"], ad["exp_avg_sq"], emas, lr=HP["lr"], beta1=HP["beta1"],
         beta2=HP["beta2"], eps=HP["eps"], wd=HP["weight_decay"], step=HP["step"], decay=w.ema_decay,
         label="model extras")


@pytest.mark.parametrize("step,beta1,beta2,eps,wd", [
    (1, 0.9, 0.999, 1e-8, 0.01),      # first step: the bias corrections are the largest
    (2, 0.8, 0.95, 1e-6, 0.1),
    (37, 0.5, 0.6, 1e-3, 0.0),
    (1000, 0.0, 0.0, 1e-8, 0.05),     # no moment memory: a sign-like step
])
def test_hyperparameters_and_steps(step, beta1, beta2, eps, wd):
    rng = np.random.default_rng(step)
    shapes = [(4096, 128), (512,), (92,), (33, 7)]
    params = [(0.02 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    grads = [(1e-2 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    m1 = [(1e-2 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    m2 = [np.square(1e-2 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    _run(params, grads, m1, m2, None, lr=3e-3, beta1=beta1, beta2=beta2, eps=eps, wd=wd, step=step, decay=0.0,
         label=f"step {step}")


def test_ragged_unaligned_empty_and_many_tensors():
    """Sizes around the 2048-element workgroup chunk, 4-byte-aligned views (scalar path), empty
    tensors, a mix of EMA and no EMA, and more tensors than one launch's table (64)."""
    import torch
    import muon_optimizer_step_amd as ms
    rng = np.random.default_rng(9)
    sizes = [1, 3, 2047, 2048, 2049, 100003, 0, 5] + [int(x) for x in rng.integers(1, 5000, size=142)]
    n = len(sizes)

    def carve(arrs, offset):
        # each tensor a view into one flat buffer, starting `offset` floats past a 16-byte boundary,
        # with 4 guard floats (kept at -7) between neighbours
        total = sum(a.size + 4 for a in arrs) + offset + 4
        flat = torch.full((total,), -7.0, dtype=torch.float32, device="cuda")
        views, used, pos = [], torch.zeros(total, dtype=torch.bool), offset
        for a in arrs:
            v = flat[pos:pos + a.size]
            v.copy_(torch.from_numpy(a.ravel()))
            views.append(v)
            used[pos:pos + a.size] = True
            pos += a.size + 4
        guards.append((flat, ~used))
        return flat, views

    guards = []

    params = [(0.02 * rng.standard_normal(k)).astype(np.float32) for k in sizes]
    grads = [(1e-3 * rng.standard_normal(k)).astype(np.float32) for k in sizes]
    m1 = [(1e-3 * rng.standard_normal(k)).astype(np.float32) for k in sizes]
    m2 = [np.square(1e-3 * rng.standard_normal(k)).astype(np.float32) for k in sizes]
    emas = [(0.02 * rng.standard_normal(k)).astype(np.float32) if i % 3 else None for i, k in enumerate(sizes)]
    views = {}
    for name, arrs, off in (("p", params, 1), ("g", grads, 0), ("m", m1, 2), ("v", m2, 0)):
        _, views[name] = carve(arrs, off)
    _, ev = carve([e if e is not None else np.zeros(0, np.float32) for e in emas], 3)
    E = [ev[i] if emas[i] is not None else None for i in range(n)]
    gu.say(f"[adamw] ragged: {n} tensors")
    ms.adamw_step(views["p"], views["g"], views["m"], views["v"], lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                  weight_decay=0.01, step=5, emas=E, ema_decay=0.99)
    torch.cuda.synchronize()
    f = gu.f32
    for i in range(n):
        if sizes[i] == 0:
            continue
        p_ref, m_ref, v_ref = oa.adamw_update(params[i], grads[i], m1[i], m2[i], lr=f(1e-3), beta1=f(0.9),
                                              beta2=f(0.999), eps=f(1e-8), wd=f(0.01), step=5)
        p_gpu = gu.host(views["p"][i])
        assert gu.rel_max(p_gpu, p_ref) <= gu.ELEM_TOL, i
        assert gu.rel_max(gu.host(views["m"][i]), m_ref) <= gu.ELEM_TOL, i
        assert gu.rel_max(gu.host(views["v"][i]), v_ref) <= gu.ELEM_TOL, i
        if emas[i] is not None:
            assert gu.rel_max(gu.host(E[i]), om.ema_update(emas[i], p_gpu, f(0.99))) <= gu.ELEM_TOL, i
    # nothing outside the tensors was written
    for flat, guard in guards:
        assert bool((flat.cpu()[guard] == -7.0).all())


def test_zero_gradients_decay_only():
    """g = 0 with zero moments: the moments stay zero and p' = (1 - lr wd) p."""
    import torch
    import muon_optimizer_step_amd as ms
    p0 = np.linspace(-1, 1, 10000, dtype=np.float32)
    P = gu.dev(p0)
    Z = [torch.zeros_like(P) for _ in range(3)]
    ms.adamw_step([P], [Z[0]], [Z[1]], [Z[2]], lr=0.1, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.5, step=3)
    torch.cuda.synchronize()
    assert torch.count_nonzero(Z[1]) == 0 and torch.count_nonzero(Z[2]) == 0
    keep = np.float32(1.0) - np.float32(0.1) * np.float32(0.5)
    assert np.array_equal(gu.host(P), p0 * keep)


def test_ten_step_trajectory():
    """Moments carried over 10 steps; each step checked against the oracle fed the GPU's state."""
    import torch
    import muon_optimizer_step_amd as ms
    w = wl.workload(2)
    nm = len(w.matrices)
    st = wl.make_state(w, 42)
    params = st["params"][nm:nm + 12]
    zeros = [np.zeros_like(p) for p in params]
    P = [gu.dev(p) for p in params]
    M = [gu.dev(z) for z in zeros]
    V = [gu.dev(z) for z in zeros]
    G = [torch.empty_like(p) for p in P]
    prep = ms.PreparedAdamW(P, G, M, V)
    for t in range(1, 11):
        grads = wl.make_adamw_state(w, 42, step=t)["grads"][:12]
        for dst, g in zip(G, grads):
            dst.copy_(torch.from_numpy(g))
        p_in, m_in, v_in = [gu.host(x) for x in P], [gu.host(x) for x in M], [gu.host(x) for x in V]
        prep(lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"], weight_decay=HP["weight_decay"], step=t)
        torch.cuda.synchronize()
        for i in range(len(P)):
            p_ref, m_ref, v_ref = oa.adamw_update(p_in[i], grads[i], m_in[i], v_in[i], lr=gu.f32(HP["lr"]),
                                                  beta1=gu.f32(HP["beta1"]), beta2=gu.f32(HP["beta2"]),
                                                  eps=gu.f32(HP["eps"]), wd=gu.f32(HP["weight_decay"]), step=t)
            assert gu.rel_max(gu.host(P[i]), p_ref) <= gu.ELEM_TOL, (t, i)
            assert gu.rel_max(gu.host(M[i]), m_ref) <= gu.ELEM_TOL, (t, i)
            assert gu.rel_max(gu.host(V[i]), v_ref) <= gu.ELEM_TOL, (t, i)
    gu.say("[adamw] 10-step trajectory ok")
