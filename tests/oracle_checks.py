"""Independent pins for the float64 oracle.

Each ``check_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with something fixed outside it: a closed form from the SVD,
a textbook special case, an invariant of the iteration, a hand-derived value,
or a number printed on the pages.  None of them re-types an oracle formula.
The same checks run once against the real oracle (tests/test_oracle_pins.py)
and once against deliberately broken copies of it (tests/test_oracle_mutants.py),
which shows that a plausible slip anywhere in the oracle trips at least one pin.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TRIPLE = (3.4445, -4.7750, 2.0315)


def _scalar_map(sigma, coeffs):
    """Compose the scalar quintics p_k(x) = a_k x + b_k x^3 + c_k x^5, p_0 first."""
    s = np.array(sigma, dtype=np.float64)
    for a, b, c in coeffs:
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def _closed_form_ns(x, coeffs):
    """U diag(phi(sigma)) V^T from the thin SVD (numpy.linalg.svd, LAPACK)."""
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    return (u * _scalar_map(s, coeffs)) @ vt


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _unit_frob(x):
    return x / np.linalg.norm(x)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _tables():
    rng = np.random.default_rng(7)
    jitter = np.array([TRIPLE] * 4) * (1 + rng.uniform(-0.05, 0.05, size=(4, 3)))
    return {
        "standard5": [TRIPLE] * 5,
        "jitter4": [tuple(r) for r in jitter],
        "cubic3": [(1.5, -0.5, 0.0)] * 3,
        "mixed": [(2.0, -1.5, 0.5), TRIPLE, (1.5, -0.5, 0.0)],
    }


SHAPES = [(8, 8), (6, 10), (16, 48), (32, 128), (5, 5)]


def check_ns_svd_closed_form(m):
    """NS on a short-side-first matrix equals U phi(S) V^T (to ~1e-12)."""
    for si, shape in enumerate(SHAPES):
        x = _unit_frob(_rand(shape, 100 + si))
        for name, tab in _tables().items():
            got = m.newton_schulz(x, tab)
            want = _closed_form_ns(x, tab)
            assert _rel(got, want) < 1e-11, (shape, name, _rel(got, want))


def check_ns_order_of_table(m):
    """The table's row k drives iteration k: a reversed schedule gives another map."""
    x = _unit_frob(_rand((12, 20), 3))
    tab = _tables()["mixed"]
    got = m.newton_schulz(x, tab)
    assert _rel(got, _closed_form_ns(x, tab)) < 1e-11
    assert _rel(got, _closed_form_ns(x, tab[::-1])) > 1e-3


def check_ns_invariants(m):
    """Transpose / orthogonal equivariance and preserved singular vectors."""
    rng = np.random.default_rng(11)
    x = _unit_frob(rng.standard_normal((10, 24)))
    tab = _tables()["jitter4"]
    o = m.newton_schulz(x, tab)
    # transpose equivariance: NS(X^T) = NS(X)^T (the iteration also runs on tall input)
    assert _rel(m.newton_schulz(x.T, tab), o.T) < 1e-11
    # orthogonal equivariance: NS(Q X R) = Q NS(X) R
    q, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    r, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    assert _rel(m.newton_schulz(q @ x @ r, tab), q @ o @ r) < 1e-11
    # singular vectors are kept: U^T O V is diagonal
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    d = u.T @ o @ vt.T
    off = d - np.diag(np.diag(d))
    assert np.abs(off).max() < 1e-11 * np.abs(np.diag(d)).max()


def check_ns_fixed_band(m):
    """Normalised inputs with sigma >= 0.01 land in the band of the scalar map.

    The band [0.68183, 1.13436] is the range of the 5-fold composed standard
    quintic over sigma in [0.01, 1] (sampled on a 2e5-point grid here).
    """
    grid = np.linspace(0.01, 1.0, 200001)
    img = _scalar_map(grid, [TRIPLE] * 5)
    lo, hi = img.min(), img.max()
    assert abs(lo - 0.68183) < 1e-4 and abs(hi - 1.13436) < 1e-4
    rng = np.random.default_rng(5)
    u, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    v, _ = np.linalg.qr(rng.standard_normal((40, 16)))
    sig = np.linspace(0.01, 1.0, 16)
    x = (u * sig) @ v.T
    o = m.newton_schulz(x, [TRIPLE] * 5)
    so = np.linalg.svd(o, compute_uv=False)
    assert so.min() >= lo - 1e-9 and so.max() <= hi + 1e-9


def check_ns_special_cases(m):
    x = _unit_frob(_rand((7, 9), 21))
    # (1, 0, 0) is the identity map; an empty table is no iteration at all
    assert _rel(m.newton_schulz(x, [(1.0, 0.0, 0.0)] * 3), x) < 1e-15
    assert _rel(m.newton_schulz(x, []), x) < 1e-15
    # the cubic Newton-Schulz (1.5, -0.5, 0) converges to the polar factor U V^T
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    xw = (u * np.linspace(0.3, 1.0, s.size)) @ vt  # well conditioned
    polar = u @ vt
    o = m.newton_schulz(xw, [(1.5, -0.5, 0.0)] * 40)
    assert _rel(o, polar) < 1e-12
    # a hand-evaluated scalar case: 1x1 input 0.5, one standard step
    # 3.4445*0.5 - 4.7750*0.125 + 2.0315*0.03125 = 1.188859375
    got = float(m.newton_schulz(np.array([[0.5]]), [TRIPLE])[0, 0])
    assert abs(got - 1.188859375) < 1e-14


def check_momentum(m):
    # hand values: buf=2, g=3, mu=0.5 -> M' = 0.5*2 + 3 = 4, U = 3 + 0.5*4 = 5 (Nesterov)
    b, u = m.momentum_update(np.array([[2.0]]), np.array([[3.0]]), 0.5, True)
    assert float(b[0, 0]) == 4.0 and float(u[0, 0]) == 5.0
    b, u = m.momentum_update(np.array([[2.0]]), np.array([[3.0]]), 0.5, False)
    assert float(b[0, 0]) == 4.0 and float(u[0, 0]) == 4.0
    # mu = 0: the buffer is the gradient, and so is U
    g = _rand((3, 4), 1)
    b, u = m.momentum_update(_rand((3, 4), 2), g, 0.0, True)
    assert np.array_equal(b, g) and np.array_equal(u, g)
    # geometric series: constant g from a zero buffer, T steps -> g (1 - mu^T) / (1 - mu)
    mu, T = 0.9, 25
    buf = np.zeros((2, 2))
    for _ in range(T):
        buf, u = m.momentum_update(buf, np.ones((2, 2)), mu, True)
    want = (1 - mu ** T) / (1 - mu)
    assert abs(buf[0, 0] - want) < 1e-12
    assert abs(u[0, 0] - (1 + mu * want)) < 1e-12


def check_row_normalize(m):
    x = _rand((5, 9), 4) * np.array([[1.0], [3.0], [0.01], [100.0], [2.0]])
    r = m.row_normalize(x)
    n = np.linalg.norm(x, axis=1)
    assert np.allclose(np.linalg.norm(r, axis=1), n / (n + 1e-7), rtol=0, atol=1e-14)
    # direction unchanged per row, rows of different shape keep their own norms
    assert np.allclose(r * (n + 1e-7)[:, None], x, rtol=1e-14, atol=0)
    # a zero row stays exactly zero
    z = x.copy()
    z[2] = 0
    assert np.all(m.row_normalize(z)[2] == 0)
    # it is a per-row operation: one row does not depend on the others
    y = x.copy()
    y[0] *= 7.0
    assert np.allclose(m.row_normalize(y)[1:], r[1:], rtol=0, atol=0)


def check_frobenius(m):
    x = _rand((6, 3), 9) * 13.0
    y = m.frobenius_normalize(x)
    assert abs(np.linalg.norm(y) - np.linalg.norm(x) / (np.linalg.norm(x) + 1e-7)) < 1e-14
    assert np.allclose(y * (np.linalg.norm(x) + 1e-7), x, rtol=1e-14, atol=0)
    assert np.all(m.frobenius_normalize(np.zeros((3, 3))) == 0)


def check_orthogonalize(m):
    tab = [TRIPLE] * 5
    rng = np.random.default_rng(31)
    for shape in [(12, 30), (30, 12), (16, 16)]:
        u = rng.standard_normal(shape) * 0.37
        o = m.orthogonalize(u, tab, row_norm=False)
        # closed form of the whole chain without row norm: U phi(S / (|u|_F + eps)) V^T
        x0 = u / (np.linalg.norm(u) + 1e-7)
        assert o.shape == u.shape
        assert _rel(o, _closed_form_ns(x0, tab)) < 1e-11, shape
        # orientation does not change the result: orthogonalize(U^T) = orthogonalize(U)^T
        assert _rel(m.orthogonalize(u.T, tab, row_norm=False), o.T) < 1e-11
    # with row norm: the closed form on the row-normalised matrix
    u = rng.standard_normal((20, 8)) * rng.uniform(0.1, 10, size=(20, 1))
    r = u / (np.linalg.norm(u, axis=1, keepdims=True) + 1e-7)
    x0 = r / (np.linalg.norm(r) + 1e-7)
    o = m.orthogonalize(u, tab, row_norm=True)
    assert _rel(o, _closed_form_ns(x0, tab)) < 1e-11
    # no iteration: O = X0
    assert _rel(m.orthogonalize(u, [], row_norm=True), x0) < 1e-15


def check_shape_scale(m):
    # out x in shapes of one layer at d = 512: only the MLP up projection is tall
    shapes = [(512, 512), (256, 512), (256, 512), (512, 512), (2048, 512), (512, 2048)]
    assert [m.shape_scale(r, c) for r, c in shapes] == [1.0, 1.0, 1.0, 1.0, 2.0, 1.0]
    assert m.shape_scale(4096, 1024) == 2.0 and m.shape_scale(9, 4) == 1.5


def check_apply_update(m):
    # hand values: W = 1, O = 1, lr = 0.1, wd = 0.5, s = 2 -> (1 - 0.05) * 1 - 0.2 = 0.75.
    # Decay applied after the update would give 0.95 * 0.8 = 0.76; decay without the
    # lr factor would give 0.5 * 1 - 0.2 = 0.3.
    w = m.apply_update(np.array([[1.0]]), np.array([[1.0]]), 0.1, 0.5, 2.0)
    assert abs(float(w[0, 0]) - 0.75) < 1e-15
    # W = 3, O = -1, lr = 0.2, wd = 0.25, s = 1 -> 0.95 * 3 + 0.2 = 3.05 (decay after: 3.04)
    w = m.apply_update(np.array([[3.0]]), np.array([[-1.0]]), 0.2, 0.25, 1.0)
    assert abs(float(w[0, 0]) - 3.05) < 1e-14
    # lr = 0 leaves W unchanged; wd = 0 is plain descent
    ww = _rand((3, 3), 8)
    oo = _rand((3, 3), 9)
    assert np.array_equal(m.apply_update(ww, oo, 0.0, 0.7, 2.0), ww)
    assert np.allclose(m.apply_update(ww, oo, 0.1, 0.0, 2.0), ww - 0.2 * oo, rtol=0, atol=1e-15)


def check_diagonal_step(m):
    """Whole step on a diagonal gradient: every stage acts on the diagonal alone.

    G = diag(g), zero momentum, Nesterov: U = (1 + mu) G.  Row norm makes each
    row +-|u|/(|u|+eps) e_i, the Frobenius scale divides by ~sqrt(n), and NS on
    a diagonal matrix is the scalar map on each entry.
    """
    n, mu, lr, wd = 6, 0.9, 0.05, 0.1
    g = np.diag(np.array([3.0, -1.0, 0.5, 2.0, -4.0, 1.5]))
    w = np.eye(n) * 0.25
    tab = [TRIPLE] * 3
    w_new, buf, o = m.muon_step_matrix(w, g, np.zeros((n, n)), lr=lr, mu=mu, nesterov=True,
                                       wd=wd, row_norm=True, coeffs=tab)
    assert np.array_equal(buf, g)
    u = (1 + mu) * np.diag(g)
    r = u / (np.abs(u) + 1e-7)
    x0 = r / (np.sqrt(np.sum(r * r)) + 1e-7)
    want_o = np.diag(_scalar_map(x0, tab))
    assert np.allclose(o, want_o, rtol=1e-13, atol=1e-15)
    assert np.allclose(w_new, (1 - lr * wd) * w - lr * want_o, rtol=1e-13, atol=1e-15)


def check_tall_step_scale(m):
    """A tall matrix is scaled by sqrt(rows/cols) and keeps its stored shape."""
    rng = np.random.default_rng(2)
    g = rng.standard_normal((12, 3))
    w = np.zeros((12, 3))
    w_new, _, o = m.muon_step_matrix(w, g, np.zeros_like(g), lr=1.0, mu=0.0, nesterov=True,
                                     wd=0.0, row_norm=False, coeffs=[TRIPLE] * 5)
    assert o.shape == (12, 3)
    x0 = g / (np.linalg.norm(g) + 1e-7)
    assert _rel(o, _closed_form_ns(x0, [TRIPLE] * 5)) < 1e-11
    assert np.allclose(w_new, -2.0 * o, rtol=1e-14, atol=0)


def check_ema(m):
    e, p = _rand((4, 5), 1), _rand((4, 5), 2)
    assert np.array_equal(m.ema_update(e, p, 1.0), e)
    assert np.array_equal(m.ema_update(e, p, 0.0), p)
    assert np.allclose(m.ema_update(e, p, 0.5), (e + p) / 2, rtol=0, atol=1e-15)
    # T steps towards a constant target: E_T = P + d^T (E_0 - P)
    d, T = 0.9965, 200
    ee = e.copy()
    for _ in range(T):
        ee = m.ema_update(ee, p, d)
    assert np.allclose(ee, p + d ** T * (e - p), rtol=1e-12, atol=1e-13)


def check_page_hyperparameters():
    """The workloads use the values the pages print (tests/golden/page_facts.json)."""
    import workloads as wl
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    w2, w3 = wl.workload(2), wl.workload(3)
    assert w2.n_params == facts["param_count_11L_512d"]["value"]
    assert abs(w2.momentum - facts["muon_momentum"]["value"]) == 0
    assert abs(w3.momentum - facts["muon_momentum_variant"]["value"]) == 0
    assert w2.lr == facts["matrix_lr"]["value"] and w3.lr == facts["matrix_lr_variant"]["value"]
    assert w2.weight_decay == facts["muon_wd"]["value"]
    assert w2.ema_decay == facts["ema_decay"]["value"] and w3.ema_decay == facts["ema_decay_variant"]["value"]
    assert wl.workload(4).ns_steps == facts["polar_express_steps"]["value"]
    arch = facts["architecture"]["value"]
    assert len(w2.matrices) == arch["layers"] * 6
    q = [s for s in w2.matrices if s[0] == "l0.q"][0]
    k = [s for s in w2.matrices if s[0] == "l0.k"][0]
    up = [s for s in w2.matrices if s[0] == "l0.up"][0]
    assert q[1:] == (arch["d_model"], arch["d_model"])
    assert k[1:] == (arch["kv_heads"] * arch["d_model"] // arch["q_heads"], arch["d_model"])
    assert up[1:] == (arch["mlp_mult"] * arch["d_model"], arch["d_model"])
    assert w3.n_params == 131_717_212  # the same list at double width (a reading)


def check_adamw_hand_values(m):
    """AdamW values derived by hand (the update of the non-matrix parameters)."""
    # Step 1 from zero moments: the bias corrections make m_hat = g and v_hat = g^2, so
    # p' = (1 - lr wd) p - lr g / (|g| + eps).  lr 0.1, wd 0.5, eps 0.5, beta1 0.9, beta2 0.99:
    #   p = 1,    g = 2:    0.95 - 0.1 * 2 / 2.5   = 0.87
    #   p = -2,   g = 0.5: -1.9  - 0.1 * 0.5 / 1.0 = -1.95
    #   p = 0.5,  g = 0:    0.475
    p, g = np.array([1.0, -2.0, 0.5]), np.array([2.0, 0.5, 0.0])
    pn, mn, vn = m.adamw_update(p, g, np.zeros(3), np.zeros(3), lr=0.1, beta1=0.9, beta2=0.99, eps=0.5,
                                wd=0.5, step=1)
    assert np.allclose(pn, [0.87, -1.95, 0.475], rtol=1e-14, atol=1e-15)
    assert np.allclose(mn, [0.2, 0.05, 0.0], rtol=1e-14, atol=0)          # (1 - beta1) g
    assert np.allclose(vn, [0.04, 0.0025, 0.0], rtol=1e-13, atol=0)       # (1 - beta2) g^2
    # A zero gradient at step 2 (beta1 0.5, beta2 0.75, eps 0, wd 0): m' = 0.15, v' = 0.03,
    # m_hat = 0.15 / 0.75 = 0.2, v_hat = 0.03 / 0.4375 = 0.0685714..., sqrt = 0.2618614682831909,
    # p' = 1 - 0.1 * 0.2 / 0.2618614682831909 = 0.9236237384174026
    pn, mn, vn = m.adamw_update([1.0], [0.0], [0.3], [0.04], lr=0.1, beta1=0.5, beta2=0.75, eps=0.0, wd=0.0,
                                step=2)
    assert np.allclose(mn, [0.15], rtol=1e-15) and np.allclose(vn, [0.03], rtol=1e-15)
    assert np.allclose(pn, [0.9236237384174026], rtol=1e-14)
    # weight decay only (zero gradient, zero moments): p' = (1 - lr wd) p exactly
    pn, _, _ = m.adamw_update([3.0], [0.0], [0.0], [0.0], lr=0.2, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.25,
                              step=5)
    assert pn[0] == 3.0 * 0.95


def check_adamw_against_torch(m):
    """torch.optim.AdamW (CPU, float64, single-tensor loop), from zero state over 4 steps, three settings."""
    import torch
    settings = [dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01),
                dict(lr=0.05, betas=(0.8, 0.95), eps=1e-6, weight_decay=0.1),
                dict(lr=0.3, betas=(0.5, 0.6), eps=1e-3, weight_decay=0.0)]
    for k, st in enumerate(settings):
        rng = np.random.default_rng(100 + k)
        p0 = rng.standard_normal((7, 5))
        tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
        opt = torch.optim.AdamW([tp], foreach=False, **st)
        p, mm, vv = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
        for t in range(1, 5):
            g = rng.standard_normal(p0.shape) * (0.1 if t % 2 else 3.0)
            tp.grad = torch.tensor(g, dtype=torch.float64)
            opt.step()
            p, mm, vv = m.adamw_update(p, g, mm, vv, lr=st["lr"], beta1=st["betas"][0], beta2=st["betas"][1],
                                       eps=st["eps"], wd=st["weight_decay"], step=t)
            state = opt.state[tp]
            assert np.allclose(p, tp.detach().numpy(), rtol=1e-12, atol=1e-14), (k, t)
            assert np.allclose(mm, state["exp_avg"].numpy(), rtol=1e-12, atol=1e-14), (k, t)
            assert np.allclose(vv, state["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-14), (k, t)


ADAMW_CHECKS = [check_adamw_hand_values, check_adamw_against_torch]


ALL_ORACLE_CHECKS = [
    check_ns_svd_closed_form, check_ns_order_of_table, check_ns_invariants,
    check_ns_fixed_band, check_ns_special_cases, check_momentum, check_row_normalize,
    check_frobenius, check_orthogonalize, check_shape_scale, check_apply_update,
    check_diagonal_step, check_tall_step_scale, check_ema,
]
