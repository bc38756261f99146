"""GPU edge cases: degenerate inputs, maximum sizes, chunking, determinism, EMA layouts."""

import numpy as np
import pytest

import oracle.muon as om
import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

STD = [list(wl.STANDARD_TRIPLE)] * 5


@pytest.mark.parametrize("ns_precision,tol", [(0, 2e-5), (1, 1e-6)])
def test_zero_ns_steps_gives_x0(ns_precision, tol):
    """ns_steps = 0: O is the row- and Frobenius-normalised update itself."""
    rng = np.random.default_rng(3)
    shapes = [(64, 200), (300, 40), (128, 128)]
    mats = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    grads = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    moms = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    emas = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    w_gpu, m_gpu, o_gpu, e_gpu = gu.gpu_step(mats, grads, moms, lr=0.1, momentum=0.5, wd=0.2, coeffs=[],
                                             ns_precision=ns_precision, emas=emas, ema_decay=0.75)
    gu.check_fused_ema(emas, w_gpu, e_gpu, 0.75)
    for i in range(len(shapes)):
        _, u = om.momentum_update(moms[i], grads[i], gu.f32(0.5), True)
        assert gu.rel_frob(o_gpu[i], om.orthogonalize(u, [], True)) <= tol
        gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.1, momentum=0.5, wd=0.2,
                        coeffs=[], nesterov=True, row_norm=True, ns_tol=tol)


def test_zero_gradient_and_zero_rows():
    """A zero update gives O = 0 and pure decay; a zero row of G stays a zero row of O."""
    rng = np.random.default_rng(4)
    w0 = rng.standard_normal((96, 160)).astype(np.float32)
    z = np.zeros((96, 160), np.float32)
    g1 = rng.standard_normal((96, 160)).astype(np.float32)
    g1[[3, 50, 95]] = 0.0
    w_gpu, m_gpu, o_gpu, _ = gu.gpu_step([w0, w0.copy()], [z, g1], [z.copy(), z.copy()], lr=0.1, momentum=0.9,
                                         wd=0.5, coeffs=STD)
    assert np.all(o_gpu[0] == 0) and np.all(m_gpu[0] == 0)
    assert gu.rel_max(w_gpu[0], (1 - gu.f32(0.1) * gu.f32(0.5)) * w0.astype(np.float64)) <= gu.ELEM_TOL
    assert np.all(o_gpu[1][[3, 50, 95]] == 0)
    gu.check_layers(w0, g1, z, w_gpu[1], m_gpu[1], o_gpu[1], lr=0.1, momentum=0.9, wd=0.5, coeffs=STD,
                    nesterov=True, row_norm=True, ns_tol=gu.NS_TOL_BF16)


def test_deterministic_and_workspace_contents_do_not_matter():
    import torch
    import muon_optimizer_step_amd as ms
    w = wl.workload(1)
    st = wl.make_state(w, 11)
    grads = wl.make_grads(w, 11, 0)
    shapes = [(r, c) for _, r, c in w.matrices]
    nbytes = ms.workspace_size(shapes)
    outs = []
    for fill in (0, 0xFF, 0x7F):  # zeros, NaN patterns, large finite values
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        P = [gu.dev(p) for p in st["params"]]
        M = [gu.dev(m) for m in st["moms"]]
        O = [torch.empty_like(p) for p in P]
        E = [gu.dev(e) for e in wl.make_independent_ema(w, 12)]
        ms.muon_step(P, [gu.dev(g) for g in grads], M, lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay,
                     coeffs=STD, update_outs=O, emas=E, ema_decay=0.9965, workspace=ws)
        torch.cuda.synchronize()
        outs.append([gu.host(t) for t in P + M + O + E])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_invalid_call_has_no_side_effects():
    import torch
    import muon_optimizer_step_amd as ms
    p = torch.ones(64, 64, device="cuda")
    g = torch.ones(64, 64, device="cuda")
    m = torch.ones(64, 64, device="cuda")
    with pytest.raises(ms.MuonError):
        ms.muon_step([p], [g], [m], lr=float("nan"), momentum=0.9, weight_decay=0.1, coeffs=STD)
    with pytest.raises(ms.MuonError):
        ms.muon_step([p], [g], [m], lr=0.1, momentum=0.9, weight_decay=0.1, coeffs=STD,
                     workspace=torch.empty(1024, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert bool((p == 1).all()) and bool((m == 1).all())


def test_many_tensors_and_shape_groups():
    """More tensors than one launch's table and more shape groups than one NS launch holds."""
    rng = np.random.default_rng(8)
    shapes = [(int(r), int(c)) for r, c in rng.integers(1, 300, size=(90, 2))]
    mats = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    grads = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    moms = [np.zeros(s, np.float32) for s in shapes]
    coeffs = wl.coeff_table(wl.workload(4), 3).tolist()
    emas = [rng.standard_normal(s).astype(np.float32) if i % 3 else None for i, s in enumerate(shapes)]
    w_gpu, m_gpu, o_gpu, e_gpu = gu.gpu_step(mats, grads, moms, lr=0.02, momentum=0.95, wd=0.1, coeffs=coeffs,
                                             emas=emas, ema_decay=0.5)
    gu.check_fused_ema(emas, w_gpu, e_gpu, 0.5)
    for i, s in enumerate(shapes):
        gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.02, momentum=0.95, wd=0.1,
                        coeffs=coeffs, nesterov=True, row_norm=True, ns_tol=gu.NS_TOL_BF16, label=f"{i} {s}")


@pytest.mark.parametrize("rows,cols", [(8192, 8192), (4096, 65536), (65536, 4096)])
def test_maximum_sizes_on_a_known_spectrum(rows, cols):
    """At the size limits, a gradient with one nonzero per short-side line.

    Then X X^T is diagonal, every NS product is exact in its zeros, and O has
    the same sparsity with entries phi(x) of the composed scalar map: the
    oracle's NS on each 1x1 entry gives the expected values.  Checked on the
    GPU with torch reductions (nothing of this size goes through the host).
    """
    import torch
    import muon_optimizer_step_amd as ms
    gu.say(f"[edge] max size {rows}x{cols}")
    m = min(rows, cols)
    gen = torch.Generator(device="cpu").manual_seed(rows + cols)
    vals = (torch.rand(m, generator=gen, dtype=torch.float64) * 2 + 0.5) * torch.where(
        torch.rand(m, generator=gen) < 0.5, -1.0, 1.0)
    pos = torch.randperm(max(rows, cols), generator=gen)[:m]
    G = torch.zeros(rows, cols, device="cuda")
    idx = torch.arange(m)
    if rows <= cols:
        G[idx.cuda(), pos.cuda()] = vals.float().cuda()
    else:
        G[pos.cuda(), idx.cuda()] = vals.float().cuda()
    P = torch.zeros_like(G)
    M = torch.zeros_like(G)
    O = torch.empty_like(G)
    E = torch.zeros_like(G)
    ms.muon_step([P], [G], [M], lr=1.0, momentum=0.0, weight_decay=0.0, coeffs=STD, row_norm=False, update_outs=[O],
                 emas=[E], ema_decay=0.5)
    torch.cuda.synchronize()
    # W' = -s*O from W = 0 and E = 0: E' = 0.5*W' exactly, over every element
    s = max(1.0, rows / cols) ** 0.5
    assert torch.equal(E, 0.5 * P)
    assert float((P + np.float32(s) * O).abs().max()) <= 1e-6 * float(O.abs().max())
    del E
    v32 = vals.float().double().numpy()
    x0 = v32 / (np.sqrt(np.sum(v32 * v32)) + 1e-7)
    want = np.array([om.newton_schulz(np.array([[x]]), STD)[0, 0] for x in x0])
    if rows <= cols:
        got = O[idx.cuda(), pos.cuda()].double().cpu().numpy()
    else:
        got = O[pos.cuda(), idx.cuda()].double().cpu().numpy()
    assert gu.rel_frob(got, want) <= gu.NS_TOL_BF16
    total = O.abs().double().sum().item()
    assert abs(total - np.abs(got).sum()) <= 1e-6 * total   # nothing off the pattern
    s = np.sqrt(max(1.0, rows / cols))
    assert gu.rel_max(P[:4].double().cpu().numpy(), -s * O[:4].double().cpu().numpy()) <= 1e-6


def test_ema_layouts_and_chunking():
    import torch
    import muon_optimizer_step_amd as ms
    rng = np.random.default_rng(12)
    sizes = [0, 1, 3, 4095, 4096, 4097, 65537] + [int(s) for s in rng.integers(1, 5000, size=300)]
    e0 = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    p0 = [rng.standard_normal(n).astype(np.float32) for n in sizes]
    # unaligned views: start one float into a bigger buffer
    big_e = torch.zeros(10001, device="cuda")
    big_p = torch.zeros(10001, device="cuda")
    big_e[1:].copy_(gu.dev(rng.standard_normal(10000).astype(np.float32)))
    big_p[1:].copy_(gu.dev(rng.standard_normal(10000).astype(np.float32)))
    for decay in (0.9965, 0.0, 1.0):
        E = [gu.dev(e) for e in e0] + [big_e[1:]]
        P = [gu.dev(p) for p in p0] + [big_p[1:]]
        ref_last = om.ema_update(gu.host(big_e[1:]), gu.host(big_p[1:]), gu.f32(decay))
        ms.ema_update(E, P, decay)
        torch.cuda.synchronize()
        for i, (e, p) in enumerate(zip(e0, p0)):
            assert gu.rel_max(gu.host(E[i]), om.ema_update(e, p, gu.f32(decay))) <= gu.ELEM_TOL, (decay, i)
        assert gu.rel_max(gu.host(E[-1]), ref_last) <= gu.ELEM_TOL
        if decay == 1.0:
            assert all(np.array_equal(gu.host(E[i]), e0[i]) for i in range(len(e0)))
        big_e[1:].copy_(gu.dev(rng.standard_normal(10000).astype(np.float32)))


def test_more_matrices_than_the_fused_apply_table():
    """80 matrices of one shape: the last NS launch cannot carry all weight
    updates, so the separate apply kernel runs after the iteration."""
    rng = np.random.default_rng(21)
    shapes = [(64, 96)] * 80
    mats = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    grads = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    moms = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    emas = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    w_gpu, m_gpu, o_gpu, e_gpu = gu.gpu_step(mats, grads, moms, lr=0.03, momentum=0.9, wd=0.1, coeffs=STD,
                                             emas=emas, ema_decay=0.9965)
    gu.check_fused_ema(emas, w_gpu, e_gpu, 0.9965)
    for i in range(0, 80, 7):
        gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.03, momentum=0.9, wd=0.1,
                        coeffs=STD, nesterov=True, row_norm=True, ns_tol=gu.NS_TOL_BF16, label=f"{i}")


def test_more_matrices_than_the_folded_frobenius_table():
    """400 matrices of one shape in one launch: more than the first Gram's table
    of row-sum spans (360), so the separate Frobenius-scale launch runs (and the
    separate apply, past the fused table)."""
    rng = np.random.default_rng(22)
    shapes = [(32, 48)] * 400
    mats = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    grads = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    moms = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    w_gpu, m_gpu, o_gpu, _ = gu.gpu_step(mats, grads, moms, lr=0.02, momentum=0.95, wd=0.0, coeffs=STD)
    for i in range(0, 400, 37):
        gu.check_layers(mats[i], grads[i], moms[i], w_gpu[i], m_gpu[i], o_gpu[i], lr=0.02, momentum=0.95, wd=0.0,
                        coeffs=STD, nesterov=True, row_norm=True, ns_tol=gu.NS_TOL_BF16, label=f"{i}")


def test_ema_and_swap_of_a_tensor_past_2_30_elements():
    """One tensor of 2^30 + 4099 elements takes two table entries (the split at
    2^30 elements): the EMA matches the oracle on slices around the split and a
    float32 device check everywhere; the swap exchanges every element exactly."""
    import torch
    import muon_optimizer_step_amd as ms
    n = (1 << 30) + 4099
    gen = torch.Generator(device="cuda").manual_seed(5)
    e = torch.rand(n, device="cuda", generator=gen)
    p = torch.rand(n, device="cuda", generator=gen)
    e0 = e.clone()
    decay = 0.99
    gu.say(f"[edges] EMA of {n} elements")
    ms.ema_update([e], [p], decay)
    torch.cuda.synchronize()
    for lo, hi in ((0, 4096), ((1 << 30) - 4096, n)):
        want = om.ema_update(e0[lo:hi].cpu().numpy(), p[lo:hi].cpu().numpy(), gu.f32(decay))
        assert gu.rel_max(e[lo:hi].cpu().numpy(), want) <= gu.ELEM_TOL, (lo, hi)
    ref = e0.mul_(decay).add_(p, alpha=1.0 - decay)
    assert float((e - ref).abs_().max()) <= 1e-6 * float(ref.abs().max())
    del ref, e0
    e1, p1 = e.clone(), p.clone()
    ms.ema_swap([e], [p])
    torch.cuda.synchronize()
    assert torch.equal(e, p1) and torch.equal(p, e1)


def test_ema_swap_is_an_exact_exchange():
    """ema_swap exchanges the buffers bit for bit (vector and scalar paths, many tensors); twice is identity."""
    import torch
    import muon_optimizer_step_amd as ms
    rng = np.random.default_rng(31)
    sizes = [4096 * 3, 1, 4095, 4097, 512, 92] + [int(x) for x in rng.integers(1, 9000, size=130)]
    total = sum(sizes) + 3 * len(sizes)
    flat_e = torch.from_numpy(rng.standard_normal(total).astype(np.float32)).cuda()
    flat_p = torch.from_numpy(rng.standard_normal(total).astype(np.float32)).cuda()
    E, P, pos = [], [], 0
    for i, k in enumerate(sizes):
        off = pos + (i % 3)          # some tensors start off the 16-byte grid
        E.append(flat_e[off:off + k])
        P.append(flat_p[off:off + k])
        pos += k + 3
    e0 = [x.clone() for x in E]
    p0 = [x.clone() for x in P]
    ms.ema_swap(E, P)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(E, p0)) and all(torch.equal(a, b) for a, b in zip(P, e0))
    ms.ema_swap(E, P)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(E, e0)) and all(torch.equal(a, b) for a, b in zip(P, p0))
