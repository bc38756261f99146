"""The seeded input generators: sizes from the pages, determinism, structure."""

import numpy as np

import workloads as wl


def test_param_counts_and_tensor_lists():
    w2 = wl.workload(2)
    assert w2.n_params == wl.PAGE_PARAM_COUNT_512 == 34_401_372
    assert len(w2.matrices) == 66 and len(w2.matrices) + len(w2.extras) == 187
    assert w2.n_matrix_elems == 31_719_424
    assert wl.workload(3).n_matrix_elems == 126_877_696
    assert wl.workload(4).matrices == w2.matrices
    assert [(r, c) for _, r, c in wl.workload(1).matrices] == [
        (512, 512), (256, 512), (256, 512), (512, 512), (2048, 512), (512, 2048)]


def test_generators_are_deterministic_and_distinct():
    w = wl.workload(1)
    a, b = wl.make_state(w, 1337), wl.make_state(w, 1337)
    c = wl.make_state(w, 42)
    for x, y, z in zip(a["params"], b["params"], c["params"]):
        assert x.dtype == np.float32 and x.flags.c_contiguous
        assert np.array_equal(x, y) and not np.array_equal(x, z)
    g0, g1 = wl.make_grads(w, 1337, 0), wl.make_grads(w, 1337, 1)
    assert not np.array_equal(g0[0], g1[0])
    assert abs(float(np.std(g0[4])) - 1e-3) < 1e-4
    assert abs(float(np.std(a["params"][4])) - 0.02) < 1e-3


def test_structured_gradients_have_rank8_plus_noise():
    w = wl.workload(4)
    g = wl.make_grads(w, 1337, 0)[1]  # 256 x 512
    s = np.linalg.svd(g.astype(np.float64), compute_uv=False)
    assert s[7] > 100 * s[8]                 # eight large directions
    assert 0.1 < s[8] < 1.0 and s[-1] > 0.05  # noise floor ~ 1e-2 (sqrt(512) +- sqrt(256))


def test_coeff_table():
    t = wl.coeff_table(wl.workload(4), 1337)
    assert t.shape == (4, 3) and t.dtype == np.float32
    base = np.array(wl.STANDARD_TRIPLE, dtype=np.float32)
    rel = t / base - 1
    assert np.all(np.abs(rel) <= 0.05 + 1e-6) and len({tuple(r) for r in t}) == 4
    t2 = wl.coeff_table(wl.workload(2), 1337)
    assert t2.shape == (5, 3) and np.all(t2 == base)
