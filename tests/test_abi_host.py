"""The C ABI on the host: the library loads, exports what include/muonstep.h
declares, sizes workspaces, and rejects bad arguments before touching a GPU.

Every call here fails validation (or only sizes a workspace), so no HIP call
is made and no GPU is needed.
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

from muon_optimizer_step_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muonstep.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_abi():
    names = _declared_functions()
    assert names == sorted(["muon_workspace_size", "muon_step", "ema_update", "ema_swap", "adamw_step",
                            "muon_last_error", "muon_version", "muon_profile_enable", "muon_profile_read",
                            "muon_plan_cache_stats", "muon_set_ns_schedule", "muon_step_static", "muon_step_ema"])


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert lib.muon_version() == 10000


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ["MUON_OK", "MUON_ERR_INVALID_ARG", "MUON_ERR_UNSUPPORTED", "MUON_ERR_WORKSPACE", "MUON_ERR_HIP",
                 "MUON_MAX_NS_STEPS", "MUON_MAX_SHORT_SIDE", "MUON_MAX_LONG_SIDE", "MUON_MAX_TENSORS",
                 "MUON_NS_BF16", "MUON_NS_FP32", "MUON_NS_BF16X3", "MUON_NS_SCHEDULE_PHASES",
                 "MUON_NS_SCHEDULE_CHAIN"]:
        m = re.search(rf"#define {name} \(?(-?\d+)\)?", text)
        assert m, name
        assert int(m.group(1)) == getattr(_lib, name), name
    assert ctypes.sizeof(_lib.MuonTensor) == 48
    assert ctypes.sizeof(_lib.AdamWTensor) == 48


# Fake, well-separated device addresses: validation only compares them.
BASE = 1 << 40


def _t(i, rows, cols, out=False, ema=False):
    span = 1 << 30
    p = BASE + 5 * i * span
    return (p, p + span, p + 2 * span, (p + 3 * span) if out else 0, (p + 4 * span) if ema else 0, rows, cols)


def _call(entries, lr=0.02, mu=0.95, nesterov=1, wd=0.1, row_norm=1, steps=5, coeffs="std",
          prec=0, ema_decay=0.9965, ws=BASE + (1 << 45), ws_bytes=1 << 40, n=None):
    lib = _lib.load()
    table = _lib.tensor_table(entries)
    if coeffs == "std":
        carr, k = _lib.coeff_array([(3.4445, -4.775, 2.0315)] * max(steps, 0))
        cptr = carr
    else:
        cptr = coeffs
    rc = lib.muon_step(table, len(entries) if n is None else n, lr, mu, nesterov, wd, row_norm, steps, cptr, prec,
                       ema_decay, ctypes.c_void_p(ws), ws_bytes, None)
    return rc, lib.muon_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n=0), _lib.MUON_ERR_INVALID_ARG, "n = 0"),
    (dict(n=_lib.MUON_MAX_TENSORS + 1), _lib.MUON_ERR_INVALID_ARG, "outside"),
    (dict(prec=3), _lib.MUON_ERR_INVALID_ARG, "ns_precision"),
    (dict(lr=float("nan")), _lib.MUON_ERR_INVALID_ARG, "finite"),
    (dict(mu=float("inf")), _lib.MUON_ERR_INVALID_ARG, "finite"),
    (dict(wd=float("-inf")), _lib.MUON_ERR_INVALID_ARG, "finite"),
    (dict(nesterov=2), _lib.MUON_ERR_INVALID_ARG, "nesterov"),
    (dict(row_norm=-1), _lib.MUON_ERR_INVALID_ARG, "row_norm"),
    (dict(steps=-1), _lib.MUON_ERR_INVALID_ARG, "ns_steps"),
    (dict(steps=_lib.MUON_MAX_NS_STEPS + 1), _lib.MUON_ERR_INVALID_ARG, "ns_steps"),
    (dict(steps=3, coeffs=None), _lib.MUON_ERR_INVALID_ARG, "ns_coeffs is NULL"),
    (dict(ema_decay=1.5), _lib.MUON_ERR_INVALID_ARG, "ema_decay"),
    (dict(ema_decay=-0.25), _lib.MUON_ERR_INVALID_ARG, "ema_decay"),
    (dict(ema_decay=float("nan")), _lib.MUON_ERR_INVALID_ARG, "ema_decay"),
    (dict(ws=0), _lib.MUON_ERR_WORKSPACE, "workspace is NULL"),
    (dict(ws=BASE + (1 << 45) + 16), _lib.MUON_ERR_WORKSPACE, "256-byte"),
    (dict(ws_bytes=1024), _lib.MUON_ERR_WORKSPACE, "needs"),
])
def test_muon_step_rejects_bad_arguments(kw, code, msg):
    rc, err = _call([_t(0, 64, 32, ema=True), _t(1, 16, 48)], **kw)
    assert rc == code and msg in err, (rc, err)


def test_muon_step_rejects_non_finite_coefficients():
    carr, _ = _lib.coeff_array([(3.4445, -4.775, 2.0315), (1.0, float("nan"), 0.0)])
    rc, err = _call([_t(0, 64, 32)], steps=2, coeffs=carr)
    assert rc == _lib.MUON_ERR_INVALID_ARG and "ns_coeffs[4]" in err


@pytest.mark.parametrize("shape,code", [
    ((0, 5), _lib.MUON_ERR_INVALID_ARG), ((5, -1), _lib.MUON_ERR_INVALID_ARG),
    ((_lib.MUON_MAX_SHORT_SIDE + 1, _lib.MUON_MAX_SHORT_SIDE + 1), _lib.MUON_ERR_UNSUPPORTED),
    ((4, _lib.MUON_MAX_LONG_SIDE + 1), _lib.MUON_ERR_UNSUPPORTED),
])
def test_muon_step_rejects_bad_shapes(shape, code):
    rc, err = _call([_t(0, *shape)])
    assert rc == code, err


def test_muon_step_rejects_null_and_aliased_buffers():
    p, g, m, o, e, r, c = _t(0, 64, 64, ema=True)
    rc, err = _call([(0, g, m, 0, 0, r, c)])
    assert rc == _lib.MUON_ERR_INVALID_ARG and "non-NULL" in err
    rc, err = _call([(p, p, m, 0, 0, r, c)])          # grad aliases param
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "overlap" in err
    rc, err = _call([(p, g, m, g + 256, 0, r, c)])    # update_out overlaps grad
    assert rc == _lib.MUON_ERR_UNSUPPORTED
    rc, err = _call([(p, g, m, 0, p + 512, r, c)])    # ema overlaps param
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "overlap" in err
    rc, err = _call([(p, g, m, 0, e + 2, r, c)])      # misaligned ema
    assert rc == _lib.MUON_ERR_INVALID_ARG and "aligned" in err
    q = _t(1, 64, 64)
    rc, err = _call([(p, g, m, 0, 0, r, c), (q[0], q[1], m + 4, 0, 0, r, c)])  # two tensors share a buffer
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "tensors 0 and 1" in err
    rc, err = _call([(p, g, m, 0, e, r, c), (q[0], q[1], q[2], 0, e + 64, r, c)])  # two tensors share an ema
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "tensors 0 and 1" in err
    rc, err = _call([(p + 2, g, m, 0, 0, r, c)])      # misaligned
    assert rc == _lib.MUON_ERR_INVALID_ARG and "aligned" in err
    rc, err = _call([(p, g, m, 0, 0, r, c)], ws=p - 256)  # workspace overlaps a tensor
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "workspace" in err
    rc, err = _call([(p, g, m, 0, e, r, c)], ws=e + 1024)  # workspace overlaps an ema
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "workspace" in err


def _ws(shapes, prec=0):
    lib = _lib.load()
    table = _lib.tensor_table((0, 0, 0, 0, 0, r, c) for r, c in shapes)
    return lib.muon_workspace_size(table, len(shapes), prec)


def test_workspace_size_properties():
    one = _ws([(512, 512)])
    # four bf16 planes of X (two ping-pong pairs) and three of the Gram-sized matrices
    assert one >= 4 * 2 * 512 * 512 + 3 * 2 * 512 * 512
    assert _ws([(512, 512)], 1) >= 4 * 2 * 512 * 512 + 2 * 4 * 512 * 512   # two fp32 X planes, A and B
    # orientation only changes the per-row sums (one float per stored row)
    assert 0 <= _ws([(2048, 512)]) - _ws([(512, 2048)]) <= 4 * (2048 - 512) + 256
    assert _ws([(100, 30)]) == _ws([(128, 128)])           # padded to 128 on both sides
    assert _ws([(512, 512)] * 22) > 21 * one
    assert _ws([(4, 4)]) % 256 == 0
    assert _ws([]) == 0 and _ws([(0, 4)]) == 0 and _ws([(4, 4)], 7) == 0
    # the compensated mode needs no more; the base mode adds the NS chain's
    # per-matrix record (64 B) and counters (two 128-byte lines, plus one status
    # block per chain launch), each region 256-byte aligned
    assert 0 <= one - _ws([(512, 512)], 2) <= 256 + 3 * 256
    assert _ws([(512, 512)] * 22) - _ws([(512, 512)] * 22, 2) <= 22 * 64 + 23 * 256 + 512


def test_ema_rejects_bad_arguments():
    lib = _lib.load()
    n = 2
    e = (ctypes.c_void_p * n)(BASE, BASE + (1 << 30))
    p = (ctypes.c_void_p * n)(BASE + (2 << 30), BASE + (3 << 30))
    ne = (ctypes.c_int64 * n)(100, 200)

    def call(e=e, p=p, ne=ne, n=n, decay=0.99):
        return lib.ema_update(e, p, ne, n, decay, None), lib.muon_last_error().decode()

    assert call(n=0)[0] == _lib.MUON_ERR_INVALID_ARG
    assert call(decay=1.5)[0] == _lib.MUON_ERR_INVALID_ARG
    assert call(decay=-0.1)[0] == _lib.MUON_ERR_INVALID_ARG
    assert call(decay=math.nan)[0] == _lib.MUON_ERR_INVALID_ARG
    bad = (ctypes.c_int64 * n)(100, -1)
    assert call(ne=bad)[0] == _lib.MUON_ERR_INVALID_ARG
    alias = (ctypes.c_void_p * n)(BASE, BASE + 200)   # param 0 overlaps ema 0's tail
    rc, err = call(p=alias)
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "overlap" in err
    nul = (ctypes.c_void_p * n)(BASE, 0)
    assert call(e=nul)[0] == _lib.MUON_ERR_INVALID_ARG
    odd = (ctypes.c_void_p * n)(BASE + 2, BASE + (1 << 30))
    assert call(e=odd)[0] == _lib.MUON_ERR_INVALID_ARG


def test_profile_read_without_events():
    lib = _lib.load()
    assert lib.muon_profile_enable(0) == 0
    assert lib.muon_profile_read(None, None, None, 0, 1) == 0


def _adam_t(i, numel, ema=False):
    span = 1 << 30
    p = BASE + 5 * i * span
    return (p, p + span, p + 2 * span, p + 3 * span, (p + 4 * span) if ema else 0, numel)


def _adam_call(entries, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01, step=10, ema_decay=0.99, n=None):
    lib = _lib.load()
    table = _lib.adamw_table(entries)
    rc = lib.adamw_step(table, len(entries) if n is None else n, lr, b1, b2, eps, wd, step, ema_decay, None)
    return rc, lib.muon_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n=0), _lib.MUON_ERR_INVALID_ARG, "n = 0"),
    (dict(n=_lib.MUON_MAX_TENSORS + 1), _lib.MUON_ERR_INVALID_ARG, "outside"),
    (dict(lr=float("nan")), _lib.MUON_ERR_INVALID_ARG, "finite"),
    (dict(wd=float("inf")), _lib.MUON_ERR_INVALID_ARG, "finite"),
    (dict(eps=-1e-8), _lib.MUON_ERR_INVALID_ARG, "eps"),
    (dict(b1=1.0), _lib.MUON_ERR_INVALID_ARG, "beta1"),
    (dict(b2=-0.5), _lib.MUON_ERR_INVALID_ARG, "beta1 and beta2"),
    (dict(b2=float("nan")), _lib.MUON_ERR_INVALID_ARG, "beta1 and beta2"),
    (dict(step=0), _lib.MUON_ERR_INVALID_ARG, "step"),
    (dict(ema_decay=1.01), _lib.MUON_ERR_INVALID_ARG, "ema_decay"),
])
def test_adamw_rejects_bad_arguments(kw, code, msg):
    rc, err = _adam_call([_adam_t(0, 1000, ema=True), _adam_t(1, 7)], **kw)
    assert rc == code and msg in err, (rc, err)


def test_adamw_rejects_bad_tensors():
    p, g, m, v, e, k = _adam_t(0, 4096, ema=True)
    assert _adam_call([(p, g, m, v, e, -1)])[0] == _lib.MUON_ERR_INVALID_ARG
    assert _adam_call([(p, g, m, v, e, 1 << 41)])[0] == _lib.MUON_ERR_UNSUPPORTED
    rc, err = _adam_call([(p, 0, m, v, e, k)])
    assert rc == _lib.MUON_ERR_INVALID_ARG and "non-NULL" in err
    rc, err = _adam_call([(p, g, m + 2, v, e, k)])
    assert rc == _lib.MUON_ERR_INVALID_ARG and "aligned" in err
    rc, err = _adam_call([(p, g, m, m + 64, e, k)])          # second moment overlaps the first
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "overlap" in err
    rc, err = _adam_call([(p, g, m, v, p + 4, k)])           # ema overlaps the parameter
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "overlap" in err
    q = _adam_t(1, 4096)
    rc, err = _adam_call([(p, g, m, v, e, k), (q[0], g + 1024, q[2], q[3], 0, k)])  # two tensors share a grad
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "tensors 0 and 1" in err


def test_streaming_entry_points_reject_huge_tensors():
    lib = _lib.load()
    e = (ctypes.c_void_p * 1)(BASE)
    p = (ctypes.c_void_p * 1)(BASE + (1 << 44))
    ne = (ctypes.c_int64 * 1)(1 << 41)
    assert lib.ema_update(e, p, ne, 1, 0.5, None) == _lib.MUON_ERR_UNSUPPORTED


def test_ema_swap_rejects_bad_arguments():
    lib = _lib.load()
    n = 2
    e = (ctypes.c_void_p * n)(BASE, BASE + (1 << 30))
    p = (ctypes.c_void_p * n)(BASE + (2 << 30), BASE + (3 << 30))
    ne = (ctypes.c_int64 * n)(100, 200)

    def call(e=e, p=p, ne=ne, n=n):
        return lib.ema_swap(e, p, ne, n, None), lib.muon_last_error().decode()

    assert call(n=0)[0] == _lib.MUON_ERR_INVALID_ARG
    assert call(ne=(ctypes.c_int64 * n)(100, -1))[0] == _lib.MUON_ERR_INVALID_ARG
    assert call(ne=(ctypes.c_int64 * n)(100, 1 << 41))[0] == _lib.MUON_ERR_UNSUPPORTED
    rc, err = call(p=(ctypes.c_void_p * n)(BASE + 64, BASE + (3 << 30)))   # param 0 inside ema 0
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "overlap" in err
    assert call(e=(ctypes.c_void_p * n)(0, BASE + (1 << 30)))[0] == _lib.MUON_ERR_INVALID_ARG
    assert call(p=(ctypes.c_void_p * n)(BASE + (2 << 30) + 1, BASE + (3 << 30)))[0] == _lib.MUON_ERR_INVALID_ARG


def test_second_call_with_the_same_signature_reuses_the_schedule():
    """muon_step plans once per signature (tensor descriptors, precision, workspace).

    Without a GPU the call fails at its first HIP call, after validation and
    planning, so the schedule cache can be observed here: the second call with
    the same descriptors is a hit, a changed pointer or shape is a new plan.
    """
    entries = [_t(0, 512, 512), _t(1, 256, 512), _t(2, 2048, 512), _t(3, 512, 2048)]
    built0, hits0, _ = _lib.plan_cache_stats()
    rc, _ = _call(entries)
    assert rc in (_lib.MUON_ERR_HIP, _lib.MUON_OK)
    built1, hits1, _ = _lib.plan_cache_stats()
    assert (built1, hits1) == (built0 + 1, hits0)
    rc, _ = _call(entries, lr=0.05, mu=0.9, steps=3)   # scalars are not part of the signature
    built2, hits2, _ = _lib.plan_cache_stats()
    assert (built2, hits2) == (built1, hits1 + 1)
    moved = list(entries)
    moved[1] = _t(7, 256, 512)                          # another buffer: another signature
    _call(moved)
    built3, hits3, _ = _lib.plan_cache_stats()
    assert (built3, hits3) == (built2 + 1, hits2)
    reshaped = list(entries)
    reshaped[0] = _t(0, 512, 384)
    _call(reshaped)
    built4, _, held = _lib.plan_cache_stats()
    assert built4 == built3 + 1 and 1 <= held <= 8
    # a rejected call plans nothing
    rc, _ = _call(entries, lr=float("nan"))
    assert rc == _lib.MUON_ERR_INVALID_ARG
    assert _lib.plan_cache_stats()[0] == built4


def test_ns_schedule_setting_is_part_of_the_signature():
    entries = [_t(20, 512, 512), _t(21, 512, 2048)]
    prev = _lib.set_ns_schedule(_lib.MUON_NS_SCHEDULE_PHASES)
    try:
        _call(entries)
        built0, _, _ = _lib.plan_cache_stats()
        _call(entries)
        assert _lib.plan_cache_stats()[0] == built0
        assert _lib.set_ns_schedule(_lib.MUON_NS_SCHEDULE_CHAIN) == _lib.MUON_NS_SCHEDULE_PHASES
        _call(entries)                                   # another schedule: another plan
        assert _lib.plan_cache_stats()[0] == built0 + 1
        with pytest.raises(_lib.MuonError):
            _lib.set_ns_schedule(7)
        assert _lib.set_ns_schedule(_lib.MUON_NS_SCHEDULE_PHASES) == _lib.MUON_NS_SCHEDULE_CHAIN
    finally:
        _lib.set_ns_schedule(prev)


def test_static_entry_rejects_what_the_static_workspace_cannot_hold():
    """muon_step_static checks the workspace it would need before any HIP call."""
    lib = _lib.load()
    entries = [_t(40 + i, 2048, 512) for i in range(30)]   # about 150 MB of workspace
    table = _lib.tensor_table(entries)
    assert lib.muon_workspace_size(table, len(entries), 0) > _lib.MUON_STATIC_WORKSPACE_BYTES
    carr, k = _lib.coeff_array([(3.4445, -4.775, 2.0315)] * 5)
    rc = lib.muon_step_static(table, len(entries), 0.02, 0.95, 1, 0.1, 1, k, carr, 0, 0.99, None)
    assert rc == _lib.MUON_ERR_WORKSPACE
    assert "static workspace" in lib.muon_last_error().decode()
    assert lib.muon_step_static(table, 0, 0.02, 0.95, 1, 0.1, 1, k, carr, 0, 0.99, None) == _lib.MUON_ERR_INVALID_ARG


def _call_ema(entries, extra, ws=BASE + (1 << 45), ws_bytes=1 << 40, n_extra=None, decay=0.9965, arrays=True):
    """muon_step_ema with the standard table; extra: list of (ema, param, numel) fake pointers."""
    lib = _lib.load()
    table = _lib.tensor_table(entries)
    carr, k = _lib.coeff_array([(3.4445, -4.775, 2.0315)] * 5)
    m = len(extra)
    e = (ctypes.c_void_p * max(1, m))(*[x[0] for x in extra])
    p = (ctypes.c_void_p * max(1, m))(*[x[1] for x in extra])
    ne = (ctypes.c_int64 * max(1, m))(*[x[2] for x in extra])
    if not arrays:
        e = p = ne = None
    rc = lib.muon_step_ema(table, len(entries), 0.02, 0.95, 1, 0.1, 1, k, carr, 0, decay, e, p, ne,
                           m if n_extra is None else n_extra, ctypes.c_void_p(ws), ws_bytes, None)
    return rc, lib.muon_last_error().decode()


EXTRA = BASE + (1 << 44)   # the other tensors' buffers, far from the matrices'


def _x(i, numel):
    return (EXTRA + 2 * i * (1 << 30), EXTRA + (2 * i + 1) * (1 << 30), numel)


def test_muon_step_ema_validates_the_extra_list_before_anything():
    mats = [_t(0, 64, 32, ema=True), _t(1, 16, 48)]
    good = [_x(0, 4096), _x(1, 17)]
    # a valid call reaches the GPU (or, without one, fails at its first HIP call): nothing here is rejected
    rc, err = _call_ema(mats, good)
    assert rc in (_lib.MUON_OK, _lib.MUON_ERR_HIP), err
    assert _call_ema(mats, good, n_extra=-1)[0] == _lib.MUON_ERR_INVALID_ARG
    assert _call_ema(mats, good, n_extra=_lib.MUON_MAX_TENSORS + 1)[0] == _lib.MUON_ERR_INVALID_ARG
    assert _call_ema(mats, good, arrays=False)[0] == _lib.MUON_ERR_INVALID_ARG
    assert _call_ema(mats, [_x(0, -1)])[0] == _lib.MUON_ERR_INVALID_ARG
    assert _call_ema(mats, [_x(0, 1 << 41)])[0] == _lib.MUON_ERR_UNSUPPORTED
    assert _call_ema(mats, [(0, EXTRA, 10)])[0] == _lib.MUON_ERR_INVALID_ARG          # NULL ema
    assert _call_ema(mats, [(EXTRA + 2, EXTRA + (1 << 30), 10)])[0] == _lib.MUON_ERR_INVALID_ARG   # misaligned
    rc, err = _call_ema(mats, [(EXTRA, EXTRA + 64, 1000)])                 # an ema overlapping its param
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "overlap" in err
    rc, err = _call_ema(mats, [_x(0, 100), (_x(1, 100)[0], _x(0, 100)[1] + 16, 100)])   # two extras share a buffer
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "overlap" in err
    p0, g0, m0, _, e0, r0, c0 = mats[0]
    for buf in (p0, g0, m0, e0):                                            # an extra buffer inside a matrix's
        rc, err = _call_ema(mats, [(EXTRA, buf + 128, 10)])
        assert rc == _lib.MUON_ERR_UNSUPPORTED and "muon_step_ema" in err, (buf, err)
    ws = BASE + (1 << 45)
    rc, err = _call_ema(mats, [(EXTRA, ws + 4096, 10)], ws=ws)              # inside the workspace
    assert rc == _lib.MUON_ERR_UNSUPPORTED and "overlap" in err
    assert _call_ema(mats, good, decay=1.5)[0] == _lib.MUON_ERR_INVALID_ARG
    # n_extra == 0 is muon_step itself, the arrays may be NULL
    rc0, _ = _call_ema(mats, [], arrays=False)
    rc1, _ = _call(mats)
    assert rc0 == rc1


def test_muon_step_ema_plans_like_muon_step():
    """The extra list is not part of the schedule signature: the same matrices reuse the schedule."""
    mats = [_t(60, 512, 512), _t(61, 256, 512)]
    _call(mats)
    built0, hits0, _ = _lib.plan_cache_stats()
    rc, err = _call_ema(mats, [_x(5, 1 << 20)])
    assert rc in (_lib.MUON_OK, _lib.MUON_ERR_HIP), err
    built1, hits1, _ = _lib.plan_cache_stats()
    assert (built1, hits1) == (built0, hits0 + 1)
