"""torch-facing binding: argument marshalling onto the C ABI, nothing else."""

from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence, Tuple

from . import _lib

# Cached workspaces, one per (device, stream), at most _MAX_WORKSPACES of them
# (least recently used first out).  Each is allocated with its stream current,
# so the caching allocator hands its memory to no other stream, and hands it
# back to that stream only in stream order once it is dropped: a workspace that
# kernels on its stream may still read is never reused under them.
_MAX_WORKSPACES = 4
_workspaces: "Dict[Tuple[int, int], object]" = {}


def _torch():
    import torch
    return torch


def _check_tensor(t, name: str, ndim: Optional[int] = None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_size(shapes: Sequence[Tuple[int, int]], ns_precision: int = _lib.MUON_NS_BF16) -> int:
    """Bytes of workspace muon_step needs for these (rows, cols) shapes."""
    table = _lib.tensor_table((0, 0, 0, 0, 0, int(r), int(c)) for r, c in shapes)
    n = _lib.load().muon_workspace_size(table, len(shapes), int(ns_precision))
    if n == 0:
        raise _lib.MuonError(_lib.MUON_ERR_INVALID_ARG, _lib.load().muon_last_error().decode())
    return int(n)


def _entries(params, grads, moms, update_outs, emas):
    """Checked descriptor tuples (param, grad, momentum, update_out, ema, rows, cols)."""
    n = len(params)
    outs = update_outs if update_outs is not None else [None] * n
    emas = emas if emas is not None else [None] * n
    if len(outs) != n or len(emas) != n:
        raise ValueError("update_outs and emas must have one entry per parameter")
    entries = []
    for i, (p, g, m, o, e) in enumerate(zip(params, grads, moms, outs, emas)):
        _check_tensor(p, f"params[{i}]", 2)
        _check_tensor(g, f"grads[{i}]", 2)
        _check_tensor(m, f"moms[{i}]", 2)
        if g.shape != p.shape or m.shape != p.shape:
            raise ValueError(f"tensor {i}: shapes differ {tuple(p.shape)} {tuple(g.shape)} {tuple(m.shape)}")
        for t, nm in ((o, "update_outs"), (e, "emas")):
            if t is not None:
                _check_tensor(t, f"{nm}[{i}]", 2)
                if t.shape != p.shape:
                    raise ValueError(f"{nm}[{i}] shape {tuple(t.shape)} != {tuple(p.shape)}")
        entries.append((p.data_ptr(), g.data_ptr(), m.data_ptr(), o.data_ptr() if o is not None else 0,
                        e.data_ptr() if e is not None else 0, p.shape[0], p.shape[1]))
    return entries


def _workspace_for(nbytes: int, device, stream):
    """A workspace of at least nbytes for kernels enqueued on `stream` (a torch stream)."""
    torch = _torch()
    index = device.index if device.index is not None else torch.cuda.current_device()
    key = (index, int(stream.cuda_stream))
    ws = _workspaces.pop(key, None)
    if ws is None or ws.numel() < nbytes:
        ws = None  # dropped on its own stream: stream-ordered reuse only
        with torch.cuda.stream(stream):
            ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _workspaces[key] = ws  # most recently used last
    while len(_workspaces) > _MAX_WORKSPACES:
        _workspaces.pop(next(iter(_workspaces)))
    return ws


def muon_step(params, grads, moms, *, lr: float, momentum: float, weight_decay: float,
              coeffs, nesterov: bool = True, row_norm: bool = True,
              ns_precision: int = _lib.MUON_NS_BF16, update_outs=None, emas=None, ema_decay: float = 0.0,
              extra_emas=None, extra_params=None, workspace=None, stream=None) -> None:
    """One Muon step over lists of 2-D fp32 tensors (params and moms updated in place).

    coeffs: ns_steps rows of (a, b, c); update_outs: optional list of tensors
    (or None entries) that receive the orthogonalised update O; emas: optional
    list of tensors (or None entries) advanced as ema = d*ema + (1-d)*W' with
    d = ema_decay, in the pass that writes W'.  extra_emas / extra_params:
    optional lists of other fp32 tensors (any shape) whose EMA is advanced with
    the same d in the same call (muon_step_ema), as ema_update after the step
    would.
    """
    lib = _lib.load()
    n = len(params)
    if len(grads) != n or len(moms) != n:
        raise ValueError("params, grads and moms must have the same length")
    entries = _entries(params, grads, moms, update_outs, emas)
    table = _lib.tensor_table(entries)
    carr, steps = _lib.coeff_array(coeffs)
    device = params[0].device if n else None
    if stream is None and n:
        stream = _torch().cuda.current_stream(device)
    if workspace is None:
        need = lib.muon_workspace_size(table, n, int(ns_precision))
        if need == 0:
            raise _lib.MuonError(_lib.MUON_ERR_INVALID_ARG, lib.muon_last_error().decode())
        workspace = _workspace_for(int(need), device, stream)
    if extra_emas is not None or extra_params is not None:
        xe, xp, xn, nx = _ema_list(extra_emas or [], extra_params or [], "extra_emas")
        rc = lib.muon_step_ema(table, n, float(lr), float(momentum), int(bool(nesterov)), float(weight_decay),
                               int(bool(row_norm)), steps, carr if steps else None, int(ns_precision),
                               float(ema_decay), xe, xp, xn, nx, ctypes.c_void_p(workspace.data_ptr()),
                               workspace.numel() * workspace.element_size(), _stream_handle(stream, device))
    else:
        rc = lib.muon_step(table, n, float(lr), float(momentum), int(bool(nesterov)), float(weight_decay),
                           int(bool(row_norm)), steps, carr if steps else None, int(ns_precision), float(ema_decay),
                           ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
                           _stream_handle(stream, device))
    _lib.check(rc)


def muon_step_static(params, grads, moms, *, lr: float, momentum: float, weight_decay: float, coeffs,
                     nesterov: bool = True, row_norm: bool = True, ns_precision: int = _lib.MUON_NS_BF16,
                     update_outs=None, emas=None, ema_decay: float = 0.0, stream=None) -> None:
    """muon_step on the library's static device workspace: allocates nothing.

    For callers that cannot allocate (graph capture, serving loops).  Calls that
    overlap in time on one GPU race on the shared static workspace.
    """
    lib = _lib.load()
    n = len(params)
    if len(grads) != n or len(moms) != n:
        raise ValueError("params, grads and moms must have the same length")
    table = _lib.tensor_table(_entries(params, grads, moms, update_outs, emas))
    carr, steps = _lib.coeff_array(coeffs)
    device = params[0].device if n else None
    rc = lib.muon_step_static(table, n, float(lr), float(momentum), int(bool(nesterov)), float(weight_decay),
                              int(bool(row_norm)), steps, carr if steps else None, int(ns_precision),
                              float(ema_decay), _stream_handle(stream, device))
    _lib.check(rc)


def _ema_list(emas, params, what: str = "emas"):
    """Checked pointer arrays (ema, params, numel) and the count of an EMA list."""
    n = len(emas)
    if len(params) != n:
        raise ValueError(f"{what} and its params must have the same length")
    e_ptrs = (ctypes.c_void_p * max(1, n))()
    p_ptrs = (ctypes.c_void_p * max(1, n))()
    numel = (ctypes.c_int64 * max(1, n))()
    for i, (e, p) in enumerate(zip(emas, params)):
        _check_tensor(e, f"{what}[{i}]")
        _check_tensor(p, f"params of {what}[{i}]")
        if e.numel() != p.numel():
            raise ValueError(f"{what}[{i}]: {e.numel()} != {p.numel()} elements")
        e_ptrs[i] = e.data_ptr()
        p_ptrs[i] = p.data_ptr()
        numel[i] = e.numel()
    return e_ptrs, p_ptrs, numel, n


def ema_update(emas, params, decay: float, stream=None) -> None:
    """emas[i] = decay * emas[i] + (1 - decay) * params[i] for fp32 tensors of any shape."""
    lib = _lib.load()
    e_ptrs, p_ptrs, numel, n = _ema_list(emas, params)
    device = emas[0].device if n else None
    rc = lib.ema_update(e_ptrs, p_ptrs, numel, n, float(decay), _stream_handle(stream, device))
    _lib.check(rc)


def _adamw_entries(params, grads, exp_avgs, exp_avg_sqs, emas):
    n = len(params)
    if len(grads) != n or len(exp_avgs) != n or len(exp_avg_sqs) != n:
        raise ValueError("params, grads, exp_avgs and exp_avg_sqs must have the same length")
    emas = emas if emas is not None else [None] * n
    if len(emas) != n:
        raise ValueError("emas must have one entry per parameter")
    entries = []
    for i, (p, g, m, v, e) in enumerate(zip(params, grads, exp_avgs, exp_avg_sqs, emas)):
        for t, nm in ((p, "params"), (g, "grads"), (m, "exp_avgs"), (v, "exp_avg_sqs")):
            _check_tensor(t, f"{nm}[{i}]")
            if t.numel() != p.numel():
                raise ValueError(f"{nm}[{i}] has {t.numel()} elements, params[{i}] {p.numel()}")
        if e is not None:
            _check_tensor(e, f"emas[{i}]")
            if e.numel() != p.numel():
                raise ValueError(f"emas[{i}] has {e.numel()} elements, params[{i}] {p.numel()}")
        entries.append((p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(),
                        e.data_ptr() if e is not None else 0, p.numel()))
    return entries


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, *, lr: float, betas=(0.9, 0.999), eps: float = 1e-8,
               weight_decay: float = 0.01, step: int, emas=None, ema_decay: float = 0.0, stream=None) -> None:
    """AdamW over lists of fp32 tensors of any shape (params and both moments updated in place).

    step counts the AdamW steps including this one (>= 1).  emas: optional list
    of tensors (or None entries) advanced as ema = d*ema + (1-d)*param' with
    d = ema_decay.
    """
    lib = _lib.load()
    entries = _adamw_entries(params, grads, exp_avgs, exp_avg_sqs, emas)
    table = _lib.adamw_table(entries)
    device = params[0].device if params else None
    rc = lib.adamw_step(table, len(entries), float(lr), float(betas[0]), float(betas[1]), float(eps),
                        float(weight_decay), int(step), float(ema_decay), _stream_handle(stream, device))
    _lib.check(rc)


class PreparedAdamW:
    """adamw_step with the tensor table marshalled once."""

    def __init__(self, params, grads, exp_avgs, exp_avg_sqs, emas=None):
        self._keep = (list(params), list(grads), list(exp_avgs), list(exp_avg_sqs), emas)
        entries = _adamw_entries(params, grads, exp_avgs, exp_avg_sqs, emas)
        self.n = len(entries)
        self.table = _lib.adamw_table(entries)
        self.device = params[0].device

    def __call__(self, *, lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, step, ema_decay=0.0, stream=None):
        rc = _lib.load().adamw_step(self.table, self.n, float(lr), float(betas[0]), float(betas[1]), float(eps),
                                    float(weight_decay), int(step), float(ema_decay),
                                    _stream_handle(stream, self.device))
        _lib.check(rc)


def ema_swap(emas, params, stream=None) -> None:
    """Exchange the contents of emas[i] and params[i] (fp32, same element count), bit for bit."""
    lib = _lib.load()
    n = len(emas)
    if len(params) != n:
        raise ValueError("emas and params must have the same length")
    e_ptrs = (ctypes.c_void_p * max(1, n))()
    p_ptrs = (ctypes.c_void_p * max(1, n))()
    numel = (ctypes.c_int64 * max(1, n))()
    for i, (e, p) in enumerate(zip(emas, params)):
        _check_tensor(e, f"emas[{i}]")
        _check_tensor(p, f"params[{i}]")
        if e.numel() != p.numel():
            raise ValueError(f"tensor {i}: {e.numel()} != {p.numel()} elements")
        e_ptrs[i], p_ptrs[i], numel[i] = e.data_ptr(), p.data_ptr(), e.numel()
    device = emas[0].device if n else None
    _lib.check(lib.ema_swap(e_ptrs, p_ptrs, numel, n, _stream_handle(stream, device)))


def profile_enable(enable: bool = True) -> None:
    _lib.check(_lib.load().muon_profile_enable(int(bool(enable))))


def profile_read(reset: bool = True) -> Dict[str, Tuple[int, float]]:
    """{kernel name: (launches, total ms)} since the last reset (synchronises on the events)."""
    lib = _lib.load()
    cap = 64
    names = ctypes.create_string_buffer(48 * cap)
    counts = (ctypes.c_int64 * cap)()
    ms = (ctypes.c_double * cap)()
    total = lib.muon_profile_read(names, counts, ms, cap, int(bool(reset)))
    if total < 0:
        _lib.check(total)
    out = {}
    for i in range(min(total, cap)):
        nm = names.raw[48 * i: 48 * (i + 1)].split(b"\0", 1)[0].decode()
        out[nm] = (int(counts[i]), float(ms[i]))
    return out


def version() -> int:
    return int(_lib.load().muon_version())


class PreparedMuonStep:
    """muon_step with the tensor table marshalled once (same tensors every call).

    Only the scalars may change between calls; the tensors, their shapes and the
    workspace are fixed at construction.
    """

    def __init__(self, params, grads, moms, *, ns_precision: int = _lib.MUON_NS_BF16, update_outs=None,
                 emas=None, extra_emas=None, extra_params=None, workspace=None, stream=None):
        if len(grads) != len(params) or len(moms) != len(params):
            raise ValueError("params, grads and moms must have the same length")
        self._keep = (list(params), list(grads), list(moms), update_outs, emas, workspace, extra_emas, extra_params)
        # the other tensors' EMA, run in the same call (muon_step_ema)
        self._extra = None
        if extra_emas is not None or extra_params is not None:
            self._extra = _ema_list(extra_emas or [], extra_params or [], "extra_emas")
        entries = _entries(params, grads, moms, update_outs, emas)
        self.n = len(entries)
        self.table = _lib.tensor_table(entries)
        self.ns_precision = int(ns_precision)
        self.device = params[0].device
        lib = _lib.load()
        need = lib.muon_workspace_size(self.table, self.n, self.ns_precision)
        if need == 0:
            raise _lib.MuonError(_lib.MUON_ERR_INVALID_ARG, lib.muon_last_error().decode())
        if workspace is None:
            # allocated on the stream the steps run on, so that its memory is
            # reused only in that stream's order once this object is dropped
            torch = _torch()
            s = stream if stream is not None else torch.cuda.current_stream(self.device)
            with torch.cuda.stream(s):
                workspace = torch.empty(int(need), dtype=torch.uint8, device=self.device)
        self.workspace = workspace
        self._ws_ptr = ctypes.c_void_p(workspace.data_ptr())
        self._ws_bytes = workspace.numel() * workspace.element_size()
        self._coeffs = None

    def __call__(self, *, lr, momentum, weight_decay, coeffs, nesterov=True, row_norm=True, ema_decay=0.0,
                 stream=None):
        if self._coeffs is None or self._coeffs[0] != coeffs:
            key = [tuple(float(v) for v in row) for row in coeffs]
            self._coeffs = (coeffs, _lib.coeff_array(key))
        carr, steps = self._coeffs[1]
        lib = _lib.load()
        if self._extra is not None:
            xe, xp, xn, nx = self._extra
            rc = lib.muon_step_ema(self.table, self.n, float(lr), float(momentum), int(bool(nesterov)),
                                   float(weight_decay), int(bool(row_norm)), steps, carr if steps else None,
                                   self.ns_precision, float(ema_decay), xe, xp, xn, nx, self._ws_ptr,
                                   self._ws_bytes, _stream_handle(stream, self.device))
        else:
            rc = lib.muon_step(self.table, self.n, float(lr), float(momentum), int(bool(nesterov)),
                               float(weight_decay), int(bool(row_norm)), steps, carr if steps else None,
                               self.ns_precision, float(ema_decay), self._ws_ptr, self._ws_bytes,
                               _stream_handle(stream, self.device))
        _lib.check(rc)


class PreparedEma:
    """ema_update with the tensor lists marshalled once."""

    def __init__(self, emas, params):
        self._keep = (list(emas), list(params))
        n = len(emas)
        self.n = n
        self.e = (ctypes.c_void_p * max(1, n))()
        self.p = (ctypes.c_void_p * max(1, n))()
        self.numel = (ctypes.c_int64 * max(1, n))()
        for i, (e, p) in enumerate(zip(emas, params)):
            _check_tensor(e, f"emas[{i}]")
            _check_tensor(p, f"params[{i}]")
            if e.numel() != p.numel():
                raise ValueError(f"tensor {i}: element counts differ")
            self.e[i], self.p[i], self.numel[i] = e.data_ptr(), p.data_ptr(), e.numel()
        self.device = emas[0].device

    def __call__(self, decay: float, stream=None):
        rc = _lib.load().ema_update(self.e, self.p, self.numel, self.n, float(decay),
                                    _stream_handle(stream, self.device))
        _lib.check(rc)
