"""ctypes declarations of the C ABI in include/muonstep.h (no torch needed here)."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuonstep.so")

MUON_OK = 0
MUON_ERR_INVALID_ARG = -1
MUON_ERR_UNSUPPORTED = -2
MUON_ERR_WORKSPACE = -3
MUON_ERR_HIP = -4
MUON_MAX_NS_STEPS = 16
MUON_MAX_SHORT_SIDE = 8192
MUON_MAX_LONG_SIDE = 65536
MUON_MAX_TENSORS = 4096
MUON_STATIC_WORKSPACE_BYTES = 64 << 20
MUON_NS_BF16 = 0
MUON_NS_FP32 = 1
MUON_NS_BF16X3 = 2
MUON_NS_SCHEDULE_PHASES = 0
MUON_NS_SCHEDULE_CHAIN = 1


class MuonTensor(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("momentum", ctypes.c_void_p),
        ("update_out", ctypes.c_void_p),
        ("ema", ctypes.c_void_p),
        ("rows", ctypes.c_int32),
        ("cols", ctypes.c_int32),
    ]


class AdamWTensor(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p),
        ("ema", ctypes.c_void_p),
        ("numel", ctypes.c_int64),
    ]


class MuonError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"muonstep error {code}: {message}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load the built HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m muon_optimizer_step_amd.build` "
            "(there is no fallback implementation)")
    # The library must run on the same HIP runtime as torch, whose device
    # pointers and streams it is handed: torch's wheel carries its own
    # libamdhip64, and loading the library first would bind it to the system
    # copy, a second runtime in the process that then finds no device.  So torch
    # (when installed) is imported first and the library links against the
    # runtime it loaded.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    f = lib.muon_workspace_size
    f.argtypes = [ctypes.POINTER(MuonTensor), ctypes.c_int32, ctypes.c_int32]
    f.restype = ctypes.c_size_t
    f = lib.muon_step
    f.argtypes = [ctypes.POINTER(MuonTensor), ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_int32,
                  ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                  ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    f.restype = ctypes.c_int
    f = lib.muon_step_ema
    f.argtypes = [ctypes.POINTER(MuonTensor), ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_int32,
                  ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                  ctypes.c_float, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                  ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    f.restype = ctypes.c_int
    f = lib.muon_step_static
    f.argtypes = [ctypes.POINTER(MuonTensor), ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_int32,
                  ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                  ctypes.c_float, ctypes.c_void_p]
    f.restype = ctypes.c_int
    f = lib.ema_update
    f.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64),
                  ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]
    f.restype = ctypes.c_int
    f = lib.ema_swap
    f.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64),
                  ctypes.c_int32, ctypes.c_void_p]
    f.restype = ctypes.c_int
    f = lib.adamw_step
    f.argtypes = [ctypes.POINTER(AdamWTensor), ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                  ctypes.c_float, ctypes.c_float, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]
    f.restype = ctypes.c_int
    lib.muon_set_ns_schedule.argtypes = [ctypes.c_int32]
    lib.muon_set_ns_schedule.restype = ctypes.c_int
    lib.muon_plan_cache_stats.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.muon_plan_cache_stats.restype = ctypes.c_int
    lib.muon_last_error.argtypes = []
    lib.muon_last_error.restype = ctypes.c_char_p
    lib.muon_version.argtypes = []
    lib.muon_version.restype = ctypes.c_int
    lib.muon_profile_enable.argtypes = [ctypes.c_int32]
    lib.muon_profile_enable.restype = ctypes.c_int
    lib.muon_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(ctypes.c_double), ctypes.c_int32, ctypes.c_int32]
    lib.muon_profile_read.restype = ctypes.c_int
    _lib = lib
    return lib


def check(rc: int) -> None:
    if rc != MUON_OK:
        raise MuonError(rc, load().muon_last_error().decode())


def tensor_table(entries) -> "ctypes.Array[MuonTensor]":
    """entries: iterable of (param, grad, momentum, update_out, ema, rows, cols) with int pointers."""
    entries = list(entries)
    arr = (MuonTensor * max(1, len(entries)))()
    for i, (p, g, m, o, e, r, c) in enumerate(entries):
        arr[i] = MuonTensor(p, g, m, o, e, r, c)
    return arr


def adamw_table(entries) -> "ctypes.Array[AdamWTensor]":
    """entries: iterable of (param, grad, exp_avg, exp_avg_sq, ema, numel) with int pointers."""
    entries = list(entries)
    arr = (AdamWTensor * max(1, len(entries)))()
    for i, e in enumerate(entries):
        arr[i] = AdamWTensor(*e)
    return arr


def coeff_array(coeffs):
    flat = [float(v) for row in coeffs for v in row]
    return (ctypes.c_float * max(1, len(flat)))(*flat), len(flat) // 3


def plan_cache_stats():
    """(schedules built, cache hits, schedules held) of muon_step's schedule cache."""
    built = ctypes.c_int64(0)
    hits = ctypes.c_int64(0)
    held = load().muon_plan_cache_stats(ctypes.byref(built), ctypes.byref(hits))
    return int(built.value), int(hits.value), int(held)


def set_ns_schedule(schedule: int) -> int:
    """Select MUON_NS_SCHEDULE_PHASES or MUON_NS_SCHEDULE_CHAIN; returns the previous setting."""
    rc = load().muon_set_ns_schedule(int(schedule))
    if rc < 0:
        check(rc)
    return int(rc)
