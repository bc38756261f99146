"""Throughput of the Muon step + weight EMA on one MI355X.

One step = muon_step over the 66 Muon matrices of the 11-layer 512d model
(momentum, MuonEq-R row norm, Frobenius scale, 5 quintic Newton-Schulz
iterations in bf16 MFMA, shape-scaled LR, decoupled weight decay, and the
matrices' weight EMA in the pass that writes W') followed by ema_update over
the remaining parameters: the EMA covers all 34,401,372 parameters.  Inputs are synthetic and seeded
(workloads.workload(2)) and resident in HBM before timing starts.

Prints one JSON line (steps/s) with a roofline entry for the dominant kernel
and the float64 CPU oracle's rate on the host as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 MFMA
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
WORKLOAD = 2
METRIC = "Muon+EMA steps/s (66-matrix 11L-512d set); NS bf16 MFMA TFLOP/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=1337)
    ap.add_argument("--workload", type=int, default=WORKLOAD, choices=(2, 3, 4),
                    help="timed workload: 2 the 11-layer 512-wide model (the metric's workload), 3 the 1024-wide "
                         "model, 4 the structured-gradient 512-wide set")
    ap.add_argument("--rotate", type=int, default=2, help="independent state copies used in turn (MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true", help="skip the steps/s of the other workloads")
    ap.add_argument("--ns-schedule", choices=("phases", "chain"), default="phases",
                    help="Newton-Schulz schedule of the timed line: one launch per phase (default) or the "
                         "persistent chain")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (counter calibration) and exit")
    ap.add_argument("--ema-only", type=int, default=0, metavar="CALLS",
                    help="only run CALLS calls of ema_update over every parameter of the workload (two state "
                         "copies in turn) and exit: the counter run of the EMA pass")
    ap.add_argument("--summarize-counters", nargs="+",
                    metavar="CSV",
                    help="FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV [EMA_FETCH_CSV EMA_WRITE_CSV]: turn "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter files of this bench, of --calibrate-copy "
                         "and of --ema-only into profiles/hbm_traffic.json, then exit (no GPU needed)")
    ap.add_argument("--summarize-mfma", nargs="+", metavar="MOPS_CSV",
                    help="MOPS_CSV [CHAIN_MOPS_CSV]: turn rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                         "SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_VALU_MFMA_MOPS_F8 counter files of this bench (and of "
                         "its chain-schedule run) into profiles/mfma_counters.json, then exit (no GPU needed)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="turn the rocprofv3 --kernel-trace --stats summary of this bench into "
                         "profiles/kernel_trace.json (average launch duration per kernel), then exit (no GPU needed)")
    ap.add_argument("--counter-run", action="store_true",
                    help="time only the step itself (no schedule comparison, AdamW, EMA or swap passes): the "
                         "run under rocprofv3 counters, whose per-kernel averages must not mix other passes")
    return ap.parse_args()


def _kernel_key(name: str) -> str:
    """Library kernel symbol -> the name the profiling hook reports."""
    import re
    m = re.search(r"ns_sym_kernel<(\d), (\d), (true|false)>", name)
    if m:
        phase, prec, comp = int(m.group(1)), int(m.group(2)), m.group(3) == "true"
        return ["ns_gram", "ns_square"][phase] + ("_fp32" if prec == 1 else ("_bf16x3" if comp else "_bf16"))
    m = re.search(r"ns_update_kernel<(\d), (true|false), (true|false)>", name)
    if m:
        prec, comp, fuse = int(m.group(1)), m.group(2) == "true", m.group(3) == "true"
        base = "ns_update_apply" if fuse else "ns_update"
        return base + ("_fp32" if prec == 1 else ("_bf16x3" if comp else "_bf16"))
    if "ns_chain_kernel" in name:
        return "ns_chain_bf16"
    for k in ("chain_setup_kernel", "prep_kernel", "apply_kernel", "ema_kernel", "frob_kernel", "adamw_kernel",
              "swap_kernel"):
        if k in name:
            return k.replace("_kernel", "")
    return "copy" if "copyBuffer" in name else name


def _per_dispatch(path: str, counter: str):
    """{kernel: mean counter value per dispatch} from a rocprofv3 counter_collection.csv."""
    import csv
    import collections
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            k = _kernel_key(r["Kernel_Name"])
            tot[k] += float(r["Counter_Value"])
            disp[k].add(r["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


COUNTER_WORKLOAD = "model11L512"   # the counter runs profile the default bench workload


def summarize_counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, ema_fetch_csv=None, ema_write_csv=None,
                       chain_fetch_csv=None, chain_write_csv=None, copy_bytes=1 << 30, out_path=None):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by the copy calibration; written to out_path
    (profiles/hbm_traffic.json by default) and returned.  The EMA-only run's ema dispatches, if given, become
    the entry "ema_full" in bytes per call (its two launches summed); the chain-schedule run's chain kernels,
    if given, their own entries."""
    cf = _per_dispatch(copy_fetch_csv, "FETCH_SIZE").get("copy")
    cw = _per_dispatch(copy_write_csv, "WRITE_SIZE").get("copy")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        if k == "copy":
            continue
        fb = fetch[k] * 1024.0 * f_scale
        wb = write[k] * 1024.0 * w_scale
        kernels[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb)}
    if ema_fetch_csv and ema_write_csv:
        ef = _per_dispatch(ema_fetch_csv, "FETCH_SIZE").get("ema")
        ew = _per_dispatch(ema_write_csv, "WRITE_SIZE").get("ema")
        if ef is not None and ew is not None:
            per_call = 2   # the 187 tensors take two launches (144 table entries per launch)
            fb, wb = ef * 1024.0 * f_scale * per_call, ew * 1024.0 * w_scale * per_call
            kernels["ema_full"] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                                   "note": "bytes per ema_update call over all parameters (two launches)"}
    if chain_fetch_csv and chain_write_csv:
        cfch = _per_dispatch(chain_fetch_csv, "FETCH_SIZE")
        cwr = _per_dispatch(chain_write_csv, "WRITE_SIZE")
        for k in ("ns_chain_bf16", "chain_setup"):
            if k in cfch and k in cwr:
                fb, wb = cfch[k] * 1024.0 * f_scale, cwr[k] * 1024.0 * w_scale
                kernels[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb)}
    out = {"source_hash": source_hash(), "workload": COUNTER_WORKLOAD, "fetch_scale": f_scale, "write_scale": w_scale,
           "calibration": f"{copy_bytes} B device-to-device copy (5 runs): FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB per dispatch",
           "kernels": kernels}
    path = out_path or os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def summarize_mfma(csv_path, chain_csv=None, out_path=None):
    """Executed MFMA flops per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16 / _F32 / _F8, 512 flops per count);
    written to out_path (profiles/mfma_counters.json by default) and returned.  chain_csv: the
    chain-schedule run, whose chain kernel gets its own entry."""
    kernels = {}
    for counter in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_INSTS_VALU_MFMA_MOPS_F8"):
        for k, v in _per_dispatch(csv_path, counter).items():
            if k == "copy":
                continue
            kernels.setdefault(k, {})[counter] = v
        if chain_csv:
            v = _per_dispatch(chain_csv, counter).get("ns_chain_bf16")
            if v is not None:
                kernels.setdefault("ns_chain_bf16", {})[counter] = v
    out = {"source_hash": source_hash(), "workload": COUNTER_WORKLOAD,
           "kernels": {k: dict(v, flops_per_launch=512.0 * sum(v.values())) for k, v in sorted(kernels.items())}}
    path = out_path or os.path.join(ROOT, "profiles", "mfma_counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def summarize_trace(stats_csv, out_path=None):
    """Average launch duration (us) and launch count per kernel from a rocprofv3 kernel_stats.csv; written
    to out_path (profiles/kernel_trace.json by default) and returned."""
    import csv
    kernels = {}
    other = {"calls": 0, "total_ns": 0.0}
    for r in csv.DictReader(open(stats_csv)):
        k = _kernel_key(r["Name"])
        # kernels that are not this library's (copies, the vendor-BLAS comparison, torch's own)
        e = other if k in ("copy", r["Name"]) else kernels.setdefault(k, {"calls": 0, "total_ns": 0.0})
        e["calls"] += int(r["Calls"])
        e["total_ns"] += float(r["TotalDurationNs"])
    out = {"source_hash": source_hash(), "workload": COUNTER_WORKLOAD,
           "kernels": {k: {"calls": v["calls"], "avg_us": round(v["total_ns"] / v["calls"] / 1e3, 3)}
                       for k, v in sorted(kernels.items())},
           "other_kernels": {"calls": other["calls"], "total_us": round(other["total_ns"] / 1e3, 1),
                             "what": "copies, the vendor-BLAS comparison leg and torch's own kernels"}}
    path = out_path or os.path.join(ROOT, "profiles", "kernel_trace.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def rocprof_avg_us(kernel: str, workload: str = COUNTER_WORKLOAD):
    """Average launch duration from the committed rocprofv3 trace summary, if it matches these sources."""
    data = _counter_file("kernel_trace.json", workload)
    if data is None:
        return None
    k = data.get("kernels", {}).get(kernel)
    return None if k is None else k.get("avg_us")


def _counter_file(name: str, workload: str):
    """A committed counter summary, if it was taken on these sources and this workload."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_hash") != source_hash() or data.get("workload", COUNTER_WORKLOAD) != workload:
        return None
    return data


def mfma_counter_flops(kernel: str, workload: str = COUNTER_WORKLOAD):
    """Executed MFMA flops per launch from the committed counter summary, if it matches these sources."""
    data = _counter_file("mfma_counters.json", workload)
    if data is None:
        return None
    k = data.get("kernels", {}).get(kernel)
    return None if k is None else k.get("flops_per_launch")


def mfma_counter_split(kernel: str, workload: str = COUNTER_WORKLOAD):
    """(bf16, fp8, fp32) executed MFMA flops per launch from the committed counter summary, or None."""
    data = _counter_file("mfma_counters.json", workload)
    if data is None:
        return None
    k = data.get("kernels", {}).get(kernel)
    if k is None:
        return None
    return tuple(512.0 * k.get(c, 0.0) for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                                                 "SQ_INSTS_VALU_MFMA_MOPS_F32"))


def calibrate_copy(mib: int) -> None:
    """A plain copy of known size: the reference for scaling FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 5}), flush=True)


def ema_only(calls: int, seed: int) -> None:
    """ema_update over every parameter of the bench workload, `calls` times, two state copies in turn."""
    import torch
    import muon_optimizer_step_amd as ms
    import workloads as wl
    w = wl.workload(WORKLOAD)
    dev = torch.device("cuda:0")
    sets = []
    for r in range(2):
        st = wl.make_state(w, seed + r)
        sets.append(ms.PreparedEma([torch.from_numpy(e).to(dev) for e in st["ema"]],
                                   [torch.from_numpy(p).to(dev) for p in st["params"]]))
    torch.cuda.synchronize()
    for i in range(calls):
        sets[i % 2](w.ema_decay)
    torch.cuda.synchronize()
    print(json.dumps({"ema_only_calls": calls, "params": w.n_params}), flush=True)


def kernel_model(w, fused=True):
    """Algorithmic work of each kernel per step: flops and HBM bytes.

    The NS phases run once per iteration (split over the lanes' launches); the
    last update carries the weight apply when `fused`, else the apply kernel
    does.  Per launch figures are these totals divided by the launches per
    step.  Bytes count each operand once at its stored width: X is a bf16 hi
    plus a byte lo (3 B; a bf16 lo, 4 B, for compensated groups below a short
    side of 192), A and B are bf16 (hi + lo for A), weights, gradients, momenta
    and EMA shadows are fp32.  The matrices' EMA rides on the weight
    apply; the ema kernel covers the other parameters.
    """
    gram_f = sq_f = 0.0
    gram_b = sq_b = upd_b = upda_b = 0.0
    elems = 0
    prep_b = 0.0
    for _, r, c in w.matrices:
        m, n = min(r, c), max(r, c)
        xb = 3.0 if m >= 192 else 4.0            # X per element: bf16 hi + byte lo (base) or bf16 lo
        gram_f += 2.0 * m * m * n
        sq_f += 2.0 * m * m * m
        gram_b += 2.0 * m * n + 4.0 * m * m      # read X hi; write A hi + lo
        sq_b += 4.0 * m * m + 2.0 * m * m        # read A hi + lo; write B
        upd_b += 2 * xb * m * n + 2.0 * m * m    # read X hi + lo and B; write X hi + lo
        upda_b += (xb + 16.0) * m * n + 2.0 * m * m  # read X hi + lo and B; read + write W and E
        prep_b += (12.0 + xb) * r * c            # read G, M; write M', X0 hi + lo
        elems += r * c
    k = w.ns_steps
    plain_updates = k - 1 if fused else k
    model = {
        "ns_gram_bf16": {"flops": k * gram_f, "bytes": k * gram_b},                        # A = X X^T
        "ns_square_bf16": {"flops": k * sq_f, "bytes": k * sq_b},                          # B = b A + c A A
        "ns_update_bf16": {"flops": plain_updates * gram_f, "bytes": plain_updates * upd_b},  # X <- a X + B X
        "prep": {"flops": 0.0, "bytes": prep_b},                         # read G, M; write M', X0 hi + lo
        "ema": {"flops": 0.0, "bytes": 12.0 * (w.n_params - elems)},     # read E, P; write E
    }
    if fused:
        model["ns_update_apply_bf16"] = {"flops": gram_f, "bytes": upda_b}  # last X, then W' and E'
    else:
        model["apply"] = {"flops": 0.0, "bytes": 20.0 * elems}           # read W, E, X hi + lo; write W, E
    # The persistent chain runs every phase of every iteration in one launch:
    # its algorithmic work is the sum of the phases above (the last update
    # carrying W' and E'), and its intermediate planes may stay in the L2.
    model["ns_chain_bf16"] = {"flops": k * (2.0 * gram_f + sq_f),
                              "bytes": k * (gram_b + sq_b) + (k - 1) * upd_b + upda_b}
    model["chain_setup"] = {"flops": 0.0, "bytes": 64.0 * len(w.matrices)}  # records written
    return model


def roof_of(kernel: str) -> str:
    """"mfma" for the Newton-Schulz products, "hbm" for the streaming passes."""
    return "mfma" if kernel.startswith("ns_") else "hbm"


def streaming_fractions(kernels, workload: str):
    """HBM rate of the streaming passes (momentum prep, EMA) by algorithmic bytes and, where the
    committed counter summary matches these sources, by FETCH_SIZE + WRITE_SIZE bytes."""
    out = {}
    for k in ("prep", "ema", "apply"):
        if k not in kernels or "bytes_per_launch" not in kernels[k]:
            continue
        d = kernels[k]
        e = {"avg_launch_us": round(d["avg_us"], 3), "algorithmic_bytes_per_launch": round(d["bytes_per_launch"]),
             "algorithmic_gbs": round(d["bytes_per_launch"] / (d["avg_us"] * 1e-6) / 1e9, 1)}
        e["algorithmic_frac"] = round(e["algorithmic_gbs"] / HBM_PEAK_GBS, 4)
        t = traffic_for(k, workload)
        if t is not None:
            e["counter_bytes_per_launch"] = t
            e["counter_gbs"] = round(t / (d["avg_us"] * 1e-6) / 1e9, 1)
            e["counter_frac"] = round(e["counter_gbs"] / HBM_PEAK_GBS, 4)
        out[k] = e
    return out


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "muon_optimizer_step_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str = COUNTER_WORKLOAD):
    """HBM bytes per launch from the committed counter summary, if it matches these sources."""
    data = _counter_file("hbm_traffic.json", workload)
    if data is None:
        return None
    k = data.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def cpu_baseline(w, seed, target_s, gpu_o=None):
    """The float64 oracle on the host: full Muon step + EMA of workload w, repeated ~target_s.

    gpu_o: the library's O for every matrix from one step on the same initial state; the oracle's first
    step is compared with it (relative Frobenius error per matrix, worst per shape)."""
    import numpy as np
    import oracle.muon as om
    import workloads as wl
    from threadpoolctl import threadpool_info, threadpool_limits
    pools = threadpool_info()
    threads = max([d.get("num_threads", 1) for d in pools] or [1])
    blas = ", ".join(sorted({f"{d.get('internal_api')} {d.get('version')}" for d in pools})) or "unknown"
    st = wl.make_state(w, seed)
    grads = wl.make_grads(w, seed, 0)
    coeffs = wl.coeff_table(w, seed).astype(np.float64)
    f = lambda x: float(np.float32(x))
    nm = len(w.matrices)

    def one_step():
        new_w, outs = [], []
        for i in range(nm):
            wn, _, o = om.muon_step_matrix(st["params"][i], grads[i], st["moms"][i], lr=f(w.lr), mu=f(w.momentum),
                                           nesterov=True, wd=f(w.weight_decay), row_norm=True, coeffs=coeffs)
            new_w.append(wn)
            outs.append(o)
        post = new_w + st["params"][nm:]
        for e, p in zip(st["ema"], post):
            om.ema_update(e, p, f(w.ema_decay))
        return outs

    reps = 0
    first = None
    t0 = time.perf_counter()
    while True:
        outs = one_step()
        if first is None:
            first = outs
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 20:
            break
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        one_step()
        el1 = time.perf_counter() - t1
    res = {"value": reps / el, "unit": "steps/s", "cores": int(threads), "host_cpus": os.cpu_count(),
           "kind": "oracle",
           "sample": f"{reps} full step(s) of the float64 NumPy oracle on the same workload "
                     f"(66 matrices + EMA over {w.n_params:,} params), {el:.1f} s",
           "blas": blas, "single_thread": {"value": 1.0 / el1, "unit": "steps/s", "sample": f"1 step, {el1:.1f} s"}}
    if gpu_o is not None:
        worst = {}
        for (name, _, _), o_ref, o_gpu in zip(w.matrices, first, gpu_o):
            err = float(np.linalg.norm(o_gpu.astype(np.float64) - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
            shape = name.split(".")[-1]
            worst[shape] = max(worst.get(shape, 0.0), err)
        res["parity_vs_library"] = {
            "ns_rel_frobenius_worst": max(worst.values()), "worst_per_shape": {k: float(f"{v:.3e}") for k, v in
                                                                               worst.items()},
            "tolerance": 2e-2, "matrices": nm,
            "what": "O of the oracle's first step against the library's O from one step on the same initial state"}
    return res


def library_outputs(w, seed):
    """O of every matrix from one muon_step of this library on a fresh copy of the initial state (float32)."""
    import torch
    import muon_optimizer_step_amd as ms
    import workloads as wl
    nm = len(w.matrices)
    st = wl.make_state(w, seed)
    dev = torch.device("cuda:0")
    P = [torch.from_numpy(p).to(dev) for p in st["params"][:nm]]
    G = [torch.from_numpy(g).to(dev) for g in wl.make_grads(w, seed, 0)]
    M = [torch.from_numpy(m).to(dev) for m in st["moms"]]
    E = [torch.from_numpy(e).to(dev) for e in st["ema"][:nm]]
    O = [torch.empty_like(p) for p in P]
    ms.muon_step(P, G, M, lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay,
                 coeffs=wl.coeff_table(w, seed).tolist(), update_outs=O, emas=E, ema_decay=w.ema_decay)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in O]


def library_ns_baseline(w, steps, stream):
    """The NS iterations of the workload built from vendor BLAS calls, for comparison.

    Per shape group (matrices stacked, short side first) and iteration:
    Xt = X^T (a copy: torch's bf16 batched products take no transposed view
    here), A = X Xt (bmm), B = b A + c A A (baddbmm), X' = a X + B X (baddbmm),
    all bf16 with fp32 accumulation inside the library, no compensation and no
    symmetry.  The inputs are random bf16 (the values do not change the time).
    Times every iteration of all matrices on one stream, without prep or apply.
    """
    import torch
    import workloads as wl
    groups = {}
    for _, r, c in w.matrices:
        m, n = min(r, c), max(r, c)
        groups[(m, n)] = groups.get((m, n), 0) + 1
    bufs = []
    g = torch.Generator(device="cuda").manual_seed(0)
    for (m, n), cnt in sorted(groups.items()):
        x = (torch.randn(cnt, m, n, device="cuda", generator=g) / (m * n) ** 0.5).to(torch.bfloat16)
        bufs.append({"x": [x, torch.empty_like(x)], "xt": torch.empty(cnt, n, m, device="cuda", dtype=torch.bfloat16),
                     "a": torch.empty(cnt, m, m, device="cuda", dtype=torch.bfloat16),
                     "b": torch.empty(cnt, m, m, device="cuda", dtype=torch.bfloat16)})
    a_, b_, c_ = wl.STANDARD_TRIPLE

    def ns(with_transpose=True):
        for it in range(w.ns_steps):
            for d in bufs:
                x, x2 = d["x"][it % 2], d["x"][(it + 1) % 2]
                if with_transpose:
                    d["xt"].copy_(x.transpose(1, 2))
                torch.bmm(x, d["xt"], out=d["a"])
                torch.baddbmm(d["a"], d["a"], d["a"], beta=b_, alpha=c_, out=d["b"])
                torch.baddbmm(x, d["b"], x, beta=a_, alpha=1.0, out=x2)

    res = {}
    with torch.cuda.stream(stream):
        for tag, wt in (("us_per_step", True), ("us_per_step_without_transposes", False)):
            for _ in range(5):
                ns(wt)
            torch.cuda.synchronize()
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            for _ in range(steps):
                ns(wt)
            e.record(stream)
            torch.cuda.synchronize()
            res[tag] = round(s.elapsed_time(e) / steps * 1e3, 2)
    flops = sum((4.0 * m * m * n + 2.0 * m ** 3) * cnt for (m, n), cnt in groups.items()) * w.ns_steps
    res["tflops_dense_formula"] = round(flops / (res["us_per_step_without_transposes"] * 1e-6) / 1e12, 1)
    try:
        res["blas"] = str(torch.backends.cuda.preferred_blas_library())
    except Exception:  # older torch
        res["blas"] = None
    res["what"] = ("the workload's NS iterations (all matrices, no prep, no apply) as torch bf16 bmm/baddbmm calls "
                   "on one stream; plain bf16 products, no compensation, no symmetry")
    return res


def time_other_config(cfg, steps, warmup, seed):
    """Steps/s of one more workload (the parity configs), same method as the main line, no profiling."""
    import torch
    import muon_optimizer_step_amd as ms
    import workloads as wl
    w = wl.workload(cfg)
    dev = torch.device("cuda:0")
    nm = len(w.matrices)
    st = wl.make_state(w, seed)
    coeffs = wl.coeff_table(w, seed).tolist()
    P = [torch.from_numpy(p).to(dev) for p in st["params"]]
    M = [torch.from_numpy(m).to(dev) for m in st["moms"]]
    E = [torch.from_numpy(e).to(dev) for e in st["ema"]] if w.ema_decay is not None else None
    # the multi-step workload draws a fresh gradient every step: two sets used in turn
    gsets = [[torch.from_numpy(g).to(dev) for g in wl.make_grads(w, seed, k)] for k in range(2 if w.steps > 1 else 1)]
    del st
    runs, workspace = [], None
    for G in gsets:
        muon = ms.PreparedMuonStep(P[:nm], G, M, ns_precision=w.ns_precision, emas=E[:nm] if E else None,
                                   workspace=workspace)
        workspace = muon.workspace
        runs.append(muon)
    ema = ms.PreparedEma(E[nm:], P[nm:]) if E and len(E) > nm else None
    stream = torch.cuda.current_stream(dev)
    decay = w.ema_decay if w.ema_decay is not None else 0.0

    def step(i):
        runs[i % len(runs)](lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay, coeffs=coeffs,
                            nesterov=w.nesterov, row_norm=w.row_norm, ema_decay=decay, stream=stream)
        if ema is not None:
            ema(decay, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    ns_flops = w.ns_steps * sum(4.0 * min(r, c) ** 2 * max(r, c) + 2.0 * min(r, c) ** 3 for _, r, c in w.matrices)
    out = {"workload": w.name, "steps_per_s": round(1.0 / el, 2), "ms_per_step": round(el * 1e3, 4),
           "ns_precision": ["bf16", "fp32"][w.ns_precision], "matrices": nm, "params": w.n_params,
           "ns_algorithmic_tflops_over_step_time": round(ns_flops / el / 1e12, 2)}
    del P, M, E, gsets, runs, ema, workspace
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.summarize_counters:
        if len(args.summarize_counters) not in (4, 6, 8):
            print("--summarize-counters takes 4, 6 or 8 files", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(summarize_counters(*args.summarize_counters), indent=1))
        return
    if args.ema_only:
        ema_only(args.ema_only, args.seed)
        return
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace), indent=1))
        return
    if args.summarize_mfma:
        print(json.dumps(summarize_mfma(*args.summarize_mfma[:2]), indent=1))
        return
    import numpy as np
    import torch
    import muon_optimizer_step_amd as ms
    import workloads as wl

    w = wl.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms.set_ns_schedule(ms.MUON_NS_SCHEDULE_CHAIN if args.ns_schedule == "chain" else ms.MUON_NS_SCHEDULE_PHASES)
    coeffs = wl.coeff_table(w, args.seed).tolist()
    nm = len(w.matrices)
    # args.rotate independent copies of the whole state (seeds seed, seed + 1, ...),
    # used in turn, so that no step finds the previous step's tensors in the
    # 256 MB MALL.  One workspace serves all of them (the steps are serial on
    # one stream).
    states = []
    ema_lists = []
    workspace = None
    for r in range(args.rotate):
        st = wl.make_state(w, args.seed + r)
        grads = wl.make_grads(w, args.seed + r, 0)
        ad = wl.make_adamw_state(w, args.seed + r)
        P = [torch.from_numpy(p).to(dev) for p in st["params"]]
        G = [torch.from_numpy(g).to(dev) for g in grads]
        M = [torch.from_numpy(m).to(dev) for m in st["moms"]]
        E = [torch.from_numpy(e).to(dev) for e in st["ema"]]
        AG, AM, AV = ([torch.from_numpy(x).to(dev) for x in ad[k]] for k in ("grads", "exp_avg", "exp_avg_sq"))
        del st, grads, ad
        muon = ms.PreparedMuonStep(P[:nm], G, M, emas=E[:nm], workspace=workspace)
        workspace = muon.workspace
        # the timed step: muon_step_ema, the other 121 tensors' EMA in the same call
        fused = ms.PreparedMuonStep(P[:nm], G, M, emas=E[:nm], extra_emas=E[nm:], extra_params=P[nm:],
                                    workspace=workspace)
        states.append((muon, ms.PreparedEma(E[nm:], P[nm:]), ms.PreparedAdamW(P[nm:], AG, AM, AV, emas=E[nm:]),
                       fused))
        ema_lists.append((E, P))
        if r == 0:
            swap_lists = (E, P)
    stream = torch.cuda.current_stream(dev)
    turn = [0]

    def step():
        # muon_step over the matrices (their EMA fused) with the EMA of the other tensors in the same call
        fused = states[turn[0] % len(states)][3]
        turn[0] += 1
        fused(lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay, coeffs=coeffs,
              ema_decay=w.ema_decay, stream=stream)

    def two_call_step():
        # the same work as two calls: muon_step, then ema_update on the other tensors
        step_muon, step_ema, _, _ = states[turn[0] % len(states)]
        turn[0] += 1
        step_muon(lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay, coeffs=coeffs,
                  ema_decay=w.ema_decay, stream=stream)
        step_ema(w.ema_decay, stream=stream)

    hp = wl.ADAMW_HPARAMS

    def adamw_only():
        _, _, step_adamw, _ = states[turn[0] % len(states)]
        turn[0] += 1
        step_adamw(lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=hp["weight_decay"],
                   step=hp["step"], ema_decay=w.ema_decay, stream=stream)

    def full_step():
        # the whole optimizer step: Muon on the matrices, AdamW on the rest, EMA on everything
        step_muon, _, step_adamw, _ = states[turn[0] % len(states)]
        turn[0] += 1
        step_muon(lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay, coeffs=coeffs,
                  ema_decay=w.ema_decay, stream=stream)
        step_adamw(lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=hp["weight_decay"],
                   step=hp["step"], ema_decay=w.ema_decay, stream=stream)

    print(f"[bench] workload {w.name}: {nm} matrices, {w.n_params:,} params, {args.rotate} state copies, "
          f"warmup {args.warmup}", flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    value = args.steps / elapsed
    print(f"[bench] timed {args.steps} steps in {elapsed * 1e3:.1f} ms", flush=True)
    # Host cost of enqueueing one step (muon_step_ema through the
    # binding): wall time of each call, the GPU idle at the start of the burst
    # and the launch queue far from full, so no call waits for the device.
    host_us = []
    for _ in range(min(args.steps, 20)):
        th = time.perf_counter()
        step()
        host_us.append((time.perf_counter() - th) * 1e6)
    torch.cuda.synchronize()
    built, hits, _ = ms.plan_cache_stats()
    host_enqueue = {"mean_us": round(float(np.mean(host_us)), 1), "p50_us": round(float(np.median(host_us)), 1),
                    "max_us": round(float(np.max(host_us)), 1), "calls": len(host_us),
                    "schedules_built": built, "schedule_cache_hits": hits,
                    "what": "host wall time per step() call (muon_step_ema), GPU work enqueued only"}

    # The other Newton-Schulz schedule on the same state, for comparison.
    other = "chain" if args.ns_schedule == "phases" else "phases"
    other_rate = None
    if not args.counter_run:
        ms.set_ns_schedule(ms.MUON_NS_SCHEDULE_CHAIN if other == "chain" else ms.MUON_NS_SCHEDULE_PHASES)
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        tc = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        other_rate = args.steps / (time.perf_counter() - tc)
        ms.set_ns_schedule(ms.MUON_NS_SCHEDULE_CHAIN if args.ns_schedule == "chain" else ms.MUON_NS_SCHEDULE_PHASES)
    two_call_rate = None
    if not args.counter_run:
        # the same work as muon_step + ema_update, two calls
        for _ in range(5):
            two_call_step()
        torch.cuda.synchronize()
        tt = time.perf_counter()
        for _ in range(args.steps):
            two_call_step()
        torch.cuda.synchronize()
        two_call_rate = args.steps / (time.perf_counter() - tt)
        print(f"[bench] {args.ns_schedule} schedule {value:.1f} steps/s, {other} schedule {other_rate:.1f} steps/s",
              flush=True)

    # Spread of single steps: an event pair around each step on the caller's
    # stream (the lanes join it before the step's last kernel).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    per_step = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    pct = lambda q: per_step[min(len(per_step) - 1, int(q * len(per_step)))]
    spread = {"p10": round(1e3 / pct(0.9), 2), "p50": round(1e3 / pct(0.5), 2), "p90": round(1e3 / pct(0.1), 2),
              "unit": "steps/s", "from": f"{args.steps} single steps timed with HIP events"}

    # Per-kernel durations: HIP events around every launch, on the launch stream.
    ms.profile_read(reset=True)
    ms.profile_enable(True)
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof_elapsed = time.perf_counter() - tp0
    ms.profile_enable(False)
    prof = ms.profile_read(reset=True)
    model = kernel_model(w, fused="ns_update_apply_bf16" in prof)
    kernels = {}
    for name, (count, total_ms) in prof.items():
        step_s = total_ms * 1e-3 / args.steps
        lps = count / args.steps
        entry = {"launches_per_step": lps, "avg_us": total_ms / max(count, 1) * 1e3, "ms_per_step": step_s * 1e3}
        if name in model:
            mm = model[name]
            entry["flops_per_step"] = mm["flops"]
            entry["bytes_per_step"] = mm["bytes"]
            entry["bytes_per_launch"] = mm["bytes"] / lps
            if mm["flops"] > 0:
                entry["tflops"] = entry["flops_per_step"] / step_s / 1e12
            entry["gbs"] = entry["bytes_per_step"] / step_s / 1e9
        kernels[name] = entry
    # The dominant kernel is the one with the most time per step in the rocprof
    # trace of the same sources (launches per step from this run times the
    # trace's average duration); without a trace, the HIP-event time decides.
    cands = [k for k in kernels if k in model]
    traced = {k: rocprof_avg_us(k, w.name) for k in cands}
    if all(traced[k] for k in cands):
        dom = max(cands, key=lambda k: kernels[k]["launches_per_step"] * traced[k])
        dom_from = "rocprof trace (launches per step x average duration)"
    else:
        dom = max(cands, key=lambda k: kernels[k]["ms_per_step"])
        dom_from = "HIP-event time per step"
    d = kernels[dom]
    # The roof of each kernel is fixed by what it computes: the Newton-Schulz
    # products are dense contractions (bf16 MFMA, dense-formula flops), the
    # streaming passes move bytes (HBM).
    if roof_of(dom) == "mfma":
        bound, achieved, peak, unit = "mfma", d["tflops"], BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", d["gbs"], HBM_PEAK_GBS, "GB/s"
    ns_names = [k for k in kernels if k.startswith("ns_")]
    ns_ms = sum(kernels[k]["ms_per_step"] for k in ns_names)
    ns_flops = sum(kernels[k].get("flops_per_step", 0.0) for k in ns_names)
    ns_tflops = ns_flops / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else None
    # executed MFMA work (counters: compensation products and symmetry savings included)
    counted = [mfma_counter_flops(k, w.name) for k in ns_names]
    ns_counted = (sum(c * kernels[k]["launches_per_step"] for c, k in zip(counted, ns_names))
                  if counted and all(c is not None for c in counted) else None)
    traffic = traffic_for(dom, w.name)
    # executed work by operand type: the square's cross terms run on the fp8 MFMA
    # (twice the bf16 rate), so the MFMA time at peak counts each type at its own peak
    split = [mfma_counter_split(k, w.name) for k in ns_names]
    if split and all(x is not None for x in split):
        ex_bf16 = sum(x[0] * kernels[k]["launches_per_step"] for x, k in zip(split, ns_names))
        ex_fp8 = sum(x[1] * kernels[k]["launches_per_step"] for x, k in zip(split, ns_names))
        mfma_at_peak_ms = (ex_bf16 / (BF16_PEAK_TFLOPS * 1e12) + ex_fp8 / (FP8_PEAK_TFLOPS * 1e12)) * 1e3
    else:
        ex_bf16 = ex_fp8 = mfma_at_peak_ms = None

    describe = {
        2: "66 matrices (11 layers x Q/K/V/O/up/down at d=512)",
        3: "66 matrices (11 layers x Q/K/V/O/up/down at d=1024)",
        4: "66 matrices (11 layers x Q/K/V/O/up/down at d=512) with rank-8 structured gradients and a drawn "
           "coefficient table",
    }[args.workload]
    out = {
        "metric": METRIC if args.workload == WORKLOAD else f"Muon+EMA steps/s ({w.name})",
        "value": round(value, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: muon_step_ema over {describe}, "
                               f"{w.ns_steps} NS steps bf16, EMA over all {w.n_params:,} fp32 params "
                               f"(the matrices' in the pass that writes W', the {len(w.extras)} other tensors' "
                               f"in the same call)",
                   "matrices": nm, "params": w.n_params, "ns_steps": w.ns_steps, "seed": args.seed,
                   "state_copies": args.rotate},
        "roofline": {"kernel": dom, "dominant_by": dom_from, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "algorithmic_flops_per_launch": round(d["flops_per_step"] / d["launches_per_step"]),
                     "algorithmic_bytes_per_launch": round(d["bytes_per_launch"]),
                     "avg_launch_us": round(d["avg_us"], 3),
                     "mfma_frac": round(d.get("tflops", 0.0) / BF16_PEAK_TFLOPS, 4),
                     "hbm_frac": round(d["gbs"] / HBM_PEAK_GBS, 4),
                     "rocprof_avg_launch_us": rocprof_avg_us(dom, w.name),
                     "rocprof_frac": (round(achieved * d["avg_us"] / rocprof_avg_us(dom, w.name) / peak, 4)
                                      if rocprof_avg_us(dom, w.name) else None),
                     "timing": "avg_launch_us from HIP events around each launch inside this run (on the launch's "
                               "stream); rocprof_avg_launch_us from profiles/kernel_trace.json of the same sources"},
        "streaming": streaming_fractions(kernels, w.name),
        "ns": {"tflops_over_summed_kernel_time": round(ns_tflops, 2) if ns_tflops else None,
               "frac_of_bf16_peak": round(ns_tflops / BF16_PEAK_TFLOPS, 4) if ns_tflops else None,
               "summed_kernel_ms_per_step": round(ns_ms, 4),
               "tflops_over_step_time": round(ns_flops / elapsed * args.steps / 1e12, 2),
               "executed_flops_per_step": ns_counted,
               "executed_tflops_over_summed_kernel_time":
                   round(ns_counted / (ns_ms * 1e-3) / 1e12, 2) if ns_counted and ns_ms > 0 else None,
               "executed_bf16_flops_per_step": ex_bf16, "executed_fp8_flops_per_step": ex_fp8,
               "mfma_busy_frac_at_peaks": (round(mfma_at_peak_ms / ns_ms, 4) if mfma_at_peak_ms and ns_ms > 0
                                           else None),
               "note": "executed work from profiles/mfma_counters.json; the fp8 share (the square's cross terms) "
                       "is priced at the 5.0 PFLOP/s fp8 peak, the bf16 share at 2.5 PFLOP/s"},
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "steps_per_s_spread": spread,
        "ns_schedule": {"timed": args.ns_schedule, "other": other,
                        "other_steps_per_s": round(other_rate, 2) if other_rate else None},
        "step_call": {"timed": "muon_step_ema (the other tensors' EMA in the same call)",
                      "two_calls_steps_per_s": round(two_call_rate, 2) if two_call_rate else None,
                      "two_calls": "muon_step, then ema_update on the 121 other tensors"},
        "ms_per_step_with_events": round(prof_elapsed / args.steps * 1e3, 4),
        "host_enqueue": host_enqueue,
        "cpu_baseline": None,
    }
    if args.counter_run:
        print(json.dumps(out), flush=True)
        return
    # AdamW on the 121 non-matrix tensors (with their EMA fused), alone and
    # inside the whole optimizer step
    for _ in range(5):
        adamw_only()
    torch.cuda.synchronize()
    ms.profile_read(reset=True)
    ms.profile_enable(True)
    for _ in range(args.steps):
        adamw_only()
    torch.cuda.synchronize()
    ms.profile_enable(False)
    aprof = ms.profile_read(reset=True)["adamw"]
    extra_elems = w.n_params - sum(r * c for _, r, c in w.matrices)
    a_bytes = 36.0 * extra_elems   # read p, g, m, v, e; write p, m, v, e
    a_us = aprof[1] / aprof[0] * 1e3
    for _ in range(5):
        full_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        full_step()
    torch.cuda.synchronize()
    full_el = (time.perf_counter() - t0) / args.steps
    out["adamw"] = {"tensors": len(w.extras), "elements": extra_elems, "hyperparameters": hp,
                    "launches_per_call": aprof[0] / args.steps, "avg_launch_us": round(a_us, 3),
                    "us_per_call": round(aprof[1] / args.steps * 1e3, 3),
                    "algorithmic_bytes_per_call": a_bytes,
                    "gbs": round(a_bytes / (aprof[1] / args.steps * 1e-3) / 1e9, 1),
                    "frac_of_hbm_peak": round(a_bytes / (aprof[1] / args.steps * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    out["full_optimizer_step"] = {"steps_per_s": round(1.0 / full_el, 2), "ms_per_step": round(full_el * 1e3, 4),
                                  "what": "muon_step on the 66 matrices (EMA fused) + adamw_step on the 121 other "
                                          "tensors (EMA fused)"}
    # The weight EMA as a pass of its own over all 187 tensors (34,401,372
    # parameters; read E and P, write E: 12 B per parameter), the state copies
    # used in turn so that no call finds its tensors in the MALL.
    full = [ms.PreparedEma(E, P) for E, P in ema_lists]
    for i in range(3):
        full[i % len(full)](w.ema_decay, stream=stream)
    torch.cuda.synchronize()
    te = time.perf_counter()
    for i in range(args.steps):
        full[i % len(full)](w.ema_decay, stream=stream)
    torch.cuda.synchronize()
    e_wall_us = (time.perf_counter() - te) / args.steps * 1e6
    ms.profile_read(reset=True)
    ms.profile_enable(True)
    for i in range(args.steps):
        full[i % len(full)](w.ema_decay, stream=stream)
    torch.cuda.synchronize()
    ms.profile_enable(False)
    eprof = ms.profile_read(reset=True)["ema"]
    e_us = eprof[1] / args.steps * 1e3          # summed launch durations per call (HIP events)
    e_bytes = 12.0 * w.n_params
    e_traffic = traffic_for("ema_full", w.name)
    out["ema_full"] = {"tensors": len(ema_lists[0][0]), "elements": w.n_params,
                       "us_per_call": round(e_wall_us, 3), "kernel_us_per_call": round(e_us, 3),
                       "launches_per_call": eprof[0] / args.steps, "algorithmic_bytes_per_call": e_bytes,
                       "gbs": round(e_bytes / (e_wall_us * 1e-6) / 1e9, 1),
                       "frac_of_hbm_peak": round(e_bytes / (e_wall_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "kernel_gbs": round(e_bytes / (e_us * 1e-6) / 1e9, 1),
                       "counter_bytes_per_call": e_traffic,
                       "counter_frac_of_hbm_peak": (round(e_traffic / (e_wall_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                                    if e_traffic else None),
                       "what": "ema_update over every parameter tensor of the model as its own pass, "
                               f"{args.steps} calls back to back on two state copies in turn"}
    # EMA swap-in over all 187 tensors (read and write both buffers: 16 B per parameter)
    sw_e, sw_p = swap_lists
    for _ in range(3):
        ms.ema_swap(sw_e, sw_p, stream=stream)
    torch.cuda.synchronize()
    ms.profile_read(reset=True)
    ms.profile_enable(True)
    for _ in range(args.steps):
        ms.ema_swap(sw_e, sw_p, stream=stream)
    torch.cuda.synchronize()
    ms.profile_enable(False)
    sprof = ms.profile_read(reset=True)["swap"]
    sw_us = sprof[1] / args.steps * 1e3
    sw_bytes = 16.0 * w.n_params
    out["ema_swap"] = {"tensors": len(sw_e), "elements": w.n_params, "us_per_call": round(sw_us, 3),
                       "launches_per_call": sprof[0] / args.steps, "algorithmic_bytes_per_call": sw_bytes,
                       "gbs": round(sw_bytes / (sw_us * 1e-6) / 1e9, 1),
                       "frac_of_hbm_peak": round(sw_bytes / (sw_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    out["library_ns"] = library_ns_baseline(w, args.steps, stream)
    print(f"[bench] adamw {out['adamw']['us_per_call']} us per call; full optimizer step "
          f"{out['full_optimizer_step']['steps_per_s']} steps/s; EMA over all parameters "
          f"{out['ema_full']['us_per_call']} us ({out['ema_full']['gbs']} GB/s)", flush=True)
    if not args.no_other_configs:
        # the other workloads (parity cases), each on its own; steps/s only
        del states, workspace
        torch.cuda.empty_cache()
        others = {}
        for cfg in (0, 1, 3, 4):
            print(f"[bench] workload {cfg}", flush=True)
            r = time_other_config(cfg, steps=max(20, args.steps // 4), warmup=5, seed=args.seed)
            others[r.pop("workload")] = r
        out["other_workloads"] = others
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.seed, args.cpu_seconds, library_outputs(w, args.seed))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
