"""Throughput of the Muon step + weight EMA on one MI355X.

One step = muon_step over the 66 Muon matrices of the 11-layer 512d model
(momentum, MuonEq-R row norm, Frobenius scale, 5 quintic Newton-Schulz
iterations in bf16 MFMA, shape-scaled LR, decoupled weight decay) followed by
ema_update over all 34,401,372 parameters.  Inputs are synthetic and seeded
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
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
WORKLOAD = 2
METRIC = "Muon+EMA steps/s (66-matrix 11L-512d set); NS bf16 MFMA TFLOP/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=1337)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    return ap.parse_args()


def kernel_work(w):
    """Algorithmic work of each kernel per step, summed over its launches (flops or HBM bytes).

    The NS kernels launch once per iteration and prep, apply and ema may be
    split into several launches by tensor-table chunking, so every rate is the
    kernel's total work per step over its total time per step.
    """
    flops_gram = flops_square = 0.0
    elems = 0
    for _, r, c in w.matrices:
        m, n = min(r, c), max(r, c)
        flops_gram += 2.0 * m * m * n
        flops_square += 2.0 * m * m * m
        elems += r * c
    return {
        "ns_gram_bf16": ("mfma", flops_gram * w.ns_steps),      # A = X X^T
        "ns_square_bf16": ("mfma", flops_square * w.ns_steps),  # B = b A + c A A
        "ns_update_bf16": ("mfma", flops_gram * w.ns_steps),    # X <- a X + B X
        "prep": ("hbm", 16.0 * elems),             # read G, M; write M, X0 (bf16 hi + lo)
        "apply": ("hbm", 12.0 * elems),            # read W, X (bf16 hi + lo); write W
        "ema": ("hbm", 12.0 * w.n_params),         # read E, P; write E
    }


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "muon_optimizer_step_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str):
    """HBM bytes per launch from the committed counter summary, if it matches these sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_hash") != source_hash():
        return None
    k = data.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def cpu_baseline(w, seed, target_s):
    """The float64 oracle on the host: full Muon step + EMA of workload w, repeated ~target_s."""
    import numpy as np
    import oracle.muon as om
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    st = wl.make_state(w, seed)
    grads = wl.make_grads(w, seed, 0)
    coeffs = wl.coeff_table(w, seed).astype(np.float64)
    f = lambda x: float(np.float32(x))
    nm = len(w.matrices)
    reps = 0
    t0 = time.perf_counter()
    while True:
        new_w = []
        for i in range(nm):
            wn, _, _ = om.muon_step_matrix(st["params"][i], grads[i], st["moms"][i], lr=f(w.lr), mu=f(w.momentum),
                                           nesterov=True, wd=f(w.weight_decay), row_norm=True, coeffs=coeffs)
            new_w.append(wn)
        post = new_w + st["params"][nm:]
        for e, p in zip(st["ema"], post):
            om.ema_update(e, p, f(w.ema_decay))
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 20:
            break
    return {"value": reps / el, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full step(s) of the float64 NumPy oracle on the same workload "
                      f"(66 matrices + EMA over {w.n_params:,} params), {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import muon_optimizer_step_amd as ms
    import workloads as wl

    w = wl.workload(WORKLOAD)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    st = wl.make_state(w, args.seed)
    grads = wl.make_grads(w, args.seed, 0)
    coeffs = wl.coeff_table(w, args.seed).tolist()
    nm = len(w.matrices)
    P = [torch.from_numpy(p).to(dev) for p in st["params"]]
    G = [torch.from_numpy(g).to(dev) for g in grads]
    M = [torch.from_numpy(m).to(dev) for m in st["moms"]]
    E = [torch.from_numpy(e).to(dev) for e in st["ema"]]
    del st, grads
    step_muon = ms.PreparedMuonStep(P[:nm], G, M)
    step_ema = ms.PreparedEma(E, P)
    stream = torch.cuda.current_stream(dev)

    def step():
        step_muon(lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay, coeffs=coeffs, stream=stream)
        step_ema(w.ema_decay, stream=stream)

    print(f"[bench] workload {w.name}: {nm} matrices, {w.n_params:,} params, warmup {args.warmup}", flush=True)
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
    work = kernel_work(w)
    kernels = {}
    for name, (count, total_ms) in prof.items():
        step_s = total_ms * 1e-3 / args.steps
        entry = {"launches_per_step": count / args.steps, "avg_us": total_ms / max(count, 1) * 1e3,
                 "ms_per_step": step_s * 1e3}
        if name in work:
            bound, amount = work[name]
            if bound == "mfma":
                entry["tflops"] = amount / step_s / 1e12
            else:
                entry["gbs"] = amount / step_s / 1e9
        kernels[name] = entry
    dom = max((k for k in kernels if k in work), key=lambda k: kernels[k]["ms_per_step"])
    bound, amount = work[dom]
    step_s = kernels[dom]["ms_per_step"] * 1e-3
    if bound == "mfma":
        achieved, peak, unit = amount / step_s / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = amount / step_s / 1e9, HBM_PEAK_GBS, "GB/s"
    ns_names = [k for k in kernels if k.startswith("ns_")]
    ns_ms = sum(kernels[k]["ms_per_step"] for k in ns_names)
    ns_flops = sum(work[k][1] for k in ns_names if k in work)
    ns_tflops = ns_flops / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else None

    out = {
        "metric": METRIC,
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
        "config": {"workload": f"{w.name}: muon_step over 66 matrices (11 layers x Q/K/V/O/up/down at d=512), "
                               f"5 NS steps bf16, then ema_update over {w.n_params:,} fp32 params",
                   "matrices": nm, "params": w.n_params, "ns_steps": w.ns_steps, "seed": args.seed},
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic_for(dom)},
        "ns": {"tflops_algorithmic": round(ns_tflops, 2) if ns_tflops else None,
               "frac_of_bf16_peak": round(ns_tflops / BF16_PEAK_TFLOPS, 4) if ns_tflops else None,
               "ms_per_step": round(ns_ms, 4)},
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "ms_per_step_with_events": round(prof_elapsed / args.steps * 1e3, 4),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.seed, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
