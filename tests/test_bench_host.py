"""Host logic of bench.py (no GPU): the one-GPU guard, the kernel-name mapping of
rocprofv3 symbols, the counter summaries behind roofline.traffic and the
executed-MFMA figures, and the algorithmic work model the roofline divides by."""

import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("symbol,key", [
    ("void muon::(anonymous namespace)::ns_sym_kernel<0, 0, false>(muon::NsArgs)", "ns_gram_bf16"),
    ("void muon::(anonymous namespace)::ns_sym_kernel<1, 0, false>(muon::NsArgs)", "ns_square_bf16"),
    ("void muon::(anonymous namespace)::ns_sym_kernel<1, 0, true>(muon::NsArgs)", "ns_square_bf16x3"),
    ("void muon::(anonymous namespace)::ns_sym_kernel<0, 1, false>(muon::NsArgs)", "ns_gram_fp32"),
    ("void muon::(anonymous namespace)::ns_update_kernel<0, false, false>(muon::NsArgs)", "ns_update_bf16"),
    ("void muon::(anonymous namespace)::ns_update_kernel<0, false, true>(muon::NsArgs)", "ns_update_apply_bf16"),
    ("void muon::(anonymous namespace)::ns_update_kernel<0, true, false>(muon::NsArgs)", "ns_update_bf16x3"),
    ("void muon::(anonymous namespace)::ns_update_kernel<1, false, true>(muon::NsArgs)", "ns_update_apply_fp32"),
    ("void muon::(anonymous namespace)::prep_kernel<0, 8>(muon::PrepArgs)", "prep"),
    ("muon::(anonymous namespace)::ema_kernel(muon::EmaArgs)", "ema"),
    ("muon::(anonymous namespace)::adamw_kernel(muon::AdamArgs)", "adamw"),
    ("__amd_rocclr_copyBuffer", "copy"),
    ("muon::(anonymous namespace)::ns_chain_kernel(muon::ChainArgs)", "ns_chain_bf16"),
    ("muon::(anonymous namespace)::chain_setup_kernel(muon::ChainSetupArgs)", "chain_setup"),
])
def test_kernel_symbols_map_to_hook_names(symbol, key):
    assert bench._kernel_key(symbol) == key


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writerows(rows)


UPD = "void muon::(anonymous namespace)::ns_update_kernel<0, false, false>(muon::NsArgs)"
GRAM = "void muon::(anonymous namespace)::ns_sym_kernel<0, 0, false>(muon::NsArgs)"


def test_traffic_summary_scales_by_the_copy_and_averages_per_dispatch(tmp_path):
    p = {k: str(tmp_path / f"{k}.csv") for k in ("fetch", "write", "cfetch", "cwrite")}
    # a 1 GiB copy that FETCH_SIZE reads as half its bytes and WRITE_SIZE as all of them
    _write_counters(p["cfetch"], [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288),
                                  (2, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288)])
    _write_counters(p["cwrite"], [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576)])
    # dispatch 1 reports in two rows (summed), dispatch 2 in one; small uploads are ignored
    _write_counters(p["fetch"], [(5, UPD, "FETCH_SIZE", 100), (5, UPD, "FETCH_SIZE", 50), (9, UPD, "FETCH_SIZE", 150),
                                 (3, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 7), (4, GRAM, "FETCH_SIZE", 10)])
    _write_counters(p["write"], [(5, UPD, "WRITE_SIZE", 80), (9, UPD, "WRITE_SIZE", 40), (4, GRAM, "WRITE_SIZE", 4)])
    out_path = str(tmp_path / "traffic.json")
    out = bench.summarize_counters(p["fetch"], p["write"], p["cfetch"], p["cwrite"], out_path=out_path)
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    upd = out["kernels"]["ns_update_bf16"]
    assert upd["fetch_bytes"] == 150 * 1024 * 2 and upd["write_bytes"] == 60 * 1024
    assert upd["bytes_per_launch"] == upd["fetch_bytes"] + upd["write_bytes"]
    assert out["kernels"]["ns_gram_bf16"]["bytes_per_launch"] == 10 * 1024 * 2 + 4 * 1024
    assert "copy" not in out["kernels"]
    assert out["source_hash"] == bench.source_hash() and out["workload"] == "model11L512"
    with open(out_path) as f:
        assert json.load(f) == out


def test_ema_only_run_becomes_the_full_ema_entry(tmp_path):
    """The EMA-only counter run (all 187 tensors, two launches per call) is reported per call."""
    p = {k: str(tmp_path / f"{k}.csv") for k in ("fetch", "write", "cfetch", "cwrite", "efetch", "ewrite")}
    EMA = "muon::(anonymous namespace)::ema_kernel(muon::EmaArgs)"
    _write_counters(p["cfetch"], [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288)])
    _write_counters(p["cwrite"], [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576)])
    _write_counters(p["fetch"], [(4, GRAM, "FETCH_SIZE", 10)])
    _write_counters(p["write"], [(4, GRAM, "WRITE_SIZE", 4)])
    _write_counters(p["efetch"], [(1, EMA, "FETCH_SIZE", 100), (2, EMA, "FETCH_SIZE", 300)])
    _write_counters(p["ewrite"], [(1, EMA, "WRITE_SIZE", 60), (2, EMA, "WRITE_SIZE", 140)])
    out = bench.summarize_counters(p["fetch"], p["write"], p["cfetch"], p["cwrite"], p["efetch"], p["ewrite"],
                                   out_path=str(tmp_path / "t.json"))
    full = out["kernels"]["ema_full"]
    assert full["fetch_bytes"] == 2 * 200 * 1024 * 2 and full["write_bytes"] == 2 * 100 * 1024
    assert "ema" not in out["kernels"] or out["kernels"]["ema"]["bytes_per_launch"] != full["bytes_per_launch"]


def test_mfma_summary_counts_512_flops_per_mop(tmp_path):
    path = str(tmp_path / "mops.csv")
    _write_counters(path, [(1, GRAM, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000), (1, GRAM, "SQ_INSTS_VALU_MFMA_MOPS_F32", 0),
                           (2, GRAM, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 3000), (2, GRAM, "SQ_INSTS_VALU_MFMA_MOPS_F32", 0)])
    out = bench.summarize_mfma(path, out_path=str(tmp_path / "mfma.json"))
    assert out["kernels"]["ns_gram_bf16"]["flops_per_launch"] == 512.0 * 2000


def test_committed_summaries_cover_the_bench_kernels():
    """The committed counter files name every kernel of the bench step (their hash decides whether
    bench.py uses them)."""
    for name in ("hbm_traffic.json", "mfma_counters.json"):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            data = json.load(f)
        assert len(data["source_hash"]) == 16
        assert data["workload"] == "model11L512"
        for k in ("prep", "ns_gram_bf16", "ns_square_bf16", "ns_update_bf16", "ns_update_apply_bf16", "ema"):
            assert k in data["kernels"], (name, k)


def test_counter_figures_are_used_only_for_the_workload_they_were_taken_on():
    """Counters taken on the 512-wide model say nothing about another workload's kernels of the same name."""
    if bench.traffic_for("ns_update_bf16", "model11L512") is None:
        pytest.skip("committed counter summaries are from other sources")
    assert bench.traffic_for("ns_update_bf16", "model11L1024") is None
    assert bench.mfma_counter_flops("ns_gram_bf16", "model11L1024") is None
    assert bench.mfma_counter_flops("ns_gram_bf16", "model11L512") > 0


def test_work_model_of_the_bench_workload():
    """Per-step algorithmic work at the bench workload: the NS flops are the dense formula
    k (4 m^2 n + 2 m^3) summed over the matrices, and the bytes follow the per-element widths
    (X 3 bytes as bf16 hi + byte lo for m >= 192, fp32 weights, gradients, momenta and EMAs)."""
    w = wl.workload(2)
    model = bench.kernel_model(w)
    k = w.ns_steps
    ns = sum(k * (4.0 * min(r, c) ** 2 * max(r, c) + 2.0 * min(r, c) ** 3) for _, r, c in w.matrices)
    got = sum(model[n]["flops"] for n in ("ns_gram_bf16", "ns_square_bf16", "ns_update_bf16", "ns_update_apply_bf16"))
    assert got == pytest.approx(ns, rel=1e-12)
    assert model["ns_chain_bf16"]["flops"] == pytest.approx(ns, rel=1e-12)   # the chain runs all of it
    per_phase = sum(model[n]["bytes"] for n in ("ns_gram_bf16", "ns_square_bf16", "ns_update_bf16",
                                                  "ns_update_apply_bf16"))
    assert model["ns_chain_bf16"]["bytes"] == pytest.approx(per_phase, rel=1e-12)
    assert ns == pytest.approx(372.8e9, rel=1e-3)
    elems = sum(r * c for _, r, c in w.matrices)
    assert elems == 31_719_424 and w.n_params == 34_401_372
    assert min(min(r, c) for _, r, c in w.matrices) >= 192          # every group is a base (3-byte X) group
    assert model["prep"]["bytes"] == 15.0 * elems                     # G, M read; M', X0 hi + lo written
    assert model["ema"]["bytes"] == 12.0 * (w.n_params - elems)       # E, P read; E written
    # the last update reads X, B, W, E and writes W', E'
    assert model["ns_update_apply_bf16"]["bytes"] == pytest.approx(
        sum(19.0 * r * c + 2.0 * min(r, c) ** 2 for _, r, c in w.matrices))
