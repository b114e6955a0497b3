"""Host-side checks of bench.py (no GPU): the algorithmic byte model against
its closed form for full routing, the HBM-counter summary and its
calibration on the copy probe, and the one-GPU contract of the command line.
"""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import get_workload  # noqa: E402


@pytest.mark.parametrize("name", ["mhar100m", "mhar350m", "mhar1b"])
def test_byte_model_closed_form(name):
    # Full routing: site s reads rows 0..s, so sum_s N_s = S (S + 1) / 2 and
    # row n is gathered by the finalize from the S - n sites that read it.
    w = get_workload(name)
    T, d, H, b, S = w.tokens, w.d, w.heads, w.elem_bytes, w.sites
    assert list(w.nsrc) == list(range(1, S + 1)) and not any(w.extra)
    reads = S * (S + 1) // 2
    fwd = reads * (T * d * b + 8 * T * H + 4 * T) + S * (4 * T * H + T * d * b)
    fin = reads * (T * d * b + 8 * T * H + 4 * T) + S * (T * w.r * b + 4 * T + 4 * T * d)
    app = sum(T * w.r * b + 4 * T + 4 * (S - n) * T * H for n in range(S))
    out, launches = bench.kernel_bytes(w, parts=0)
    assert out["fwd"] == fwd and launches["fwd"] == S
    assert out["finalize"] == fin and launches["finalize"] == S
    assert out["score"] == app and launches["score"] == S


def test_byte_model_1b_forward_per_launch():
    # the figure the bench line and the HBM counters of the 1B bank compare
    out, launches = bench.kernel_bytes(get_workload("mhar1b"), parts=0)
    assert out["fwd"] / launches["fwd"] == 1635581952


def _write_pmc(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        for disp, kernel, value in rows:
            wr.writerow({"Dispatch_Id": disp, "Kernel_Name": kernel, "Counter_Name": counter,
                         "Counter_Value": value})


def test_counter_summary_is_calibrated_on_the_copy_probe(tmp_path, monkeypatch):
    copy = 1 << 20
    # FETCH_SIZE reads half of what the copy probe fetched, WRITE_SIZE all of it
    fwd = "void attnres::(anonymous namespace)::k_fwd<unsigned short, 5, unsigned short>(...)"
    probe = "void attnres::(anonymous namespace)::k_probe_copy(...)"
    _write_pmc(tmp_path / "pmc_FETCH_SIZE", "FETCH_SIZE",
               [(1, probe, copy / 2 / 1024), (2, fwd, 100.0), (3, fwd, 300.0)])
    _write_pmc(tmp_path / "pmc_WRITE_SIZE", "WRITE_SIZE",
               [(1, probe, copy / 1024), (2, fwd, 10.0), (3, fwd, 30.0)])
    text = bench.summarize_counters(str(tmp_path), "toy", copy, "cmd")
    fields = {ln.split()[1]: ln.split() for ln in text.splitlines() if ln.startswith("kernel ")}
    assert "scale FETCH_SIZE 2.000000 WRITE_SIZE 1.000000" in text
    assert fields["fwd"][2] == "2"                       # dispatches
    assert float(fields["fwd"][5]) == 200.0 * 1024 * 2   # mean fetch, calibrated bytes
    assert float(fields["fwd"][6]) == 20.0 * 1024        # mean write, calibrated bytes
    # the stored summary is used only while the kernel sources match its hash
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    with open(bench.counters_path("toy"), "w") as f:
        f.write(text)
    assert bench.load_counters("toy")["fwd"] == (200.0 * 1024 * 2, 20.0 * 1024)
    # the microbatch total: every routing dispatch, the probes left out
    total = 2 * (200.0 * 1024 * 2 + 20.0 * 1024)
    assert bench.load_counters("toy")["_total"] == total
    m = bench.measured_fields("toy", 2.0, 1000000)
    assert m["hbm_bytes_per_microbatch"] == int(total)
    assert m["achieved_gbps"] == round(total / 2.0 / 1e6, 1)
    assert m["model_gbps"] == 0.5 and m["alg_bytes_per_microbatch"] == 1000000
    with open(bench.counters_path("toy"), "w") as f:
        f.write(text.replace(bench.source_hash("toy"), "0" * 16))
    assert bench.load_counters("toy") is None


def test_phase_traffic_of_the_delta_and_list_lines(tmp_path, monkeypatch):
    """The roofline traffic of the delta and list lines is measured bytes in
    the unit of their `achieved` figure: one call's backward phase holds its
    recomputed forward, null sums and dq reductions; the list backward its dq
    reduction."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    h = bench.source_hash("delta8b")
    n = bench.DELTA_SITES
    fwd, bwd, null, red = (100.0, 10.0), (300.0, 200.0), (5.0, 1.0), (2.0, 0.0)
    total = 2 * n * sum(fwd) + n * sum(bwd) + 2 * n * sum(null) + 3 * n * sum(red)
    with open(bench.counters_path("delta8b"), "w") as f:
        f.write(f"source_hash {h}\n"
                f"kernel delta_fwd {2 * n} 0 0 {fwd[0]} {fwd[1]}\n"
                f"kernel delta_bwd {n} 0 0 {bwd[0]} {bwd[1]}\n"
                f"kernel delta_null {2 * n} 0 0 {null[0]} {null[1]}\n"
                f"kernel dq_reduce {3 * n} 0 0 {red[0]} {red[1]}\n"
                f"hbm_bytes_per_microbatch {total}\n")
    assert bench.delta_traffic("delta8b", "delta_fwd") == 110
    assert bench.delta_traffic("delta8b", "delta_bwd") == 110 + 500 + 2 * 6 + 3 * 2
    with open(bench.counters_path("list_lr"), "w") as f:
        f.write(f"source_hash {bench.source_hash('list_lr')}\n"
                "kernel list_fwd 1 0 0 70 7\nkernel list_bwd 1 0 0 90 40\n"
                "kernel dq_reduce 1 0 0 3 1\nhbm_bytes_per_microbatch 211\n")
    assert bench.list_traffic("list_lr", "list_fwd") == 77
    assert bench.list_traffic("list_lr", "list_bwd") == 134
    assert bench.list_traffic("list_d513", "list_bwd") is None  # no summary


@pytest.mark.parametrize("name,kind", [
    ("void attnres::(anonymous namespace)::k_fwd<unsigned short, 5, unsigned short>(...)", "fwd"),
    ("void attnres::(anonymous namespace)::k_bwd_site_w<unsigned short, 5>(...)", "bwd_site"),
    ("void attnres::(anonymous namespace)::k_score_mfma<5, 2>(...)", "score"),
    ("void attnres::(anonymous namespace)::k_delta_fwd_s<unsigned short, 8>(...)", "delta_fwd"),
    ("void attnres::(anonymous namespace)::k_delta_bwd<unsigned short, 8>(...)", "delta_bwd"),
    ("void attnres::(anonymous namespace)::k_delta_null_vec<unsigned short>(...)", "delta_null"),
    ("void attnres::(anonymous namespace)::k_list_bwd<unsigned short, 8>(...)", "list_bwd"),
    ("void attnres::(anonymous namespace)::k_finalize_cols<unsigned short, 2, float>(...)",
     "finalize"),
])
def test_kernel_kinds(name, kind):
    assert bench.kind_of(name) == kind


def test_source_hash_follows_the_workload_path():
    assert bench.path_of("delta8b") == "delta" and bench.path_of("list_lr") == "list"
    assert bench.path_of("mhar1b") == "bank" and bench.path_of("k3_blocks") == "bank"
    assert bench.source_hash("mhar1b") == bench.source_hash("k3")
    assert bench.source_hash("mhar1b") != bench.source_hash("delta8b")
    assert bench.source_hash("list_lr") != bench.source_hash("delta8b")


def test_kernel_stats_summary(tmp_path):
    path = tmp_path / "run_kernel_stats.csv"
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                           "Percentage", "MinNs", "MaxNs", "StdDev"])
        wr.writeheader()
        wr.writerow({"Name": "void attnres::(anonymous namespace)::k_fwd<unsigned short, 5>(x)",
                     "Calls": 4, "TotalDurationNs": 4000, "AverageNs": 1000, "Percentage": 80,
                     "MinNs": 900, "MaxNs": 1100, "StdDev": 1})
        wr.writerow({"Name": "k_probe_copy", "Calls": 1, "TotalDurationNs": 1000,
                     "AverageNs": 1000, "Percentage": 20, "MinNs": 1000, "MaxNs": 1000,
                     "StdDev": 0})
    text = bench.summarize_kernel_stats(str(path), "toy", "cmd", "note")
    assert "| k_fwd<unsigned short, 5> | 4 | 4.0 | 1.00 | 0.90 | 1.10 | 80.0% |" in text
    assert text.index("k_fwd") < text.index("k_probe_copy")


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_cpu_baseline_chunks_cover_every_token_once():
    import threading

    seen, lock = [], threading.Lock()

    def prepare(n):
        def run(lo, hi):
            with lock:
                seen.append((n, lo, hi))
        return run

    res = bench.oracle_baseline(prepare, 1000, "ms/microbatch", "toy", tokens=37)
    chunks = sorted((lo, hi) for n, lo, hi in seen if n == 37)
    assert chunks[0][0] == 0 and chunks[-1][1] == 37
    assert all(a[1] == b[0] for a, b in zip(chunks, chunks[1:]))
    assert res["cores"] == len(chunks) <= bench.oracle_cores() <= 16
    assert res["kind"] == "oracle" and res["unit"] == "ms/microbatch"
    # the default sample is sized from a one-thread probe on a few tokens
    seen.clear()
    bench.oracle_baseline(prepare, 64, "ms/read", "toy")
    assert seen[0] == (16, 0, 16)


def test_transient_gradient_bytes_follow_the_site_pass(monkeypatch):
    """The work-group-wide site pass (rows no wave covers in whole tokens)
    forms each transient source's gradient: its bytes move from the finalize
    to the site pass, and a site that finalizes nothing launches nothing."""
    assert bench.site_pass_is_wave_owned(get_workload("mhar1b"))
    assert not bench.site_pass_is_wave_owned(get_workload("k3"))
    assert not bench.site_pass_is_wave_owned(get_workload("lr_h8"))
    w = get_workload("k3")
    T, d, r, H, b = w.tokens, w.d, w.r, w.heads, w.elem_bytes
    fused, fl = bench.kernel_bytes(w, parts=512)
    monkeypatch.setattr(bench, "site_pass_is_wave_owned", lambda w: True)
    apart, al = bench.kernel_bytes(w, parts=512)
    n = sum(w.extra)
    assert fused["bwd_site"] - apart["bwd_site"] == n * (4 * T * d + r * b)
    job = T * d * b + 8 * T * H + 4 * T + T * r * b + 4 * T + 4 * T * d  # one site's gather
    assert apart["finalize"] - fused["finalize"] == n * job
    rows_final = sum(1 for s in range(w.sites) if w.nsrc[s] > (w.nsrc[s - 1] if s else 0))
    assert fl["finalize"] == rows_final and al["finalize"] == w.sites
