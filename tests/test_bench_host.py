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
    with open(bench.counters_path("toy"), "w") as f:
        f.write(text.replace(bench.source_hash(), "0" * 16))
    assert bench.load_counters("toy") is None


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
