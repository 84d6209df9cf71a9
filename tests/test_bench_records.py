"""The measurement code's profile records (bench.py --record / --pmc-summary and
the roofline fields built from them), on small synthetic rocprofv3 CSV files:
no GPU involved."""
import csv
import importlib
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PMC_FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
              "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
              "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
              "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_pmc(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=PMC_FIELDS)
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Agent_Id": 1, "Queue_Id": 1,
                        "Process_Id": 1, "Thread_Id": 1, "Grid_Size": 131072, "Kernel_Id": 3,
                        "Kernel_Name": kernel, "Workgroup_Size": 512, "LDS_Block_Size": 0,
                        "Scratch_Size": 0, "VGPR_Count": 88, "Accum_VGPR_Count": 0,
                        "SGPR_Count": 64, "Counter_Name": counter, "Counter_Value": value,
                        "Start_Timestamp": 0, "End_Timestamp": 1})


@pytest.fixture()
def tree(tmp_path):
    """A copy of bench.py and the kernel sources (their hash keys the records)."""
    shutil.copy(os.path.join(ROOT, "bench.py"), tmp_path / "bench.py")
    shutil.copytree(os.path.join(ROOT, "group_quantized_moe_dsq_amd", "csrc"),
                    tmp_path / "group_quantized_moe_dsq_amd" / "csrc")
    return tmp_path


def run_bench(tree, *args):
    r = subprocess.run([sys.executable, str(tree / "bench.py"), *args], cwd=tree,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stdout


def load_bench(tree):
    sys.path.insert(0, str(tree))
    try:
        if "bench" in sys.modules:
            del sys.modules["bench"]
        return importlib.import_module("bench")
    finally:
        sys.path.remove(str(tree))


GMM = "void dsq::gmm_kernel<8, 4, 1, true>(dsq::GmmArgs)"


def make_records(tree):
    # the copy calibration: 1 GiB read and written, FETCH_SIZE reads half
    write_pmc(tree / "c.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0),
                               ("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    run_bench(tree, "--record", "calibration", "--pmc", "c.csv")
    with open(tree / "kt.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow([GMM, 100, 85000000, 850000.0, 50.0, 840000, 860000, 1.0])
        w.writerow(["void dsq::gmm_kernel<8, 4, 1, false>(dsq::GmmArgs)", 100, 45000000,
                    450000.0, 25.0, 440000, 460000, 1.0])
        w.writerow(["void at::native::fill(float*)", 5, 1000, 200.0, 0.0, 100, 300, 1.0])
    write_pmc(tree / "f.csv", [(GMM, "FETCH_SIZE", 2.0e6), (GMM, "FETCH_SIZE", 2.2e6)])
    write_pmc(tree / "w.csv", [(GMM, "WRITE_SIZE", 1000.0), (GMM, "WRITE_SIZE", 1000.0)])
    run_bench(tree, "--record", "moe256", "--kt", "kt.csv", "--pmc", "f.csv", "w.csv")
    with open(tree / "profiles" / "records.json") as fh:
        return json.load(fh)


def test_record_contents(tree):
    recs = make_records(tree)
    cal = recs["calibration"]
    assert cal["fetch_scale"] == pytest.approx(2.0) and cal["write_scale"] == pytest.approx(1.0)
    w = recs["workloads"]["moe256"]
    k = w["kernels"]["dsq::gmm_kernel<8, 4, 1, true>"]
    assert k["avg_us"] == 850.0 and k["calls"] == 100
    assert k["FETCH_SIZE"] == pytest.approx(2.1e6)  # mean over dispatches
    assert k["WRITE_SIZE"] == pytest.approx(1000.0) and k["dispatches_counted"] == 2
    assert "dsq::gmm_kernel<8, 4, 1, false>" in w["kernels"]
    assert not any("fill" in name for name in w["kernels"])  # library kernels only
    assert any("--only moe256" in c and "--kernel-trace" in c for c in w["commands"])
    assert any("--pmc FETCH_SIZE" in c for c in w["commands"])


def test_roofline_from_record(tree):
    make_records(tree)
    bench = load_bench(tree)
    algo = 4_000_000_000
    e = bench.roofline_entry("moe256", "dsq::gmm_kernel<8, 4, 1, true>", "hbm", algo,
                             "algorithmic_bytes")
    assert e["kernel"] == "dsq::gmm_kernel<8, 4, 1, true>"
    assert e["kernel_us"] == 850.0
    assert e["achieved"] == pytest.approx(algo / 850e-6 / 1e9, abs=0.1)
    assert e["frac"] == pytest.approx(e["achieved"] / 8000.0, abs=1e-4)
    # FETCH 2.1e6 KiB x 2.0 + WRITE 1000 KiB x 1.0
    assert e["traffic"] == int(2.1e6 * 1024 * 2.0 + 1000 * 1024 * 1.0)
    # a prefix picks the kernel of the family with the most GPU time
    e2 = bench.roofline_entry("moe256", "dsq::gmm_kernel<8", "hbm", algo, "algorithmic_bytes")
    assert e2["kernel"] == "dsq::gmm_kernel<8, 4, 1, true>"
    # no record of another workload: the fields stay null
    e3 = bench.roofline_entry("moe1", "dsq::dec_gateup_kernel", "hbm", algo, "algorithmic_bytes")
    assert e3["kernel_us"] is None and e3["achieved"] is None and e3["traffic"] is None


def test_record_invalid_after_source_change(tree):
    make_records(tree)
    with open(tree / "group_quantized_moe_dsq_amd" / "csrc" / "gmm.hip", "a") as fh:
        fh.write("\n// changed\n")
    bench = load_bench(tree)
    e = bench.roofline_entry("moe256", "dsq::gmm_kernel<8, 4, 1, true>", "hbm", 1, "algorithmic_bytes")
    assert e["kernel_us"] is None and e["traffic"] is None and "note" in e


def test_pmc_summary(tree):
    write_pmc(tree / "f.csv", [(GMM, "FETCH_SIZE", 2.0e6), (GMM, "FETCH_SIZE", 4.0e6),
                               ("void at::native::fill(float*)", "FETCH_SIZE", 1.0)])
    out = run_bench(tree, "--pmc-summary", "f.csv")
    assert "dsq::gmm_kernel<8, 4, 1, true>" in out and "dispatches=2" in out
    assert "3e+06" in out and "fill" not in out


def test_kernel_name():
    bench = load_bench(__import__("pathlib").Path(ROOT))
    assert bench._kernel_name(GMM) == "dsq::gmm_kernel<8, 4, 1, true>"
    assert bench._kernel_name("dsq::gemm_prep_kernel(float const*, int)") == "dsq::gemm_prep_kernel"
    assert bench._kernel_name("void dsq::splitk_reduce_kernel<4>(float const*, float*, int)") == \
        "dsq::splitk_reduce_kernel<4>"
