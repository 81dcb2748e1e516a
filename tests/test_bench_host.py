"""Host-side logic of the benchmark and of the seeded input generators (CPU):
the one-GPU guard, the source hash that ties counter summaries to the code
they were taken from, the traffic lookup, the algorithmic byte counts and the
generators' conventions."""
import importlib.util
import json
import os
import shutil
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

from ssim_loss_amd.inputs import WORKLOADS, make_pair, smooth_field

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.fixture
def source_copy(tmp_path, monkeypatch):
    """The library's sources copied to a scratch tree the hash is taken over."""
    bench = load_bench()
    csrc = tmp_path / "ssim_loss_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "ssim_loss_amd", "csrc"), csrc)
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    return bench, csrc


def test_source_hash_ignores_comments_and_white_space_runs_but_not_code(source_copy):
    bench, csrc = source_copy
    h0 = bench.source_hash()
    assert h0 == load_bench().source_hash()  # the copy hashes as the tree does
    hpp = csrc / "ssim_fused.hpp"
    text = hpp.read_text()

    hpp.write_text(text + "\n// a comment\n/* and a\n   block comment */\n\n")
    assert bench.source_hash() == h0
    # runs of white space count as one space
    hpp.write_text(text.replace("constexpr int kXYRing = 20;", "constexpr  int   kXYRing =\n   20;"))
    assert bench.source_hash() == h0

    hpp.write_text(text.replace("constexpr int kXYRing = 20;", "constexpr int kXYRing = 24;"))
    assert bench.source_hash() != h0
    hpp.write_text(text)
    assert bench.source_hash() == h0


def test_source_hash_keeps_string_literals(source_copy):
    bench, csrc = source_copy
    h0 = bench.source_hash()
    api = csrc / "ssim_api.hip"
    text = api.read_text()
    assert '"' in text
    # a // inside a string literal is code, not the start of a comment
    first = text.index('"')
    api.write_text(text[:first + 1] + "// " + text[first + 1:])
    assert bench.source_hash() != h0


def _args(workload, dtype="float32"):
    return SimpleNamespace(workload=workload, dtype=dtype)


def test_traffic_lookup_requires_the_same_code_workload_and_dtype(tmp_path, monkeypatch):
    bench = load_bench()
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    h = bench.source_hash()
    rec = {"workload": "1080p-valid", "dtype": "float32", "source_sha256_16": h,
           "bytes_per_launch": {"ssim_loss_and_grad": 123456789}}
    (tmp_path / "hbm_traffic_1080p-valid.json").write_text(json.dumps(rec))
    assert bench.measured_traffic(_args("1080p-valid"), "ssim_loss_and_grad") == 123456789
    assert bench.measured_traffic(_args("1080p-valid"), "ssim_forward") is None
    assert bench.measured_traffic(_args("1080p-same"), "ssim_loss_and_grad") is None
    assert bench.measured_traffic(_args("1080p-valid", "bfloat16"), "ssim_loss_and_grad") is None

    (tmp_path / "hbm_traffic_1080p-valid.json").write_text(
        json.dumps(dict(rec, source_sha256_16="0" * 16)))
    assert bench.measured_traffic(_args("1080p-valid"), "ssim_loss_and_grad") is None

    (tmp_path / "hbm_traffic_1080p-valid-bfloat16.json").write_text(
        json.dumps(dict(rec, dtype="bfloat16")))
    assert bench.measured_traffic(_args("1080p-valid", "bfloat16"), "ssim_loss_and_grad") == 123456789


def test_committed_traffic_summaries_name_their_workload_and_dtype():
    d = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(d) if n.startswith("hbm_traffic_") and n.endswith(".json")]
    assert names
    for n in names:
        with open(os.path.join(d, n)) as f:
            rec = json.load(f)
        tag = n[len("hbm_traffic_"):-len(".json")]
        want = rec["workload"] if rec.get("dtype", "float32") == "float32" else \
            f"{rec['workload']}-{rec['dtype']}"
        assert tag == want
        assert len(rec["source_sha256_16"]) == 16
        assert all(v > 0 for v in rec["bytes_per_launch"].values())


@pytest.mark.parametrize("padding", ["valid", "same"])
def test_algorithmic_bytes_of_the_designs(padding):
    bench = load_bench()
    shape = (2, 3, 40, 52)
    N, C, H, W = shape
    e_in = N * C * H * W
    e_out = N * C * ((H - 10) * (W - 10) if padding == "valid" else H * W)
    for eb in (4, 2):
        b = bench.algorithmic_bytes(shape, padding, eb)
        # one launch: both images in, both gradients out, nothing else
        assert b["ssim_loss_and_grad"] == 4 * eb * e_in
        # the recomputing backward moves what the one launch moves; the
        # recompute step adds a forward that reads both images again
        assert b["ssim_backward_recompute"] == b["ssim_loss_and_grad"]
        assert b["ssim_forward(inference)"] == 2 * eb * e_in
        # saved maps: four fp32 statistics written once and read once
        assert (b["ssim_forward"] + b["ssim_backward"]
                - b["ssim_forward(inference)"] - b["ssim_backward_recompute"]) == 32 * e_out
        # cached reference: y's map is read instead of y's gradient written
        assert b["ssim_loss_and_grad_ref"] == 3 * eb * e_in + 4 * e_out
    assert bench.algorithmic_bytes(shape, padding, 4)["ssim_loss_and_grad"] == \
        2 * bench.algorithmic_bytes(shape, padding, 2)["ssim_loss_and_grad"]


def test_algorithmic_flops_order_the_designs():
    bench = load_bench()
    f = bench.algorithmic_flops((1, 3, 1080, 1920), "valid")
    assert f["ssim_forward"] == f["ssim_forward(inference)"]
    # the one launch does the recomputing backward's work plus the loss
    assert f["ssim_backward_recompute"] < f["ssim_loss_and_grad"]
    assert f["ssim_loss_and_grad"] < f["ssim_forward"] + f["ssim_backward_recompute"]
    # the cached reference blurs three quantities each way instead of four
    assert f["ssim_loss_and_grad_ref"] < f["ssim_loss_and_grad"]


def test_generators_are_seeded_fp32_in_the_unit_interval():
    for kind in ("uniform", "field"):
        x, y = make_pair((2, 3, 24, 40), kind, 0.05, seed=7)
        x2, y2 = make_pair((2, 3, 24, 40), kind, 0.05, seed=7)
        assert x.dtype == np.float32 and y.dtype == np.float32
        assert x.flags["C_CONTIGUOUS"] and y.flags["C_CONTIGUOUS"]
        assert np.array_equal(x, x2) and np.array_equal(y, y2)
        assert x.min() >= 0.0 and x.max() <= 1.0 and y.min() >= 0.0 and y.max() <= 1.0
        x3, _ = make_pair((2, 3, 24, 40), kind, 0.05, seed=8)
        assert not np.array_equal(x, x3)
    v1, v2 = make_pair((1, 2, 12, 14, 16), "uniform", 0.05, seed=3)
    assert v1.shape == (1, 2, 12, 14, 16) and v1.dtype == np.float32
    assert v1.min() >= 0.0 and v2.max() <= 1.0


def test_second_image_is_the_first_plus_clamped_gaussian_noise():
    x, y = make_pair((1, 3, 256, 256), "uniform", 0.05, seed=0)
    d = (y.astype(np.float64) - x.astype(np.float64))
    inner = (y > 0.0) & (y < 1.0)  # entries the clamp left alone
    assert abs(d[inner].mean()) < 2e-3
    assert abs(d[inner].std() - 0.05) < 2e-3
    # near the ends of the interval the noise is clamped onto them
    assert (y == 1.0).any() and (y == 0.0).any()
    x0, y0 = make_pair((1, 1, 16, 16), "uniform", 0.0, seed=0)
    assert np.array_equal(x0, y0)


def test_per_image_seeds_draw_image_n_from_seed_plus_n():
    x, y = make_pair((3, 2, 20, 24), "field", 0.03, seed=5, per_image_seed=True)
    for n in range(3):
        xn, yn = make_pair((1, 2, 20, 24), "field", 0.03, seed=5 + n, per_image_seed=True)
        assert np.array_equal(x[n], xn[0]) and np.array_equal(y[n], yn[0])


def test_smooth_field_spans_the_unit_interval():
    f = smooth_field(np.random.default_rng(1), 3, 64, 96)
    assert f.shape == (3, 64, 96)
    for c in range(3):
        # min-max rescaled to [0, 1] before the +-0.02 texture and the clamp
        assert f[c].min() <= 0.02 and f[c].max() >= 0.98


def test_workload_table_matches_the_benchmark_configurations():
    shapes = {w.name: (w.shape, w.padding) for w in WORKLOADS.values()}
    assert shapes["tiny-64"] == ((1, 1, 64, 64), "valid")
    assert shapes["small-256"] == ((1, 3, 256, 256), "valid")
    assert shapes["1080p-valid"] == ((1, 3, 1080, 1920), "valid")
    assert shapes["1080p-same"] == ((1, 3, 1080, 1920), "same")
    assert shapes["4k-batch8"] == ((8, 3, 2160, 3840), "valid")
    assert WORKLOADS["4k-batch8"].per_image_seed
    assert WORKLOADS["1080p-valid"].kind == "field" and WORKLOADS["4k-batch8"].kind == "uniform"


def test_profile_summaries_from_rocprof_csvs(tmp_path):
    """bench.py --summarize: the kernel-trace table, the HBM traffic scaled by
    the 512 MiB calibration copy, and the derived SQ figures, from CSVs laid
    out as a --profile run leaves them (synthetic values)."""
    import csv
    import json

    import bench

    out = tmp_path / "prof"

    def write(key, fname, rows):
        d = out / key / "host" / "123"
        d.mkdir(parents=True, exist_ok=True)
        with open(d / fname, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=list(rows[0]))
            w.writeheader()
            w.writerows(rows)

    k = "(anonymous namespace)::ssim_loss_grad_kernel(ssim_dev::Params)"
    cp = "void at::native::vectorized_elementwise_kernel<4, copy_kernel...>"
    write("trace", "run_kernel_stats.csv",
          [{"Name": k, "Calls": "10", "TotalDurationNs": "500000", "AverageNs": "50000",
            "Percentage": "90.0", "MinNs": "49000", "MaxNs": "51000"}])
    write("trace", "run_kernel_trace.csv",
          [{"Kernel_Name": k, "Start_Timestamp": str(100 * i), "End_Timestamp": str(100 * i + 50)}
           for i in range(8)])

    def pmc(key, counter, kval, cval):
        rows = [{"Dispatch_Id": str(i), "Kernel_Name": k, "Counter_Name": counter,
                 "Counter_Value": str(kval)} for i in range(4)]
        rows += [{"Dispatch_Id": str(10 + i), "Kernel_Name": cp, "Counter_Name": counter,
                  "Counter_Value": str(cval)} for i in range(3)]
        # small staging copies of the same kernel must not dilute the calibration
        rows += [{"Dispatch_Id": str(20 + i), "Kernel_Name": cp, "Counter_Name": counter,
                  "Counter_Value": "2.5"} for i in range(4)]
        write(key, "p_counter_collection.csv", rows)

    pmc("fetch", "FETCH_SIZE", 50000, 262144)   # the copy reads half: scale 2
    pmc("write", "WRITE_SIZE", 48828.125, 524288)
    rows = []
    for i in range(4):
        for c, v in (("SQ_WAVES", 4096), ("SQ_INSTS_VALU", 3.0e7), ("SQ_WAVE_CYCLES", 8.0e7),
                     ("SQ_ACTIVE_INST_VALU", 2.4e7)):
            rows.append({"Dispatch_Id": str(i), "Kernel_Name": k, "Counter_Name": c,
                         "Counter_Value": str(v)})
    write("sq_a", "p_counter_collection.csv", rows)
    write("sq_c", "p_counter_collection.csv",
          [{"Dispatch_Id": "0", "Kernel_Name": k, "Counter_Name": "GRBM_GUI_ACTIVE",
            "Counter_Value": str(8 * 2.4e9 * 50e-6)}])

    prof = tmp_path / "profiles"
    bench.summarize_profile("1080p-valid", "float32", str(out), profiles_dir=str(prof))
    tr = json.loads((prof / "hbm_traffic_1080p-valid.json").read_text())
    assert tr["fetch_scale"] == 2.0 and tr["write_scale"] == 1.0
    assert tr["detail"]["ssim_loss_and_grad"]["read_bytes"] == 50000 * 1024 * 2
    assert tr["bytes_per_launch"]["ssim_loss_and_grad"] == 50000 * 2048 + 50000000
    assert tr["source_sha256_16"] == bench.source_hash()
    sq = json.loads((prof / "sq_counters_1080p-valid.json").read_text())
    d = sq["derived"]["ssim_loss_and_grad"]
    assert d["valu_insts_per_wave"] == round(3.0e7 / 4096, 1)
    assert d["valu_active_share_of_wave_cycles"] == 0.3
    assert abs(d["clock_ghz"] - 2.4) < 1e-3
    assert d["trace_avg_us"] == 50.0
    md = (prof / "ssim_kernels_1080p-valid_kernel_trace.md").read_text()
    assert "ssim_loss_and_grad" in md and "| 10 | 50.00 |" in md
