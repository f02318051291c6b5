"""Host logic of bench.py (no GPU): the single-GPU guard, the rocprofv3 counter parsing behind the
measured-traffic figure, and the rule that a traffic record counts only for the decode sources it
was taken on."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_rows_are_summed_per_dispatch(bench, tmp_path):
    p = tmp_path / "run_counter_collection.csv"
    rows = [("1", "decode_mfma_kernel<2, 2>", "FETCH_SIZE", 10.0), ("1", "decode_mfma_kernel<2, 2>", "FETCH_SIZE", 5.5),
            ("2", "decode_mfma_kernel<2, 2>", "FETCH_SIZE", 7.0), ("2", "decode_mfma_kernel<2, 2>", "WRITE_SIZE", 99.0),
            ("3", "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)]
    with open(p, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for r in rows:
            f.write(f'{r[0]},"{r[1]}",{r[2]},{r[3]}\n')
    assert sorted(bench._per_dispatch(str(p), "FETCH_SIZE", "decode_mfma_kernel")) == [7.0, 15.5]
    assert bench._per_dispatch(str(p), "WRITE_SIZE", "decode_mfma_kernel") == [99.0]
    assert bench._per_dispatch(str(p), "FETCH_SIZE", "copyBuffer") == [512.0]


def test_traffic_record_must_match_the_decode_sources(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "decode_{}_traffic.json"))
    assert bench.measured_traffic("llama2_7b_decode") is None                      # no record
    rec = {"decode_source_sha256_16": bench.source_hash(bench.DECODE_SOURCES), "bytes_per_launch": 123.0}
    (tmp_path / "decode_llama2_7b_decode_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("llama2_7b_decode") == 123.0
    rec["decode_source_sha256_16"] = "0" * 16                                        # taken on other sources
    (tmp_path / "decode_llama2_7b_decode_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("llama2_7b_decode") is None


def test_oracle_baseline_and_estimator_quality_on_a_small_workload(bench):
    """The cpu_baseline leg on a scaled-down workload: at least two whole units, the thread counts, and
    estimator-quality figures in their ranges (the oracle's 1-bit keys correlate with the exact scores;
    a perfect estimate would give a cosine of 1 and a relative RMSE of 0)."""
    import seeded_inputs as si
    w = si.WORKLOADS["llama3_8b_gqa_decode"].scaled(B=1, Hq=8, Hkv=2, N=400)
    base, quality = bench.cpu_baseline(w, 0.01)
    assert base["kind"] == "oracle" and base["cores"] >= 1 and base["host_cores"] >= 1
    assert base["value"] > 0 and "2 of 2" in base["sample"]
    q = quality[w.name]
    assert q["heads"] == 8 and q["keys"] == 8 * 400
    assert 0.0 < q["score_rmse_rel"] < 1.0 and 0.5 < q["score_corr"] <= 1.0
    assert -1.0 <= q["output_cosine_min"] <= q["output_cosine_mean"] <= 1.0
    assert 0.5 < q["output_cosine_keys_only_mean"] <= 1.0
    one = bench.estimator_quality(w, (0, 1))
    assert one["heads"] == 4 and one["units"] == [[0, 1]]


def test_quality_figures_of_exact_estimates(bench):
    import numpy as np
    s = [np.array([1.0, -2.0, 3.0])]
    o = [np.array([0.5, 0.25])]
    q = bench._quality(s, s, o, o, o)
    assert q["score_rmse"] == 0.0 and q["score_rmse_rel"] == 0.0
    assert abs(q["output_cosine_mean"] - 1.0) < 1e-15 and abs(q["score_corr"] - 1.0) < 1e-15
