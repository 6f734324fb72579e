"""bench.py: the host-side accounting (CPU) and the JSON line of a short run
on the GPU."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_recurrent_weight_amd.inputs import WORKLOADS  # noqa: E402


def test_algorithmic_bytes():
    """q, k, v and o once in the io dtype, beta and lambda once in fp32 (beta
    per column for Falcon-2), the final state once in fp32."""
    assert bench.algorithmic_bytes(WORKLOADS["c2"]) == 52_690_944
    assert bench.algorithmic_bytes(WORKLOADS["c3"]) == 204_865_536
    assert bench.algorithmic_bytes(WORKLOADS["c4"]) == 407_896_064
    c1 = WORKLOADS["c1"]
    assert bench.algorithmic_bytes(c1) == 4 * 64 * 16 * 4 + 2 * 64 * 4 + 16 * 16 * 4


def test_algorithmic_bytes_backward_c2():
    """q, k, v, d_o read and d_q, d_k, d_v written in bf16 (7 x 64 x 2 bytes
    per head-token), four fp32 scalars per head-token, and three fp32 states
    per head."""
    n = 8 * 12 * 1024
    assert bench.algorithmic_bytes_bwd(WORKLOADS["c2"]) == n * (7 * 64 * 2 + 16) + 96 * 64 * 64 * 4 * 3
    # 42 64^3-sized product terms per head and 64-token chunk at d_k = d_v = 64
    assert bench.algorithmic_flops_bwd(WORKLOADS["c2"]) == 96 * 16 * 42 * 64 ** 3


def test_algorithmic_flops_c2():
    """Falcon-1 chunk form: 2C(d_k + d_v) + 6 d_k d_v per head-token."""
    w = WORKLOADS["c2"]
    assert bench.algorithmic_flops(w) == w.batch * w.heads * w.seqlen * (2 * 64 * 128 + 6 * 64 * 64)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


@pytest.mark.gpu
def test_bench_line_contract():
    """A short run prints one JSON line with the keys and the roofline and
    CPU-baseline objects the measurement contract names."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--cpu-seconds", "0.5"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("c2")
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert cb["single_core_value"] > 0 and cb["cpu_model"]
    assert d["value"] > 0 and abs(d["value"] - 8 * 12 * 1024 / (d["ms_per_step"] * 1e-3)) < 1e-3 * d["value"]


def _fake_db(path, counter, rows, top=()):
    """A stand-in for a rocprofv3 results database: the two tables and the
    columns that the summary reads."""
    import sqlite3
    con = sqlite3.connect(path)
    con.execute("create table top_kernels (name text, total_calls int, average real, total_duration real)")
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into top_kernels values (?, ?, ?, ?)", top)
    con.executemany("insert into counters_collection values (?, ?, ?)", [(k, counter, v) for k, v in rows])
    con.commit()
    con.close()


def test_rocprof_summary_calibrates_on_the_largest_copy(tmp_path):
    """The runtime's copy kernel also uploads the inputs: the calibration is
    the largest of its dispatches (256 MiB read as 131072 KiB by FETCH_SIZE,
    written as 262144 KiB by WRITE_SIZE gives scale factors 2 and 1)."""
    k = "void falcon::(anonymous namespace)::a1_output<false>(falcon::ChunkAArgs)"
    copy = bench.COPY_KERNEL
    _fake_db(tmp_path / "s.db", "X", [], top=[(k, 3, 50.0, 150.0)])
    _fake_db(tmp_path / "f.db", "FETCH_SIZE", [(copy, 12.0), (copy, 131072.0), (copy, 40.0), (k, 1000.0), (k, 1000.0)])
    _fake_db(tmp_path / "w.db", "WRITE_SIZE", [(copy, 8.0), (copy, 262144.0), (k, 500.0)])
    text = bench.rocprof_summary("c3", ["a1_output"], str(tmp_path / "s.db"), str(tmp_path / "f.db"),
                                 str(tmp_path / "w.db"), "cmd")
    assert "scale factors 2.0 (fetch) and 1.0 (write)" in text
    # per dispatch: 1000 KiB fetched x 2 + 500 KiB written x 1
    assert "traffic_bytes_per_call: %d" % ((2 * 1000 + 500) * 1024) in text
    assert "| `%s` | 3 | 50.000 |" % k in text


def test_mfma_summary_busy_fraction(tmp_path):
    """SQ_VALU_MFMA_BUSY_CYCLES over (CUs x SIMDs x kernel cycles at the peak
    clock), weighted by kernel time for the call."""
    a = "void falcon::(anonymous namespace)::ka(falcon::X)"
    b = "void falcon::(anonymous namespace)::kb(falcon::X)"
    _fake_db(tmp_path / "s.db", "X", [], top=[(a, 5, 10.0, 50.0), (b, 5, 30.0, 150.0)])
    import sqlite3
    _fake_db(tmp_path / "m.db", "SQ_VALU_MFMA_BUSY_CYCLES", [(a, 0.5 * 1024 * 10.0 * 2400), (b, 0.1 * 1024 * 30.0 * 2400)])
    text = bench.mfma_summary(str(tmp_path / "m.db"), str(tmp_path / "s.db"))
    assert "| 0.5000 |" in text and "| 0.1000 |" in text
    frac = float(text.split("mfma_busy_frac_per_call: ")[1].split()[0])
    assert abs(frac - (0.5 * 10 + 0.1 * 30) / 40) < 1e-6
