"""bench.py's command line, without a GPU: the one-GPU contract and the
counter-summary lookup."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def test_source_hash_ignores_comments_only():
    a = "int f(int x) { return x + 1; } // add one\n/* block */"
    b = "// header\nint f(int x)\n{\n    return x + 1; /* same code */\n}\n"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_every_workload_names_its_counter_summary_format():
    # Each workload's dominant call names a profiles/<call>_<workload>_counters.txt
    # summary that carries the fields bench.py reads.
    names = {"vec16m": "sum", "vec16m_fused": "sum_max_min", "vec16m_atomic": "sum_accum",
             "vec1g": "sum", "colprod4k": "colprod_f32", "colprod_int": "colprod_i16",
             "cols4k": "sum_cols", "rows1000": "rows_sum", "rows32": "rows_sum"}
    for wl, call in names.items():
        path = os.path.join(ROOT, "profiles", "%s_%s_counters.txt" % (call, wl))
        assert os.path.exists(path), path
        text = open(path).read()
        for key in ("kernel_source_sha256_16", "traffic_bytes_per_launch",
                    "algorithmic_bytes_per_launch", "fetch_factor", "write_factor"):
            assert key + " = " in text, (path, key)
