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


def _source_tree(tmp_path):
    """A copy of the kernel and planning sources, laid out as in the repo
    (csrc/ two levels below the include/ directory)."""
    import shutil
    csrc = tmp_path / "pkg" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    for f in bench.SOURCES_1D:
        dst = csrc / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.CSRC, f), dst)
    return str(csrc)


def test_planning_change_invalidates_traffic(tmp_path):
    """A counter summary stops counting once the kernel source OR the host
    planning (grid sizes, workgroups per CU) differs from the one it was
    taken on."""
    csrc = _source_tree(tmp_path)
    prof = tmp_path / "profiles"
    prof.mkdir()
    wl = bench.Workload("vec1g", "", {}, [], ["sum"], bench.SOURCES_1D, [])
    (prof / "sum_vec1g_counters.txt").write_text(
        "# test\nkernel_source_sha256_16 = %s\ntraffic_bytes_per_launch = 123\n"
        % bench.source_hash(bench.SOURCES_1D, csrc))
    assert bench.committed_traffic(wl, "sum", str(prof), csrc) == 123.0
    assert "api.hip" in bench.SOURCES_1D and "internal.hpp" in bench.SOURCES_1D
    for f, old, new in (("internal.hpp", "#define RED_STREAM_WG_PER_CU 2",
                         "#define RED_STREAM_WG_PER_CU 3"),
                        ("api.hip", "kPartialBytes = size_t(16) << 20",
                         "kPartialBytes = size_t(8) << 20"),
                        ("reduce1d.hip", "if (grid > 1)", "if (grid > 2)")):
        path = os.path.join(csrc, f)
        text = open(path).read()
        assert old in text, (f, old)
        open(path, "w").write(text.replace(old, new, 1))
        assert bench.committed_traffic(wl, "sum", str(prof), csrc) is None, f
        open(path, "w").write(text)
        assert bench.committed_traffic(wl, "sum", str(prof), csrc) == 123.0
    # a comment-only change keeps the summary
    path = os.path.join(csrc, "internal.hpp")
    open(path, "a").write("\n// a comment\n")
    assert bench.committed_traffic(wl, "sum", str(prof), csrc) == 123.0


def test_cpu_threads_respects_the_job_share(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert 1 <= bench.cpu_threads() <= 3
    monkeypatch.setenv("OMP_NUM_THREADS", "")
    assert bench.cpu_threads() == len(os.sched_getaffinity(0))


def test_cpu_baseline_reports_threads_and_single_core():
    """Both oracle modes are timed; the threaded one is the baseline."""
    import numpy as np
    import oracle
    x = np.linspace(-1, 1, 1 << 16, dtype=np.float32)
    wl = bench.Workload("t", "", {}, [], [], [], bench.vector_cpu(oracle.get(), x, (False,)))
    b = bench.cpu_baseline(wl, 0.05)
    assert b["kind"] == "oracle" and b["value"] > 0
    assert b["single_core"] is None or (b["single_core"]["cores"] == 1 and b["cores"] >= 2)


def test_against_ceiling_picks_the_same_byte_count():
    ceiling = {"big": {"bytes": 4 << 30, "gbs_mean": 7400.0},
               "128MiB": {"bytes": 128 << 20, "gbs_mean": 6700.0},
               "256MiB": {"bytes": 256 << 20, "gbs_mean": 6900.0}}
    e = bench.against_ceiling({"bytes": 134283264, "gbs_mean": 6300.0}, ceiling)
    assert e["read_ceiling"] == "128MiB" and abs(e["of_read_ceiling"] - 6300 / 6700) < 1e-4
    e = bench.against_ceiling({"bytes": 262406144, "gbs_mean": 6660.0}, ceiling)
    assert e["read_ceiling"] == "256MiB"
    e = bench.against_ceiling({"bytes": 540672, "gbs_mean": 100.0}, ceiling)
    assert "read_ceiling" not in e and "of_read_ceiling" not in e


def test_variant_without_a_workload_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "rows32",
                           "--variant", "atomic"], capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "no atomic variant" in proc.stderr and "vec1g" in proc.stderr
    assert proc.stdout == ""


def test_every_variant_names_a_workload():
    for base in ("vec1g", "vec16m"):
        for v in ("fused", "atomic"):
            assert "%s_%s" % (base, v) in bench.WORKLOADS
