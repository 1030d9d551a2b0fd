"""Host-side behaviour of bench.py that needs no GPU: the one-GPU refusal, row
selection errors, the rocprofv3 trace summary, and that the decode GEMV's
stored HBM traffic belongs to the kernel source in the tree (so the bench
line reports it rather than null)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + list(args),
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_unknown_row_is_refused():
    r = _run("--rows", "step,nonsense")
    assert r.returncode == 2
    assert "nonsense" in r.stderr


def test_gemv_traffic_matches_the_kernel_source():
    b = _bench()
    h = b.source_hash("tq_gemv_m1.hip")
    assert h is not None
    assert list(b.GEMV_TRAFFIC) == [h], "re-measure FETCH_SIZE/WRITE_SIZE for the current kernel"
    algorithmic = 57802752  # codes and scales of the 72-matrix stack at G = 128
    assert 1.0 <= b.GEMV_TRAFFIC[h] / algorithmic < 1.1


def test_trace_summary_tables(tmp_path, capsys):
    stats = tmp_path / "stats.csv"
    stats.write_text("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs\n"
                     "\"void tq::(anonymous namespace)::k_a<128>(int)\",2,3000,1500,75,1000,2000\n"
                     "k_b,1,1000,1000,25,1000,1000\n")
    trace = tmp_path / "trace.csv"
    trace.write_text("Kernel_Name,Grid_Size_X,Grid_Size_Y,Workgroup_Size_X,Start_Timestamp,End_Timestamp\n"
                     "\"void tq::(anonymous namespace)::k_a<128>(int)\",512,1,256,0,1000\n"
                     "\"void tq::(anonymous namespace)::k_a<128>(int)\",512,1,256,5000,7000\n"
                     "k_b,64,2,128,9000,10000\n")
    _bench().trace_summary([str(stats), str(trace)])
    out = capsys.readouterr().out.splitlines()
    assert "| tq::k_a<128> | 2 | 1.50 | 1.00 | 2.00 | 75.0% |" in out
    assert "| k_b | 1 | 1.00 | 1.00 | 1.00 | 25.0% |" in out
    assert "| tq::k_a<128> | 512 | 1 | 256 | 2 | 1.50 | 1.00 | 2.00 |" in out
    assert "| k_b | 64 | 2 | 128 | 1 | 1.00 | 1.00 | 1.00 |" in out
