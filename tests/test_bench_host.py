"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal and the rule that the
measured HBM traffic of the rasterizer is reported only for the source it was measured on."""
import importlib.util
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def test_committed_traffic_summary_matches_the_current_rasterizer():
    """The committed counter summary was taken on this very raster.hip, so the bench reports its
    bytes (a summary of another source would be refused)."""
    b = load_bench()
    t = b.measured_traffic()
    assert t is not None and t > 1e8


def test_traffic_of_another_source_is_not_reported(tmp_path):
    b = load_bench()
    src = tmp_path / "raster.hip"
    shutil.copy(b.RASTER_SRC, src)
    with open(src, "a") as f:
        f.write("\n// another source\n")
    b.RASTER_SRC = str(src)
    assert b.measured_traffic() is None
    # and a summary without the bytes line is ignored
    summ = tmp_path / "traffic.md"
    lines = [l for l in open(b.TRAFFIC_FILE) if not l.startswith("- hbm bytes per launch")]
    summ.write_text("".join(lines))
    b.RASTER_SRC = os.path.join(ROOT, "differentiable_raster_amd", "csrc", "raster.hip")
    b.TRAFFIC_FILE = str(summ)
    assert b.measured_traffic() is None


def test_alu_peak_is_the_published_float32_vector_rate():
    b = load_bench()
    assert abs(b.ALU_PEAK_TFLOPS - 157.3) < 0.1
