"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU needed).

* The C-ABI library's host code (argument checks, workspace carving, launch set-up) built with
  both sanitizers, driven by the whole C-ABI test module (every entry point's rejections).
* The oracle's C code built with both sanitizers, driven by its projection, rasterization,
  backward and error-model tests.
Each runs in a child process with the sanitizer runtime preloaded; any report aborts it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def run_child(code, env_extra, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=timeout,
                       cwd=ROOT)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    return out


def test_library_host_code_under_sanitizers(tmp_path):
    from differentiable_raster_amd import build
    lib = build.build_sanitized(str(tmp_path / "san"))
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {TESTS!r}]\n"
            "import differentiable_raster_amd.gsmi as g\n"
            f"g.load({lib!r})\n"
            "import pytest\n"
            f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', {os.path.join(TESTS, 'test_abi.py')!r}]))\n")
    out = run_child(code, {"LD_PRELOAD": build.asan_runtime()})
    assert " passed" in out


def test_oracle_under_sanitizers(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "osan"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc has no shared ASan runtime")
    files = [os.path.join(TESTS, f) for f in ("test_oracle_project.py", "test_oracle_raster.py",
                                              "test_oracle_backward.py", "test_oracle_error_model.py",
                                              "test_oracle_project_backward.py")]
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {TESTS!r}]\n"
            "import pytest\n"
            f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu and not slow', *{files!r}]))\n")
    out = run_child(code, {"LD_PRELOAD": asan, "GS_ORACLE_LIB": lib, "OMP_NUM_THREADS": "4"})
    assert " passed" in out
