"""bench.py's refusals that need no GPU: more than one GPU, the fp32 tiny
layer (a parity-test size, not a timed layer), and the library-GEMM
comparison on the layer given by its Hessian (no X).  Each exits with
status 2 and a message before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          cwd=ROOT, capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_tiny_fp32_layer_is_not_a_bench_line():
    r = _bench("--config", "1")
    assert r.returncode == 2
    assert "parity-test size" in r.stderr
    assert r.stdout.strip() == ""


def test_library_gemm_needs_activations():
    r = _bench("--config", "5", "--library-gemm")
    assert r.returncode == 2
    assert "has no bf16 X" in r.stderr
    assert r.stdout.strip() == ""
