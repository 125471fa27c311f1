"""Build libpwq.so (the HIP/C-ABI library) in-tree for gfx950.

    python -m post_weight_quantization_19_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpwq.so")
PROBE = os.path.join(HERE, "peak_probe")
SOURCES = ["pwq_api.hip", "hessian.hip", "cholesky.hip", "sweep.hip", "order.hip", "rate.hip",
           "ssqr.hip", "min_pivot.hip", "oaem.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source into libpwq.so; returns the library path."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-result", "-o", LIB + ".tmp"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """Compile the peak probe executable (a measurement aid next to the library)."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", PROBE + ".tmp", os.path.join(CSRC, "peak_probe.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (peak_probe):\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(PROBE + ".tmp", PROBE)
    return PROBE


if __name__ == "__main__":
    print(build(verbose=True))
