"""Build libpwq.so (the HIP/C-ABI library) in-tree for gfx950.

    python -m post_weight_quantization_19_amd.build            the library
    python -m post_weight_quantization_19_amd.build --sanitized  also the
        host-sanitized copy (_build/san/libpwq_san.so) for the ABI tests
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


FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"]
OBJDIR = os.path.join(HERE, "_build")


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({what}):\n" + err)
    return err


def build(verbose: bool = False) -> str:
    """Compile every source (one object each, in parallel) and link
    libpwq.so; returns the library path."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def compile_one(i):
        return _run([hipcc(), *FLAGS, "-c", "-o", objs[i], os.path.join(CSRC, SOURCES[i])],
                    SOURCES[i])
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        errs = list(ex.map(compile_one, range(len(SOURCES))))
    errs.append(_run([hipcc(), *FLAGS, "-shared", "-o", LIB + ".tmp", *objs], "link"))
    err = "\n".join(e for e in errs if e.strip())
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    build_probe(verbose)
    return LIB


SAN_DIR = os.path.join(OBJDIR, "san")
SAN_LIB = os.path.join(SAN_DIR, "libpwq_san.so")
# Host code only: every sanitizer flag goes to the host pass (-Xarch_host
# before each), the device code is compiled as usual.
SAN_FLAGS = [x for opt in ["-fsanitize=" + k for k in ("address", "undefined")] +
             ["-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
             for x in ("-Xarch_host", opt)]


def build_host_sanitized(verbose: bool = False) -> str:
    """A second build of the library whose host code (argument validation,
    workspace carving, launch set-up) carries AddressSanitizer and
    UndefinedBehaviorSanitizer checks, for the CPU tests of the C ABI.  The
    sanitizer runtime is not linked in: a process loads the library with the
    runtime preloaded (LD_PRELOAD)."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(SAN_DIR, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN_FLAGS
    objs = [os.path.join(SAN_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def compile_one(i):
        return _run([hipcc(), *flags, "-c", "-o", objs[i], os.path.join(CSRC, SOURCES[i])],
                    SOURCES[i] + " (host sanitizers)")
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        errs = list(ex.map(compile_one, range(len(SOURCES))))
    errs.append(_run([hipcc(), *FLAGS, "-shared", "-o", SAN_LIB + ".tmp", *objs],
                     "link (host sanitizers)"))
    err = "\n".join(e for e in errs if e.strip())
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


def sanitizer_runtime():
    """The clang AddressSanitizer runtime of the ROCm toolchain (None if absent)."""
    import glob
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


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
    if "--sanitized" in sys.argv[1:]:
        print(build_host_sanitized(verbose=True))
