"""Build libflint_moe.so (all HIP sources of csrc/) for gfx950 with hipcc, in-tree.

``python -m int4_expert_ffn_amd.build --phase-ts`` builds the profiling
variant libflint_moe_phase.so instead: the decode kernel then records the wall
clock at each phase of the layers of a call (flint_moe_debug_phase_ts), read by
``bench.py --phase-table``.

``--asan`` builds libflint_moe_asan.so: the same library with AddressSanitizer
on its host code only (the runtime's argument checks, allocation, failure and
release paths); device code is built as usual.  It needs the sanitizer runtime
preloaded (``asan_runtime()``); ``tests/test_abi_asan.py`` runs the C ABI's
host paths through it.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libflint_moe.so")
LIB_PHASE = os.path.join(HERE, "libflint_moe_phase.so")
LIB_ASAN = os.path.join(HERE, "libflint_moe_asan.so")
ARCH = "gfx950"


def asan_runtime() -> str:
    """Path of the host AddressSanitizer runtime of the ROCm compiler (to preload)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build(verbose: bool = False, phase_ts: bool = False, asan: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    lib = LIB_PHASE if phase_ts else LIB_ASAN if asan else LIB
    tmp = lib + ".tmp"
    extra = ["-DFLINT_PHASE_TS"] if phase_ts else []
    if asan:   # host code only: each sanitizer flag right after -Xarch_host
        extra += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-shared-libsan"]
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(HERE, "..", "include"), "-o", tmp] + extra + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if verbose and msg:
        print(msg)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, phase_ts="--phase-ts" in sys.argv[1:], asan="--asan" in sys.argv[1:]))
