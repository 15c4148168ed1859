"""Builds libssm_scan.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Run as ``python -m selective_state_space_38_amd.build`` or call ``build()``.
Always recompiles.  Needs only hipcc (no GPU).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssm_scan.so")
# the roofline ceiling probes: a library of their own, not part of the scan's ABI
MICRO_LIB = os.path.join(HERE, "libssm_micro.so")
MICRO_SOURCE = "micro.hip"
# (source, object name, extra flags): the forward is compiled once per
# activation type so the two halves build in parallel
SOURCES = [
    ("api.hip", "api", []),
    ("scan_fwd.hip", "scan_fwd_f32", ["-DSSM_FWD_DTYPE=0"]),
    ("scan_fwd.hip", "scan_fwd_bf16", ["-DSSM_FWD_DTYPE=1"]),
    ("scan_bwd.hip", "scan_bwd", []),
    ("state_update.hip", "state_update", []),
    ("carry.hip", "carry", []),
    ("conv1d.hip", "conv1d", []),
    ("gemm.hip", "gemm", []),
]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed-FP32 instructions stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


# hipBLASLt runs the Mamba block's projection GEMMs
LINK_LIBS = ["-L/opt/rocm/lib", "-lhipblaslt"]


# The host-sanitized build: AddressSanitizer and UndefinedBehaviorSanitizer on
# the host code only (argument checks, planning, workspace arithmetic); the
# device code is compiled as in the product build.  Loaded with the ASan
# runtime preloaded, for the CPU tests of the argument checks.
SANITIZED_DIR = os.path.join(HERE, "_build", "asan")
SANITIZED_LIB = os.path.join(SANITIZED_DIR, "libssm_scan.so")
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _check(proc, verbose):
    out, _ = proc.communicate()
    msgs = "\n".join(line for line in out.splitlines() if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)


def build(verbose=False):
    """Compiles every source to an object in parallel, then links the
    shared library (replacing the old one only on success)."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs, procs = [], []
    for src, name, extra in SOURCES:
        obj = os.path.join(objdir, name + ".o")
        objs.append(obj)
        procs.append(_run([hipcc()] + compile_flags + extra +
                          ["-c", os.path.join(CSRC, src), "-o", obj], verbose))
    micro_tmp = MICRO_LIB + ".tmp"
    procs.append(_run([hipcc()] + HIPCC_FLAGS + [os.path.join(CSRC, MICRO_SOURCE), "-o",
                                                 micro_tmp], verbose))
    for proc in procs:
        _check(proc, verbose)
    tmp = LIB + ".tmp"
    _check(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs +
                ["-o", tmp] + LINK_LIBS, verbose), verbose)
    os.replace(tmp, LIB)
    os.replace(micro_tmp, MICRO_LIB)
    return LIB


def asan_runtime():
    """Path of the compiler's shared ASan runtime (to preload), or None."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin",
                         "clang")
    for cand in (clang, "/opt/rocm/lib/llvm/bin/clang"):
        if os.path.exists(cand):
            out = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 capture_output=True, text=True).stdout.strip()
            if os.path.isabs(out) and os.path.exists(out):
                return out
    return None


def build_host_sanitized(verbose=False):
    """Builds the host-sanitized library into SANITIZED_DIR unless it is newer
    than every source; returns its path."""
    include = os.path.join(os.path.dirname(HERE), "include")
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + \
        [os.path.join(include, f) for f in os.listdir(include)]
    if os.path.exists(SANITIZED_LIB) and \
            os.path.getmtime(SANITIZED_LIB) > max(os.path.getmtime(f) for f in srcs):
        return SANITIZED_LIB
    os.makedirs(SANITIZED_DIR, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"] + SANITIZE_HOST
    objs, procs = [], []
    for src, name, extra in SOURCES:
        obj = os.path.join(SANITIZED_DIR, name + ".o")
        objs.append(obj)
        procs.append(_run([hipcc()] + compile_flags + extra +
                          ["-c", os.path.join(CSRC, src), "-o", obj], verbose))
    for proc in procs:
        _check(proc, verbose)
    tmp = SANITIZED_LIB + ".tmp"
    _check(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + SANITIZE_HOST + objs +
                ["-o", tmp] + LINK_LIBS, verbose), verbose)
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
