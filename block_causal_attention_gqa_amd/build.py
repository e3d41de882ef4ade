"""Build the C-ABI library ``libbc.so`` from the HIP sources in ``csrc/``.

    python -m block_causal_attention_gqa_amd.build

Compiles every ``csrc/*.hip`` for gfx950 with hipcc into an in-tree shared
library next to this file.  Packed-fp32 instructions are disabled on the
device side (``-packed-fp32-ops``); the host pass only warns about the flag.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbc.so")
ARCH = os.environ.get("BC_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def asan_runtime():
    """Path of the compiler's shared AddressSanitizer runtime, or None."""
    root = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root)) if os.path.isdir(root) else []:
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def build(verbose=False, asan=False, out=None):
    """Compile and link libbc.so (always rebuilds).  Returns the library path.

    asan=True instruments the host code only (argument validation, split
    plan, scheduler) with AddressSanitizer; the device code is built as
    usual.  Such a library is loaded with the runtime from asan_runtime()
    preloaded.  ``out`` overrides the output path."""
    lib = out or LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-result",
           "-I", os.path.join(HERE, "..", "include")]
    if asan:
        cmd += ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                "-shared-libasan"]
    cmd += [*sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if proc.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (proc.returncode, out))
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
