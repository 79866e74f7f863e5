"""Build step: compile the HIP sources into the in-tree C-ABI shared library.

``hipcc --offload-arch=gfx950`` cross-compiles without a GPU.  Packed-fp32
VALU forms are disabled for device code (``-packed-fp32-ops``); hipcc's host
pass warns that it does not know the feature, which is harmless.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libpagedprefill.so"
SOURCES = [os.path.join(HERE, "csrc", "prefill_attention.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
         "-I" + os.path.join(ROOT, "include"),
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def library_path() -> str:
    return os.path.join(HERE, LIB_NAME)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``libpagedprefill.so`` (always rebuilds)."""
    out = library_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, errs))
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
