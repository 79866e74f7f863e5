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


def build(verbose: bool = False, defines=None, out=None) -> str:
    """Compile every HIP source into ``libpagedprefill.so`` (always rebuilds).

    ``defines`` (``{"PREFILL_TILE_D128": "4,32,4,2,1"}``) and ``out`` build a
    variant of the library elsewhere, e.g. another tile shape for a sweep; the
    in-tree library is then left as it is.
    """
    out = out or library_path()
    tmp = out + ".tmp%d" % os.getpid()
    dflags = ["-D%s=%s" % (k, v) for k, v in (defines or {}).items()]
    cmd = [HIPCC] + FLAGS + dflags + SOURCES + ["-o", tmp]
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
    import argparse
    ap = argparse.ArgumentParser(description="build the HIP library (or a variant of it)")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="preprocessor define, e.g. PREFILL_TILE_D128=4,32,4,2,1")
    ap.add_argument("--out", default=None, help="output path (default: the in-tree library)")
    a = ap.parse_args()
    defs = dict(d.split("=", 1) for d in a.define)
    print(build(verbose=True, defines=defs, out=a.out))
