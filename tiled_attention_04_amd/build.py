"""Compile the HIP library libfa_mi355x.so in-tree for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = [os.path.join(HERE, "csrc", "fa_api.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms are disabled on purpose (see the kernel header)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False, out=None, extra=()):
    """Always recompiles; returns the path of the built library.  `out` and
    `extra` build a variant (the tests' LDS race-check library)."""
    out = out or LIB_PATH
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + list(extra) + SOURCES + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
