"""Build libfm.so (HIP, gfx950) in-tree with hipcc.

    python -m mask_aware_sparse_amd.build [--debug]

Produces mask_aware_sparse_amd/libfm.so from csrc/*.hip and csrc/*.cpp.  Cross-compiles
without a GPU.  Every call compiles (no staleness check)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-result",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def build(debug=False, out=OUT, extra=()):
    cmd = [HIPCC] + FLAGS + list(extra) + (["-g"] if debug else []) + sources() + ["-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfm.so")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv))
