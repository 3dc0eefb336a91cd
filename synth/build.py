"""Build libsynth.so (host + gfx950 device generator) with hipcc."""

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(root, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "csrc", "synth.hip")
    out = os.path.join(_HERE, "libsynth.so")
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           # host and device must round identically: no contraction into FMA
           "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wl,-rpath,/opt/rocm/lib", "-pthread", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
