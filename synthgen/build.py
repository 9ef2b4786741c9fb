"""Build the synthetic-input generator library (host + gfx950 device code)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "csrc", "synth.hip")
    out = os.path.join(HERE, "libsynth.so")
    tmp = out + ".tmp"
    cmd = ["hipcc", "-O3", "--offload-arch=gfx950", "-shared", "-fPIC", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-ffp-contract=off", "-o", tmp, src, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("synth build failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(" ".join(cmd))
    return out


if __name__ == "__main__":
    print(build(verbose=True))
