"""Build synth/libmla_synth.so, the GPU twin of the seeded input generator."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "libmla_synth.so")
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, os.path.join(HERE, "gpu_gen.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT if not verbose else None)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
