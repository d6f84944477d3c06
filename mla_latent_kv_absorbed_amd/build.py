"""Build the MLA library: mla_latent_kv_absorbed_amd/lib/libmla.so (gfx950).

Plain hipcc, one shared library, no torch involved.  Packed-fp32 VALU
instructions are disabled for every HIP source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "decode.hip", "decode_fp8.hip", "kernels.hip", "prefill.hip", "probe.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def lib_path() -> str:
    return os.path.join(HERE, "lib", "libmla.so")


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(HERE, "lib"), exist_ok=True)
    out = lib_path()
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *[os.path.join(HERE, "csrc", s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
