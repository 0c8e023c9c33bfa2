"""Build libdflash.so in-tree with hipcc for gfx950."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdflash.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src, device in (("host.cpp", False), ("api.cpp", False), ("kernels.hip", True), ("tree.hip", True),
                        ("sample.hip", True)):
        obj = os.path.join(objdir, src + ".o")
        cmd = [hipcc] + (HIP_FLAGS if device else ["-O2", "-std=c++17", "-fPIC", "-Wall"])
        cmd += ["-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    # a kernel whose host stub was not emitted would only fail at load time
    undef = subprocess.run(["nm", "-u", tmp], capture_output=True, text=True).stdout
    missing = [l.split()[-1] for l in undef.splitlines() if "dflash" in l]
    if missing:
        raise RuntimeError(f"libdflash.so has undefined library symbols: {missing[:4]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
