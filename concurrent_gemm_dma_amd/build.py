"""Build libc3.so for gfx950: hipcc for the kernels, clang++ for host-only sources.

The library links against the HIP and ROCr runtimes that PyTorch itself loads (torch/lib), so a
process that uses torch for device memory and streams holds exactly one HIP runtime and one ROCr
runtime: torch's streams, allocations and agents are then the library's too.
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libc3.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions stay off (the compiler must not form v_pk_* fp32 ops)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__"]


def torch_lib_dir() -> str:
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("torch is not importable; its HIP runtime is what libc3 links against")
    d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
    for name in ("libamdhip64.so", "libhsa-runtime64.so"):
        if not os.path.exists(os.path.join(d, name)):
            raise RuntimeError(f"{name} not found in {d}")
    return d


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "unknown target feature" not in l and "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, save_temps: bool = False, defines=(), out: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile every source and link `out`. `defines` are extra -D flags for the HIP sources."""
    os.makedirs(build_dir, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    inc = [f"-I{INCLUDE}", f"-I{CSRC}", f"-I{ROCM}/include"]
    jobs = []
    objs = []
    for src in sources():
        path = os.path.join(CSRC, src)
        obj = os.path.join(build_dir, src + ".o")
        objs.append(obj)
        if src.endswith(".hip"):
            cmd = [hipcc] + HIP_FLAGS + [f"-D{d}" for d in defines] + inc + ["-c", path, "-o", obj]
            if save_temps:
                cmd += ["-save-temps=obj"]
        else:
            cmd = [clangxx] + HOST_FLAGS + inc + ["-c", path, "-o", obj]
        jobs.append(cmd)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tlib = torch_lib_dir()
    tmp = out + ".tmp"
    link = [clangxx, "-shared", "-o", tmp] + objs + [
        f"-L{tlib}", "-l:libamdhip64.so", "-l:libhsa-runtime64.so", f"-Wl,-rpath,{tlib}",
        "-Wl,--no-undefined", "-lpthread",
    ]
    _run(link, verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv))
