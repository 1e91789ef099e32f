"""Build libcsa2.so (the gfx950 HIP kernels plus the C-ABI) in-tree with hipcc, and
libcsa2_debug.so, the same library with the device-side precondition checks on."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libcsa2.so")
DEBUG_LIB = os.path.join(HERE, "libcsa2_debug.so")
ROOF_LIB = os.path.join(HERE, "libcsa2_roofline.so")
SOURCES = ["quant_append.hip", "index.hip", "index_head.hip", "attend.hip", "csa2_abi.cpp"]
HEADERS = ["codec.hpp", "kernels.hpp", "block_ops.hpp", "dev_check.hpp", "quant_entry.hpp", "index_common.hpp"]
ARCH = "gfx950"


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(CSRC, h) for h in HEADERS] + [
        os.path.join(INCLUDE, "csa2.h")]


def build_roofline(verbose: bool = False) -> str:
    """libcsa2_roofline.so: the streaming-read ceiling kernel the benchmark
    reports the indexer scan against (a measurement helper, not the method)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}", "-I", INCLUDE, "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(CSRC, "stream_ceiling.hip"), "-o", ROOF_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(ROOF_LIB + ".tmp", ROOF_LIB)
    return ROOF_LIB


def build(verbose: bool = False, jobs: int = 4, debug: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    build_dir = os.path.join(HERE, "_build", "debug" if debug else "release")
    lib = DEBUG_LIB if debug else LIB
    os.makedirs(build_dir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-Wall",
              # keep the compiler from forming packed fp32 instructions
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              # IEEE fp32 division and sqrt (the quantisers divide by the scale)
              "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=fast"]
    if debug:
        # the checks on, and the internal namespace renamed, so that the two
        # libraries can be loaded into one process side by side
        common += ["-DCSA2_DEBUG", "-Dcsa2=csa2_debug"]
    objs = []
    procs = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(build_dir, s + ".o")
        lang = ["-x", "hip"] if s.endswith(".cpp") else []
        cmd = [hipcc] + common + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), s))
        objs.append(obj)
        if len(procs) >= jobs:
            p, name = procs.pop(0)
            if p.wait() != 0:
                raise RuntimeError(f"hipcc failed on {name}")
    for p, name in procs:
        if p.wait() != 0:
            raise RuntimeError(f"hipcc failed on {name}")
    link = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", lib + ".tmp"] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, debug=True)
    build_roofline(verbose=True)
    sys.exit(0)
