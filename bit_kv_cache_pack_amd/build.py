"""Builds libkvq.so (HIP kernels + C ABI) for gfx950, in-tree, with hipcc.

    python -m bit_kv_cache_pack_amd.build [-v]

Every translation unit is compiled with -ffp-contract=off (the quantizer and the window
scores are bit-reproducible only without contraction; the attention kernels spell their
fused multiply-adds explicitly) and with packed fp32 instructions disabled. The attention
kernels and the quantizer are also compiled with -fno-honor-nans: their inputs are taken
to be finite, so a running minimum or maximum needs no NaN quieting of its operands
(which doubles its instruction count).
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["api.hip", "quant.hip", "attention.hip", "decode.hip", "windows.hip", "probe.hip"]
PER_SOURCE = {"attention.hip": ["-fno-honor-nans"], "decode.hip": ["-fno-honor-nans"], "quant.hip": ["-fno-honor-nans"]}
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags(extra=()):
    return list(extra) + ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool, obj_dir: str = OBJ_DIR, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags(list(extra) + PER_SOURCE.get(src, [])) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s%s" % (src, r.stdout, r.stderr))
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile and link; ``defines`` (NAME=VALUE strings) are passed as -D flags and compiled
    into an object folder of their own, so a variant does not overwrite the default objects."""
    extra = ["-D" + d for d in defines]
    obj_dir = OBJ_DIR if not defines else OBJ_DIR + "_" + "_".join(d.replace("=", "") for d in defines)
    os.makedirs(obj_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, obj_dir, extra), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
