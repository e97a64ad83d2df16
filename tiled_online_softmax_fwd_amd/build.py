"""Build libattn.so (the HIP kernels + C ABI) in-tree for gfx950.

Every source in csrc/ is compiled to an object with hipcc in parallel, then
linked into tiled_online_softmax_fwd_amd/libattn.so.  Packed-fp32 VALU
instructions are disabled for all device code.

The same sources are also built with ATTN_LDS_POISON into
libattn_poison.so, a debug library whose LDS copies first fill their
destination with NaN (a read that is not ordered after a copy's completion
then sees NaN); tests/test_gpu_lds_poison.py runs it beside libattn.so.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
LIB_POISON = os.path.join(HERE, "libattn_poison.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
SOURCES = ["attn_api.cpp", "naive.hip", "decode.hip", "bwd.hip", "fwd_inst_bf16.hip", "fwd_inst_f16.hip", "fwd_inst_f32.hip", "fwd_inst_sparse.hip", "probe.hip"]

# (output library, object directory, extra flags)
VARIANTS = {"": (LIB, OBJ_DIR, []),
            "poison": (LIB_POISON, OBJ_DIR + "_poison", ["-DATTN_LDS_POISON"])}


def _compile(src: str, variant: str, verbose: bool) -> str:
    _, obj_dir, extra = VARIANTS[variant]
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} ({variant or 'release'}):\n{r.stderr}")
    return obj


def _link(variant: str, objs, verbose: bool) -> str:
    lib = VARIANTS[variant][0]
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + list(objs)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({variant or 'release'}):\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, jobs: int = 0, variants=("", "poison")) -> str:
    """Compile and link every variant; returns the path of libattn.so."""
    for v in variants:
        os.makedirs(VARIANTS[v][1], exist_ok=True)
    work = [(s, v) for v in variants for s in SOURCES]
    jobs = jobs or min(len(work), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda sv: _compile(sv[0], sv[1], verbose), work))
    for v in variants:
        _link(v, [o for o, (_, vv) in zip(objs, work) if vv == v], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, variants=("",) if "--release-only" in sys.argv else ("", "poison")))
