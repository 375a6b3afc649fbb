"""Build libkvarn.so (the C-ABI library of hand-written gfx950 HIP kernels).

hipcc, offload arch gfx950 only.  Packed-fp32 VALU instructions are disabled
(-target-feature -packed-fp32-ops): every fp32 operation in the kernels is a
plain per-lane instruction.  The library is built in-tree next to this file.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvarn.so")
# streaming reference kernels for bench.py only (not part of the library's ABI)
STREAM_SRC = "bench_stream.hip"
STREAM_LIB = os.path.join(HERE, "libkvarn_streamref.so")
SOURCES = ["kvarn_abi.cpp", "kvarn_quantize.hip", "kvarn_dequantize.hip", "kvarn_attention.hip",
           "kvarn_attention_fp16.hip", "kvarn_scratch.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-function",
]


# per-file code generation options: the attention kernel keeps its
# matrix-core results in ordinary VGPRs (no accumulator-register copies)
FILE_FLAGS = {"kvarn_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + FILE_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, "\n".join(msgs)))
    if verbose and msgs:
        print("\n".join(msgs))
    return out


def _link(objs, lib, verbose):
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + [STREAM_SRC]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:-1], LIB, verbose)
    _link(objs[-1:], STREAM_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
