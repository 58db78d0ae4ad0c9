"""Build libsparse_attn.so (gfx950) in-tree with hipcc.

Every translation unit under csrc/ is compiled for --offload-arch=gfx950 and
linked into top_indexer_sparse_amd/libsparse_attn.so.  Packed-fp32 VALU
instructions are disabled for all device code.

`build.py --sanitize` builds libsparse_attn_san.so instead: the same sources
with AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
(argument validation, launchers); device code is built as usual.  It is for
CPU runs of the ABI tests with the clang ASan runtime preloaded.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsparse_attn.so")
OBJ_SAN = os.path.join(HERE, "_build_san")
LIB_SAN = os.path.join(HERE, "libsparse_attn_san.so")
# host-side sanitizers: each -fsanitize= applies to the host pass only
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer"]
SOURCES = ["api.cpp", "indexer.hip", "topk.hip", "mla.hip", "block_sparse.hip",
           "prefill.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall",
         "-Wno-unused-command-line-argument"]


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(OBJ_SAN if sanitize else OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    extra = SAN_FLAGS if sanitize else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # host pass: harmless unknown-feature note
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    obj_dir, lib = (OBJ_SAN, LIB_SAN) if sanitize else (OBJ, LIB)
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    link = ["-shared-libsan", *SAN_FLAGS] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, *objs, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
