"""Build libbsa.so (all HIP kernels + the C-ABI layer) for gfx950, in-tree, and the
checked build libbsa_checked.so (-DBSA_CHECKED: kernels test the list indices they read).

Usage: python -m block_sparse_attention_mask_amd.build   (or call build() / build_all()).
"""
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["nabla.hip", "sta.hip", "mask_ops.hip", "attn.hip", "attn_bwd.hip", "reorder.hip", "api.cpp"]
LIB = os.path.join(PKG, "libbsa.so")
CHECKED_LIB = os.path.join(PKG, "libbsa_checked.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src, obj, checked=False):
    cmd = [HIPCC] + FLAGS + (["-DBSA_CHECKED"] if checked else []) + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                                     "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = True, variants=(False,)) -> str:
    """Compile and link the production library (variant False) and/or the checked one
    (True); all objects are compiled in one pool. Returns the last library built."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.time()
    jobs, libs = [], []
    for checked in variants:
        bdir = os.path.join(PKG, "_build_checked" if checked else "_build")
        os.makedirs(bdir, exist_ok=True)
        objs = [os.path.join(bdir, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
        jobs += [(s, o, checked) for s, o in zip(SOURCES, objs)]
        libs.append((objs, CHECKED_LIB if checked else LIB))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _compile(*j), jobs))
    for objs, lib in libs:
        _link(objs, lib)
        if verbose:
            print(f"built {lib} in {time.time() - t0:.1f}s", file=sys.stderr)
    return libs[-1][1]


def build_all(verbose: bool = True) -> str:
    return build(verbose, variants=(False, True))


if __name__ == "__main__":
    build_all() if "--all" in sys.argv else build()
