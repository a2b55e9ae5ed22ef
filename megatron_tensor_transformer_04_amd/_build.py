"""Compile the HIP library libtpmlp.so for gfx950, in-tree, with hipcc.

The sources (csrc/ and include/) are first copied to a snapshot directory
under _build/, so that edits made while a build runs cannot reach a compiler
half way through (hipcc reads the sources once for the device pass and again
for the host pass). Each source is compiled to an object in parallel (the MLP
shard's launch sequences are split by storage type for that), then the
objects are linked into one shared library (MLP shard and attention shard
entry points).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtpmlp.so")
SOURCES = [os.path.join(CSRC, n) for n in ("mlp_bf16.hip", "mlp_f16.hip", "tp_attn.hip", "tp_attn_flash.hip", "mlp_f32.hip", "tp_mlp.hip")]
OBJDIR = os.path.join(PKG, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed-fp32 VALU forms stay off: scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")


def build(out: str = LIB, extra_flags=(), verbose: bool = False) -> str:
    """Compile SOURCES into `out` (atomically replaced) and return its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    snap = os.path.join(OBJDIR, "src")
    shutil.rmtree(snap, ignore_errors=True)
    shutil.copytree(CSRC, os.path.join(snap, "csrc"))
    shutil.copytree(INCLUDE, os.path.join(snap, "include"))
    s_csrc, s_inc = os.path.join(snap, "csrc"), os.path.join(snap, "include")
    objs = [os.path.join(OBJDIR, os.path.splitext(os.path.basename(s))[0] + ".o") for s in SOURCES]
    cmds = [[cc, *HIPCC_FLAGS, *extra_flags, "-I", s_inc, "-I", s_csrc, "-c",
             os.path.join(s_csrc, os.path.basename(src)), "-o", obj]
            for src, obj in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = out + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
