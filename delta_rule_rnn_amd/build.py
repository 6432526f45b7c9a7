"""Build the gfx950 shared library (libdeltarule.so) in-tree with hipcc.

Each kernel family is its own translation unit (csrc/*.hip); they compile in
parallel to objects under _build/ and link into one shared library."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ("deltarule.hip", "k_intra.hip", "k_inter.hip", "k_seg.hip", "k_bwd.hip", "k_gradb.hip", "k_misc.hip",
           "k_noalloc.hip")
LIB = os.path.join(HERE, "libdeltarule.so")
OBJDIR = os.path.join(os.path.dirname(HERE), "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no packed fp32 VALU instructions in device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res.stderr


def _fresh(obj: str) -> bool:
    """True when obj and its dependency file exist and obj is newer than every
    file the dependency file lists."""
    dep = obj[:-2] + ".d"
    if not (os.path.exists(obj) and os.path.exists(dep)):
        return False
    t = os.path.getmtime(obj)
    text = open(dep).read().replace("\\\n", " ")
    files = text.split(":", 1)[1].split() if ":" in text else []
    return all(os.path.exists(f) and os.path.getmtime(f) <= t for f in files)


def build_library(out: str = LIB, extra=None, verbose: bool = False, jobs: int = 0,
                  incremental: bool = False) -> str:
    """Compile every translation unit (or, with incremental, only those whose
    object is older than a file it includes) and link the library."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, *(extra or []), "-MMD", "-MF", o[:-2] + ".d", "-c", "-o", o, os.path.join(CSRC, s)]
            for s, o in zip(srcs, objs) if not (incremental and not extra and _fresh(o))]
    jobs = jobs or max(1, min(len(cmds), 16, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        logs = list(ex.map(_run, cmds))
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp", *objs])
    if verbose:
        print("\n".join(logs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=False))
