"""Build libdg.so (HIP, gfx950) in-tree: `python -m block_denoising_step_amd.build`."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdg.so")
SOURCES = ["dg_host.cpp", "sampler.hip", "selfcond.hip", "attn.hip", "kvcache.hip", "inject.hip"]
# measurement kernels (achievable ceilings), a library of their own
PROBE_LIB = os.path.join(HERE, "libdg_probe.so")
PROBE_SOURCES = ["probe.hip"]

# Packed-fp32 instructions are kept out of every code object (the compiler would
# otherwise form v_pk_* from plain float code).
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source to an object, then link libdg.so and libdg_probe.so. Always
    recompiles."""
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *HIP_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if verbose and out.strip():
            print(out)
        if p.returncode != 0:
            failed.append((src, out))
    if failed:
        raise RuntimeError("libdg build failed:\n" + "\n".join(f"== {s}\n{o}" for s, o in failed))
    probe_objs = objs[len(SOURCES):]
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, probe_objs)):
        tmp = lib + ".tmp"
        link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{os.path.basename(lib)} link failed:\n" + r.stdout)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
