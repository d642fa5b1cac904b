"""Build the HIP library libattn.so in-tree with hipcc for gfx950.

Usage: python -m io_aware_exact_06_amd.build   (or __graft_entry__.build()).
Every HIP source is compiled with packed-fp32 instructions disabled; the
objects are linked into one shared library next to this file.  The
instruction-rate probe (csrc/rate_probe.hip) becomes the executable
rate_probe beside it, the dQ atomic-add probe (csrc/atomic_probe.hip) the
executable atomic_probe, and the MFMA/vector co-issue probe
(csrc/issue_probe.hip) the executable issue_probe.  libattn_cstep.so is the
same library with the hand-scheduled loops compiled out, for the tests that
compare the two bitwise.  Before compiling, the
generators csrc/gen_fwd_loop.py, csrc/gen_dq_loop.py and csrc/gen_dkdv_loop.py
rewrite csrc/attn_fwd_loop.inc, csrc/attn_dq_loop.inc and csrc/attn_dkdv_loop.inc
(the hand-scheduled loops of the three kernels) if their output changed.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn.so")
# The same library with the hand-scheduled loops compiled out (every tile through
# the C++ steps): the GPU tests compare the two bitwise.
CSTEP_LIB = os.path.join(HERE, "libattn_cstep.so")
CSTEP_DEFS = ["-DATTN_FWD_ASM=0", "-DATTN_DQ_ASM=0", "-DATTN_DKDV_ASM=0"]
CSTEP_SOURCES = ["attn_fwd.hip", "attn_bwd.hip"]
PROBE = os.path.join(HERE, "rate_probe")  # instruction-rate microbenchmark (an executable)
ATOMIC_PROBE = os.path.join(HERE, "atomic_probe")  # dQ atomic-add rate microbenchmark (an executable)
ISSUE_PROBE = os.path.join(HERE, "issue_probe")  # MFMA / vector co-issue microbenchmark (an executable)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_unfused.hip", "attn_noalloc.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I" + INCLUDE, "-I" + CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]


def _compile(src: str, defs: tuple = (), tag: str = "") -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + tag + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _build_probe(src: str = "rate_probe.hip", out: str = None) -> None:
    out = out or PROBE
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *COMMON, "-x", "hip", os.path.join(CSRC, src), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    os.replace(tmp, out)


def generate() -> None:
    """Regenerate the inline-assembly includes of the forward, dQ and dK/dV kernels."""
    sys.path.insert(0, CSRC)
    try:
        import gen_dkdv_loop
        import gen_dq_loop
        import gen_fwd_loop
    finally:
        sys.path.pop(0)
    gen_fwd_loop.main(os.path.join(CSRC, "attn_fwd_loop.inc"))
    gen_dkdv_loop.main(os.path.join(CSRC, "attn_dkdv_loop.inc"))
    gen_dq_loop.main(os.path.join(CSRC, "attn_dq_loop.inc"))


def _link(objs: list, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    generate()
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + len(CSTEP_SOURCES) + 3) as ex:
        probes = [ex.submit(_build_probe), ex.submit(_build_probe, "atomic_probe.hip", ATOMIC_PROBE),
                  ex.submit(_build_probe, "issue_probe.hip", ISSUE_PROBE)]
        cstep = [ex.submit(_compile, src, tuple(CSTEP_DEFS), ".cstep") for src in CSTEP_SOURCES]
        objs = list(ex.map(_compile, SOURCES))
        cobjs = {src: f.result() for src, f in zip(CSTEP_SOURCES, cstep)}
        for p in probes:
            p.result()
    _link(objs, LIB)
    _link([cobjs.get(src, obj) for src, obj in zip(SOURCES, objs)], CSTEP_LIB)
    if verbose:
        print("built", LIB, "and", CSTEP_LIB)
    return LIB


if __name__ == "__main__":
    build()
