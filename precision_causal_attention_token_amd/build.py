"""Build libflamia.so (all HIP sources, gfx950) in place, next to this file.

`build(debug=True)` builds the test variant instead (FLAMIA_DEBUG_DUMP: the same kernels plus
copies of their intermediates into caller buffers, see include/flamia_debug.h) into
tests/_build/libflamia_debug.so; the product never loads it."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libflamia.so")
DEBUG_LIB = os.path.join(os.path.dirname(HERE), "tests", "_build", "libflamia_debug.so")
SOURCES = ["flamia_api.hip", "quantize.hip", "worklist.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_dqp.hip", "attn_small.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed FP32 instructions stay off (only scalar float code is generated)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    return out


def build(verbose=False, debug=False):
    """Each source compiled to an object in its own hipcc process (in parallel), then linked."""
    out_lib = DEBUG_LIB if debug else LIB
    os.makedirs(os.path.dirname(out_lib), exist_ok=True)
    tag = "%s.%d" % ("dbg" if debug else "rel", os.getpid())
    objdir = os.path.join(os.path.dirname(out_lib), "_obj")
    os.makedirs(objdir, exist_ok=True)
    defs = ["-DFLAMIA_DEBUG_DUMP"] if debug else []
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, "%s.%s.o" % (s, tag))
        jobs.append((obj, [HIPCC] + FLAGS + defs + ["-c", os.path.join(CSRC, s), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    objs = [o for o, _ in jobs]
    try:
        with ThreadPoolExecutor(workers) as ex:
            outs = list(ex.map(_run, [c for _, c in jobs]))
        tmp = out_lib + ".tmp%d" % os.getpid()
        outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]))
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
        if not os.listdir(objdir):
            os.rmdir(objdir)
    out = "\n".join(o for o in outs if o.strip())
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, out_lib)
    return out_lib


if __name__ == "__main__":
    print(build(verbose=True, debug="--debug" in sys.argv))
