"""Build ``libqrita.so`` for gfx950 with hipcc (in-tree, next to this file).

The kernels live in separate translation units (the streaming pass and the
two tail tiers) that compile in parallel; the host API links them.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqrita.so")
OBJDIR = os.path.join(HERE, "_build")
UNITS = ["qrita.hip", "pass1.hip", "tail_light.hip", "tail_heavy.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res


def build(verbose: bool = False) -> str:
    sys.path.insert(0, CSRC)
    try:
        import gen_delta_lut  # noqa: WPS433
        gen_delta_lut.main()
    finally:
        sys.path.pop(0)
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(OBJDIR, u.replace(".hip", ".o")) for u in UNITS]
    cmds = [[HIPCC, *FLAGS, *inc, "-c", "-o", o, os.path.join(CSRC, u)] for u, o in zip(UNITS, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
