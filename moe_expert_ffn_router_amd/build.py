"""Build libmoe.so in-tree with hipcc for gfx950.

    python moe_expert_ffn_router_amd/build.py      (or __graft_entry__.build())

Every call recompiles. Flags: one target (gfx950); packed-fp32 instructions
disabled; fp32 division and sqrt correctly rounded (the FP8 quantiser's
decisions depend on it); hidden visibility so that only the C ABI of
include/moe.h is exported.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe.so")
SOURCES = ["moe_api.hip", "moe_route.hip", "moe_align.hip", "moe_ffn.hip", "moe_gemm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *CFLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 1)) as ex:
        logs = list(ex.map(_run, cmds))
    tmp = OUT + ".tmp"
    logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, OUT)
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
