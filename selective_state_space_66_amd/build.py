"""Build the HIP library in-tree: hipcc for gfx950, one shared object.  Each
source is compiled to an object file of its own, several at a time, and the
objects are linked into the library.

    python -m selective_state_space_66_amd.build
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssm66_hip.so")
SOURCES = ["ssm_api.hip", "scan_fwd.hip", "scan_tpar.hip", "scan_wave8.hip", "scan_bwd.hip", "scan_bwd_wave.hip", "step.hip", "conv1d.hip", "ssd.hip",
           "probe.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    # packed fp32 (v_pk_fma_f32 and friends) stays off: ordinary fp32 VALU only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    return r.returncode, msgs


def build(verbose: bool = False, extra_flags=None) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [hipcc()] + HIPCC_FLAGS + list(extra_flags or [])
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [flags + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        results = list(pool.map(lambda c: _run(c, verbose), cmds))
    msgs = [m for _, ms in results for m in ms]
    if any(rc != 0 for rc, _ in results):
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed")
    rc, link_msgs = _run(flags + ["-shared"] + objs + ["-o", LIB + ".tmp"], verbose)
    msgs += link_msgs
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc link failed")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
