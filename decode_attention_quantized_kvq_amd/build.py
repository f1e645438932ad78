"""Builds libkvq.so (host code + gfx950 kernels) in this package's directory.

Usage: python -m decode_attention_quantized_kvq_amd.build [--phase-stamps]
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvq.so")
SOURCES = ["kvq_host.cpp", "kvq_append.hip", "kvq_decode.hip", "kvq_decode_w4.hip",
           "kvq_decode_mixed.hip", "kvq_decode_w2.hip", "kvq_dequant.hip"]
OBJDIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no AGPR round trips when the softmax
    # rescales them
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-function",
]


def _run(cmds, verbose):
    """Runs the commands in parallel; raises with their messages on failure."""
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
    failed, msgs = False, []
    for p in procs:
        text = p.communicate()[0].strip()
        # the host pass does not know the device target feature; that is expected
        msgs += [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        failed |= p.returncode != 0
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compiles every source (in parallel) and links libkvq.so (or `out`);
    returns its path.  defines: extra -D macros for variant builds."""
    objdir = os.path.join(OBJDIR, os.path.basename(out))
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
    _run([[HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)],
         verbose)
    tmp = out + ".tmp"
    _run([[HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]], verbose)
    os.replace(tmp, out)
    return out


# An instrumented build, libkvq_phases.so: every decode workgroup stamps the
# real-time counter at each phase into the workspace (bench.py --phases).
PHASES_LIB = os.path.join(PKG, "libkvq_phases.so")


if __name__ == "__main__":
    if "--phase-stamps" in sys.argv:
        print(build(verbose="-q" not in sys.argv, out=PHASES_LIB, defines=["KVQ_PHASE_STAMPS"]))
    else:
        print(build(verbose="-q" not in sys.argv))
