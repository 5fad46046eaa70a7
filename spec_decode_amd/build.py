"""Build libkda.so (gfx950) in-tree with hipcc.

Every HIP source under csrc/ is compiled for gfx950 only, with packed-FP32
instruction selection disabled, into an object of its own (in parallel, under
spec_decode_amd/_build/), and the objects are linked into
spec_decode_amd/libkda.so.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["abi.hip", "plan.hip", "decay.hip", "commit.hip", "fused.hip", "fused_conv.hip",
           "fused_conv_packed.hip", "fused_conv_window_major.hip", "gate_proj.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result", "-Wno-unused-variable",
]


def _filtered(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines()
                     if "target feature" not in l and "not a recognized feature" not in l
                     and l.strip())


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = _filtered(res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err:
        print(err, file=sys.stderr)


# Measurement variants: built on request only, each into a directory of its own
# (load one with KDA_LIBRARY=<path> to time it in place of the product library).
VARIANTS = {
    # the verify kernel's row dots on plain FP32 FMAs instead of MFMA
    "valu_dots": ["-DKDA_VALU_DOTS=1"],
    # the streaming FP32 commit's fold on plain FP32 FMAs instead of MFMA
    "valu_fold": ["-DKDA_VALU_FOLD=1"],
}


def build(verbose: bool = False, extra=(), variant: str = "") -> str:
    obj_dir, lib = OBJ, LIB
    if variant:
        extra = (*extra, *VARIANTS[variant])
        obj_dir = os.path.join(OBJ, variant)
        lib = os.path.join(HERE, "_variants", variant, "libkda.so")
        os.makedirs(os.path.dirname(lib), exist_ok=True)
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, *extra, "-c", "-o", o, os.path.join(CSRC, s)]
            for s, o in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    var = next((a.split("=", 1)[1] for a in sys.argv[1:] if a.startswith("--variant=")), "")
    print(build(verbose="-v" in sys.argv, variant=var))
