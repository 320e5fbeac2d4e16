"""Build libkvs.so (all HIP sources under csrc/) for gfx950 with hipcc, in-tree.

Usage: python prompt_token_importance_amd/build.py   (or call build()).  Run
it as a file: importing the package loads libkvs.so, which may be missing or
older than the sources.  Each source compiles to an object of its own, in
parallel, under prompt_token_importance_amd/_build/; one hipcc call links them.
"""
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkvs.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("KVS_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # Never emit packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax work reads them directly, no
    # v_accvgpr_read copies.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _filter(text):
    return [l for l in text.splitlines() if "packed-fp32-ops" not in l]


def build(verbose: bool = False) -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    procs = []
    for src in sources():
        obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o")
        cmd = [hipcc, *FLAGS, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    failed = False
    for obj, p in procs:
        out, _ = p.communicate()
        lines = _filter(out)
        if p.returncode != 0:
            failed = True
            sys.stderr.write("\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in procs], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write("\n".join(_filter(res.stdout + res.stderr)) + "\n")
        raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
