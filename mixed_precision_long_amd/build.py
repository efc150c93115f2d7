"""Builds libapa.so (every HIP source in csrc/) for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libapa.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # loadable by the HIP runtime PyTorch ships as well as by the system one
    "-mcode-object-version=5",
    "-ffp-contract=off",
    # never emit packed FP32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]

# Per-source extras.  Pass 1 issues the next tile's score MFMAs in the middle
# of the current tile so they overlap the vote and the P V product; machine
# sinking would move them to the loop latch (and force the K prefetch into
# temporaries plus copies that wait on the loads just issued).  Kernels whose
# registers exceed the 256 vector registers (one wave per SIMD, D >= 256) keep
# their MFMA accumulators in vector registers with the VGPR form of the MFMA
# instructions; otherwise the compiler takes the accumulation-register form
# for every MFMA and copies the accumulators to vector registers and back in
# every tile (hundreds of copies per tile; code up to D = 128 is unchanged).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {
    "pass1.hip": ["-mllvm", "-disable-machine-sink", *VGPR_FORM],
    "fused.hip": ["-mllvm", "-disable-machine-sink", *VGPR_FORM],
    "fa16.hip": VGPR_FORM,
    "big16.hip": VGPR_FORM,
}


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link one shared library (always recompiles)."""
    inc = ["-I", os.path.join(HERE, "..", "include")]
    tmpdir = tempfile.mkdtemp(prefix="apa_build_")
    try:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append(["hipcc", *FLAGS, *EXTRA.get(os.path.basename(src), []), *inc, "-c",
                         "-o", obj, src])
        with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp%d" % os.getpid()
        _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
