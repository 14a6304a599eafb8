"""Build libretention.so (HIP, gfx950 only) in-tree.

    python -m retention_chunkwise_amd._build

compiles every source under csrc/ with hipcc for --offload-arch=gfx950 and
links them into retention_chunkwise_amd/libretention.so.  Packed fp32 vector
instructions are disabled for all device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libretention.so")
SOURCES = ["capi.hip", "walk.hip", "walk_ret_bf16.hip", "walk_ret_f32.hip", "walk_lin_bf16.hip",
           "walk_lin_f32.hip", "walk_norm_f32.hip", "rownorm.hip", "decode.hip", "seg_ret_bf16_c64.hip", "seg_ret_bf16_c128.hip",
           "seg_lin_bf16_c64.hip", "seg_lin_bf16_c128.hip", "seg_rev_bf16_c64.hip", "seg_rev_bf16_c128.hip",
           "seg_norm_bf16_c64.hip", "seg_norm_bf16_c128.hip", "gla.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libretention)")


def common_flags() -> list[str]:
    return ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="retbuild_") as tmp:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmds.append([cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj])

        def run(cmd):
            r = subprocess.run(cmd, capture_output=True, text=True)
            return cmd, r

        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for cmd, r in ex.map(run, cmds):
                # hipcc's host pass warns that it does not know the packed-fp32
                # feature flag; that line is expected and harmless.
                msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
                        if "not a recognized feature" not in ln]
                if verbose or r.returncode != 0:
                    sys.stderr.write("\n".join(msgs) + ("\n" if msgs else ""))
                if r.returncode != 0:
                    raise RuntimeError(f"hipcc failed: {' '.join(cmd)}")
        out_tmp = LIB + ".tmp"
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc link failed")
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
