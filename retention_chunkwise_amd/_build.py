"""Build libretention.so (HIP, gfx950 only) in-tree.

    python -m retention_chunkwise_amd._build [-v] [--incremental] [--sanitize-host]

compiles every source under csrc/ with hipcc for --offload-arch=gfx950 and
links them into retention_chunkwise_amd/libretention.so.  Packed fp32 vector
instructions are disabled for all device code (-packed-fp32-ops).
--incremental keeps the objects and hipcc's dependency files under _build/ at
the repository root and recompiles only the sources whose object is older than
the source or any header it includes.  --sanitize-host builds a separate copy,
_build/asan/libretention.so, whose host code (argument validation, planning,
launch set-up) runs under AddressSanitizer and UndefinedBehaviorSanitizer; the
device code is compiled exactly as in the normal build.  Loading it needs the
clang ASan runtime preloaded (asan_runtime() names it); the CPU tests do that.
--debug builds retention_chunkwise_amd/libretention_debug.so with -DRET_DEBUG:
the LDS hazard self-check, where the segment walks, the state kernel, the fused
backward walk and the gated walk overwrite every LDS buffer that has gone dead
with NaN words until it is refilled.  Its outputs must equal the normal
build's bit for bit; a GPU test compares them.
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
DEBUG_LIB = os.path.join(HERE, "libretention_debug.so")
SOURCES = ["capi.hip", "walk.hip", "walk_ret_bf16.hip", "walk_ret_f32.hip", "walk_lin_bf16.hip",
           "walk_lin_f32.hip", "walk_norm_f32.hip", "rownorm.hip", "decode.hip", "seg_ret_bf16_c64.hip", "seg_ret_bf16_c128.hip",
           "seg_lin_bf16_c64.hip", "seg_lin_bf16_c128.hip", "seg_norm_bf16_c64.hip", "seg_norm_bf16_c128.hip", "seg_bwd_bf16.hip", "gla.hip"]
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


# host-only sanitizers: each -fsanitize= applies to the host pass alone
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(os.path.dirname(HERE), "_build", "asan", "libretention.so")


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime the sanitized build links to."""
    out = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


OBJ_CACHE = os.path.join(os.path.dirname(HERE), "_build")


def _stale(obj: str, src: str) -> bool:
    """True when obj is missing or older than src or a file its depfile lists."""
    dep = obj[:-2] + ".d"
    if not (os.path.exists(obj) and os.path.exists(dep)):
        return True
    t = os.path.getmtime(obj)
    text = open(dep).read().replace("\\\n", " ")
    files = text.split(":", 1)[1].split() if ":" in text else [src]
    return any(not os.path.exists(f) or os.path.getmtime(f) > t for f in files + [src])


def build(verbose: bool = False, incremental: bool = False, sanitize_host: bool = False, debug: bool = False) -> str:
    cc = hipcc()
    extra = SANITIZE_HOST if sanitize_host else (["-DRET_DEBUG"] if debug else [])
    lib = SANITIZED_LIB if sanitize_host else (DEBUG_LIB if debug else LIB)
    if sanitize_host:
        incremental = True
    with tempfile.TemporaryDirectory(prefix="retbuild_") as tmp:
        if sanitize_host:
            odir = os.path.dirname(SANITIZED_LIB)
        elif incremental:
            odir = os.path.join(OBJ_CACHE, "debug") if debug else OBJ_CACHE
        else:
            odir = tmp
        os.makedirs(odir, exist_ok=True)
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(odir, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            path = os.path.join(CSRC, src)
            if incremental and not _stale(obj, path):
                continue
            cmds.append([cc, *common_flags(), *extra, "-MD", "-MF", obj[:-2] + ".d", "-c", path, "-o", obj])

        def run(cmd):
            r = subprocess.run(cmd, capture_output=True, text=True)
            return cmd, r

        with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, len(cmds))) as ex:
            for cmd, r in ex.map(run, cmds):
                # hipcc's host pass warns that it does not know the packed-fp32
                # feature flag; that line is expected and harmless.
                msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
                        if "not a recognized feature" not in ln]
                if verbose or r.returncode != 0:
                    sys.stderr.write("\n".join(msgs) + ("\n" if msgs else ""))
                if r.returncode != 0:
                    raise RuntimeError(f"hipcc failed: {' '.join(cmd)}")
        out_tmp = lib + ".tmp"
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra,
                *(["-Xarch_host", "-shared-libasan"] if sanitize_host else []), "-o", out_tmp, *objs]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc link failed")
        os.replace(out_tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv,
                sanitize_host="--sanitize-host" in sys.argv, debug="--debug" in sys.argv))
