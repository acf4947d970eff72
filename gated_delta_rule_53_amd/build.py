"""Build libkda.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_chunk.hip", "kda_backward.hip", "dplr_chunk.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled: plain float code only.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-ffp-contract=fast", "-munsafe-fp-atomics"]


# Host-only sanitizers for the entry points' validation and planning code (device
# code is compiled as usual): every -fsanitize= goes right after -Xarch_host.
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-shared-libasan"]
SAN_LIB = os.path.join(HERE, "_build_san", "libkda_san.so")


def build(verbose: bool = False, jobs: int = 4, sanitize_host: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libkda.so; returns its path.  With
    sanitize_host, kda_api.hip's host code is built with AddressSanitizer and
    UndefinedBehaviorSanitizer into _build_san/libkda_san.so instead (the process that
    loads it must preload clang's ASan runtime)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build_san" if sanitize_host else "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        san = SAN_HOST_FLAGS if sanitize_host and src == "kda_api.hip" else []
        cmd = [hipcc, *HIPCC_FLAGS, *san, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{text}")
        if verbose and text.strip():
            print(text)
    target = SAN_LIB if sanitize_host else LIB
    tmp = target + f".tmp{os.getpid()}"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SAN_HOST_FLAGS if sanitize_host else []), "-o",
           tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize_host="--sanitize-host" in sys.argv))
