"""Build libgdn.so in-tree with hipcc for gfx950.

    python -m gated_delta_rule_79_amd.build [-v] [-j N] [-i] [--sanitize]

Every HIP source under csrc/ is compiled to an object under _build/ and the
objects are linked into gated_delta_rule_79_amd/libgdn.so (written to a
temporary name first, then renamed, so a half-built library is never seen).

--sanitize builds a second library, _build/asan/libgdn_asan.so, whose host
code (argument validation, workspace sizing, dispatch) carries
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is the
same.  tests/test_abi_sanitized.py runs the C-ABI tests against it on the
CPU.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libgdn_asan.so")
# sanitizers on the host side only (each flag behind -Xarch_host)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]

SOURCES = ["gdn_api.hip", "gdn_decode.hip", "gdn_fwd.hip", "gdn_bwd.hip", "gdn_tree.hip",
           "gdn_prologue.hip"]
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix accumulators in ordinary VGPRs: the kernels scale and convert
    # them between products, which AGPR accumulators turn into copies
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _stale(src: str, obj: str) -> bool:
    """An object is stale when it is missing or older than its source or any
    header under csrc/ or include/."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, src)]
    for d in (CSRC, INCLUDE):
        deps += [os.path.join(d, f) for f in os.listdir(d) if f.endswith((".h", ".hpp"))]
    return any(os.path.getmtime(x) > t for x in deps)


def _compile(src: str, verbose: bool, incremental: bool = False, sanitize: bool = False) -> str:
    obj = os.path.join(ASAN_DIR if sanitize else BUILD, os.path.splitext(src)[0] + ".o")
    if incremental and not _stale(src, obj):
        return obj
    cmd = [_hipcc(), *CFLAGS, *(SAN if sanitize else []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None,
          incremental: bool = False, sanitize: bool = False) -> str:
    """Compile every source (incremental: only those whose object is stale)
    and link the library (sanitize: the host-sanitized variant)."""
    os.makedirs(ASAN_DIR if sanitize else BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, incremental, sanitize), SOURCES))
    lib = ASAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs,
           *(["-fsanitize=address,undefined", "-shared-libsan"] if sanitize else []),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    ap.add_argument("-i", "--incremental", action="store_true",
                    help="recompile only sources whose object is stale")
    ap.add_argument("--sanitize", action="store_true",
                    help="build the host-sanitized variant _build/asan/libgdn_asan.so")
    a = ap.parse_args()
    print(build(a.verbose, a.jobs, a.incremental, a.sanitize))


if __name__ == "__main__":
    main()
