"""Kernel resources of the built library, read from its own gfx950 code
objects on the CPU: no kernel may use scratch memory except the backward
gradient kernel, whose register spills are known and bounded.

Scratch use without spills means a private array or a real call inside a
kernel (a staging lambda the compiler stopped inlining once put the
convolution prep's K, V and q pieces in scratch and doubled its time); this
catches that at build time.  The library is this repository's own build:
its .hip_fatbin section holds one clang offload bundle per source file, and
llvm-readelf prints each code object's kernel metadata."""

import os
import re
import shutil
import struct
import subprocess

import pytest

from gated_delta_rule_79_amd import _lib

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
# bytes of scratch per lane the gradient kernel's spills may take (measured:
# 12, 116 and 452 for gate none, scalar, per-channel)
GRAD_SCRATCH_MAX = 512


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


def _kernel_scratch(lib_path, tmp_path):
    """{kernel symbol: private segment bytes per lane} over every gfx950
    code object of the library."""
    objcopy, readelf = _tool("llvm-objcopy"), _tool("llvm-readelf")
    if objcopy is None or readelf is None:
        pytest.skip("llvm-objcopy / llvm-readelf not found")
    fat = tmp_path / "fat.bin"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", lib_path,
                    str(tmp_path / "stripped.so")], check=True, capture_output=True)
    blob = fat.read_bytes()
    out = {}
    n = 0
    for m in re.finditer(re.escape(MAGIC), blob):
        # bundle header: magic, entry count, then (offset, size, triple
        # length, triple) per entry, offsets from the bundle start
        p = m.start()
        (count,) = struct.unpack_from("<Q", blob, p + len(MAGIC))
        q = p + len(MAGIC) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", blob, q)
            q += 24
            triple = blob[q:q + tlen].decode()
            q += tlen
            if not triple.endswith("gfx950"):
                continue
            co = tmp_path / f"co{n}.o"
            n += 1
            co.write_bytes(blob[p + off:p + off + size])
            notes = subprocess.run([readelf, "--notes", str(co)], check=True,
                                   capture_output=True, text=True).stdout
            # a kernel's map lists .args (whose entries have .name too), then
            # its own .name, then .private_segment_fixed_size
            name = None
            for line in notes.splitlines():
                mn = re.match(r"\s*(?:- )?\.name:\s+(\S+)", line)
                if mn:
                    name = mn.group(1)
                mp = re.match(r"\s*\.private_segment_fixed_size:\s+(\d+)", line)
                if mp:
                    out[name] = int(mp.group(1))
    return out


def test_no_kernel_uses_scratch_but_the_gradient_spills(tmp_path):
    path = _lib.LIB_PATH
    if not os.path.exists(path):
        pytest.skip("libgdn.so not built")
    scratch = _kernel_scratch(path, tmp_path)
    # every kernel family of the library is there
    for fam in ("fwd_prep_sg_kernel", "fwd_prep_kernel", "fwd_trans_kernel",
                "fwd_combine_kernel", "fwd_scan_kernel", "bwd_grad_kernel",
                "bwd_scan_lds_kernel", "decode_kernel", "tree_commit_kernel",
                "prologue_kernel"):
        assert any(fam in k for k in scratch), fam
    bad = {k: v for k, v in scratch.items() if v > 0 and "bwd_grad_kernel" not in k}
    assert not bad, bad
    grad = {k: v for k, v in scratch.items() if "bwd_grad_kernel" in k}
    assert max(grad.values()) <= GRAD_SCRATCH_MAX, grad
