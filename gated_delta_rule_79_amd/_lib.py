"""ctypes loader for libgdn.so (built in-tree by ``build.py``).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  There is no CPU fallback; a missing library raises.
"""

from __future__ import annotations

import ctypes
import os

# the in-tree library; GDN_LIBRARY names another build of it (for example
# the host-sanitized one the C-ABI tests also run against)
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

# status codes (include/gdn.h)
GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE = 0, 1, 2, 3
GDN_ERR_UNSUPPORTED, GDN_ERR_ALIGN, GDN_ERR_WORKSPACE, GDN_ERR_HIP = 4, 5, 6, 7
GDN_ERR_SCRATCH = 8
NOALLOC_SCRATCH_BYTES = 256 << 20  # GDN_NOALLOC_SCRATCH_BYTES
GDN_F32, GDN_BF16 = 0, 1
GDN_GATE_NONE, GDN_GATE_SCALAR, GDN_GATE_CHANNEL = 0, 1, 2

EXPORTED = (
    "gdn_abi_version", "gdn_status_str", "gdn_chunk_fwd_workspace",
    "gdn_chunk_fwd", "gdn_chunk_bwd_workspace", "gdn_chunk_bwd",
    "gdn_decode_step", "gdn_test_set_fail_launch", "gdn_profile_enable",
    "gdn_profile_read",
    "gdn_chunk_fwd_product_workspace", "gdn_chunk_fwd_product",
    "gdn_chunk_fwd_qknorm", "gdn_tree_verify_workspace", "gdn_tree_verify",
    "gdn_tree_commit", "gdn_decode_step_product", "gdn_chunk_fwd_noalloc",
    "gdn2_chunk_fwd", "gdn2_decode_step", "gdn_chunk_fwd_qknorm_workspace",
    "gdn_chunk_fwd_conv_workspace", "gdn_chunk_fwd_conv", "gdn_prologue_fwd",
    "gdn_prologue_bwd_workspace", "gdn_prologue_bwd",
)
STAGE_COUNT = 12
STAGES = ("chunk_map", "fwd_prep", "fwd_scan", "decode", "bwd_states",
          "bwd_scan", "bwd_grad", "other", "fwd_trans", "fwd_combine", "tree_commit",
          "prologue")


class GdnProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("nseq", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("io_dtype", ctypes.c_int32), ("gate_dtype", ctypes.c_int32),
        ("gate", ctypes.c_int32), ("seg_chunks", ctypes.c_int32),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(text)
        self.status = status


_LIB = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and type the library.  Raises if it has not been built."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"libgdn.so not found at {p}: build it with "
            "`python -m gated_delta_rule_79_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    pp = ctypes.POINTER(GdnProblem)
    lib.gdn_abi_version.restype = i32
    lib.gdn_abi_version.argtypes = []
    lib.gdn_status_str.restype = ctypes.c_char_p
    lib.gdn_status_str.argtypes = [i32]
    lib.gdn_chunk_fwd_workspace.restype = i32
    lib.gdn_chunk_fwd_workspace.argtypes = [pp, ctypes.POINTER(sz)]
    lib.gdn_chunk_bwd_workspace.restype = i32
    lib.gdn_chunk_bwd_workspace.argtypes = [pp, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd.restype = i32
    lib.gdn_chunk_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_bwd.restype = i32
    lib.gdn_chunk_bwd.argtypes = [pp] + [vp] * 15 + [sz, vp]
    lib.gdn_decode_step.restype = i32
    lib.gdn_decode_step.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_profile_enable.restype = None
    lib.gdn_profile_enable.argtypes = [i32]
    lib.gdn_profile_read.restype = i32
    lib.gdn_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int32)]
    lib.gdn_test_set_fail_launch.restype = None
    lib.gdn_test_set_fail_launch.argtypes = [i32]
    lib.gdn_chunk_fwd_product_workspace.restype = i32
    lib.gdn_chunk_fwd_product_workspace.argtypes = [pp, i32, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd_product.restype = i32
    lib.gdn_chunk_fwd_product.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_fwd_qknorm.restype = i32
    lib.gdn_chunk_fwd_qknorm.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_tree_verify_workspace.restype = i32
    lib.gdn_tree_verify_workspace.argtypes = [pp, ctypes.POINTER(sz)]
    lib.gdn_tree_verify.restype = i32
    lib.gdn_tree_verify.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_decode_step_product.restype = i32
    lib.gdn_decode_step_product.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_noalloc.restype = i32
    lib.gdn_chunk_fwd_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn2_chunk_fwd.restype = i32
    lib.gdn2_chunk_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn2_decode_step.restype = i32
    lib.gdn2_decode_step.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_qknorm_workspace.restype = i32
    lib.gdn_chunk_fwd_qknorm_workspace.argtypes = [pp, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd_conv_workspace.restype = i32
    lib.gdn_chunk_fwd_conv_workspace.argtypes = [pp, i32, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd_conv.restype = i32
    lib.gdn_chunk_fwd_conv.argtypes = [pp, i32] + [vp] * 12 + [sz, vp]
    lib.gdn_prologue_fwd.restype = i32
    lib.gdn_prologue_fwd.argtypes = [pp, i32, i32, i32, vp, vp, vp, vp]
    lib.gdn_prologue_bwd_workspace.restype = i32
    lib.gdn_prologue_bwd_workspace.argtypes = [pp, i32, i32, ctypes.POINTER(sz)]
    lib.gdn_prologue_bwd.restype = i32
    lib.gdn_prologue_bwd.argtypes = [pp, i32, i32, i32] + [vp] * 6 + [sz, vp]
    lib.gdn_tree_commit.restype = i32
    lib.gdn_tree_commit.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
    if path is None:
        _LIB = lib
    return lib


def check(status: int, what: str) -> None:
    if status != GDN_OK:
        lib = load()
        raise GdnError(status, f"{what}: {lib.gdn_status_str(status).decode()}")
