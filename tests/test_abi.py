"""The C ABI of libgdn on the CPU: the library loads, exports every function
include/gdn.h declares, and rejects bad arguments before launching anything.

Every call here either fails validation or runs with the launch-failure test
hook set, so no kernel is ever launched (fake device pointers are safe)."""

import ctypes
import os
import re

import pytest

from gated_delta_rule_79_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

A = 0x10000  # fake, 16-byte aligned "device" addresses (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libgdn.so not built")
    lib = _lib.load()
    lib.gdn_test_set_fail_launch(1)
    yield lib
    lib.gdn_test_set_fail_launch(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.gdn_abi_version() == 6
    for s in range(8):
        txt = lib.gdn_status_str(s).decode()
        assert txt.startswith("GDN_")
    assert lib.gdn_status_str(99).decode() == "GDN_ERR_UNKNOWN"


def prob(**kw):
    p = _lib.GdnProblem()
    d = dict(B=1, T=64, H=2, dk=128, dv=128, chunk=64, nseq=0, cu_seqlens=None,
             io_dtype=_lib.GDN_BF16, gate_dtype=_lib.GDN_BF16,
             gate=_lib.GDN_GATE_SCALAR)
    d.update(kw)
    for k, v in d.items():
        setattr(p, k, v)
    return p


def ws_bytes(lib, p):
    n = ctypes.c_size_t(0)
    st = lib.gdn_chunk_fwd_workspace(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def fwd(lib, p, ws=None, **ptr):
    d = dict(q=A, k=A, v=A, beta=A, la=A, s0=None, o=A, sf=None)
    d.update(ptr)
    st, need = ws_bytes(lib, p)
    if st != 0:
        need = 0
    return lib.gdn_chunk_fwd(ctypes.byref(p), d["q"], d["k"], d["v"], d["beta"],
                             d["la"], d["s0"], d["o"], d["sf"],
                             A if ws is None else ws, need, None)


def test_valid_call_reaches_launch(lib):
    # validation passes, the test hook turns the launch into GDN_ERR_HIP
    assert fwd(lib, prob()) == _lib.GDN_ERR_HIP


@pytest.mark.parametrize("kw,status", [
    (dict(dk=48), _lib.GDN_ERR_UNSUPPORTED),
    (dict(dk=256), _lib.GDN_ERR_UNSUPPORTED),
    (dict(dv=24), _lib.GDN_ERR_UNSUPPORTED),
    (dict(dv=272), _lib.GDN_ERR_UNSUPPORTED),
    (dict(chunk=128), _lib.GDN_ERR_UNSUPPORTED),
    (dict(chunk=8), _lib.GDN_ERR_UNSUPPORTED),
    (dict(gate=3), _lib.GDN_ERR_UNSUPPORTED),
    (dict(io_dtype=2), _lib.GDN_ERR_DTYPE),
    (dict(gate_dtype=-1), _lib.GDN_ERR_DTYPE),
    (dict(B=0), _lib.GDN_ERR_SHAPE),
    (dict(H=0), _lib.GDN_ERR_SHAPE),
    (dict(T=-1), _lib.GDN_ERR_SHAPE),
    (dict(nseq=-2), _lib.GDN_ERR_SHAPE),
    (dict(nseq=3, B=2, cu_seqlens=A), _lib.GDN_ERR_SHAPE),
    (dict(nseq=3, cu_seqlens=None), _lib.GDN_ERR_NULL),
    (dict(nseq=0, cu_seqlens=A), _lib.GDN_ERR_SHAPE),
    (dict(nseq=3, cu_seqlens=A + 2), _lib.GDN_ERR_ALIGN),
    (dict(T=(1 << 31) - 1, H=1024), _lib.GDN_ERR_SHAPE),
])
def test_problem_validation(lib, kw, status):
    p = prob(**kw)
    assert fwd(lib, p) == status
    st, _ = ws_bytes(lib, p)
    assert st == status


def test_null_problem(lib):
    n = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace(None, ctypes.byref(n)) == _lib.GDN_ERR_NULL
    assert lib.gdn_chunk_fwd_workspace(ctypes.byref(prob()), None) == _lib.GDN_ERR_NULL
    assert lib.gdn_chunk_fwd(None, A, A, A, A, A, None, A, None, A, 0, None) == _lib.GDN_ERR_NULL


@pytest.mark.parametrize("name", ["q", "k", "v", "beta", "la", "o"])
def test_pointer_checks(lib, name):
    assert fwd(lib, prob(), **{name: None}) == _lib.GDN_ERR_NULL
    assert fwd(lib, prob(), **{name: A + 8}) == _lib.GDN_ERR_ALIGN


def test_optional_pointers(lib):
    assert fwd(lib, prob(), s0=A + 4) == _lib.GDN_ERR_ALIGN
    assert fwd(lib, prob(), sf=A + 4) == _lib.GDN_ERR_ALIGN
    assert fwd(lib, prob(), s0=A, sf=A) == _lib.GDN_ERR_HIP
    # gate none: log_alpha may be NULL
    assert fwd(lib, prob(gate=_lib.GDN_GATE_NONE), la=None) == _lib.GDN_ERR_HIP


def test_empty_sequence_needs_no_pointers(lib):
    p = prob(T=0)
    st, need = ws_bytes(lib, p)
    assert st == 0 and need == 0
    assert lib.gdn_chunk_fwd(ctypes.byref(p), None, None, None, None, None, None,
                             None, None, None, 0, None) == _lib.GDN_ERR_HIP


def test_workspace_checks(lib):
    p = prob()
    st, need = ws_bytes(lib, p)
    assert st == 0 and need > 0
    assert lib.gdn_chunk_fwd(ctypes.byref(p), A, A, A, A, A, None, A, None, A,
                             need - 1, None) == _lib.GDN_ERR_WORKSPACE
    assert lib.gdn_chunk_fwd(ctypes.byref(p), A, A, A, A, A, None, A, None, None,
                             need, None) == _lib.GDN_ERR_WORKSPACE
    assert lib.gdn_chunk_fwd(ctypes.byref(p), A, A, A, A, A, None, A, None, A + 4,
                             need, None) == _lib.GDN_ERR_ALIGN


def test_workspace_scales_with_problem(lib):
    _, a = ws_bytes(lib, prob(T=64))
    _, b = ws_bytes(lib, prob(T=128))
    _, c = ws_bytes(lib, prob(T=64, H=4))
    assert b == 2 * a and c == 2 * a
    # varlen: one chunk slot per sequence more than the dense bound, plus the map
    _, d = ws_bytes(lib, prob(T=64, nseq=3, cu_seqlens=A))
    assert d > a


def seg_bytes(nsegs, H, dk, dv, ob):
    al = lambda x: (x + 255) // 256 * 256
    return nsegs * H * (2 * al(dk * dv * 4) + al((dk // 16) * ((dk + 31) // 32) * 512 * ob))


def test_workspace_of_segmented_state_pass(lib):
    try:
        lib.gdn_set_segment_chunks(-1)
        _, off = ws_bytes(lib, prob(T=640))
        _, off_big = ws_bytes(lib, prob(T=4096, H=16))
        lib.gdn_set_segment_chunks(3)           # 10 chunks -> 4 segments
        _, seg3 = ws_bytes(lib, prob(T=640))
        assert seg3 - off == seg_bytes(4, 2, 128, 128, 2)
        _, seg3f = ws_bytes(lib, prob(T=640, io_dtype=_lib.GDN_F32))
        lib.gdn_set_segment_chunks(-1)
        _, offf = ws_bytes(lib, prob(T=640, io_dtype=_lib.GDN_F32))
        assert seg3f - offf == seg_bytes(4, 2, 128, 128, 4)
        # automatic: 16 (sequence, head) workgroups of 64 chunks; filling 256
        # CUs takes segments of 64 * 16 / 256 = 4 chunks, raised to the floor
        # ceil(sqrt(64 / 2.56)) = 5: 13 segments per sequence
        lib.gdn_set_segment_chunks(0)
        _, auto = ws_bytes(lib, prob(T=4096, H=16))
        assert auto - off_big == seg_bytes(13, 16, 128, 128, 2)
        # enough (sequence, head) workgroups (16 x 16 = 256): no split
        _, a = ws_bytes(lib, prob(B=16, T=4096, H=16))
        lib.gdn_set_segment_chunks(-1)
        _, b = ws_bytes(lib, prob(B=16, T=4096, H=16))
        assert a == b
        # 8 x 16 = 128 workgroups of 64 chunks: segments of 64 * 128 / 256 =
        # 32 chunks, 2 per sequence
        lib.gdn_set_segment_chunks(0)
        _, a = ws_bytes(lib, prob(B=8, T=4096, H=16))
        assert a - b // 2 == seg_bytes(8 * 2, 16, 128, 128, 2)
        # long chains: 16 workgroups of 1024 chunks -> 64-chunk segments
        _, a = ws_bytes(lib, prob(T=65536, H=16))
        lib.gdn_set_segment_chunks(-1)
        _, b = ws_bytes(lib, prob(T=65536, H=16))
        lib.gdn_set_segment_chunks(0)
        assert a - b == seg_bytes(16, 16, 128, 128, 2)
        # short chains (fewer than 8 chunks) are never split
        _, a = ws_bytes(lib, prob(T=448, H=16))
        lib.gdn_set_segment_chunks(-1)
        _, b = ws_bytes(lib, prob(T=448, H=16))
        lib.gdn_set_segment_chunks(0)
        assert a == b
        # varlen with a forced split: segment table + buffers for at most
        # nchunks / L + nseq slots
        lib.gdn_set_segment_chunks(2)
        _, v2 = ws_bytes(lib, prob(T=640, nseq=3, cu_seqlens=A))
        lib.gdn_set_segment_chunks(-1)
        _, v0 = ws_bytes(lib, prob(T=640, nseq=3, cu_seqlens=A))
        nch = 10 + 3
        slots = nch // 2 + 3
        al = lambda x: (x + 255) // 256 * 256
        assert v2 - v0 == seg_bytes(slots, 2, 128, 128, 2) + al(slots * 16) + al(4 * 4)
    finally:
        lib.gdn_set_segment_chunks(0)


def test_decode_validation(lib):
    p = prob(B=4, T=0)
    args = [A, A, A, A, A, A, A, None]
    assert lib.gdn_decode_step(ctypes.byref(p), *args) == _lib.GDN_ERR_HIP
    assert lib.gdn_decode_step(None, *args) == _lib.GDN_ERR_NULL
    assert lib.gdn_decode_step(ctypes.byref(prob(dk=20)), *args) == _lib.GDN_ERR_UNSUPPORTED
    assert lib.gdn_decode_step(ctypes.byref(prob(B=0)), *args) == _lib.GDN_ERR_SHAPE
    bad = list(args)
    bad[5] = None      # state
    assert lib.gdn_decode_step(ctypes.byref(p), *bad) == _lib.GDN_ERR_NULL
    bad[5] = A + 2
    assert lib.gdn_decode_step(ctypes.byref(p), *bad) == _lib.GDN_ERR_ALIGN


def test_bwd_validation(lib):
    p = prob()
    n = ctypes.c_size_t(0)
    assert lib.gdn_chunk_bwd_workspace(ctypes.byref(p), ctypes.byref(n)) == 0
    args = [A] * 6 + [A, None] + [A] * 5 + [None]
    st = lib.gdn_chunk_bwd(ctypes.byref(p), *args, A, n.value, None)
    assert st == _lib.GDN_ERR_HIP
    bad = list(args)
    bad[6] = None      # d_o
    assert lib.gdn_chunk_bwd(ctypes.byref(p), *bad, A, n.value, None) == _lib.GDN_ERR_NULL
    bad = list(args)
    bad[12] = None     # dlog_alpha with a gate
    assert lib.gdn_chunk_bwd(ctypes.byref(p), *bad, A, n.value, None) == _lib.GDN_ERR_NULL


def test_python_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        _lib.load(str(tmp_path / "missing.so"))


def test_product_workspace_and_rejections(lib):
    """Householder-product forward: nh steps per token run as nh * T steps,
    so its workspace is the forward's for nh * T; other nh and the
    per-channel gate are rejected before any launch."""
    n = ctypes.c_size_t(0)
    for nh in (1, 2, 4):
        st = lib.gdn_chunk_fwd_product_workspace(ctypes.byref(prob(T=100)), nh,
                                                 ctypes.byref(n))
        assert st == _lib.GDN_OK
        st2, ref = ws_bytes(lib, prob(T=100 * nh))
        assert st2 == _lib.GDN_OK and n.value == ref
    for nh in (0, 3, 8, -1):
        assert lib.gdn_chunk_fwd_product_workspace(
            ctypes.byref(prob(T=100)), nh, ctypes.byref(n)) == _lib.GDN_ERR_UNSUPPORTED
    assert lib.gdn_chunk_fwd_product_workspace(
        ctypes.byref(prob(T=100, gate=_lib.GDN_GATE_CHANNEL)), 2,
        ctypes.byref(n)) == _lib.GDN_ERR_UNSUPPORTED
    assert lib.gdn_chunk_fwd_product_workspace(None, 2, ctypes.byref(n)) == _lib.GDN_ERR_NULL
    # null pointers are rejected before any launch
    st = lib.gdn_chunk_fwd_product(ctypes.byref(prob(T=100)), 2, None, A, A, A, A,
                                   None, A, None, A, 1 << 30, None)
    assert st == _lib.GDN_ERR_NULL


def test_qknorm_rejections(lib):
    """The forward that normalises q and k itself: the per-channel gate is
    rejected, null pointers and a short workspace are caught before any
    launch."""
    st = lib.gdn_chunk_fwd_qknorm(ctypes.byref(prob(T=100, gate=_lib.GDN_GATE_CHANNEL)),
                                  A, A, A, A, A, None, A, None, A, 1 << 30, None)
    assert st == _lib.GDN_ERR_UNSUPPORTED
    assert lib.gdn_chunk_fwd_qknorm(None, A, A, A, A, A, None, A, None, A, 1 << 30,
                                    None) == _lib.GDN_ERR_NULL
    st = lib.gdn_chunk_fwd_qknorm(ctypes.byref(prob(T=100)), None, A, A, A, A,
                                  None, A, None, A, 1 << 30, None)
    assert st == _lib.GDN_ERR_NULL
    st = lib.gdn_chunk_fwd_qknorm(ctypes.byref(prob(T=100)), A, A, A, A, A,
                                  None, A, None, A, 1, None)
    assert st == _lib.GDN_ERR_WORKSPACE


def test_tree_rejections_before_launch(lib):
    """Draft trees: more nodes than the chunk (dense), the per-channel gate,
    null or misaligned parent / accepted arrays are rejected before any
    launch; the verification workspace is the forward's for the same sizes."""
    n = ctypes.c_size_t(0)
    st = lib.gdn_tree_verify_workspace(ctypes.byref(prob(T=16, chunk=16)), ctypes.byref(n))
    st2, ref = ws_bytes(lib, prob(T=16, chunk=16))
    assert st == _lib.GDN_OK and st2 == _lib.GDN_OK and n.value == ref
    assert lib.gdn_tree_verify_workspace(ctypes.byref(prob(T=40, chunk=32)),
                                         ctypes.byref(n)) == _lib.GDN_ERR_SHAPE
    assert lib.gdn_tree_verify_workspace(
        ctypes.byref(prob(T=16, chunk=16, gate=_lib.GDN_GATE_CHANNEL)),
        ctypes.byref(n)) == _lib.GDN_ERR_UNSUPPORTED
    p = prob(T=16, chunk=16)
    assert lib.gdn_tree_verify(ctypes.byref(p), None, A, A, A, A, A, None, A, A, 1 << 30,
                               None) == _lib.GDN_ERR_NULL
    assert lib.gdn_tree_verify(ctypes.byref(p), A + 2, A, A, A, A, A, None, A, A, 1 << 30,
                               None) == _lib.GDN_ERR_ALIGN
    assert lib.gdn_tree_verify(ctypes.byref(p), A, A, A, A, A, A, None, A, A, 1,
                               None) == _lib.GDN_ERR_WORKSPACE
    assert lib.gdn_tree_commit(ctypes.byref(p), A, None, A, A, A, A, A,
                               None) == _lib.GDN_ERR_NULL
    assert lib.gdn_tree_commit(ctypes.byref(p), A, A, A, A, A, A, None,
                               None) == _lib.GDN_ERR_NULL
    assert lib.gdn_tree_commit(ctypes.byref(prob(T=40, chunk=32)), A, A, A, A, A, A, A,
                               None) == _lib.GDN_ERR_SHAPE


def test_decode_product_rejections(lib):
    """Product decode: nh outside {1, 2, 4} and the per-channel gate are
    rejected, null pointers caught, before any launch."""
    p = prob(B=4, T=1)
    for nh in (0, 3, 8):
        assert lib.gdn_decode_step_product(ctypes.byref(p), nh, A, A, A, A, A, A, A,
                                           None) == _lib.GDN_ERR_UNSUPPORTED
    pc = prob(B=4, T=1, gate=_lib.GDN_GATE_CHANNEL)
    assert lib.gdn_decode_step_product(ctypes.byref(pc), 2, A, A, A, A, A, A, A,
                                       None) == _lib.GDN_ERR_UNSUPPORTED
    assert lib.gdn_decode_step_product(ctypes.byref(p), 2, None, A, A, A, A, A, A,
                                       None) == _lib.GDN_ERR_NULL
    assert lib.gdn_decode_step_product(ctypes.byref(p), 2, A, A, A, A, A, None, A,
                                       None) == _lib.GDN_ERR_NULL
