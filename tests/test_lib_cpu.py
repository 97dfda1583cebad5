"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects invalid arguments before touching the device."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mcs.h")

L = pytest.importorskip("sparse_attention_diffusion_mcs_amd._lib")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mcs_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libmcs.so not built")
    return L.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert set(names) == set(L.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.mcs_version() == L.MCS_VERSION == 3
    assert lib.mcs_status_string(0) == b"MCS_SUCCESS"
    assert lib.mcs_status_string(6) == b"MCS_ERROR_HIP"
    assert lib.mcs_status_string(99) == b"MCS_UNKNOWN_STATUS"
    assert lib.mcs_last_hip_error() == 0


def _desc(H=2, N=100, d=64, dt=1, scale=0.0):
    return L.AttnDesc(H, N, d, dt, scale)


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


FAKE = ctypes.c_void_p(0x7f0000000000)        # 256-aligned, never dereferenced: validation fails first
FAKE_MIS = ctypes.c_void_p(0x7f0000000008)
NULL = ctypes.c_void_p(0)


def test_dense_validation(lib):
    f = lib.mcs_dense_attn
    assert f(None, FAKE, FAKE, FAKE, FAKE, NULL) == L.MCS_ERROR_INVALID_VALUE
    assert f(ctypes.byref(_desc(d=96)), FAKE, FAKE, FAKE, FAKE, NULL) == L.MCS_ERROR_UNSUPPORTED_SHAPE
    assert f(ctypes.byref(_desc(dt=7)), FAKE, FAKE, FAKE, FAKE, NULL) == L.MCS_ERROR_UNSUPPORTED_SHAPE
    assert f(ctypes.byref(_desc(H=-1)), FAKE, FAKE, FAKE, FAKE, NULL) == L.MCS_ERROR_INVALID_VALUE
    assert f(ctypes.byref(_desc(N=(1 << 24) + 1)), FAKE, FAKE, FAKE, FAKE, NULL) == L.MCS_ERROR_UNSUPPORTED_SHAPE
    assert f(ctypes.byref(_desc(scale=float("nan"))), FAKE, FAKE, FAKE, FAKE, NULL) == L.MCS_ERROR_INVALID_VALUE
    assert f(ctypes.byref(_desc()), NULL, FAKE, FAKE, FAKE, NULL) == L.MCS_ERROR_INVALID_VALUE
    assert f(ctypes.byref(_desc()), FAKE, FAKE, FAKE_MIS, FAKE, NULL) == L.MCS_ERROR_MISALIGNED
    # empty problems are valid no-ops, whatever the pointers
    assert f(ctypes.byref(_desc(H=0)), NULL, NULL, NULL, NULL, NULL) == L.MCS_SUCCESS
    assert f(ctypes.byref(_desc(N=0)), NULL, NULL, NULL, NULL, NULL) == L.MCS_SUCCESS


def test_meta_layout(lib):
    H, N, d, G = 3, 1000, 128, 64
    keep, kp = _i32([64, 100, 1000])
    m = L.Meta()
    assert lib.mcs_meta_layout(ctypes.byref(_desc(H, N, d)), G, kp, ctypes.byref(m)) == L.MCS_SUCCESS
    ng = -(-N // G)
    assert (m.version, m.num_heads, m.seq_len, m.head_dim, m.group_size, m.num_groups) == (3, H, N, d, G, ng)
    assert m.total_idx == ng * keep.sum() and m.max_keep == 1000 and m.base is None
    assert m.residual_dtype == L.MCS_DTYPE_FP32 and m.reserved == 0
    offs = [m.off_perm, m.off_keep, m.off_idx_start, m.off_sched, m.off_count, m.off_order, m.off_idx,
            m.off_residual]
    sizes = [H * N * 4, H * 4, H * 8, H * 4, H * ng * 4, H * ng * 4, m.total_idx * 4, H * N * d * 4]
    assert all(o % 256 == 0 for o in offs)
    for (o, s), o2 in zip(zip(offs, sizes), offs[1:] + [m.bytes]):
        assert o + s <= o2
    assert lib.mcs_meta_bytes(ctypes.byref(_desc(H, N, d)), G, kp) == m.bytes
    # a bf16 residual: the same regions, the residual region half as large
    mb16 = L.Meta()
    assert lib.mcs_meta_layout_ex(ctypes.byref(_desc(H, N, d)), G, kp, L.MCS_DTYPE_BF16,
                                  ctypes.byref(mb16)) == L.MCS_SUCCESS
    assert mb16.residual_dtype == L.MCS_DTYPE_BF16 and mb16.off_residual == m.off_residual
    assert mb16.bytes == m.off_residual + H * N * d * 2
    # bf16 residuals exist for bf16 problems only; other codes are refused
    assert lib.mcs_meta_layout_ex(ctypes.byref(_desc(H, N, d, dt=0)), G, kp, L.MCS_DTYPE_BF16,
                                  ctypes.byref(mb16)) == L.MCS_ERROR_INVALID_VALUE
    assert lib.mcs_meta_layout_ex(ctypes.byref(_desc(H, N, d)), G, kp, 7, ctypes.byref(mb16)) == L.MCS_ERROR_INVALID_VALUE
    # invalid keep / group
    bad, bp = _i32([64, 0, 5])
    assert lib.mcs_meta_layout(ctypes.byref(_desc(H, N, d)), G, bp, ctypes.byref(m)) == L.MCS_ERROR_INVALID_VALUE
    bad, bp = _i32([64, 1001, 5])
    assert lib.mcs_meta_bytes(ctypes.byref(_desc(H, N, d)), G, bp) == 0
    assert lib.mcs_meta_layout(ctypes.byref(_desc(H, N, d)), 32, kp, ctypes.byref(m)) == L.MCS_ERROR_UNSUPPORTED_SHAPE
    assert lib.mcs_meta_layout(ctypes.byref(_desc(H, N, d)), G, None, ctypes.byref(m)) == L.MCS_ERROR_INVALID_VALUE


def test_workspace_bytes(lib):
    d = _desc(4, 1000, 64)
    one = lib.mcs_select_workspace_bytes(ctypes.byref(d), 64, 1)
    two = lib.mcs_select_workspace_bytes(ctypes.byref(d), 64, 2)
    # 16 groups x (N rounded up to 64 key scores + 16 block scores rounded up to 64) x float32,
    # plus the N rows' log-sum-exp (float32, rounded up to 256 bytes) and, for bf16 problems,
    # the head's V rounded to float16 [N][d]
    per = 16 * (1024 + 64) * 4 + 4096 + 1000 * 64 * 2
    assert two - one == per
    assert lib.mcs_select_workspace_bytes(ctypes.byref(d), 64, 99) == lib.mcs_select_workspace_bytes(
        ctypes.byref(d), 64, 4)
    assert lib.mcs_select_workspace_bytes(ctypes.byref(d), 48, 1) == 0
    # a bf16 residual adds each head's float32 dense output [N][d]
    opts = L.SelectOptions(0, 1, 1, 0, 0, 0, L.MCS_DTYPE_BF16, 0.0, None, 0)
    one16 = lib.mcs_select_workspace_bytes_ex(ctypes.byref(d), 64, 1, ctypes.byref(opts))
    two16 = lib.mcs_select_workspace_bytes_ex(ctypes.byref(d), 64, 2, ctypes.byref(opts))
    assert two16 - one16 == per + 1000 * 64 * 4 and one16 == one + 1000 * 64 * 4
    assert lib.mcs_select_workspace_bytes_ex(ctypes.byref(d), 64, 1, None) == one
    opts.residual_dtype = 5
    assert lib.mcs_select_workspace_bytes_ex(ctypes.byref(d), 64, 1, ctypes.byref(opts)) == 0


def test_select_validation(lib):
    H, N, d = 2, 100, 64
    keep, kp = _i32([10, 20])
    proj = np.zeros((8, d), np.float32)
    pp = proj.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    m = L.Meta()
    D = ctypes.byref(_desc(H, N, d))
    mb = lib.mcs_meta_bytes(D, 64, kp)
    wb = lib.mcs_select_workspace_bytes(D, 64, 1)
    sel = lib.mcs_select
    args = lambda **kw: [kw.get("desc", D), FAKE, FAKE, FAKE, kw.get("G", 64), kw.get("keep", kp),
                         kw.get("proj", pp), kw.get("meta", FAKE), kw.get("mb", mb), kw.get("ws", FAKE),
                         kw.get("wb", wb), kw.get("od", NULL), kw.get("out", ctypes.byref(m)), NULL]
    assert sel(*args(G=96)) == L.MCS_ERROR_UNSUPPORTED_SHAPE
    assert sel(*args(proj=None)) == L.MCS_ERROR_INVALID_VALUE
    assert sel(*args(meta=NULL)) == L.MCS_ERROR_INVALID_VALUE
    assert sel(*args(meta=FAKE_MIS)) == L.MCS_ERROR_MISALIGNED
    assert sel(*args(ws=FAKE_MIS)) == L.MCS_ERROR_MISALIGNED
    assert sel(*args(od=FAKE_MIS)) == L.MCS_ERROR_MISALIGNED
    assert sel(*args(mb=mb - 1)) == L.MCS_ERROR_BUFFER_TOO_SMALL
    assert sel(*args(wb=wb - 1)) == L.MCS_ERROR_BUFFER_TOO_SMALL
    assert sel(*args(out=None)) == L.MCS_ERROR_INVALID_VALUE
    bad, bp = _i32([0, 20])
    assert sel(*args(keep=bp)) == L.MCS_ERROR_INVALID_VALUE
    # empty problem: validates, fills the descriptor, launches nothing
    m0 = L.Meta()
    D0 = ctypes.byref(_desc(0, N, d))
    assert sel(D0, NULL, NULL, NULL, 64, kp, pp, NULL, 0, NULL, 0, NULL, ctypes.byref(m0), NULL) == L.MCS_SUCCESS
    assert m0.version == L.MCS_META_VERSION == 3 and m0.num_heads == 0 and m0.bytes == 0


def test_select_ex_options_validation(lib):
    """Bad ablation options are rejected before anything is launched."""
    H, N, d = 2, 128, 64
    keep, kp = _i32([64, 128])
    proj = np.zeros((8, d), np.float32)
    pp = proj.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    m = L.Meta()
    D = ctypes.byref(_desc(H, N, d))
    mb = lib.mcs_meta_bytes(D, 64, kp)
    wb = lib.mcs_select_workspace_bytes(D, 64, 1)

    def call(opts, desc=D, keep_p=kp):
        return lib.mcs_select_ex(desc, FAKE, FAKE, FAKE, 64, keep_p, pp, ctypes.byref(opts), FAKE, mb, FAKE, wb,
                                 NULL, ctypes.byref(m), NULL)

    O = L.SelectOptions
    assert call(O(4, 1, 1)) == L.MCS_ERROR_INVALID_VALUE          # unknown grouping
    assert call(O(0, 32, 1)) == L.MCS_ERROR_INVALID_VALUE         # block size other than 1 / 64
    assert call(O(0, 1, 2)) == L.MCS_ERROR_INVALID_VALUE          # residual flag not 0 / 1
    assert call(O(0, 1, 1, 2, 8, 8)) == L.MCS_ERROR_INVALID_VALUE   # grid given to a non-grid grouping
    assert call(O(3, 1, 1)) == L.MCS_ERROR_INVALID_VALUE          # Z-curve without a grid
    assert call(O(3, 1, 1, 2, 8, 9)) == L.MCS_ERROR_INVALID_VALUE   # grid holds more than N tokens
    assert call(O(3, 1, 1, 1, 2, 2048)) == L.MCS_ERROR_INVALID_VALUE  # a dimension above 1024
    odd, op = _i32([64, 100])
    assert call(O(0, 64, 1), keep_p=op) == L.MCS_ERROR_UNSUPPORTED_SHAPE   # keep not whole blocks
    d2 = ctypes.byref(_desc(H, 130, d))
    assert call(O(1, 64, 0), desc=d2) == L.MCS_ERROR_UNSUPPORTED_SHAPE     # N not whole blocks
    # the options do not bypass the ordinary checks
    zero, zp = _i32([0, 64])
    assert call(O(1, 1, 0), keep_p=zp) == L.MCS_ERROR_INVALID_VALUE
    # tracing events: at most MCS_SELECT_PHASES, an array when any, no null handle
    evs = (ctypes.c_void_p * 6)(*([FAKE.value] * 6))
    ep = ctypes.cast(evs, ctypes.POINTER(ctypes.c_void_p))
    assert call(O(0, 1, 1, 0, 0, 0, 0, 0.0, ep, L.MCS_SELECT_PHASES + 1)) == L.MCS_ERROR_INVALID_VALUE
    assert call(O(0, 1, 1, 0, 0, 0, 0, 0.0, None, 1)) == L.MCS_ERROR_INVALID_VALUE
    assert call(O(0, 1, 1, 0, 0, 0, 0, 0.0, ep, -1)) == L.MCS_ERROR_INVALID_VALUE
    evs[1] = None
    assert call(O(0, 1, 1, 0, 0, 0, 0, 0.0, ep, 2)) == L.MCS_ERROR_INVALID_VALUE
    # extensions: residual dtype, retained-mass target in [0, 1] with single-token selection
    assert call(O(0, 1, 1, 0, 0, 0, 3)) == L.MCS_ERROR_INVALID_VALUE
    assert call(O(0, 1, 1, 0, 0, 0, 0, -0.5)) == L.MCS_ERROR_INVALID_VALUE
    assert call(O(0, 1, 1, 0, 0, 0, 0, 1.5)) == L.MCS_ERROR_INVALID_VALUE
    assert call(O(0, 1, 1, 0, 0, 0, 0, float("nan"))) == L.MCS_ERROR_INVALID_VALUE
    d64 = ctypes.byref(_desc(H, 128, d))
    assert call(O(1, 64, 1, 0, 0, 0, 0, 0.9), desc=d64) == L.MCS_ERROR_INVALID_VALUE
    # bf16 residual of a float32 problem
    assert call(O(0, 1, 1, 0, 0, 0, 1), desc=ctypes.byref(_desc(H, N, d, dt=0))) == L.MCS_ERROR_INVALID_VALUE


def test_sparse_validation(lib):
    H, N, d = 2, 100, 64
    keep, kp = _i32([10, 20])
    m = L.Meta()
    assert lib.mcs_meta_layout(ctypes.byref(_desc(H, N, d)), 64, kp, ctypes.byref(m)) == L.MCS_SUCCESS
    m.base = FAKE.value
    f = lib.mcs_sparse_attn
    for bad in (_desc(H + 1, N, d), _desc(H, N + 1, d), _desc(H, N, 128), _desc(H, N, d, dt=0)):
        assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, ctypes.byref(m), FAKE, NULL) == L.MCS_ERROR_META_MISMATCH
    m2 = L.Meta.from_buffer_copy(m)
    m2.version = 1
    assert f(ctypes.byref(_desc(H, N, d)), FAKE, FAKE, FAKE, ctypes.byref(m2), FAKE, NULL) == L.MCS_ERROR_META_MISMATCH
    m5 = L.Meta.from_buffer_copy(m)
    m5.residual_dtype = L.MCS_DTYPE_BF16   # the regions of an fp32 layout under a bf16 label
    assert f(ctypes.byref(_desc(H, N, d)), FAKE, FAKE, FAKE, ctypes.byref(m5), FAKE, NULL) == L.MCS_ERROR_META_MISMATCH
    m5.residual_dtype = 9
    assert f(ctypes.byref(_desc(H, N, d)), FAKE, FAKE, FAKE, ctypes.byref(m5), FAKE, NULL) == L.MCS_ERROR_META_MISMATCH
    assert f(ctypes.byref(_desc(H, N, d)), FAKE, FAKE, FAKE, None, FAKE, NULL) == L.MCS_ERROR_INVALID_VALUE
    assert f(ctypes.byref(_desc(H, N, d)), FAKE, FAKE, FAKE, ctypes.byref(m), NULL, NULL) == L.MCS_ERROR_INVALID_VALUE
    m3 = L.Meta.from_buffer_copy(m)
    m3.base = FAKE_MIS.value
    assert f(ctypes.byref(_desc(H, N, d)), FAKE, FAKE, FAKE, ctypes.byref(m3), FAKE, NULL) == L.MCS_ERROR_MISALIGNED
    m4 = L.Meta.from_buffer_copy(m)
    m4.base = None
    assert f(ctypes.byref(_desc(H, N, d)), FAKE, FAKE, FAKE, ctypes.byref(m4), FAKE, NULL) == L.MCS_ERROR_INVALID_VALUE


def test_meta_init_validation(lib):
    H, N, d = 2, 100, 64
    keep, kp = _i32([10, 20])
    m = L.Meta()
    D = ctypes.byref(_desc(H, N, d))
    mb = lib.mcs_meta_bytes(D, 64, kp)
    assert lib.mcs_meta_init(D, 64, kp, NULL, mb, ctypes.byref(m), NULL) == L.MCS_ERROR_INVALID_VALUE
    assert lib.mcs_meta_init(D, 64, kp, FAKE_MIS, mb, ctypes.byref(m), NULL) == L.MCS_ERROR_MISALIGNED
    assert lib.mcs_meta_init(D, 64, kp, FAKE, mb - 4, ctypes.byref(m), NULL) == L.MCS_ERROR_BUFFER_TOO_SMALL
    assert lib.mcs_meta_init(D, 64, kp, FAKE, mb, None, NULL) == L.MCS_ERROR_INVALID_VALUE


def test_max_seq_len_boundary(lib):
    """N = MCS_MAX_SEQ_LEN is accepted and N + 1 rejected (host-side layout
    only); the binding's constant is the header's."""
    import re
    hdr = open(os.path.join(ROOT, "include", "mcs.h")).read()
    assert re.search(r"#define MCS_MAX_SEQ_LEN \(1 << (\d+)\)", hdr).group(1) == "22"
    assert L.MCS_MAX_SEQ_LEN == 1 << 22
    keep, kp = _i32([64])
    for d in (64, 128):
        assert lib.mcs_meta_bytes(ctypes.byref(_desc(1, L.MCS_MAX_SEQ_LEN, d)), 64, kp) > 0
        assert lib.mcs_meta_bytes(ctypes.byref(_desc(1, L.MCS_MAX_SEQ_LEN + 1, d)), 64, kp) == 0
        assert lib.mcs_select_workspace_bytes(ctypes.byref(_desc(1, L.MCS_MAX_SEQ_LEN + 1, d)), 64, 1) == 0


def test_sparse_attn_rejects_edited_layouts(lib):
    """A metadata struct whose regions do not sit where the layout puts them
    is refused before any launch (fake, aligned device pointers: nothing may
    run)."""
    H, N, d, G = 2, 1000, 128, 64
    keep, kp = _i32([64, 100])
    good = L.Meta()
    assert lib.mcs_meta_layout(ctypes.byref(_desc(H, N, d)), G, kp, ctypes.byref(good)) == L.MCS_SUCCESS
    for field, delta in (("off_residual", 256), ("off_idx", -256), ("off_perm", 256), ("bytes", 256),
                         ("off_count", 256), ("off_order", 256), ("total_idx", 64),
                         ("total_idx", -good.total_idx - 1)):
        m = L.Meta()
        ctypes.pointer(m)[0] = good
        m.base = FAKE
        setattr(m, field, getattr(m, field) + delta)
        st = lib.mcs_sparse_attn(ctypes.byref(_desc(H, N, d)), FAKE, FAKE, FAKE, ctypes.byref(m), FAKE, NULL)
        assert st == L.MCS_ERROR_META_MISMATCH, (field, delta, st)


@pytest.mark.parametrize("debug", ["0", "1"])
def test_valid_call_without_a_device_reports_the_hip_error(debug):
    """On a host with no GPU a valid call passes validation, its launch fails
    and the call returns MCS_ERROR_HIP with the HIP code kept for
    mcs_last_hip_error (hipErrorNoDevice), also in the debug mode
    (MCS_DEBUG=1) that synchronises after every launch.  Run in a child
    process; skipped where a device exists, since the pointers are fake."""
    import os
    import subprocess
    import sys

    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: the fake pointers must not reach a kernel")
    code = (
        "import ctypes, sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from sparse_attention_diffusion_mcs_amd import _lib as L\n"
        "lib = L.lib()\n"
        "d = L.AttnDesc(1, 64, 64, 1, 0.0)\n"
        "f = ctypes.c_void_p(0x7f0000000000)\n"
        "st = lib.mcs_dense_attn(ctypes.byref(d), f, f, f, f, None)\n"
        "print(st, lib.mcs_last_hip_error())\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, MCS_DEBUG=debug))
    assert r.returncode == 0, r.stderr[-2000:]
    st, err = (int(x) for x in r.stdout.split()[-2:])
    assert st == L.MCS_ERROR_HIP and err == 100


def test_noalloc_refuses_shapes_beyond_its_array(lib):
    """mcs_select_noalloc refuses a shape whose fixed workspace plus one
    head's scores exceed MCS_NOALLOC_SCRATCH_BYTES before any other check or
    device call (the long-video layer: 357 MB of scores per head), and takes
    the ordinary validation path otherwise."""
    keep, kp = _i32([3776] * 24)
    proj = np.zeros((8, 128), np.float32)
    pp = proj.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    m = L.Meta()
    big = _desc(24, 75600, 128)
    assert lib.mcs_select_workspace_bytes(ctypes.byref(big), 64, 1) > L.MCS_NOALLOC_SCRATCH_BYTES
    assert lib.mcs_select_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, 64, kp, pp, None, FAKE, 1 << 40, NULL,
                                  ctypes.byref(m), NULL) == L.MCS_ERROR_BUFFER_TOO_SMALL
    small = _desc(2, 1000, 128)
    keep2, kp2 = _i32([0, 64])
    assert lib.mcs_select_noalloc(ctypes.byref(small), FAKE, FAKE, FAKE, 64, kp2, pp, None, FAKE, 1 << 30, NULL,
                                  ctypes.byref(m), NULL) == L.MCS_ERROR_INVALID_VALUE
    assert lib.mcs_select_noalloc(ctypes.byref(small), FAKE, FAKE, FAKE, 96, kp, pp, None, FAKE, 1 << 30, NULL,
                                  ctypes.byref(m), NULL) == L.MCS_ERROR_UNSUPPORTED_SHAPE
