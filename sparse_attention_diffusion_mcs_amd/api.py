"""Python binding of libmcs: marshals torch tensors (device memory and the
current HIP stream) into the C ABI.  Every step of the computation runs in the
library's HIP kernels; there is no fallback path."""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib as L


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return L.MCS_DTYPE_BF16
    if t.dtype == torch.float32:
        return L.MCS_DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_qkv(q, k, v):
    for t in (q, k, v):
        if not isinstance(t, torch.Tensor) or t.dim() != 3:
            raise ValueError("q, k, v must be [H, N, d] tensors")
        if not t.is_cuda:
            raise ValueError("q, k, v must be device tensors")
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def _check_out(out, q):
    """A caller-supplied output must be a contiguous device tensor of q's
    shape and dtype: the kernels write all of [H, N, d] from its pointer."""
    if not isinstance(out, torch.Tensor) or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous device tensor")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError(f"out must be {tuple(q.shape)} {q.dtype}, got {tuple(out.shape)} {out.dtype}")
    if out.device != q.device:
        raise ValueError(f"out must be on {q.device}, got {out.device}")


def _check_bytes(buf, name, device):
    """Metadata and workspace buffers are contiguous uint8 tensors on the
    inputs' device: their element count is the byte size handed to the
    library."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous() or buf.dtype != torch.uint8:
        raise ValueError(f"{name} must be a contiguous uint8 device tensor")
    if buf.device != device:
        raise ValueError(f"{name} must be on {device}, got {buf.device}")


def desc_for(q: torch.Tensor, scale: float | None = None) -> L.AttnDesc:
    H, N, d = q.shape
    return L.AttnDesc(H, N, d, _dtype_code(q), float(scale) if scale else 0.0)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream, device):
    """The HIP stream handle for a call on `device`: the given stream, which
    must belong to that device, or the device's current stream."""
    s = stream if stream is not None else torch.cuda.current_stream(device)
    if s.device != device:
        raise ValueError(f"stream belongs to {s.device}, the tensors to {device}")
    return ctypes.c_void_p(s.cuda_stream)


def _keep_array(keep, H) -> np.ndarray:
    arr = np.ascontiguousarray(np.broadcast_to(np.asarray(keep, dtype=np.int32), (H,)), dtype=np.int32)
    return arr


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class MetaCache:
    """Cached selection metadata: a device buffer plus its mcs_meta descriptor.

    Region views (all on the device): perm int32 [H, N], keep int32 [H],
    idx_start int64 [H], sched int32 [H], count int32 [H, num_groups] (keys
    kept per group), order int32 [H, num_groups] (launch order of the groups
    in the sparse passes), idx int32 [total_idx] (per group a slot of keep[h]
    indices, the first count[h, g] valid) and residual [H, N, d] (float32 or
    bfloat16, rows in group order)."""

    def __init__(self, meta: L.Meta, buffer: torch.Tensor):
        self.meta = meta
        self.buffer = buffer

    def _region(self, off, count, dtype, shape):
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return self.buffer[off:off + nbytes].view(dtype).view(*shape)

    @property
    def num_heads(self):
        return self.meta.num_heads

    @property
    def seq_len(self):
        return self.meta.seq_len

    @property
    def group_size(self):
        return self.meta.group_size

    @property
    def num_groups(self):
        return self.meta.num_groups

    @property
    def perm(self):
        m = self.meta
        return self._region(m.off_perm, m.num_heads * m.seq_len, torch.int32, (m.num_heads, m.seq_len))

    @property
    def keep(self):
        m = self.meta
        return self._region(m.off_keep, m.num_heads, torch.int32, (m.num_heads,))

    @property
    def idx_start(self):
        m = self.meta
        return self._region(m.off_idx_start, m.num_heads, torch.int64, (m.num_heads,))

    @property
    def sched(self):
        m = self.meta
        return self._region(m.off_sched, m.num_heads, torch.int32, (m.num_heads,))

    @property
    def count(self):
        m = self.meta
        return self._region(m.off_count, m.num_heads * m.num_groups, torch.int32, (m.num_heads, m.num_groups))

    @property
    def order(self):
        m = self.meta
        return self._region(m.off_order, m.num_heads * m.num_groups, torch.int32, (m.num_heads, m.num_groups))

    @property
    def idx(self):
        m = self.meta
        return self._region(m.off_idx, m.total_idx, torch.int32, (m.total_idx,))

    @property
    def residual(self):
        m = self.meta
        dt = torch.bfloat16 if m.residual_dtype == L.MCS_DTYPE_BF16 else torch.float32
        return self._region(m.off_residual, m.num_heads * m.seq_len * m.head_dim, dt,
                            (m.num_heads, m.seq_len, m.head_dim))

    def head_idx(self, h: int, keep_h: int) -> torch.Tensor:
        """Index slots of head h as [num_groups, keep_h] (group g's first
        count[h, g] entries are its kept keys)."""
        start = int(self.idx_start[h].item())
        return self.idx[start:start + self.num_groups * keep_h].view(self.num_groups, keep_h)

    @property
    def nbytes(self) -> int:
        return int(self.meta.bytes)


def dense_attn(q, k, v, out=None, scale=None, stream=None):
    """Dense attention O = softmax(scale q k^T) v per head (mcs_dense_attn)."""
    _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    desc = desc_for(q, scale)
    st = _stream(stream, q.device)
    with torch.cuda.device(q.device):  # launches go to the calling thread's current device
        L.check(L.lib().mcs_dense_attn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), st),
                "mcs_dense_attn")
    return out


def topk_rows(scores, k, out=None, stream=None):
    """The selection's top-k on caller score rows (mcs_topk_rows): for each
    row of the float32 [rows, n] CUDA tensor `scores` (unit column stride,
    row stride a multiple of 4), the ascending indices of its k largest
    scores, ties to the lower index, as int32 [rows, k]."""
    if not isinstance(scores, torch.Tensor) or scores.dtype != torch.float32 or scores.dim() != 2:
        raise TypeError("scores must be a float32 tensor [rows, n]")
    if not scores.is_cuda or scores.stride(1) != 1:
        raise ValueError("scores must be a CUDA tensor with unit column stride")
    rows, n = scores.shape
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    if out.dtype != torch.int32 or tuple(out.shape) != (rows, k) or not out.is_contiguous() or \
            out.device != scores.device:
        raise ValueError(f"out must be a contiguous int32 [{rows}, {k}] tensor on {scores.device}")
    ld = scores.stride(0)
    need = (scores.storage_offset() + (rows - 1) * ld + -(-n // 4) * 4) * 4
    if rows and (ld % 4 or ld < n or need > scores.untyped_storage().nbytes()):
        raise ValueError("scores needs a row stride that is a multiple of 4 and at least n, and storage for the "
                         "last row's n scores rounded up to 4")
    st = _stream(stream, scores.device)
    fp = ctypes.cast(ctypes.c_void_p(scores.data_ptr()), ctypes.POINTER(ctypes.c_float))
    with torch.cuda.device(scores.device):
        L.check(L.lib().mcs_topk_rows(fp, ld, rows, n, k, _ptr(out), st), "mcs_topk_rows")
    return out


_RESIDUAL_DTYPES = {"fp32": L.MCS_DTYPE_FP32, "bf16": L.MCS_DTYPE_BF16}


def _residual_code(residual_dtype) -> int:
    if residual_dtype not in _RESIDUAL_DTYPES:
        raise ValueError(f"residual_dtype must be one of {sorted(_RESIDUAL_DTYPES)}")
    return _RESIDUAL_DTYPES[residual_dtype]


def meta_layout(H, N, d, dtype_code, group_size, keep, residual_dtype="fp32") -> L.Meta:
    desc = L.AttnDesc(H, N, d, dtype_code, 0.0)
    ka = _keep_array(keep, H)
    m = L.Meta()
    L.check(L.lib().mcs_meta_layout_ex(ctypes.byref(desc), group_size, _i32p(ka), _residual_code(residual_dtype),
                                       ctypes.byref(m)), "mcs_meta_layout_ex")
    return m


def workspace_bytes(q, group_size, heads_per_chunk=None, residual_dtype="fp32") -> int:
    desc = desc_for(q)
    hc = q.shape[0] if heads_per_chunk is None else heads_per_chunk
    opts = L.SelectOptions(L.MCS_GROUPING_HASH, 1, 1, 0, 0, 0, _residual_code(residual_dtype), 0.0, None, 0)
    return int(L.lib().mcs_select_workspace_bytes_ex(ctypes.byref(desc), group_size, hc, ctypes.byref(opts)))


def meta_init(q, group_size, keep, meta_buf=None, stream=None, residual_dtype="fp32") -> MetaCache:
    """Lays out an empty metadata buffer (keep/idx_start/sched written, every
    group's count set to keep[h], the launch order 0 .. num_groups-1;
    perm/idx/residual to be filled by the caller) (mcs_meta_init_ex)."""
    if not isinstance(q, torch.Tensor) or not q.is_cuda:
        raise ValueError("q must be a device tensor")
    desc = desc_for(q)
    H, N, d = q.shape
    ka = _keep_array(keep, H)
    layout = meta_layout(H, N, d, _dtype_code(q), group_size, keep, residual_dtype)
    if meta_buf is None:
        meta_buf = torch.empty(max(int(layout.bytes), 256), dtype=torch.uint8, device=q.device)
    _check_bytes(meta_buf, "meta_buf", q.device)
    m = L.Meta()
    st = _stream(stream, q.device)
    with torch.cuda.device(q.device):
        L.check(L.lib().mcs_meta_init_ex(ctypes.byref(desc), group_size, _i32p(ka), _residual_code(residual_dtype),
                                         _ptr(meta_buf), meta_buf.numel(), ctypes.byref(m), st), "mcs_meta_init_ex")
    return MetaCache(m, meta_buf)


def select(q, k, v, group_size, keep, proj, scale=None, meta_buf=None, workspace=None, heads_per_chunk=None,
           return_dense=False, stream=None, grouping="hash", kv_block=1, residual=True, grid=None, dense_out=None,
           phase_events=None, noalloc=False, residual_dtype="fp32", keep_mass=0.0):
    """Selection step (mcs_select; mcs_select_ex for the other groupings --
    "raster", "centred", "morton" with the (T, Y, X) `grid` -- the
    failure-mode ablations kv_block 64, residual False, and tracing).  The
    step's exact dense output is written to `dense_out` when given (a tensor
    like q), else to a new tensor when return_dense is set.  `phase_events`:
    up to MCS_SELECT_PHASES torch.cuda.Event objects, recorded on the stream
    as the grouping, dense pass, key scores, top-k and residual pass are
    launched.  With noalloc the call is mcs_select_noalloc: the workspace is
    the library's own per-device array (no `workspace` may be given).
    Extensions: residual_dtype "bf16" caches the residual in bfloat16;
    keep_mass in (0, 1] keeps, per group, the fewest keys reaching that
    retained probability mass, at most `keep` (their number is in the
    metadata's count region).  Returns (MetaCache, dense output or None)."""
    _check_qkv(q, k, v)
    H, N, d = q.shape
    desc = desc_for(q, scale)
    ka = _keep_array(keep, H)
    pj = np.ascontiguousarray(np.asarray(proj, dtype=np.float32))
    if pj.shape != (L.MCS_HASH_BITS, d):
        raise ValueError(f"proj must be [{L.MCS_HASH_BITS}, {d}]")
    rcode = _residual_code(residual_dtype)
    ml = L.Meta()
    st_l = L.lib().mcs_meta_layout_ex(ctypes.byref(desc), group_size, _i32p(ka), rcode, ctypes.byref(ml))
    if st_l != L.MCS_SUCCESS:
        raise L.McsError(st_l, "mcs_meta_layout_ex")
    nbytes = int(ml.bytes)
    if meta_buf is None:
        meta_buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _check_bytes(meta_buf, "meta_buf", q.device)
    if noalloc:
        if workspace is not None or heads_per_chunk is not None:
            raise ValueError("noalloc uses the library's own workspace")
    else:
        if workspace is None:
            workspace = torch.empty(max(workspace_bytes(q, group_size, heads_per_chunk, residual_dtype), 256),
                                    dtype=torch.uint8, device=q.device)
        _check_bytes(workspace, "workspace", q.device)
    if dense_out is not None:
        _check_out(dense_out, q)
        o_dense = dense_out
    else:
        o_dense = torch.empty_like(q) if return_dense else None
    m = L.Meta()
    pjp = pj.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    st = _stream(stream, q.device)
    ev_arr = None
    if phase_events:
        if len(phase_events) > L.MCS_SELECT_PHASES:
            raise ValueError(f"at most {L.MCS_SELECT_PHASES} phase events")
        handles = []
        for ev in phase_events:
            if ev.cuda_event == 0:  # torch creates the HIP event on its first record
                ev.record(torch.cuda.current_stream(q.device))
            handles.append(ev.cuda_event)
        ev_arr = (ctypes.c_void_p * len(handles))(*handles)
    if (grouping == "hash" and kv_block == 1 and residual and ev_arr is None and not noalloc and rcode == 0
            and keep_mass == 0):
        with torch.cuda.device(q.device):
            L.check(L.lib().mcs_select(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), group_size, _i32p(ka), pjp,
                                       _ptr(meta_buf), meta_buf.numel(), _ptr(workspace), workspace.numel(),
                                       _ptr(o_dense), ctypes.byref(m), st), "mcs_select")
    else:
        codes = {"hash": L.MCS_GROUPING_HASH, "raster": L.MCS_GROUPING_RASTER,
                 "centred": L.MCS_GROUPING_CENTRED_HASH, "morton": L.MCS_GROUPING_MORTON}
        if grouping not in codes:
            raise ValueError(f"unknown grouping {grouping!r}")
        gt, gy, gx = (int(x) for x in grid) if grouping == "morton" else (0, 0, 0)
        opts = L.SelectOptions(codes[grouping], int(kv_block), 1 if residual else 0, gt, gy, gx, rcode,
                               float(keep_mass),
                               ctypes.cast(ev_arr, ctypes.POINTER(ctypes.c_void_p)) if ev_arr is not None else None,
                               len(phase_events) if ev_arr is not None else 0)
        with torch.cuda.device(q.device):
            if noalloc:
                L.check(L.lib().mcs_select_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), group_size,
                                                   _i32p(ka), pjp, ctypes.byref(opts), _ptr(meta_buf),
                                                   meta_buf.numel(), _ptr(o_dense), ctypes.byref(m), st),
                        "mcs_select_noalloc")
            else:
                L.check(L.lib().mcs_select_ex(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), group_size, _i32p(ka),
                                              pjp, ctypes.byref(opts), _ptr(meta_buf), meta_buf.numel(),
                                              _ptr(workspace), workspace.numel(), _ptr(o_dense), ctypes.byref(m),
                                              st), "mcs_select_ex")
    return MetaCache(m, meta_buf), o_dense


def sparse_attn(q, k, v, meta: MetaCache, out=None, scale=None, stream=None):
    """Reuse step (mcs_sparse_attn): attention over each group's cached keys
    plus the cached residual, output in original token order."""
    _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    _check_bytes(meta.buffer, "the metadata buffer", q.device)
    desc = desc_for(q, scale)
    st = _stream(stream, q.device)
    with torch.cuda.device(q.device):
        L.check(L.lib().mcs_sparse_attn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(meta.meta),
                                        _ptr(out), st), "mcs_sparse_attn")
    return out
