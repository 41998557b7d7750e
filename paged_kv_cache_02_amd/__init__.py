"""Paged attention on AMD MI355X: thin Python binding of libpa.so.

Every function here has the name of the C entry point it wraps
(include/pa.h) and does argument marshalling only: it checks tensor
layouts, fills the host descriptor, allocates outputs with torch when the
caller passes none, and calls the library on torch's current HIP stream.
All attention work runs in the library's HIP kernels; there is no fallback.
If libpa.so is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_OK, PA_ERR_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_METADATA, PA_ERR_NO_PAGES = range(7)
PA_BF16, PA_F32 = 0, 1
PA_PATH_DECODE, PA_PATH_DECODE_SPLIT, PA_PATH_PREFILL, PA_PATH_DECODE_BALANCED = 0, 1, 2, 3
PATH_NAMES = {PA_PATH_DECODE: "decode", PA_PATH_DECODE_SPLIT: "decode_split",
              PA_PATH_PREFILL: "prefill", PA_PATH_DECODE_BALANCED: "decode_balanced"}


class PaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {pa_status_str(code)}")


class pa_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages",
        "max_pages_per_seq", "total_q", "max_seq_len", "max_q_len", "dtype")]


class pa_plan_info(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("grid_x", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]


_lib = None

_P = ctypes.c_void_p
_D = ctypes.POINTER(pa_desc)
_SIGS = {
    "pa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_workspace_bytes": (ctypes.c_size_t, [_D, ctypes.c_int32]),
    "pa_plan": (ctypes.c_int, [_D, ctypes.c_int32, ctypes.POINTER(pa_plan_info)]),
    "pa_decode": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                 ctypes.c_size_t, _P]),
    "pa_decode_noalloc": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]),
    "pa_split_merge": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int32,
                                      _P, ctypes.c_size_t, _P, _P, _P]),
    "pa_prefill_chunk": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                        _P, ctypes.c_size_t, _P]),
    "pa_mixed_attention": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                          _P]),
    "pa_merge_partials": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, _P, _P, _P, ctypes.c_int32, _P, _P]),
    "pa_gather_kv": (ctypes.c_int, [_D, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "pa_read_blocks": (ctypes.c_int, [_P, ctypes.c_int64, _P, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "pa_validate_metadata": (ctypes.c_int, [_D, _P, _P, _P, _P]),
    "pa_append_kv": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "pa_pool_create": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]),
    "pa_pool_destroy": (None, [_P]),
    "pa_pool_num_free": (ctypes.c_int32, [_P]),
    "pa_pool_alloc": (ctypes.c_int, [_P, ctypes.c_int32, _P]),
    "pa_pool_free": (ctypes.c_int, [_P, _P, ctypes.c_int32]),
    "pa_pool_reserve": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32]),
    "pa_pool_release": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "pa_pool_refcount": (ctypes.c_int32, [_P, ctypes.c_int32]),
    "pa_pool_share": (ctypes.c_int, [_P, _P, ctypes.c_int32]),
    "pa_pool_fork": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "pa_pool_cow": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "pa_copy_pages": (ctypes.c_int, [_D, _P, _P, _P, _P, ctypes.c_int32, _P]),
    "pa_decode_dense": (ctypes.c_int, [_D, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]),
    "pa_direct_workspace_bytes": (ctypes.c_size_t, [_D]),
    "pa_decode_direct": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
}
EXPORTED = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m paged_kv_cache_02_amd.build or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def pa_status_str(code: int) -> str:
    return lib().pa_status_str(int(code)).decode()


def _check(code: int, where: str):
    if code != PA_OK:
        raise PaError(code, where)


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_desc(q: torch.Tensor, k_pool: torch.Tensor, page_table: torch.Tensor,
              seq_lens: torch.Tensor, max_seq_len: Optional[int] = None,
              max_q_len: Optional[int] = None, q_offsets: Optional[torch.Tensor] = None) -> pa_desc:
    """Host descriptor from tensor shapes; max_seq_len/max_q_len are read
    from the device (a synchronization) only when not given."""
    total_q, Hq, d = q.shape
    NP, Hkv, P, d2 = k_pool.shape
    if d2 != d:
        raise ValueError("q and k_pool head_dim differ")
    B, MP = page_table.shape
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    if max_q_len is None:
        if q_offsets is None:
            max_q_len = 1 if B else 0
        else:
            max_q_len = int((seq_lens - q_offsets).max().item()) if B else 0
    return pa_desc(B, Hq, Hkv, d, P, NP, MP, total_q, int(max_seq_len), int(max_q_len),
                   _dtype_code(q))


def _desc_dict(desc: pa_desc) -> dict:
    return {n: getattr(desc, n) for n, _ in pa_desc._fields_}


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------
def pa_plan(desc: pa_desc, cu_count: int = 0) -> dict:
    info = pa_plan_info()
    _check(lib().pa_plan(ctypes.byref(desc), int(cu_count), ctypes.byref(info)), "pa_plan")
    return {"path": PATH_NAMES[info.path], "num_splits": info.num_splits, "grid_x": info.grid_x,
            "workspace_bytes": int(info.workspace_bytes)}


def pa_workspace_bytes(desc: pa_desc, num_splits: int) -> int:
    return int(lib().pa_workspace_bytes(ctypes.byref(desc), int(num_splits)))


def _alloc_out(q, out, lse, want_lse=True):
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    return out, lse


NOALLOC_SCRATCH_BYTES = 32 << 20


def pa_decode_noalloc(q, k_pool, v_pool, page_table, seq_lens, q_offsets, scale, *, out, lse,
                      max_seq_len=None, desc=None):
    """pa_decode on the library's fixed device scratch: the C call allocates
    nothing (out and lse are the caller's)."""
    desc = desc or make_desc(q, k_pool, page_table, seq_lens, max_seq_len)
    _check(lib().pa_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                   _ptr(page_table), _ptr(seq_lens), _ptr(q_offsets),
                                   float(scale), _ptr(out), _ptr(lse), _stream(q.device)),
           "pa_decode_noalloc")
    return out, lse


def pa_decode(q, k_pool, v_pool, page_table, seq_lens, q_offsets, scale, *,
              max_seq_len=None, out=None, lse=None, workspace=None, desc=None):
    """Single-token decode; returns (out, lse)."""
    desc = desc or make_desc(q, k_pool, page_table, seq_lens, max_seq_len)
    out, lse = _alloc_out(q, out, lse)
    plan = pa_plan(desc)
    if workspace is None and plan["workspace_bytes"]:
        workspace = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_decode(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                           _ptr(page_table), _ptr(seq_lens), _ptr(q_offsets), float(scale),
                           _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(q.device)),
           "pa_decode")
    return out, lse


def pa_decode_dense(q, k_cache, v_cache, seq_lens, scale, *, desc, out=None, lse=None):
    """Decode over a dense cache [B, Hkv, MP * P, d] (no page table; MP =
    desc.max_pages_per_seq); returns (out, lse)."""
    out, lse = _alloc_out(q, out, lse)
    _check(lib().pa_decode_dense(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(seq_lens), float(scale), _ptr(out), _ptr(lse), _stream(q.device)),
           "pa_decode_dense")
    return out, lse


def pa_decode_direct(q, k_pool, v_pool, page_table, seq_lens, scale, *, desc, out=None, lse=None,
                     workspace=None):
    """Decode through the page table without the flash fusion (scores stored,
    softmax, then values); returns (out, lse)."""
    out, lse = _alloc_out(q, out, lse)
    need = int(lib().pa_direct_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_direct(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                  _ptr(page_table), _ptr(seq_lens), float(scale), _ptr(out), _ptr(lse),
                                  _ptr(workspace), ws_bytes, _stream(q.device)), "pa_decode_direct")
    return out, lse


def pa_split_merge(q, k_pool, v_pool, page_table, seq_lens, q_offsets, scale, num_splits, *,
                   max_seq_len=None, out=None, lse=None, workspace=None, desc=None):
    """Split-K decode with num_splits partitions; returns (out, lse, workspace)
    (the workspace holds the partials after the call)."""
    desc = desc or make_desc(q, k_pool, page_table, seq_lens, max_seq_len)
    out, lse = _alloc_out(q, out, lse)
    need = pa_workspace_bytes(desc, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pa_split_merge(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(page_table), _ptr(seq_lens), _ptr(q_offsets), float(scale),
                                int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                                _stream(q.device)), "pa_split_merge")
    return out, lse, workspace


def split_partials_view(desc: pa_desc, workspace: torch.Tensor, num_splits: int):
    """(o_part [B,Hq,S,d], lse_part [B,Hq,S]) float32 views of a split workspace."""
    B, Hq, d, S = desc.num_seqs, desc.num_q_heads, desc.head_dim, num_splits
    o_bytes = (B * Hq * S * d * 4 + 255) // 256 * 256
    f = workspace.view(torch.uint8)
    o = f[:B * Hq * S * d * 4].view(torch.float32).view(B, Hq, S, d)
    l = f[o_bytes:o_bytes + B * Hq * S * 4].view(torch.float32).view(B, Hq, S)
    return o, l


def pa_prefill_chunk(q, k_pool, v_pool, page_table, seq_lens, q_offsets, scale, *,
                     q_starts=None, max_seq_len=None, max_q_len=None, out=None, lse=None,
                     workspace=None, split=True, desc=None):
    """Chunked prefill; returns (out, lse).  split=False runs without a
    workspace (every query tile over its whole key range)."""
    desc = desc or make_desc(q, k_pool, page_table, seq_lens, max_seq_len, max_q_len, q_offsets)
    out, lse = _alloc_out(q, out, lse)
    if split and workspace is None:
        need = pa_plan(desc)["workspace_bytes"]
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_prefill_chunk(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                  _ptr(page_table), _ptr(seq_lens), _ptr(q_offsets),
                                  _ptr(q_starts), float(scale), _ptr(out), _ptr(lse),
                                  _ptr(workspace), ws_bytes, _stream(q.device)),
           "pa_prefill_chunk")
    return out, lse


def pa_mixed_attention(q, k_pool, v_pool, page_table, seq_lens, q_offsets, scale, *,
                       q_starts=None, max_seq_len=None, max_q_len=None, out=None, lse=None,
                       desc=None):
    """One continuous-batching round in one launch: rows with n_r = 1 are
    decoded, chunks with n_r > 1 prefilled; returns (out, lse)."""
    desc = desc or make_desc(q, k_pool, page_table, seq_lens, max_seq_len, max_q_len, q_offsets)
    out, lse = _alloc_out(q, out, lse)
    _check(lib().pa_mixed_attention(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                    _ptr(page_table), _ptr(seq_lens), _ptr(q_offsets),
                                    _ptr(q_starts), float(scale), _ptr(out), _ptr(lse),
                                    _stream(q.device)),
           "pa_mixed_attention")
    return out, lse


def bind_mixed_attention(q, k_pool, v_pool, page_table, seq_lens, q_offsets, scale, *, out, lse,
                         desc, q_starts=None) -> "BoundCall":
    """pa_mixed_attention with fixed arguments (see BoundCall)."""
    keep = (desc, q, k_pool, v_pool, page_table, seq_lens, q_offsets, q_starts, out, lse)
    return BoundCall("pa_mixed_attention", keep, ctypes.byref(desc), _ptr(q), _ptr(k_pool),
                     _ptr(v_pool), _ptr(page_table), _ptr(seq_lens), _ptr(q_offsets),
                     _ptr(q_starts), float(scale), _ptr(out), _ptr(lse), _stream(q.device))


class BoundCall:
    """One library call with its arguments marshalled once, for launch loops
    in which the per-call Python cost would otherwise starve the GPU queue.
    It keeps the tensors alive; they must not be reallocated between calls
    (in-place updates of their contents are fine).  The stream is the current
    stream at bind time."""

    def __init__(self, name: str, keep, *args):
        self.name = name
        self.fn = getattr(lib(), name)
        self.args = args
        self.keep = keep

    def __call__(self):
        _check(self.fn(*self.args), self.name)


def bind_decode(q, k_pool, v_pool, page_table, seq_lens, q_offsets, scale, *, out, lse,
                workspace, desc) -> BoundCall:
    """pa_decode with fixed arguments (see BoundCall)."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    keep = (desc, q, k_pool, v_pool, page_table, seq_lens, q_offsets, out, lse, workspace)
    return BoundCall("pa_decode", keep, ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                     _ptr(page_table), _ptr(seq_lens), _ptr(q_offsets), float(scale), _ptr(out),
                     _ptr(lse), _ptr(workspace), ws_bytes, _stream(q.device))


def bind_prefill_chunk(q, k_pool, v_pool, page_table, seq_lens, q_offsets, scale, *, q_starts,
                       out, lse, workspace, desc) -> BoundCall:
    """pa_prefill_chunk with fixed arguments (see BoundCall)."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    keep = (desc, q, k_pool, v_pool, page_table, seq_lens, q_offsets, q_starts, out, lse, workspace)
    return BoundCall("pa_prefill_chunk", keep, ctypes.byref(desc), _ptr(q), _ptr(k_pool),
                     _ptr(v_pool), _ptr(page_table), _ptr(seq_lens), _ptr(q_offsets),
                     _ptr(q_starts), float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                     ws_bytes, _stream(q.device))


def pa_merge_partials(o_part, lse_part, out_dtype=torch.bfloat16, *, out=None, lse=None):
    """Merge o_part [rows, heads, S, d] / lse_part [rows, heads, S]; returns (out, lse)."""
    rows, heads, S, d = o_part.shape
    if out is None:
        out = torch.empty(rows, heads, d, dtype=out_dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty(rows, heads, dtype=torch.float32, device=o_part.device)
    _check(lib().pa_merge_partials(rows, heads, S, d, _ptr(o_part), _ptr(lse_part), _ptr(out),
                                   _dtype_code(out), _ptr(lse), _stream(o_part.device)),
           "pa_merge_partials")
    return out, lse


def pa_gather_kv(k_pool, v_pool, page_table, req, seq_len, *, desc=None, seq_lens=None):
    """Contiguous copies [seq_len, Hkv, d] of request req's keys and values."""
    NP, Hkv, P, d = k_pool.shape
    if desc is None:
        B, MP = page_table.shape
        desc = pa_desc(B, Hkv, Hkv, d, P, NP, MP, B, int(seq_len), 1, _dtype_code(k_pool))
    k_out = torch.empty(seq_len, Hkv, d, dtype=k_pool.dtype, device=k_pool.device)
    v_out = torch.empty_like(k_out)
    _check(lib().pa_gather_kv(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                              int(req), int(seq_len), _ptr(k_out), _ptr(v_out),
                              _stream(k_pool.device)), "pa_gather_kv")
    return k_out, v_out


def pa_read_blocks(buf, order, block_bytes, sink):
    """Read the blocks of the uint8 device tensor buf (block_bytes each) in
    the order of the int32 device tensor order, XOR-folding every word into
    the int32 device tensor sink (one element, zeroed by the caller): the
    decode kernels' K/V read pattern on its own, for timing."""
    _check(lib().pa_read_blocks(_ptr(buf), int(buf.numel()) // int(block_bytes), _ptr(order),
                                int(order.numel()), int(block_bytes), _ptr(sink), _stream(buf.device)),
           "pa_read_blocks")


def bind_read_blocks(buf, order, block_bytes, sink) -> BoundCall:
    """pa_read_blocks with fixed arguments (see BoundCall)."""
    keep = (buf, order, sink)
    return BoundCall("pa_read_blocks", keep, _ptr(buf), int(buf.numel()) // int(block_bytes), _ptr(order),
                     int(order.numel()), int(block_bytes), _ptr(sink), _stream(buf.device))


def pa_validate_metadata(desc: pa_desc, page_table, seq_lens, q_offsets=None) -> int:
    """Returns the status code (PA_OK or PA_ERR_METADATA); synchronizes."""
    return int(lib().pa_validate_metadata(ctypes.byref(desc), _ptr(page_table), _ptr(seq_lens),
                                          _ptr(q_offsets), _stream(page_table.device)))


def pa_append_kv(k_new, v_new, k_pool, v_pool, page_table, seq_lens, q_offsets, *,
                 q_starts=None, max_seq_len=None, max_q_len=None, desc=None):
    """Write the new K/V rows [total_q, Hkv, d] into their page slots (in
    place in k_pool / v_pool)."""
    desc = desc or make_desc(k_new, k_pool, page_table, seq_lens, max_seq_len, max_q_len, q_offsets)
    _check(lib().pa_append_kv(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(page_table),
                              _ptr(seq_lens), _ptr(q_offsets), _ptr(q_starts), _ptr(k_pool),
                              _ptr(v_pool), _stream(k_new.device)), "pa_append_kv")


def bind_append_kv(k_new, v_new, k_pool, v_pool, page_table, seq_lens, q_offsets, *, q_starts,
                   desc) -> BoundCall:
    """pa_append_kv with fixed arguments (see BoundCall)."""
    keep = (desc, k_new, v_new, k_pool, v_pool, page_table, seq_lens, q_offsets, q_starts)
    return BoundCall("pa_append_kv", keep, ctypes.byref(desc), _ptr(k_new), _ptr(v_new),
                     _ptr(page_table), _ptr(seq_lens), _ptr(q_offsets), _ptr(q_starts),
                     _ptr(k_pool), _ptr(v_pool), _stream(k_new.device))


def pa_copy_pages(k_pool, v_pool, src_ids, dst_ids, *, desc):
    """Copy whole pages (K and V, all KV heads) src_ids[i] -> dst_ids[i]
    (device int32 tensors), in place in the pools: the device half of a
    copy on write (PagePool.cow)."""
    n = int(src_ids.numel())
    if int(dst_ids.numel()) != n:
        raise ValueError("src_ids and dst_ids must have the same length")
    _check(lib().pa_copy_pages(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool), _ptr(src_ids),
                               _ptr(dst_ids), n, _stream(k_pool.device)), "pa_copy_pages")


class PagePool:
    """The library's host page allocator (pa_pool_*): page ids on demand, a
    request's page-table row grown by whole pages and released at the end,
    pages shared between rows by reference count with copy on write.
    Page-table rows are host numpy int32 arrays; copy them to the device
    before a kernel reads them."""

    def __init__(self, num_pages: int):
        h = ctypes.c_void_p()
        _check(lib().pa_pool_create(int(num_pages), ctypes.byref(h)), "pa_pool_create")
        self._h = h
        self.num_pages = int(num_pages)

    def close(self):
        if getattr(self, "_h", None):
            lib().pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return int(lib().pa_pool_num_free(self._h))

    @staticmethod
    def _i32(a):
        import numpy as np
        if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous):
            raise ValueError("page-table rows and id lists must be contiguous int32 numpy arrays")
        return a.ctypes.data_as(ctypes.c_void_p)

    def alloc(self, n: int):
        import numpy as np
        ids = np.empty(max(int(n), 0), np.int32)
        _check(lib().pa_pool_alloc(self._h, int(n), self._i32(ids) if n > 0 else None), "pa_pool_alloc")
        return ids

    def free(self, ids):
        import numpy as np
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        _check(lib().pa_pool_free(self._h, self._i32(ids) if ids.size else None, int(ids.size)),
               "pa_pool_free")

    def reserve(self, row, old_len: int, new_len: int, page_size: int = 16):
        """Grow page-table row `row` (int32 numpy view, edited in place)."""
        _check(lib().pa_pool_reserve(self._h, self._i32(row), int(row.size), int(old_len),
                                     int(new_len), int(page_size)), "pa_pool_reserve")

    def release(self, row, length: int, page_size: int = 16):
        _check(lib().pa_pool_release(self._h, self._i32(row), int(row.size), int(length),
                                     int(page_size)), "pa_pool_release")

    def refcount(self, page_id: int) -> int:
        return int(lib().pa_pool_refcount(self._h, int(page_id)))

    def share(self, ids):
        import numpy as np
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        _check(lib().pa_pool_share(self._h, self._i32(ids) if ids.size else None, int(ids.size)),
               "pa_pool_share")

    def fork(self, src_row, dst_row, length: int, page_size: int = 16):
        """dst_row starts as a sharer of src_row's pages for `length` keys."""
        _check(lib().pa_pool_fork(self._h, self._i32(src_row), self._i32(dst_row), int(dst_row.size),
                                  int(length), int(page_size)), "pa_pool_fork")

    def cow(self, row, logical_page: int):
        """Make logical page `logical_page` of `row` private before a write;
        returns (old_id, new_id), equal when no copy is needed."""
        old = ctypes.c_int32(-1)
        new = ctypes.c_int32(-1)
        _check(lib().pa_pool_cow(self._h, self._i32(row), int(row.size), int(logical_page),
                                 ctypes.byref(old), ctypes.byref(new)), "pa_pool_cow")
        return int(old.value), int(new.value)


__all__ = ["pa_desc", "pa_plan_info", "PaError", "lib", "make_desc", "pa_plan",
           "pa_workspace_bytes", "pa_decode", "pa_split_merge", "pa_prefill_chunk",
           "pa_merge_partials", "pa_gather_kv", "pa_read_blocks", "bind_read_blocks", "pa_validate_metadata", "pa_status_str",
           "split_partials_view", "pa_append_kv", "bind_append_kv", "PagePool", "BoundCall",
           "bind_decode", "bind_prefill_chunk", "pa_copy_pages", "pa_decode_dense",
           "pa_decode_direct", "pa_mixed_attention", "bind_mixed_attention", "EXPORTED"]
