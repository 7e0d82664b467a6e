"""Python binding of libhwkv, the per-head windowed KV cache runtime for MI355X.

A thin ctypes layer over the C ABI declared in ``include/hwkv.h``: the
functions keep the C names and only marshal arguments (torch tensors become
device pointers, the current torch stream becomes the HIP stream).  Every
step of the path runs in the library's HIP kernels; PyTorch only provides
device memory and streams.  There is no CPU fallback: if ``libhwkv.so`` is
missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhwkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libhwkv.so is not built (%s); build it with head_windowed_kv_amd._build "
                      "or __graft_entry__.build()" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

HWKV_F32 = 0
HWKV_BF16 = 1
HWKV_F16 = 2
ABI_VERSION = 3

STATUS_NAMES = {0: "HWKV_OK", 1: "HWKV_ERR_INVALID_ARG", 2: "HWKV_ERR_UNSUPPORTED",
                3: "HWKV_ERR_MISALIGNED", 4: "HWKV_ERR_CAPACITY", 5: "HWKV_ERR_ABI_MISMATCH",
                6: "HWKV_ERR_HIP", 7: "HWKV_ERR_OVERFLOW"}

#: every symbol the C ABI exports
EXPORTED = ("hwkv_abi_version", "hwkv_last_error", "hwkv_layout_create", "hwkv_layout_destroy",
            "hwkv_layout_query", "hwkv_mem_estimate", "hwkv_capacity_check", "hwkv_table_fill",
            "hwkv_meta_fill", "hwkv_meta_fingerprint",
            "hwkv_workspace_bytes", "hwkv_append", "hwkv_decode_split", "hwkv_decode_merge",
            "hwkv_decode_attn", "hwkv_decode_split_append", "hwkv_decode_append_attn",
            "hwkv_decode_append_attn_static", "hwkv_step_workspace_bytes",
            "hwkv_decode_step",
            "hwkv_prefill_workspace_bytes", "hwkv_prefill_attn", "hwkv_prefill_attn_exact")


class hwkv_layout_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("n_layers", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32), ("max_window", ctypes.c_int32),
                ("blocks_per_seq", ctypes.c_int64), ("n_work", ctypes.c_int64),
                ("block_bytes", ctypes.c_uint64), ("meta_bytes", ctypes.c_uint64),
                ("fingerprint", ctypes.c_uint64)]


class hwkv_cache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("pool_bytes", ctypes.c_uint64),
                ("block_ids", ctypes.c_void_p), ("table_rows", ctypes.c_int64),
                ("meta", ctypes.c_void_p), ("meta_fingerprint", ctypes.c_uint64)]


_i32, _i64, _u64, _f32, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                               ctypes.c_float, ctypes.c_void_p)
_P = ctypes.POINTER

_lib.hwkv_abi_version.restype = ctypes.c_uint32
_lib.hwkv_abi_version.argtypes = []
_lib.hwkv_last_error.restype = ctypes.c_char_p
_lib.hwkv_last_error.argtypes = []
_lib.hwkv_layout_create.restype = ctypes.c_int
_lib.hwkv_layout_create.argtypes = [_i32, _i32, _vp, _i32, _i32, ctypes.c_int, _i32, _P(_vp)]
_lib.hwkv_layout_destroy.restype = None
_lib.hwkv_layout_destroy.argtypes = [_vp]
_lib.hwkv_layout_query.restype = ctypes.c_int
_lib.hwkv_layout_query.argtypes = [_vp, _P(hwkv_layout_desc), _vp, _vp, _vp]
_lib.hwkv_mem_estimate.restype = ctypes.c_int
_lib.hwkv_mem_estimate.argtypes = [_vp, _i64, _P(_u64)]
_lib.hwkv_capacity_check.restype = ctypes.c_int
_lib.hwkv_capacity_check.argtypes = [_vp, _i64, _u64, _P(_i64), _P(_i32), _P(_i32)]
_lib.hwkv_table_fill.restype = ctypes.c_int
_lib.hwkv_table_fill.argtypes = [_vp, _i64, _vp]
_lib.hwkv_meta_fill.restype = ctypes.c_int
_lib.hwkv_meta_fill.argtypes = [_vp, _vp, _u64]
_lib.hwkv_meta_fingerprint.restype = ctypes.c_int
_lib.hwkv_meta_fingerprint.argtypes = [_vp, _u64, _P(_u64)]
_lib.hwkv_workspace_bytes.restype = ctypes.c_int
_lib.hwkv_workspace_bytes.argtypes = [_vp, _i32, _i32, _i32, _i32, _P(_u64)]
_lib.hwkv_append.restype = ctypes.c_int
_lib.hwkv_append.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp,
                             _vp]
_lib.hwkv_decode_split.restype = ctypes.c_int
_lib.hwkv_decode_split.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _i32, _vp, _vp, _i32, _vp,
                                   _f32, _vp, _u64, _vp]
_lib.hwkv_decode_merge.restype = ctypes.c_int
_lib.hwkv_decode_merge.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _i32, _vp, _i32, _vp, _u64,
                                   _vp, ctypes.c_int, _vp]
_lib.hwkv_decode_attn.restype = ctypes.c_int
_lib.hwkv_decode_attn.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _i32, _vp, _vp, _i32, _vp,
                                  _f32, _vp, _u64, _vp, ctypes.c_int, _vp]
_lib.hwkv_decode_split_append.restype = ctypes.c_int
_lib.hwkv_decode_split_append.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _i32, _vp, _vp, _vp,
                                          _vp, _i32, _vp, _f32, _vp, _u64, _vp]
_lib.hwkv_decode_append_attn.restype = ctypes.c_int
_lib.hwkv_decode_append_attn.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _i32, _vp, _vp, _vp,
                                         _vp, _i32, _vp, _f32, _vp, _u64, _vp, ctypes.c_int, _vp]
_lib.hwkv_decode_append_attn_static.restype = ctypes.c_int
_lib.hwkv_decode_append_attn_static.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _i32, _vp, _vp,
                                                _vp, _vp, _i32, _vp, _f32, _vp, ctypes.c_int,
                                                _vp]
#: bytes of the library's static decode scratch (hwkv_decode_append_attn_static)
STATIC_SCRATCH_BYTES = 64 << 20
_lib.hwkv_step_workspace_bytes.restype = ctypes.c_int
_lib.hwkv_step_workspace_bytes.argtypes = [_vp, _i32, _i32, _i32, _i32, _P(_u64)]
_lib.hwkv_decode_step.restype = ctypes.c_int
_lib.hwkv_decode_step.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                  _i32, _vp, _f32, _vp, _u64, _vp, ctypes.c_int, _vp]
_lib.hwkv_prefill_workspace_bytes.restype = ctypes.c_int
_lib.hwkv_prefill_workspace_bytes.argtypes = [_vp, _i32, _i32, _i32, _P(_u64)]
_lib.hwkv_prefill_attn.restype = ctypes.c_int
_lib.hwkv_prefill_attn.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _vp, _vp, _i32, _i32, _vp,
                                   _vp, _vp, _vp, _u64, _vp, ctypes.c_int, _f32, _vp]
_lib.hwkv_prefill_attn_exact.restype = ctypes.c_int
_lib.hwkv_prefill_attn_exact.argtypes = [_vp, _P(hwkv_cache), _i32, _i32, _vp, _vp, _i32, _i32,
                                         _vp, _vp, _vp, _vp, ctypes.c_int, _f32, _vp]


class HwkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), msg))
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))


def _check(status: int) -> None:
    if status != 0:
        raise HwkvError(status, _lib.hwkv_last_error().decode("utf-8", "replace"))


def hwkv_abi_version() -> int:
    return int(_lib.hwkv_abi_version())


def hwkv_last_error() -> str:
    return _lib.hwkv_last_error().decode("utf-8", "replace")


def _dtype_code(dtype) -> int:
    if dtype in (torch.bfloat16, "bf16", HWKV_BF16):
        return HWKV_BF16
    if dtype in (torch.float32, "f32", HWKV_F32):
        return HWKV_F32
    if dtype in (torch.float16, "f16", HWKV_F16):
        return HWKV_F16
    raise ValueError("dtype must be torch.bfloat16, torch.float16 or torch.float32, got %r"
                     % (dtype,))


def torch_dtype(code: int) -> torch.dtype:
    return {HWKV_BF16: torch.bfloat16, HWKV_F16: torch.float16}.get(code, torch.float32)


class Layout:
    """Owns one immutable ``hwkv_layout`` (released on garbage collection)."""

    _destroy = _lib.hwkv_layout_destroy

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and not getattr(self, "_freed", False):
            self._freed = True
            self._destroy(h)

    def desc(self) -> hwkv_layout_desc:
        return hwkv_layout_query(self)[0]


def hwkv_layout_create(windows, block_size: int, head_dim: int, dtype,
                       split_tokens: int = 0) -> Layout:
    """windows: [n_layers][n_kv_heads] ints (layer-major)."""
    w = np.ascontiguousarray(np.asarray(windows, dtype=np.int64))
    if w.ndim != 2:
        raise ValueError("windows must be 2-D [n_layers][n_kv_heads]")
    if w.size and (w.min() < -2 ** 31 or w.max() >= 2 ** 31):
        raise ValueError("window outside int32")
    w = w.astype(np.int32)
    out = ctypes.c_void_p()
    _check(_lib.hwkv_layout_create(w.shape[0], w.shape[1], w.ctypes.data_as(_vp), block_size,
                                   head_dim, _dtype_code(dtype), split_tokens, ctypes.byref(out)))
    return Layout(out.value)


def hwkv_layout_query(layout: Layout):
    """Returns (desc, windows [L][H] int32, nblocks [L][H] int32, head_offsets [L*H+1] int64)."""
    d = hwkv_layout_desc()
    _check(_lib.hwkv_layout_query(layout.handle, ctypes.byref(d), None, None, None))
    n = d.n_layers * d.n_kv_heads
    w = np.zeros(n, np.int32)
    nb = np.zeros(n, np.int32)
    off = np.zeros(n + 1, np.int64)
    _check(_lib.hwkv_layout_query(layout.handle, ctypes.byref(d), w.ctypes.data_as(_vp),
                                  nb.ctypes.data_as(_vp), off.ctypes.data_as(_vp)))
    return d, w.reshape(d.n_layers, d.n_kv_heads), nb.reshape(d.n_layers, d.n_kv_heads), off


def hwkv_mem_estimate(layout: Layout, n_seqs: int) -> int:
    b = ctypes.c_uint64()
    _check(_lib.hwkv_mem_estimate(layout.handle, n_seqs, ctypes.byref(b)))
    return int(b.value)


def hwkv_capacity_check(layout: Layout, n_seqs: int, pool_bytes: int):
    """None if the pool holds n_seqs rows, else (seq_row, layer, head, message)
    of the first head whose blocks do not fit."""
    row, layer, head = ctypes.c_int64(-1), ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = _lib.hwkv_capacity_check(layout.handle, n_seqs, pool_bytes, ctypes.byref(row),
                                  ctypes.byref(layer), ctypes.byref(head))
    if st == 0:
        return None
    if STATUS_NAMES.get(st) != "HWKV_ERR_CAPACITY":
        _check(st)
    return int(row.value), int(layer.value), int(head.value), hwkv_last_error()


def hwkv_table_fill(layout: Layout, n_seqs: int) -> np.ndarray:
    d = layout.desc()
    ids = np.zeros(max(n_seqs, 0) * d.blocks_per_seq, np.int32)
    _check(_lib.hwkv_table_fill(layout.handle, n_seqs, ids.ctypes.data_as(_vp)))
    return ids.reshape(n_seqs, d.blocks_per_seq)


def hwkv_meta_fill(layout: Layout) -> np.ndarray:
    d = layout.desc()
    buf = np.zeros(d.meta_bytes, np.uint8)
    _check(_lib.hwkv_meta_fill(layout.handle, buf.ctypes.data_as(_vp), d.meta_bytes))
    return buf


def hwkv_meta_fingerprint(meta_host: np.ndarray) -> int:
    """The layout fingerprint a host copy of a meta blob carries."""
    buf = np.ascontiguousarray(meta_host, dtype=np.uint8)
    fp = ctypes.c_uint64()
    _check(_lib.hwkv_meta_fingerprint(buf.ctypes.data_as(_vp), buf.size, ctypes.byref(fp)))
    return int(fp.value)


def hwkv_workspace_bytes(layout: Layout, layer_begin: int, n_layers: int, n_seqs: int,
                         n_q_heads: int) -> int:
    b = ctypes.c_uint64()
    _check(_lib.hwkv_workspace_bytes(layout.handle, layer_begin, n_layers, n_seqs, n_q_heads,
                                     ctypes.byref(b)))
    return int(b.value)


# ---------------------------------------------------------------------------
# device side: torch tensors provide memory, the current torch stream the queue
# ---------------------------------------------------------------------------

def _alloc_aligned(nbytes: int, device, align: int = 256) -> torch.Tensor:
    """A uint8 device tensor of nbytes whose data pointer is `align`-aligned."""
    t = torch.empty(nbytes + align, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % align
    return t[off:off + nbytes]


@dataclass
class Cache:
    """Caller-owned device memory of one cache: pool, block tables and meta."""
    layout: Layout
    pool: torch.Tensor        # uint8 [pool_bytes]
    block_ids: torch.Tensor   # int32 [table_rows][blocks_per_seq]
    meta: torch.Tensor        # uint8 [meta_bytes]
    meta_fingerprint: int = 0  # fingerprint the blob carries (hwkv_meta_fingerprint)

    @property
    def table_rows(self) -> int:
        return int(self.block_ids.shape[0])

    def view(self) -> hwkv_cache:
        return hwkv_cache(self.pool.data_ptr(), self.pool.numel(), self.block_ids.data_ptr(),
                          self.table_rows, self.meta.data_ptr(), self.meta_fingerprint)


def make_cache(layout: Layout, n_seqs: int, device="cuda", block_ids: Optional[np.ndarray] = None,
               pool_bytes: Optional[int] = None, fill: Optional[int] = None) -> Cache:
    """Allocate the pool (exactly hwkv_mem_estimate bytes unless pool_bytes is
    given), upload the block tables (default layout unless block_ids is given)
    and the meta blob."""
    nbytes = hwkv_mem_estimate(layout, n_seqs) if pool_bytes is None else pool_bytes
    pool = _alloc_aligned(nbytes, device)
    if fill is not None:
        pool.fill_(fill)
    ids = hwkv_table_fill(layout, n_seqs) if block_ids is None else np.asarray(block_ids, np.int32)
    d = layout.desc()
    tbl = _alloc_aligned(ids.size * 4, device).view(torch.int32).view(ids.shape[0],
                                                                     d.blocks_per_seq)
    tbl.copy_(torch.from_numpy(np.ascontiguousarray(ids)))
    meta_host = hwkv_meta_fill(layout)
    meta = _alloc_aligned(meta_host.size, device)
    meta.copy_(torch.from_numpy(meta_host))
    return Cache(layout, pool, tbl, meta, hwkv_meta_fingerprint(meta_host))


def make_workspace(layout: Layout, layer_begin: int, n_layers: int, n_seqs: int, n_q_heads: int,
                   device="cuda") -> torch.Tensor:
    return _alloc_aligned(max(hwkv_workspace_bytes(layout, layer_begin, n_layers, n_seqs,
                                                   n_q_heads), 256), device)


def hwkv_step_workspace_bytes(layout: Layout, layer_begin: int, n_layers: int, n_seqs: int,
                              n_q_heads: int) -> int:
    b = ctypes.c_uint64()
    _check(_lib.hwkv_step_workspace_bytes(layout.handle, layer_begin, n_layers, n_seqs,
                                          n_q_heads, ctypes.byref(b)))
    return int(b.value)


def make_step_workspace(layout: Layout, layer_begin: int, n_layers: int, n_seqs: int,
                        n_q_heads: int, device="cuda") -> torch.Tensor:
    """Workspace of hwkv_decode_step, zero-filled once (its arrival counters
    must start at zero; every call leaves them at zero)."""
    ws = _alloc_aligned(hwkv_step_workspace_bytes(layout, layer_begin, n_layers, n_seqs,
                                                  n_q_heads), device)
    ws.zero_()
    return ws


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(name: str, t: Optional[torch.Tensor], shape, dtype) -> None:
    """The C ABI sees only pointers: make sure each tensor really has the
    extent the call will touch (a short tensor would be read out of bounds)."""
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))


def _expect_opt(name: str, t: Optional[torch.Tensor], shape, dtype) -> None:
    if t is not None:
        _expect(name, t, shape, dtype)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def hwkv_append(cache: Cache, layer_begin: int, n_layers: int, pos0: torch.Tensor,
                k: torch.Tensor, v: torch.Tensor, seq_slots: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """k, v: [n_layers][n_seqs][n_new][n_kv_heads][head_dim] device tensors."""
    d = cache.layout.desc()
    n_seqs, n_new = int(k.shape[1]), int(k.shape[2])
    kv_shape = (n_layers, n_seqs, n_new, d.n_kv_heads, d.head_dim)
    _expect("k", k, kv_shape, torch_dtype(d.dtype))
    _expect("v", v, kv_shape, torch_dtype(d.dtype))
    _expect("pos0", pos0, (n_seqs,), torch.int64)
    _expect_opt("seq_slots", seq_slots, (n_seqs,), torch.int32)
    cv = cache.view()
    _check(_lib.hwkv_append(cache.layout.handle, ctypes.byref(cv), layer_begin, n_layers, n_seqs,
                            _ptr(seq_slots), _ptr(pos0), n_new, _ptr(k), _ptr(v),
                            _stream(stream)))


def hwkv_decode_split(cache: Cache, layer_begin: int, n_layers: int, ctx_len: torch.Tensor,
                      q: torch.Tensor, scale: float, workspace: torch.Tensor,
                      seq_slots: Optional[torch.Tensor] = None, stream=None) -> None:
    """q: [n_layers][n_seqs][n_q_heads][head_dim]."""
    d = cache.layout.desc()
    _expect("q", q, (n_layers, q.shape[1], q.shape[2], d.head_dim), torch_dtype(d.dtype))
    _expect("ctx_len", ctx_len, (q.shape[1],), torch.int64)
    _expect_opt("seq_slots", seq_slots, (q.shape[1],), torch.int32)
    cv = cache.view()
    _check(_lib.hwkv_decode_split(cache.layout.handle, ctypes.byref(cv), layer_begin, n_layers,
                                  int(q.shape[1]), _ptr(seq_slots), _ptr(ctx_len), int(q.shape[2]),
                                  _ptr(q), scale, _ptr(workspace), workspace.numel(),
                                  _stream(stream)))


def hwkv_decode_merge(cache: Cache, layer_begin: int, n_layers: int, ctx_len: torch.Tensor,
                      workspace: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    d = cache.layout.desc()
    if out.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise ValueError("out must be float32, bfloat16 or float16")
    _expect("out", out, (n_layers, out.shape[1], out.shape[2], d.head_dim), out.dtype)
    _expect("ctx_len", ctx_len, (out.shape[1],), torch.int64)
    cv = cache.view()
    _check(_lib.hwkv_decode_merge(cache.layout.handle, ctypes.byref(cv), layer_begin, n_layers,
                                  int(out.shape[1]), _ptr(ctx_len), int(out.shape[2]),
                                  _ptr(workspace), workspace.numel(), _ptr(out),
                                  _dtype_code(out.dtype), _stream(stream)))


def hwkv_decode_attn(cache: Cache, layer_begin: int, n_layers: int, ctx_len: torch.Tensor,
                     q: torch.Tensor, scale: float, workspace: torch.Tensor, out: torch.Tensor,
                     seq_slots: Optional[torch.Tensor] = None, stream=None) -> None:
    """out: [n_layers][n_seqs][n_q_heads][head_dim] float32 or bfloat16."""
    d = cache.layout.desc()
    _expect("q", q, (n_layers, q.shape[1], q.shape[2], d.head_dim), torch_dtype(d.dtype))
    if out.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise ValueError("out must be float32, bfloat16 or float16")
    _expect("out", out, tuple(q.shape), out.dtype)
    _expect("ctx_len", ctx_len, (q.shape[1],), torch.int64)
    _expect_opt("seq_slots", seq_slots, (q.shape[1],), torch.int32)
    cv = cache.view()
    _check(_lib.hwkv_decode_attn(cache.layout.handle, ctypes.byref(cv), layer_begin, n_layers,
                                 int(q.shape[1]), _ptr(seq_slots), _ptr(ctx_len), int(q.shape[2]),
                                 _ptr(q), scale, _ptr(workspace), workspace.numel(), _ptr(out),
                                 _dtype_code(out.dtype), _stream(stream)))


def _decode_with_append(fn, cache: Cache, layer_begin: int, n_layers: int, pos: torch.Tensor,
                     k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, scale: float,
                     workspace: torch.Tensor, out: torch.Tensor,
                     seq_slots: Optional[torch.Tensor] = None, stream=None) -> None:
    d = cache.layout.desc()
    n_seqs, n_q = int(q.shape[1]), int(q.shape[2])
    _expect("q", q, (n_layers, n_seqs, n_q, d.head_dim), torch_dtype(d.dtype))
    kv_shape = (n_layers, n_seqs, d.n_kv_heads, d.head_dim)
    if k_new.dim() == 5:
        kv_shape = (n_layers, n_seqs, 1, d.n_kv_heads, d.head_dim)
    _expect("k_new", k_new, kv_shape, torch_dtype(d.dtype))
    _expect("v_new", v_new, kv_shape, torch_dtype(d.dtype))
    if out.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise ValueError("out must be float32, bfloat16 or float16")
    _expect("out", out, tuple(q.shape), out.dtype)
    _expect("pos", pos, (n_seqs,), torch.int64)
    _expect_opt("seq_slots", seq_slots, (n_seqs,), torch.int32)
    cv = cache.view()
    _check(fn(cache.layout.handle, ctypes.byref(cv), layer_begin, n_layers, n_seqs,
              _ptr(seq_slots), _ptr(pos), _ptr(k_new), _ptr(v_new), n_q, _ptr(q), scale,
              _ptr(workspace), workspace.numel(), _ptr(out), _dtype_code(out.dtype),
              _stream(stream)))


def hwkv_decode_split_append(cache: Cache, layer_begin: int, n_layers: int, pos: torch.Tensor,
                             k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                             scale: float, workspace: torch.Tensor,
                             seq_slots: Optional[torch.Tensor] = None, stream=None) -> None:
    """First stage of hwkv_decode_append_attn; follow with hwkv_decode_merge
    at ctx_len = pos + 1."""
    d = cache.layout.desc()
    n_seqs, n_q = int(q.shape[1]), int(q.shape[2])
    _expect("q", q, (n_layers, n_seqs, n_q, d.head_dim), torch_dtype(d.dtype))
    kv_shape = (n_layers, n_seqs, d.n_kv_heads, d.head_dim)
    if k_new.dim() == 5:
        kv_shape = (n_layers, n_seqs, 1, d.n_kv_heads, d.head_dim)
    _expect("k_new", k_new, kv_shape, torch_dtype(d.dtype))
    _expect("v_new", v_new, kv_shape, torch_dtype(d.dtype))
    _expect("pos", pos, (n_seqs,), torch.int64)
    _expect_opt("seq_slots", seq_slots, (n_seqs,), torch.int32)
    cv = cache.view()
    _check(_lib.hwkv_decode_split_append(cache.layout.handle, ctypes.byref(cv), layer_begin,
                                         n_layers, n_seqs, _ptr(seq_slots), _ptr(pos),
                                         _ptr(k_new), _ptr(v_new), n_q, _ptr(q), scale,
                                         _ptr(workspace), workspace.numel(), _stream(stream)))


def hwkv_decode_append_attn(cache: Cache, layer_begin: int, n_layers: int, pos: torch.Tensor,
                            k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                            scale: float, workspace: torch.Tensor, out: torch.Tensor,
                            seq_slots: Optional[torch.Tensor] = None, stream=None) -> None:
    """Append of the token at position pos[b] and decode at context pos[b]+1
    in two launches (the split stage appends).  k_new, v_new:
    [n_layers][n_seqs][n_kv_heads][head_dim] (or with a unit token axis);
    q, out: [n_layers][n_seqs][n_q_heads][head_dim]; workspace: make_workspace."""
    _decode_with_append(_lib.hwkv_decode_append_attn, cache, layer_begin, n_layers, pos, k_new,
                        v_new, q, scale, workspace, out, seq_slots, stream)


def hwkv_decode_append_attn_static(cache: Cache, layer_begin: int, n_layers: int,
                                   pos: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                   q: torch.Tensor, scale: float, out: torch.Tensor,
                                   seq_slots: Optional[torch.Tensor] = None, stream=None) -> None:
    """hwkv_decode_append_attn with the split records in the library's static
    scratch (no workspace argument; the call allocates nothing)."""
    d = cache.layout.desc()
    n_seqs, n_q = int(q.shape[1]), int(q.shape[2])
    _expect("q", q, (n_layers, n_seqs, n_q, d.head_dim), torch_dtype(d.dtype))
    kv_shape = (n_layers, n_seqs, d.n_kv_heads, d.head_dim)
    if k_new.dim() == 5:
        kv_shape = (n_layers, n_seqs, 1, d.n_kv_heads, d.head_dim)
    _expect("k_new", k_new, kv_shape, torch_dtype(d.dtype))
    _expect("v_new", v_new, kv_shape, torch_dtype(d.dtype))
    if out.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise ValueError("out must be float32, bfloat16 or float16")
    _expect("out", out, tuple(q.shape), out.dtype)
    _expect("pos", pos, (n_seqs,), torch.int64)
    _expect_opt("seq_slots", seq_slots, (n_seqs,), torch.int32)
    cv = cache.view()
    _check(_lib.hwkv_decode_append_attn_static(
        cache.layout.handle, ctypes.byref(cv), layer_begin, n_layers, n_seqs, _ptr(seq_slots),
        _ptr(pos), _ptr(k_new), _ptr(v_new), n_q, _ptr(q), scale, _ptr(out),
        _dtype_code(out.dtype), _stream(stream)))


def hwkv_decode_step(cache: Cache, layer_begin: int, n_layers: int, pos: torch.Tensor,
                     k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, scale: float,
                     workspace: torch.Tensor, out: torch.Tensor,
                     seq_slots: Optional[torch.Tensor] = None, stream=None) -> None:
    """The same step in one launch (the last split of each head merges);
    workspace: make_step_workspace."""
    _decode_with_append(_lib.hwkv_decode_step, cache, layer_begin, n_layers, pos, k_new, v_new,
                        q, scale, workspace, out, seq_slots, stream)


def hwkv_prefill_workspace_bytes(layout: Layout, layer: int, n_seqs: int, n_chunk: int) -> int:
    b = ctypes.c_uint64()
    _check(_lib.hwkv_prefill_workspace_bytes(layout.handle, layer, n_seqs, n_chunk,
                                             ctypes.byref(b)))
    return int(b.value)


def make_prefill_workspace(layout: Layout, layer: int, n_seqs: int, n_chunk: int,
                           device="cuda") -> torch.Tensor:
    """Workspace of hwkv_prefill_attn (at least 256 bytes, so never empty)."""
    return _alloc_aligned(max(hwkv_prefill_workspace_bytes(layout, layer, n_seqs, n_chunk), 256),
                          device)


def hwkv_prefill_attn(cache: Cache, layer: int, pos0: torch.Tensor, q: torch.Tensor,
                      k: torch.Tensor, v: torch.Tensor, workspace: Optional[torch.Tensor],
                      out: torch.Tensor, scale: float, seq_slots: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """q, out: [n_seqs][n_chunk][n_q_heads][head_dim]; k, v: [n_seqs][n_chunk][n_kv][head_dim].
    P enters the P.V product in fp16; workspace: make_prefill_workspace (None
    for fp16 caches, which need none)."""
    _prefill(_lib.hwkv_prefill_attn, cache, layer, pos0, q, k, v, workspace, out, scale,
             seq_slots, stream)


def hwkv_prefill_attn_exact(cache: Cache, layer: int, pos0: torch.Tensor, q: torch.Tensor,
                            k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, scale: float,
                            seq_slots: Optional[torch.Tensor] = None, stream=None) -> None:
    """hwkv_prefill_attn with P split into two bf16 products for bf16 caches (no workspace)."""
    _prefill(_lib.hwkv_prefill_attn_exact, cache, layer, pos0, q, k, v, None, out, scale,
             seq_slots, stream)


def _prefill(fn, cache, layer, pos0, q, k, v, workspace, out, scale, seq_slots, stream) -> None:
    d = cache.layout.desc()
    n_seqs, n_chunk, n_q = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    _expect("q", q, (n_seqs, n_chunk, n_q, d.head_dim), torch_dtype(d.dtype))
    _expect("k", k, (n_seqs, n_chunk, d.n_kv_heads, d.head_dim), torch_dtype(d.dtype))
    _expect("v", v, (n_seqs, n_chunk, d.n_kv_heads, d.head_dim), torch_dtype(d.dtype))
    if out.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise ValueError("out must be float32, bfloat16 or float16")
    _expect("out", out, tuple(q.shape), out.dtype)
    _expect("pos0", pos0, (n_seqs,), torch.int64)
    _expect_opt("seq_slots", seq_slots, (n_seqs,), torch.int32)
    cv = cache.view()
    head = (cache.layout.handle, ctypes.byref(cv), layer, int(q.shape[0]), _ptr(seq_slots),
            _ptr(pos0), int(q.shape[1]), int(q.shape[2]), _ptr(q), _ptr(k), _ptr(v))
    tail = (_ptr(out), _dtype_code(out.dtype), scale, _stream(stream))
    if fn is _lib.hwkv_prefill_attn:
        # None is passed on as a null workspace of 0 bytes, which the library
        # accepts only where none is needed (fp16 caches)
        if workspace is not None and (workspace.dtype != torch.uint8 or
                                      workspace.device != out.device):
            raise ValueError("workspace must be a uint8 tensor on the device of out "
                             "(make_prefill_workspace)")
        _check(fn(*head, _ptr(workspace), 0 if workspace is None else workspace.numel(),
                  *tail))
    else:
        _check(fn(*head, *tail))


def loaded_library_path() -> str:
    return LIB_PATH
