"""CPU oracle of the per-head windowed KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports it and it never imports the product.

The arithmetic lives in ``hwkv_oracle.c`` (plain C, fp64, OpenMP over
independent outputs); this module only marshals numpy arrays to it.  Every
function follows a definition from the pages on HeadWiseKV's grouped-cache
runtime (cited in the C source by page title and section).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hwkv_oracle.c")
_LIB = os.path.join(_HERE, "libhwkv_oracle.so")

ELEM_F32 = 0
ELEM_BF16 = 1
ELEM_F16 = 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP) into ``libhwkv_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i32, i64, u64, dbl, vp = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.hwkvref_blocks.restype = i64
        lib.hwkvref_blocks.argtypes = [i64, i64]
        lib.hwkvref_layout.restype = i64
        lib.hwkvref_layout.argtypes = [i32, i32, vp, i32, vp, vp]
        lib.hwkvref_mem_estimate.restype = u64
        lib.hwkvref_mem_estimate.argtypes = [i32, i32, vp, i32, i32, i32, i64]
        lib.hwkvref_default_table.restype = None
        lib.hwkvref_default_table.argtypes = [i64, i64, vp]
        lib.hwkvref_ring_slot.restype = None
        lib.hwkvref_ring_slot.argtypes = [i64, i32, i32, vp, vp]
        lib.hwkvref_append.restype = i32
        lib.hwkvref_append.argtypes = [vp, u64, vp, i64, vp, i32, i32, i32, i32,
                                       i32, i32, i32, i32, vp, vp, i32, vp, vp]
        for name in ("hwkvref_decode", "hwkvref_decode_masked"):
            f = getattr(lib, name)
            f.restype = i32
            f.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                          i64, dbl, vp]
        lib.hwkvref_prefill.restype = i32
        lib.hwkvref_prefill.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32, vp,
                                        vp, vp, vp, vp, vp, i64, i32, vp, dbl, vp]
        lib.hwkvref_widen.restype = None
        lib.hwkvref_widen.argtypes = [vp, i64, i32, vp]
        lib.hwkvref_threads.restype = i32
        lib.hwkvref_threads.argtypes = []
        lib.hwkvref_set_threads.restype = None
        lib.hwkvref_set_threads.argtypes = [i32]
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def elem_code(raw: np.ndarray) -> int:
    """fp32 arrays are float32; bf16 arrays are carried as their uint16 bits;
    fp16 arrays are numpy float16 (also only bits to the C side)."""
    if raw.dtype == np.float32:
        return ELEM_F32
    if raw.dtype == np.uint16:
        return ELEM_BF16
    if raw.dtype == np.float16:
        return ELEM_F16
    raise TypeError("oracle inputs are float32, bf16 bits (uint16) or float16, got %s"
                    % raw.dtype)


def widen(raw: np.ndarray) -> np.ndarray:
    """The oracle's own widening of stored elements to float64."""
    raw = np.ascontiguousarray(raw)
    out = np.zeros(raw.size, np.float64)
    _load().hwkvref_widen(_ptr(raw), raw.size, elem_code(raw), _ptr(out))
    return out.reshape(raw.shape)


def threads() -> int:
    return int(_load().hwkvref_threads())


def set_threads(n: int) -> None:
    _load().hwkvref_set_threads(int(n))


def blocks(window: int, block_size: int) -> int:
    return int(_load().hwkvref_blocks(int(window), int(block_size)))


def layout(windows: np.ndarray, block_size: int):
    """Returns (nblocks [L*H] int32, head_off [L*H+1] int64, blocks_per_seq)."""
    w = _i32(windows)
    n_layers, n_kv = w.shape
    nb = np.zeros(n_layers * n_kv, np.int32)
    off = np.zeros(n_layers * n_kv + 1, np.int64)
    bps = _load().hwkvref_layout(n_layers, n_kv, _ptr(w), int(block_size), _ptr(nb), _ptr(off))
    if bps < 0:
        raise ValueError("invalid layout")
    return nb, off, int(bps)


def mem_estimate(windows: np.ndarray, block_size: int, head_dim: int, elem_bytes: int,
                 n_seqs: int) -> int:
    w = _i32(windows)
    n_layers, n_kv = w.shape
    return int(_load().hwkvref_mem_estimate(n_layers, n_kv, _ptr(w), int(block_size),
                                            int(head_dim), int(elem_bytes), int(n_seqs)))


def default_table(n_seqs: int, blocks_per_seq: int) -> np.ndarray:
    ids = np.zeros(n_seqs * blocks_per_seq, np.int32)
    _load().hwkvref_default_table(int(n_seqs), int(blocks_per_seq), _ptr(ids))
    return ids.reshape(n_seqs, blocks_per_seq)


def ring_slot(t: int, block_size: int, nblocks: int):
    j = np.zeros(1, np.int32)
    r = np.zeros(1, np.int32)
    _load().hwkvref_ring_slot(int(t), int(block_size), int(nblocks), _ptr(j), _ptr(r))
    return int(j[0]), int(r[0])


def append(pool: np.ndarray, block_ids: np.ndarray, windows: np.ndarray, block_size: int,
           head_dim: int, layer_begin: int, pos0: Sequence[int], k: np.ndarray,
           v: np.ndarray, seq_slots: Optional[Sequence[int]] = None) -> None:
    """In-place model of the append on a host copy of the pool (uint8 bytes).

    k, v: [n_layers][n_seqs][n_new][n_kv_heads][head_dim] float32 or bf16 bits.
    """
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    w = _i32(windows)
    ids = _i32(block_ids)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    n_layers, n_seqs, n_new, n_kv, d = k.shape
    assert v.shape == k.shape and d == head_dim and n_kv == w.shape[1]
    slots = None if seq_slots is None else _i32(seq_slots)
    p0 = _i64(pos0)
    rc = _load().hwkvref_append(_ptr(pool), pool.nbytes, _ptr(ids), ids.shape[0], _ptr(w),
                                w.shape[0], w.shape[1], int(block_size), int(head_dim),
                                elem_code(k), int(layer_begin), n_layers, n_seqs,
                                _ptr(slots), _ptr(p0), n_new, _ptr(k), _ptr(v))
    if rc != 0:
        raise ValueError("oracle append rejected its arguments (%d)" % rc)


def decode(windows: np.ndarray, ctx_len: Sequence[int], q: np.ndarray, k_hist: np.ndarray,
           v_hist: np.ndarray, hist_base: Sequence[int], scale: float,
           masked: bool = False) -> np.ndarray:
    """Windowed decode attention in fp64.

    windows: [n_layers][n_kv]; q: [n_layers][n_seqs][n_q][d];
    k_hist, v_hist: [n_layers][n_seqs][T][n_kv][d] holding positions
    [hist_base[b], hist_base[b]+T).  Returns float64 shaped like q.
    """
    w = _i32(windows)
    q = np.ascontiguousarray(q)
    k_hist = np.ascontiguousarray(k_hist)
    v_hist = np.ascontiguousarray(v_hist)
    n_layers, n_seqs, n_q, d = q.shape
    _, _, T, n_kv, _ = k_hist.shape
    assert w.shape == (n_layers, n_kv) and n_q % n_kv == 0
    assert k_hist.dtype == q.dtype == v_hist.dtype
    out = np.zeros(q.shape, np.float64)
    L = _i64(ctx_len)
    base = _i64(hist_base)
    fn = _load().hwkvref_decode_masked if masked else _load().hwkvref_decode
    rc = fn(n_layers, n_seqs, n_kv, n_q // n_kv, d, elem_code(q), _ptr(w), _ptr(L), _ptr(q),
            _ptr(k_hist), _ptr(v_hist), _ptr(base), T, float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments (%d)" % rc)
    return out


def prefill(windows: Sequence[int], pos0: Sequence[int], q: np.ndarray, k_chunk: np.ndarray,
            v_chunk: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray,
            hist_base: Sequence[int], scale: float,
            rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Windowed causal prefill of one layer in fp64.

    q: [n_seqs][n][n_q][d]; k_chunk, v_chunk: [n_seqs][n][n_kv][d];
    k_hist, v_hist: [n_seqs][T][n_kv][d] for positions [hist_base[b], +T).
    Returns float64 [n_seqs][len(rows)][n_q][d].
    """
    w = _i32(windows)
    q = np.ascontiguousarray(q)
    k_chunk = np.ascontiguousarray(k_chunk)
    v_chunk = np.ascontiguousarray(v_chunk)
    k_hist = np.ascontiguousarray(k_hist)
    v_hist = np.ascontiguousarray(v_hist)
    n_seqs, n, n_q, d = q.shape
    n_kv = k_chunk.shape[2]
    T = k_hist.shape[1]
    r = _i32(np.arange(n) if rows is None else rows)
    p0 = _i64(pos0)
    base = _i64(hist_base)
    out = np.zeros((n_seqs, r.size, n_q, d), np.float64)
    rc = _load().hwkvref_prefill(n_seqs, n_kv, n_q // n_kv, d, elem_code(q), _ptr(w),
                                 _ptr(p0), n, _ptr(q), _ptr(k_chunk), _ptr(v_chunk),
                                 _ptr(k_hist), _ptr(v_hist), _ptr(base), T,
                                 r.size, _ptr(r), float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments (%d)" % rc)
    return out
