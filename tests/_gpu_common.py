"""Helpers shared by the GPU parity tests (imported only by tests marked gpu)."""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

import oracle
import synth

BF16_TOL = 2e-3
F32_TOL = 1e-5
# Regression bound for decode with fp32 outputs, far below the acceptance
# gates: the kernels accumulate exact 16-bit products in fp32 and measure
# ~3e-7 row error even over 64K-token windows.  On these near-uniform 64K
# windows one token dropped or counted twice moves a row's error by about
# 4e-3, only ~2x the 2e-3 gate, so this bound is what catches an off-by-one
# at a split or ring seam.
DECODE_REGRESSION_TOL = 1e-5
# fp16 caches: inputs are exact 16-bit values and the kernels accumulate in
# fp32 exactly as for bf16, so the bf16 gate applies
F16_TOL = 2e-3


def tol(dtype) -> float:
    return F32_TOL if dtype == torch.float32 else BF16_TOL


def say(*a):
    """Print and flush a line that names the case about to run on the GPU."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def hw():
    import head_windowed_kv_amd as m  # fails loudly when libhwkv.so is missing
    return m


def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda", 0)


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over output rows of max|o - r| / max|r| (rows = last axis)."""
    o = out.reshape(-1, out.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.abs(o - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if o.size else 0.0


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 (round to nearest even via torch) -> fp64."""
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_ulps_apart(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place between two bf16-valued arrays."""
    ia = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64)
    ib = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64)
    # map sign-magnitude to a monotone integer line
    ia = np.where(ia < 0, -32768 - ia, ia)
    ib = np.where(ib < 0, -32768 - ib, ib)
    return np.abs(ia - ib)


def f16_ulps_apart(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in binary16 units in the last place; each array is rounded
    to binary16 first (numpy rounds to nearest even)."""
    ia = a.astype(np.float16).view(np.int16).astype(np.int64)
    ib = b.astype(np.float16).view(np.int16).astype(np.int64)
    ia = np.where(ia < 0, -32768 - ia, ia)
    ib = np.where(ib < 0, -32768 - ib, ib)
    return np.abs(ia - ib)


@dataclass
class DecodeCase:
    """A cache filled by appending a logical token stream, plus one decode step.

    For sequence b the history holds positions [base[b], ctx[b]-1); the decode
    step appends position ctx[b]-1 and attends at context ctx[b]."""
    lay: object
    cache: object
    windows: np.ndarray
    dtype: torch.dtype
    head_dim: int
    group: int
    ctx: List[int]
    base: List[int]
    slots: Optional[List[int]]
    q: torch.Tensor = None
    k_hist: np.ndarray = None   # host raw [n_layers][n_seqs][T][n_kv][d]
    v_hist: np.ndarray = None
    k_new: torch.Tensor = None  # device [n_layers][n_seqs][1][n_kv][d]
    v_new: torch.Tensor = None
    T: int = 0
    extras: dict = field(default_factory=dict)


def build_decode_case(windows, dtype, head_dim, group, ctx, seed, split_tokens=0,
                      slots=None, table_rows=None, block_ids=None, hist_margin=37,
                      fill=0xFF, chunk=None, block_size=16) -> DecodeCase:
    """Fill a cache (pool pre-filled with NaN bytes so that any read outside
    what was appended shows up) by appending each sequence's history."""
    H = hw()
    dev = device()
    windows = np.asarray(windows, np.int32)
    n_layers, n_kv = windows.shape
    n_seqs = len(ctx)
    lay = H.hwkv_layout_create(windows, block_size, head_dim, dtype, split_tokens)
    rows = table_rows or n_seqs
    cache = H.make_cache(lay, rows, device=dev, block_ids=block_ids, fill=fill)
    wmax = int(windows.max())
    base = [max(0, c - 1 - (wmax + hist_margin)) for c in ctx]
    T = max(c - b for c, b in zip(ctx, base))
    n_q = n_kv * group
    g = synth.gen(seed, dev)
    q = synth.randn((n_layers, n_seqs, n_q, head_dim), dtype, g, std=1.0 / math.sqrt(head_dim))
    raw_dt = {torch.float32: np.float32, torch.float16: np.float16}.get(dtype, np.uint16)
    k_hist = np.zeros((n_layers, n_seqs, T, n_kv, head_dim), raw_dt)
    v_hist = np.zeros_like(k_hist)
    k_new = torch.empty((n_layers, n_seqs, 1, n_kv, head_dim), dtype=dtype, device=dev)
    v_new = torch.empty_like(k_new)
    for b in range(n_seqs):
        nh = ctx[b] - 1 - base[b]
        kb = synth.randn((n_layers, 1, nh + 1, n_kv, head_dim), dtype, g)
        vb = synth.randn((n_layers, 1, nh + 1, n_kv, head_dim), dtype, g)
        k_hist[:, b, :nh + 1] = synth.to_raw(kb[:, 0])
        v_hist[:, b, :nh + 1] = synth.to_raw(vb[:, 0])
        k_new[:, b] = kb[:, 0, nh:]
        v_new[:, b] = vb[:, 0, nh:]
        slot = torch.tensor([slots[b] if slots else b], dtype=torch.int32, device=dev)
        step = chunk or max(nh, 1)
        t = 0
        while t < nh:
            n = min(step, nh - t)
            pos = torch.tensor([base[b] + t], dtype=torch.int64, device=dev)
            H.hwkv_append(cache, 0, n_layers, pos, kb[:, :, t:t + n].contiguous(),
                          vb[:, :, t:t + n].contiguous(), seq_slots=slot)
            t += n
    torch.cuda.synchronize()
    return DecodeCase(lay, cache, windows, dtype, head_dim, group, list(ctx), base, slots, q,
                      k_hist, v_hist, k_new, v_new, T)


def run_decode_step(c: DecodeCase, out_dtype=torch.float32, layer_begin=0, n_layers=None,
                    scale=None, split_only=False):
    """Append position ctx-1 of every sequence, then decode at ctx."""
    H = hw()
    dev = device()
    n_layers = c.windows.shape[0] if n_layers is None else n_layers
    n_seqs = len(c.ctx)
    slots = None if c.slots is None else torch.tensor(c.slots, dtype=torch.int32, device=dev)
    pos = torch.tensor([x - 1 for x in c.ctx], dtype=torch.int64, device=dev)
    ctx = torch.tensor(c.ctx, dtype=torch.int64, device=dev)
    H.hwkv_append(c.cache, layer_begin, n_layers, pos,
                  c.k_new[layer_begin:layer_begin + n_layers].contiguous(),
                  c.v_new[layer_begin:layer_begin + n_layers].contiguous(), seq_slots=slots)
    n_q = c.windows.shape[1] * c.group
    ws = H.make_workspace(c.lay, layer_begin, n_layers, n_seqs, n_q, device=dev)
    out = torch.full((n_layers, n_seqs, n_q, c.head_dim), float("nan"), dtype=out_dtype,
                     device=dev)
    s = 1.0 / math.sqrt(c.head_dim) if scale is None else scale
    H.hwkv_decode_attn(c.cache, layer_begin, n_layers, ctx,
                       c.q[layer_begin:layer_begin + n_layers].contiguous(), s, ws, out,
                       seq_slots=slots)
    torch.cuda.synchronize()
    return out


def oracle_decode(c: DecodeCase, layer_begin=0, n_layers=None, scale=None) -> np.ndarray:
    n_layers = c.windows.shape[0] if n_layers is None else n_layers
    sl = slice(layer_begin, layer_begin + n_layers)
    s = 1.0 / math.sqrt(c.head_dim) if scale is None else scale
    return oracle.decode(c.windows[sl], c.ctx, synth.to_raw(c.q[sl]), c.k_hist[sl], c.v_hist[sl],
                         c.base, s)


def layer_seed(seed: int, layer: int) -> int:
    return seed * 100003 + layer


def gen_layer_kv(seed: int, layer: int, n_seqs: int, n_tok: int, n_kv: int, d: int, dtype,
                 dev):
    """K/V of one layer's token stream, [1][n_seqs][n_tok][n_kv][d]; the same
    (seed, layer) always regenerates the same values on the same device."""
    g = synth.gen(layer_seed(seed, layer), dev)
    k = synth.randn((1, n_seqs, n_tok, n_kv, d), dtype, g)
    v = synth.randn((1, n_seqs, n_tok, n_kv, d), dtype, g)
    return k, v


@dataclass
class StackCase:
    """All sequences share one context L.  Layer l's stream holds positions
    [base, L] (history plus the token of the decode step), base = L - n_hist,
    n_hist = min(L, largest ring capacity)."""
    lay: object
    cache: object
    windows: np.ndarray
    dtype: torch.dtype
    head_dim: int
    group: int
    L: int
    n_seqs: int
    seed: int
    n_hist: int
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor


def build_stack_case(windows, dtype, head_dim, group, L, n_seqs, seed, split_tokens=0,
                     block_size=16):
    H = hw()
    dev = device()
    windows = np.asarray(windows, np.int32)
    n_layers, n_kv = windows.shape
    lay = H.hwkv_layout_create(windows, block_size, head_dim, dtype, split_tokens)
    cache = H.make_cache(lay, n_seqs, device=dev, fill=0xFF)
    cap = int(((windows.astype(np.int64) + block_size - 1) // block_size * block_size).max())
    n_hist = min(L, cap)
    base = L - n_hist
    q = synth.randn((n_layers, n_seqs, n_kv * group, head_dim), dtype, synth.gen(seed, dev),
                    std=1.0 / math.sqrt(head_dim))
    k_new = torch.empty((n_layers, n_seqs, 1, n_kv, head_dim), dtype=dtype, device=dev)
    v_new = torch.empty_like(k_new)
    pos = torch.full((n_seqs,), base, dtype=torch.int64, device=dev)
    for l in range(n_layers):
        k, v = gen_layer_kv(seed, l, n_seqs, n_hist + 1, n_kv, head_dim, dtype, dev)
        if n_hist > 0:
            H.hwkv_append(cache, l, 1, pos, k[:, :, :n_hist].contiguous(),
                          v[:, :, :n_hist].contiguous())
        k_new[l] = k[0, :, n_hist:]
        v_new[l] = v[0, :, n_hist:]
        del k, v
    torch.cuda.synchronize()
    return StackCase(lay, cache, windows, dtype, head_dim, group, L, n_seqs, seed, n_hist, q,
                     k_new, v_new)


def stack_step(c: StackCase, out_dtype=torch.float32):
    """Append token L of every layer and sequence (one launch), then decode all
    layers at context L+1 (one split and one merge launch)."""
    H = hw()
    dev = device()
    n_layers, n_kv = c.windows.shape
    pos = torch.full((c.n_seqs,), c.L, dtype=torch.int64, device=dev)
    ctx = torch.full((c.n_seqs,), c.L + 1, dtype=torch.int64, device=dev)
    H.hwkv_append(c.cache, 0, n_layers, pos, c.k_new, c.v_new)
    ws = H.make_workspace(c.lay, 0, n_layers, c.n_seqs, n_kv * c.group, device=dev)
    out = torch.full((n_layers, c.n_seqs, n_kv * c.group, c.head_dim), float("nan"),
                     dtype=out_dtype, device=dev)
    H.hwkv_decode_attn(c.cache, 0, n_layers, ctx, c.q, 1.0 / math.sqrt(c.head_dim), ws, out)
    torch.cuda.synchronize()
    return out


def stack_oracle_layer(c: StackCase, layer: int) -> np.ndarray:
    """Oracle output of one layer, from the regenerated logical stream."""
    n_layers, n_kv = c.windows.shape
    k, v = gen_layer_kv(c.seed, layer, c.n_seqs, c.n_hist + 1, n_kv, c.head_dim, c.dtype,
                        device())
    kh, vh = synth.to_raw(k), synth.to_raw(v)
    del k, v
    return oracle.decode(c.windows[layer:layer + 1], [c.L + 1] * c.n_seqs,
                         synth.to_raw(c.q[layer:layer + 1]), kh, vh,
                         [c.L - c.n_hist] * c.n_seqs, 1.0 / math.sqrt(c.head_dim))
