"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no part of the attention or cache arithmetic: it only draws
random tensors of the workloads' shapes and converts bf16 tensors to the raw
uint16 bit patterns that the CPU oracle reads.  Values are drawn in fp32 and
rounded once to bf16 (round-to-nearest-even, torch's ``.to``), so both sides
consume identical bits.

Workload shapes follow the HeadWiseKV write-up (KnoAI), sections 摘要
(112K / 161K contexts) and 核心技术 1-2 (window levels 1024 / 4096 / 16384 /
65536; 8 KV heads per layer, 48 layers; the two printed window vectors).
"""
from __future__ import annotations

import numpy as np
import torch

#: window levels printed for the per-head window vector (HeadWiseKV page,
#: 核心技术 1, definition of w_i)
WINDOW_LEVELS = (1024, 4096, 16384, 65536)

#: the two window vectors printed in the policy example (HeadWiseKV page,
#: 核心技术 2, the YAML policy), layer_id 0 and layer_id 1
YAML_LAYER0 = (4096, 4096, 16384, 16384, 65536, 65536, 65536, 65536)
YAML_LAYER1 = (1024, 4096, 4096, 16384, 16384, 65536, 65536, 65536)

#: "K" read as 1024 tokens
CTX_112K = 112 * 1024
CTX_161K = 161 * 1024


def stack_windows(n_layers: int = 48, n_kv_heads: int = 8, seed: int = 0) -> np.ndarray:
    """Per-(layer, head) windows drawn from the four levels with weights
    0.2/0.3/0.3/0.2, layer-major, from ``numpy.random.default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    w = rng.choice(np.array(WINDOW_LEVELS), size=(n_layers, n_kv_heads),
                   p=[0.2, 0.3, 0.3, 0.2])
    return w.astype(np.int32)


def hybrid_windows(n_layers: int = 48, n_kv_heads: int = 8, swa: int = 4096, every: int = 4,
                   seed: int = 0) -> np.ndarray:
    """A hybrid stack: layer l with l % every == every - 1 is a global layer
    whose per-head windows are those of ``stack_windows(..., seed)``; every
    other layer is a sliding-window layer whose heads all keep ``swa`` tokens."""
    w = stack_windows(n_layers, n_kv_heads, seed)
    w[(np.arange(n_layers) % every) != every - 1] = swa
    return w


def gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, dtype: torch.dtype, generator: torch.Generator, std: float = 1.0,
          device=None) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 on the generator's device, rounded once to dtype."""
    dev = generator.device if device is None else device
    x = torch.randn(tuple(shape), generator=generator, dtype=torch.float32, device=dev)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def to_raw(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor's stored values: float32 stays float32,
    bfloat16 becomes its uint16 bit patterns, float16 stays float16."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.numpy()
    raise TypeError("unsupported dtype %s" % t.dtype)


def raw_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of float32 / bf16-bit arrays to float64."""
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float16:
        return a.astype(np.float64)
    raise TypeError(a.dtype)


def cb_contexts(n_seqs: int = 32, seed: int = 1) -> np.ndarray:
    """Context lengths of the continuous decode batch: uniform integers in
    [4K, 160K] from numpy default_rng(seed)."""
    return np.random.default_rng(seed).integers(4096, 160 * 1024, n_seqs, endpoint=True)


def fill_normal(buf_u8: torch.Tensor, seed: int, progress: bool = False) -> None:
    """Fill a raw byte buffer (a whole KV pool) with N(0,1) bf16 values from
    torch's generator, in pieces of 2^29 elements (a line per 16 GiB when
    progress is set)."""
    import sys
    import time
    g = torch.Generator(device=buf_u8.device)
    g.manual_seed(int(seed))
    x = buf_u8.view(torch.bfloat16)
    step = 1 << 29
    t0 = time.time()
    for n, i in enumerate(range(0, x.numel(), step)):
        x[i:i + step].normal_(generator=g)
        if progress and n % 16 == 15:
            torch.cuda.synchronize()
            print("fill: %.0f GiB in %.1f s" % ((i + step) * 2 / 2 ** 30, time.time() - t0),
                  file=sys.stderr, flush=True)
