"""Mixed stacks through the same runtime, on the GPU, against the fp64 oracle.

Covers the layouts beyond the 48-layer benchmark's: fp16 caches, block sizes
32..256 (powers of two; the decode kernel walks 16-token tiles, so the block
size changes only the addressing), uniform-window (sliding-window) layers,
full-attention heads (a window longer than any context) and windows that are
not multiples of the block size.  Bitwise gate: the same logical cache gives
the same output bits whatever the block size and however its blocks are
numbered."""
import math

import numpy as np
import pytest
import torch

import synth
from _gpu_common import (DECODE_REGRESSION_TOL, build_decode_case, build_stack_case, device, hw,
                         oracle_decode, row_rel_err, run_decode_step, say, stack_oracle_layer,
                         stack_step, to_host_f64, tol)

pytestmark = pytest.mark.gpu


def _check(case, out):
    ref = oracle_decode(case)
    got = to_host_f64(out)
    assert np.all(np.isfinite(got))
    err = row_rel_err(got, ref)
    say("max row rel err", err)
    assert err <= tol(case.dtype), err


@pytest.mark.parametrize("d,G", [(128, 3), (64, 2), (128, 1), (64, 8), (128, 6)])
def test_f16_decode_instances(d, G):
    windows = [[40, 700, 1, 2100], [16, 333, 1025, 64]]
    say("f16 decode", d, G)
    c = build_decode_case(windows, torch.float16, d, G, [5, 900, 2500], seed=701, split_tokens=256)
    _check(c, run_decode_step(c))


@pytest.mark.parametrize("dtype,G", [(torch.bfloat16, 1), (torch.bfloat16, 3), (torch.float16, 2),
                                     (torch.float16, 4), (torch.bfloat16, 6), (torch.float16, 8)])
def test_head_dim_256_decode(dtype, G):
    """head_dim 256 (16-bit caches, GQA groups 1 to 8): one 16-byte chunk per
    lane of 32-lane row groups."""
    windows = [[40, 700, 1, 2100], [16, 333, 1025, 64]]
    say("head_dim 256 decode", dtype, G)
    c = build_decode_case(windows, dtype, 256, G, [5, 900, 2500], seed=706, split_tokens=256,
                          block_size=32)
    _check(c, run_decode_step(c))


@pytest.mark.parametrize("G", [3, 8])
def test_head_dim_256_steps_bitwise(G):
    """The appending entry points at head_dim 256 equal append + decode_attn."""
    H = hw()
    dev = device()
    windows = [[64, 1000, 17], [300, 16, 2048]]
    ctx = [2049, 16, 48]
    mk = dict(seed=707, split_tokens=512, chunk=300)
    eager = build_decode_case(windows, torch.bfloat16, 256, G, ctx, **mk)
    two = build_decode_case(windows, torch.bfloat16, 256, G, ctx, **mk)
    one = build_decode_case(windows, torch.bfloat16, 256, G, ctx, **mk)
    say("head_dim 256 steps", G)
    o_e = run_decode_step(eager)
    pos = torch.tensor([x - 1 for x in ctx], device=dev)
    o_t = torch.full_like(o_e, float("nan"))
    H.hwkv_decode_append_attn(two.cache, 0, 2, pos, two.k_new, two.v_new, two.q, 1 / 16.0,
                              H.make_workspace(two.lay, 0, 2, 3, 3 * G, device=dev), o_t)
    o_o = torch.full_like(o_e, float("nan"))
    H.hwkv_decode_step(one.cache, 0, 2, pos, one.k_new, one.v_new, one.q, 1 / 16.0,
                       H.make_step_workspace(one.lay, 0, 2, 3, 3 * G, device=dev), o_o)
    torch.cuda.synchronize()
    assert torch.equal(o_e, o_t) and torch.equal(o_e, o_o)
    assert torch.equal(eager.cache.pool, two.cache.pool)
    assert torch.equal(eager.cache.pool, one.cache.pool)
    _check(eager, o_e)


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
def test_block_sizes_match_oracle_and_block_size_16_bitwise(bs):
    """Ragged windows (not multiples of the block size), permuted block ids,
    sequence slots; bit-identical to the same cache built with 16-token
    blocks (same split length, same 16-token tiles)."""
    windows = [[1, 15, 17, 100, 513, 1500, 3000, 256], [300, 2048, 7, 4096, 600, 33, 1024, 5000]]
    ctx = [1, 2, 17, 600, 3001, 9000]
    slots = [5, 0, 7, 2, 1, 6]
    say("block size", bs)
    lay = hw().hwkv_layout_create(np.array(windows, np.int32), bs, 128, torch.bfloat16, 512)
    bps = lay.desc().blocks_per_seq
    perm = np.random.default_rng(bs).permutation(8 * bps).astype(np.int32).reshape(8, bps)
    c = build_decode_case(windows, torch.bfloat16, 128, 3, ctx, seed=702, split_tokens=512,
                          slots=slots, table_rows=8, block_ids=perm, chunk=777, block_size=bs)
    out = run_decode_step(c)
    _check(c, out)
    c16 = build_decode_case(windows, torch.bfloat16, 128, 3, ctx, seed=702, split_tokens=512,
                            slots=slots, table_rows=8, chunk=777, block_size=16)
    assert torch.equal(out, run_decode_step(c16))


@pytest.mark.parametrize("bs,dtype", [(32, torch.float16), (64, torch.bfloat16),
                                      (256, torch.float32)])
def test_fused_step_with_other_block_sizes(bs, dtype):
    """The single-launch step writes the new token into blocks of any size:
    output and pool equal append + decode_attn bit for bit."""
    H = hw()
    dev = device()
    windows = [[64, 1000, 17], [300, 16, 2048]]
    ctx = [2049, 16, 48, 1000]
    mk = dict(seed=703, split_tokens=512, chunk=300, block_size=bs)
    eager = build_decode_case(windows, dtype, 64, 2, ctx, **mk)
    fused = build_decode_case(windows, dtype, 64, 2, ctx, **mk)
    say("fused step, block size", bs, dtype)
    o_e = run_decode_step(eager)
    ws = H.make_step_workspace(fused.lay, 0, 2, len(ctx), 6, device=dev)
    o_f = torch.full_like(o_e, float("nan"))
    H.hwkv_decode_step(fused.cache, 0, 2, torch.tensor([x - 1 for x in ctx], device=dev),
                       fused.k_new, fused.v_new, fused.q, 1.0 / math.sqrt(64), ws, o_f)
    torch.cuda.synchronize()
    assert torch.equal(o_e, o_f)
    assert torch.equal(eager.cache.pool, fused.cache.pool)
    _check(fused, o_f)


def test_mixed_stack_swa_full_and_per_head_layers():
    """One stack: a sliding-window layer (every head the same 4096 window), a
    full-attention layer (windows far beyond any context), a per-head layer
    from the printed policy, and a layer of windows that are no multiple of
    the block size; fp16 cache in 64-token blocks, four sequences."""
    windows = [[4096] * 8, [1 << 16] * 8, list(synth.YAML_LAYER1),
               [1000, 3, 77, 4097, 65, 129, 1, 2500]]
    ctx = [7000, 130, 4097, 20000]
    say("mixed stack")
    c = build_decode_case(windows, torch.float16, 128, 3, ctx, seed=704, split_tokens=1024,
                          block_size=64, hist_margin=20, chunk=4096)
    _check(c, run_decode_step(c))


def test_full_attention_layer_equals_all_tokens():
    """A window longer than the context attends to every token: the oracle
    (pinned against SDPA without a mask) and the kernel agree on it."""
    c = build_decode_case([[1 << 15, 1 << 15]], torch.bfloat16, 128, 2, [3333, 17], seed=705,
                          hist_margin=10 ** 7)
    assert c.base == [0, 0]
    _check(c, run_decode_step(c))


@pytest.mark.parametrize("kind", ["stack48_f16_block64", "hybrid48_swa4096_every4th_global"])
def test_mixed_stack_configs_at_full_size(kind):
    """The mixed-stack configurations the benchmark times, at full size (48
    layers, context 112K, batch 1): the headline's windows on an fp16 cache in
    64-token blocks, and the hybrid stack (sliding-window layers of 4096 with
    every fourth layer per-head global).  Sampled sliding-window and global
    layers against the oracle; the benchmark's launch (appending split + merge
    with bf16 output) equals the three-launch step's fp32 results rounded."""
    H = hw()
    dev = device()
    if kind == "stack48_f16_block64":
        windows, dtype, bs, layers = synth.stack_windows(48, 8, 0), torch.float16, 64, (0, 23, 47)
    else:
        windows, dtype, bs, layers = synth.hybrid_windows(48, 8, 4096, 4, 0), torch.bfloat16, 16, \
            (0, 3, 22, 47)
    say("mixed config", kind, ": fill")
    c = build_stack_case(windows, dtype, 128, 3, synth.CTX_112K, 1, seed=706, block_size=bs)
    say("mixed config", kind, ": step")
    out = stack_step(c)
    got = to_host_f64(out)
    assert np.all(np.isfinite(got))
    worst = 0.0
    for l in layers:
        worst = max(worst, row_rel_err(got[l:l + 1], stack_oracle_layer(c, l)))
    say("mixed config", kind, "max row rel err (sampled layers)", worst)
    assert worst <= tol(dtype)
    ws = H.make_workspace(c.lay, 0, 48, 1, 24, device=dev)
    o16 = torch.empty(out.shape, dtype=torch.bfloat16, device=dev)
    H.hwkv_decode_append_attn(c.cache, 0, 48, torch.tensor([synth.CTX_112K], device=dev),
                              c.k_new, c.v_new, c.q, 1.0 / math.sqrt(128), ws, o16)
    torch.cuda.synchronize()
    assert torch.equal(o16, out.to(torch.bfloat16))


@pytest.mark.parametrize("group,head_dim", [(4, 128), (8, 128), (8, 256)])
def test_gqa_stacks_at_full_size(group, head_dim):
    """The GQA-group configurations the benchmark times, at full size: the
    headline's 48-layer stack (windows of seed 0, context 112K, batch 1, bf16)
    with 4 or 8 query heads per KV head.  Sampled layers against the oracle,
    within the decode regression bound; the benchmark's launch (appending
    split + merge, bf16 output) equals the three-launch step's fp32 results
    rounded to bf16."""
    H = hw()
    dev = device()
    windows = synth.stack_windows(48, 8, 0)
    n_q = 8 * group
    say("gqa stack G", group, "d", head_dim, ": fill")
    c = build_stack_case(windows, torch.bfloat16, head_dim, group, synth.CTX_112K, 1, seed=707)
    say("gqa stack G", group, "d", head_dim, ": step")
    out = stack_step(c)
    got = to_host_f64(out)
    assert np.all(np.isfinite(got))
    worst = 0.0
    for l in (0, 29, 47):
        worst = max(worst, row_rel_err(got[l:l + 1], stack_oracle_layer(c, l)))
    say("gqa stack G", group, "d", head_dim, "max row rel err (sampled layers)", worst)
    assert worst <= tol(torch.bfloat16)
    assert worst <= DECODE_REGRESSION_TOL, worst
    ws = H.make_workspace(c.lay, 0, 48, 1, n_q, device=dev)
    o16 = torch.empty(out.shape, dtype=torch.bfloat16, device=dev)
    H.hwkv_decode_append_attn(c.cache, 0, 48, torch.tensor([synth.CTX_112K], device=dev),
                              c.k_new, c.v_new, c.q, 1.0 / math.sqrt(head_dim), ws, o16)
    torch.cuda.synchronize()
    assert torch.equal(o16, out.to(torch.bfloat16))
