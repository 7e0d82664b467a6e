"""Decode parity on the GPU against the fp64 oracle.

Metric (per output row = one (layer, sequence, query head)):
max|o - r| / max|r| <= 2e-3 for bf16 caches, <= 1e-5 for fp32 caches, with fp32
outputs; bf16 outputs must be within one bf16 ulp of the oracle rounded to
bf16.  Bitwise gates: w = 1 returns the newest V row exactly, and results do
not depend on batch composition or on the physical block ids."""
import math

import numpy as np
import pytest
import torch

import synth
from _gpu_common import (BF16_TOL, DECODE_REGRESSION_TOL, F32_TOL, bf16_round, bf16_ulps_apart,
                         build_decode_case, build_stack_case, device, f16_ulps_apart, hw, oracle_decode, row_rel_err,
                         run_decode_step, say, stack_oracle_layer, stack_step, to_host_f64)

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return BF16_TOL if dtype == torch.bfloat16 else F32_TOL


def _check(case, out, **kw):
    ref = oracle_decode(case, **kw)
    got = to_host_f64(out)
    assert np.all(np.isfinite(got))
    err = row_rel_err(got, ref)
    say("max row rel err", err)
    assert err <= _tol(case.dtype), err
    assert err <= DECODE_REGRESSION_TOL, err
    return got, ref


def test_tiny_config():
    """1 layer, 2 KV heads, 4 query heads, d=64, fp32, w=[32,128]: one append
    of 256 tokens, then one decode step (token 256 appended, L=257)."""
    say("tiny config")
    c = build_decode_case([[32, 128]], torch.float32, 64, 2, [257], seed=101, hist_margin=10 ** 6)
    assert c.base == [0]
    out = run_decode_step(c)
    _check(c, out)


@pytest.mark.parametrize("split", [16, 64, 512, 2048])
def test_bf16_ragged_windows_and_contexts(split):
    windows = [[1, 15, 17, 100, 512, 513, 1500, 3000],
               [16, 2048, 7, 4096, 600, 33, 1024, 5000]]
    ctx = [1, 2, 17, 600, 3001, 9000]
    say("ragged bf16 split", split)
    c = build_decode_case(windows, torch.bfloat16, 128, 3, ctx, seed=301, split_tokens=split,
                          slots=[5, 0, 7, 2, 1, 6], table_rows=8, chunk=777)
    out = run_decode_step(c)
    _check(c, out)


@pytest.mark.parametrize("dtype,d,G", [(torch.bfloat16, 64, 2), (torch.float32, 128, 3),
                                       (torch.float32, 64, 4), (torch.bfloat16, 128, 1),
                                       (torch.bfloat16, 128, 4), (torch.bfloat16, 128, 6),
                                       (torch.bfloat16, 64, 8), (torch.float32, 64, 1)])
def test_instances(dtype, d, G):
    windows = [[40, 700, 1], [2100, 16, 333]]
    say("instance", dtype, d, G)
    c = build_decode_case(windows, dtype, d, G, [5, 900, 2500], seed=302, split_tokens=256)
    out = run_decode_step(c)
    _check(c, out)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 6, 8])
def test_mfma_loop_every_instance(dtype, d, G):
    """Every 16-bit decode instance (the MFMA block loop) against the oracle:
    windows whose tiles leave waves with odd and even tile counts, one of 1
    token, a partial last block and a partial first block; the pool starts as
    NaN bytes, so any row outside a window that reached a product would
    show."""
    windows = [[1, 47, 700], [2100, 16, 333]]
    say("mfma instance", dtype, d, G)
    c = build_decode_case(windows, dtype, d, G, [5, 901, 2500], seed=304, split_tokens=256)
    out = run_decode_step(c)
    _check(c, out)


@pytest.mark.parametrize("d,G", [(128, 6), (128, 8), (64, 6)])
def test_fp32_large_groups(d, G):
    """fp32 caches keep the per-lane loop; its large-group instances hold
    more than 256 registers per lane (values parked in AGPRs)."""
    windows = [[40, 700, 1], [2100, 16, 333]]
    say("fp32 instance", d, G)
    c = build_decode_case(windows, torch.float32, d, G, [5, 900, 2500], seed=305, split_tokens=256)
    out = run_decode_step(c)
    _check(c, out)


def test_layer_subrange_and_scale():
    windows = [[64, 128], [300, 16], [1000, 5], [77, 4000]]
    say("layer subrange")
    c = build_decode_case(windows, torch.bfloat16, 128, 3, [4500, 333], seed=303)
    out = run_decode_step(c, layer_begin=1, n_layers=2, scale=0.05)
    _check(c, out, layer_begin=1, n_layers=2, scale=0.05)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_w1_returns_newest_v_bitwise(dtype, d):
    say("w=1 bitwise", dtype, d)
    c = build_decode_case([[1, 1, 1]], dtype, d, 3, [1, 50, 1000], seed=304)
    out = run_decode_step(c)
    got = out.cpu()
    for b in range(3):
        for i in range(9):
            want = c.v_new[0, b, 0, i // 3].float().cpu()
            assert torch.equal(got[0, b, i], want), (b, i)


def test_bf16_output_within_one_ulp():
    windows = [[128, 1024, 4096, 33]]
    say("bf16 output")
    c = build_decode_case(windows, torch.bfloat16, 128, 3, [5000, 70], seed=305)
    out = run_decode_step(c, out_dtype=torch.bfloat16)
    ref = bf16_round(oracle_decode(c))
    ulps = bf16_ulps_apart(to_host_f64(out), ref)
    assert ulps.max() <= 1, ulps.max()


def test_f16_output_within_one_ulp():
    """fp16 outputs (here from a bf16 cache): the fp32 result rounded to
    nearest even, within one binary16 ulp of the oracle rounded the same way."""
    windows = [[128, 1024, 4096, 33]]
    say("f16 output")
    c = build_decode_case(windows, torch.bfloat16, 128, 3, [5000, 70], seed=308)
    out = run_decode_step(c, out_dtype=torch.float16)
    ulps = f16_ulps_apart(out.cpu().numpy().astype(np.float64), oracle_decode(c))
    assert ulps.max() <= 1, ulps.max()


def test_batch_composition_is_bitwise_invariant():
    windows = [[100, 2000, 700]]
    ctx = [3000, 10, 1500, 2222]
    say("batch composition")
    c = build_decode_case(windows, torch.bfloat16, 128, 2, ctx, seed=306, split_tokens=256)
    full = run_decode_step(c)
    H = hw()
    dev = device()
    for b in range(len(ctx)):
        # decode sequence b alone (its token is already appended)
        ws = H.make_workspace(c.lay, 0, 1, 1, 6, device=dev)
        out = torch.empty((1, 1, 6, 128), dtype=torch.float32, device=dev)
        H.hwkv_decode_attn(c.cache, 0, 1, torch.tensor([ctx[b]], device=dev), c.q[:, b:b + 1].contiguous(),
                           1.0 / math.sqrt(128), ws, out,
                           seq_slots=torch.tensor([b], dtype=torch.int32, device=dev))
        torch.cuda.synchronize()
        assert torch.equal(out[0, 0], full[0, b]), b


def test_block_table_permutation_is_bitwise_invariant():
    windows = [[48, 1000], [16, 300]]
    ctx = [1200, 800]
    say("table permutation")
    c1 = build_decode_case(windows, torch.bfloat16, 128, 3, ctx, seed=307)
    bps = c1.lay.desc().blocks_per_seq
    perm = np.random.default_rng(1).permutation(2 * bps).astype(np.int32).reshape(2, bps)
    c2 = build_decode_case(windows, torch.bfloat16, 128, 3, ctx, seed=307, block_ids=perm)
    o1 = run_decode_step(c1)
    o2 = run_decode_step(c2)
    assert torch.equal(o1, o2)
    _check(c2, o2)


def test_needle_at_the_window_edge():
    """A key aligned with q and scaled up placed at L-w dominates the output;
    at L-w-1 it is outside the window and has no effect."""
    H = hw()
    dev = device()
    d, w, L = 128, 1000, 5000
    for pos, inside in ((L - w, True), (L - w - 1, False), (L - 1, True)):
        say("needle", pos, inside)
        c = build_decode_case([[w]], torch.bfloat16, d, 1, [L], seed=308)
        # overwrite the stored key of `pos` with a needle c*q (score ~ 60)
        qv = c.q[0, 0, 0].float()
        needle = (qv / qv.norm() * (60.0 * math.sqrt(d) / qv.norm())).to(torch.bfloat16)
        kn = needle.reshape(1, 1, 1, 1, d).contiguous()
        vn = synth.randn((1, 1, 1, 1, d), torch.bfloat16, synth.gen(9, dev))
        c.k_hist[0, 0, pos - c.base[0], 0] = synth.to_raw(needle)
        c.v_hist[0, 0, pos - c.base[0], 0] = synth.to_raw(vn[0, 0, 0, 0])
        if pos == L - 1:  # the decode step's own token
            c.k_new[0, 0, 0, 0] = needle
            c.v_new[0, 0, 0, 0] = vn[0, 0, 0, 0]
        else:  # overwrite the stored history row
            H.hwkv_append(c.cache, 0, 1, torch.tensor([pos], device=dev), kn, vn)
        out = run_decode_step(c)
        got, ref = _check(c, out)
        vfloat = vn[0, 0, 0, 0].double().cpu().numpy()
        if inside:
            assert np.abs(got[0, 0, 0] - vfloat).max() < 1e-3
        else:
            assert np.abs(got[0, 0, 0] - vfloat).max() > 0.1


def test_invalid_context_values():
    """ctx_len <= 0 gives zeros; a slot outside the table gives NaN; neither
    faults and the other sequences are unaffected."""
    H = hw()
    dev = device()
    c = build_decode_case([[64, 300]], torch.bfloat16, 128, 2, [400, 400, 400], seed=309)
    good = run_decode_step(c)
    ws = H.make_workspace(c.lay, 0, 1, 3, 4, device=dev)
    out = torch.empty((1, 3, 4, 128), dtype=torch.float32, device=dev)
    say("invalid ctx values")
    H.hwkv_decode_attn(c.cache, 0, 1, torch.tensor([400, 0, 400], device=dev), c.q, 1 / math.sqrt(128),
                       ws, out, seq_slots=torch.tensor([0, 1, 9], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(out[0, 0], good[0, 0])
    assert torch.all(out[0, 1] == 0)
    assert torch.all(torch.isnan(out[0, 2]))


@pytest.mark.parametrize("split", [0, 2048])
def test_single_layer_config(split):
    """1 layer, 8 KV x 3 query heads, d=128, bf16, windows of the printed
    policy's layer 0, context 32768, batch 8: every output row, at the
    default split length and at the one the benchmark times (2048)."""
    say("single-layer config: fill, split", split)
    c = build_stack_case([synth.YAML_LAYER0], torch.bfloat16, 128, 3, 32768, 8, seed=102,
                         split_tokens=split)
    say("single-layer config: step")
    out = stack_step(c)
    ref = stack_oracle_layer(c, 0)
    err = row_rel_err(to_host_f64(out[0:1]), ref)
    say("single-layer max row rel err", err)
    assert err <= BF16_TOL
    assert err <= DECODE_REGRESSION_TOL, err
    # the benchmark's launch: the appending split (rewriting the same token)
    # and the merge, bf16 output = the fp32 results rounded to bf16
    H = hw()
    dev = device()
    ws = H.make_workspace(c.lay, 0, 1, 8, 24, device=dev)
    o16 = torch.empty((1, 8, 24, 128), dtype=torch.bfloat16, device=dev)
    H.hwkv_decode_append_attn(c.cache, 0, 1, torch.full((8,), 32768, device=dev), c.k_new,
                              c.v_new, c.q, 1.0 / math.sqrt(128), ws, o16)
    torch.cuda.synchronize()
    assert torch.equal(o16, out.to(torch.bfloat16))


def test_stack48_config():
    """48 layers, 8 KV x 3 query heads, d=128, bf16, windows drawn from
    {1K,4K,16K,64K} (seed 0), context 112K, batch 1: one decode step over all
    layers in one launch each of append, split and merge; every output row."""
    w = synth.stack_windows(48, 8, 0)
    say("stack48 config: fill")
    c = build_stack_case(w, torch.bfloat16, 128, 3, synth.CTX_112K, 1, seed=103)
    say("stack48 config: step")
    out = stack_step(c)
    got = to_host_f64(out)
    worst = 0.0
    for l in range(48):
        ref = stack_oracle_layer(c, l)
        worst = max(worst, row_rel_err(got[l:l + 1], ref))
    say("stack48 max row rel err", worst)
    assert worst <= BF16_TOL
    assert worst <= DECODE_REGRESSION_TOL, worst
