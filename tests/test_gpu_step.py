"""The single-launch decode step (hwkv_decode_step) on the GPU.

It must have exactly the effect of hwkv_append of the new token followed by
hwkv_decode_attn at context pos+1: the same output bits and the same pool
bytes, on twin caches filled identically.  It is also checked against the
fp64 oracle, over consecutive steps on one workspace (the arrival counters
are re-armed by every call), through window wraparound, on degenerate
inputs, under HIP-graph capture of per-layer launches, and at the full size
of the 48-layer 112K stack."""
import math

import numpy as np
import pytest
import torch

import synth
from _gpu_common import (BF16_TOL, DECODE_REGRESSION_TOL, F32_TOL, build_decode_case,
                         build_stack_case, device, hw, oracle_decode, row_rel_err, run_decode_step, say, stack_oracle_layer,
                         stack_step, to_host_f64)

pytestmark = pytest.mark.gpu


def _fused(c, out_dtype=torch.float32, layer_begin=0, n_layers=None, scale=None, ws=None,
           two_launch=False):
    H = hw()
    dev = device()
    n_layers = c.windows.shape[0] if n_layers is None else n_layers
    n_seqs = len(c.ctx)
    n_q = c.windows.shape[1] * c.group
    slots = None if c.slots is None else torch.tensor(c.slots, dtype=torch.int32, device=dev)
    pos = torch.tensor([x - 1 for x in c.ctx], dtype=torch.int64, device=dev)
    if ws is None:
        mk = H.make_workspace if two_launch else H.make_step_workspace
        ws = mk(c.lay, layer_begin, n_layers, n_seqs, n_q, device=dev)
    out = torch.full((n_layers, n_seqs, n_q, c.head_dim), float("nan"), dtype=out_dtype,
                     device=dev)
    s = 1.0 / math.sqrt(c.head_dim) if scale is None else scale
    sl = slice(layer_begin, layer_begin + n_layers)
    fn = H.hwkv_decode_append_attn if two_launch else H.hwkv_decode_step
    fn(c.cache, layer_begin, n_layers, pos, c.k_new[sl].contiguous(), c.v_new[sl].contiguous(),
       c.q[sl].contiguous(), s, ws, out, seq_slots=slots)
    torch.cuda.synchronize()
    return out


def _twins(*args, **kw):
    return build_decode_case(*args, **kw), build_decode_case(*args, **kw)


CASES = [
    # (windows, dtype, d, G, ctx, split, slots, rows)
    ([[1, 15, 17, 100, 512, 513, 1500, 3000], [16, 2048, 7, 4096, 600, 33, 1024, 5000]],
     torch.bfloat16, 128, 3, [1, 2, 17, 600, 3001, 9000], 256, [5, 0, 7, 2, 1, 6], 8),
    ([[32, 128]], torch.float32, 64, 2, [257, 31, 129], 0, None, None),
    ([[40, 700, 1], [2100, 16, 333]], torch.bfloat16, 64, 4, [5, 900, 2500], 64, None, None),
    ([[64, 1000, 17], [300, 16, 2048]], torch.float32, 128, 1, [2049, 16, 48], 16, None, None),
]


@pytest.mark.parametrize("two_launch", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_step_equals_append_then_attn(case, two_launch):
    """hwkv_decode_step (one launch) and hwkv_decode_append_attn (split stage
    appends, then merge) against the three-call path."""
    windows, dtype, d, G, ctx, split, slots, rows = CASES[case]
    say("fused step vs append+attn, case", case, "two launches" if two_launch else "one launch")
    eager, fused = _twins(windows, dtype, d, G, ctx, seed=601 + case, split_tokens=split,
                          slots=slots, table_rows=rows, chunk=333)
    o_e = run_decode_step(eager)
    o_f = _fused(fused, two_launch=two_launch)
    assert torch.equal(o_e, o_f)
    assert torch.equal(eager.cache.pool, fused.cache.pool)
    ref = oracle_decode(fused)
    err = row_rel_err(to_host_f64(o_f), ref)
    say("fused max row rel err", err)
    assert err <= (BF16_TOL if dtype == torch.bfloat16 else F32_TOL)
    assert err <= DECODE_REGRESSION_TOL, err


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_step_bf16_output_and_layer_subrange(out_dtype):
    windows = [[64, 128], [300, 16], [1000, 5], [77, 4000]]
    say("fused step: 16-bit output, layer subrange", out_dtype)
    eager, fused = _twins(windows, torch.bfloat16, 128, 3, [4500, 333], seed=611)
    o_e = run_decode_step(eager, out_dtype=out_dtype, layer_begin=1, n_layers=2, scale=0.05)
    o_f = _fused(fused, out_dtype=out_dtype, layer_begin=1, n_layers=2, scale=0.05)
    assert torch.equal(o_e, o_f)
    assert torch.equal(eager.cache.pool, fused.cache.pool)
    # the two stage calls of the two-launch step: split (appending), merge
    H = hw()
    dev = device()
    st = build_decode_case(windows, torch.bfloat16, 128, 3, [4500, 333], seed=611)
    pos = torch.tensor([4499, 332], dtype=torch.int64, device=dev)
    ws = H.make_workspace(st.lay, 1, 2, 2, 24, device=dev)
    o_s = torch.full_like(o_e, float("nan"))
    H.hwkv_decode_split_append(st.cache, 1, 2, pos, st.k_new[1:3].contiguous(),
                               st.v_new[1:3].contiguous(), st.q[1:3].contiguous(), 0.05, ws)
    H.hwkv_decode_merge(st.cache, 1, 2, pos + 1, ws, o_s)
    torch.cuda.synchronize()
    assert torch.equal(o_e, o_s)
    assert torch.equal(eager.cache.pool, st.cache.pool)


def test_consecutive_steps_through_wraparound():
    """Eight steps in a row on one step workspace, contexts chosen so that
    windows wrap and the new token crosses block and split boundaries; every
    step of both appending entry points equals the two-call path bit for
    bit."""
    H = hw()
    dev = device()
    windows = [[16, 40, 1024, 1], [33, 256, 17, 2000]]
    ctx = [15, 1020, 2043, 250]
    eager, fused = _twins(windows, torch.bfloat16, 128, 2, ctx, seed=612, split_tokens=256)
    two = build_decode_case(windows, torch.bfloat16, 128, 2, ctx, seed=612, split_tokens=256)
    n_layers, n_kv = 2, 4
    n_seqs, n_q = len(ctx), 8
    ws_f = H.make_step_workspace(fused.lay, 0, n_layers, n_seqs, n_q, device=dev)
    ws_e = H.make_workspace(eager.lay, 0, n_layers, n_seqs, n_q, device=dev)
    ws_t = H.make_workspace(two.lay, 0, n_layers, n_seqs, n_q, device=dev)
    o_e = torch.empty((n_layers, n_seqs, n_q, 128), dtype=torch.float32, device=dev)
    o_f = torch.empty_like(o_e)
    o_t = torch.empty_like(o_e)
    g = synth.gen(613, dev)
    scale = 1.0 / math.sqrt(128)
    for step in range(8):
        say("consecutive fused step", step)
        k = synth.randn((n_layers, n_seqs, 1, n_kv, 128), torch.bfloat16, g)
        v = synth.randn((n_layers, n_seqs, 1, n_kv, 128), torch.bfloat16, g)
        q = synth.randn((n_layers, n_seqs, n_q, 128), torch.bfloat16, g, std=scale)
        pos = torch.tensor([c - 1 + step for c in ctx], dtype=torch.int64, device=dev)
        H.hwkv_append(eager.cache, 0, n_layers, pos, k, v)
        H.hwkv_decode_attn(eager.cache, 0, n_layers, pos + 1, q, scale, ws_e, o_e)
        H.hwkv_decode_step(fused.cache, 0, n_layers, pos, k, v, q, scale, ws_f, o_f)
        H.hwkv_decode_append_attn(two.cache, 0, n_layers, pos, k, v, q, scale, ws_t, o_t)
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_f), step
        assert torch.equal(o_e, o_t), step
        assert torch.equal(eager.cache.pool, fused.cache.pool), step
        assert torch.equal(eager.cache.pool, two.cache.pool), step
    # the counters are back at zero after every call
    rec = H.hwkv_workspace_bytes(fused.lay, 0, n_layers, n_seqs, n_q)
    off = (rec + 255) // 256 * 256
    assert int(ws_f[off:].view(torch.int32).abs().sum()) == 0


def test_degenerate_positions_and_slots():
    """pos < 0: zeros and no append; a slot outside the table: NaN and no
    append; the other sequences are unaffected."""
    H = hw()
    dev = device()
    c = build_decode_case([[64, 300]], torch.bfloat16, 128, 2, [400, 400, 400], seed=614)
    good = _fused(c)
    pool_before = c.cache.pool.clone()
    ws = H.make_step_workspace(c.lay, 0, 1, 3, 4, device=dev)
    out = torch.empty((1, 3, 4, 128), dtype=torch.float32, device=dev)
    say("fused step: degenerate positions and slots")
    # sequence 0 repeats its token (same slot, same bytes): identical output
    H.hwkv_decode_step(c.cache, 0, 1, torch.tensor([399, -1, 399], device=dev), c.k_new,
                       c.v_new, c.q, 1 / math.sqrt(128), ws, out,
                       seq_slots=torch.tensor([0, 1, 9], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(out[0, 0], good[0, 0])
    assert torch.all(out[0, 1] == 0)
    assert torch.all(torch.isnan(out[0, 2]))
    assert torch.equal(c.cache.pool, pool_before)
    # the workspace still works for a normal call afterwards
    H.hwkv_decode_step(c.cache, 0, 1, torch.tensor([399, 399, 399], device=dev), c.k_new,
                       c.v_new, c.q, 1 / math.sqrt(128), ws, out)
    torch.cuda.synchronize()
    assert torch.equal(out, good)
    # the two-launch entry point on the same degenerate inputs
    ws2 = H.make_workspace(c.lay, 0, 1, 3, 4, device=dev)
    out2 = torch.empty_like(out)
    H.hwkv_decode_append_attn(c.cache, 0, 1, torch.tensor([399, -1, 399], device=dev), c.k_new,
                              c.v_new, c.q, 1 / math.sqrt(128), ws2, out2,
                              seq_slots=torch.tensor([0, 1, 9], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(out2[0, 0], good[0, 0])
    assert torch.all(out2[0, 1] == 0)
    assert torch.all(torch.isnan(out2[0, 2]))
    assert torch.equal(c.cache.pool, pool_before)


def test_per_layer_step_graph_replays():
    """Per-layer hwkv_decode_step launches captured once in a HIP graph;
    every replay equals the eager two-call step on a twin cache."""
    H = hw()
    dev = device()
    windows = [[64, 1000, 17], [300, 16, 2048], [5, 700, 128]]
    ctx = [2500, 90]
    n_layers, n_kv, G, d = 3, 3, 2, 128
    eager, graphd = _twins(windows, torch.bfloat16, d, G, ctx, seed=615, split_tokens=256)
    n_seqs = len(ctx)
    scale = 1.0 / math.sqrt(d)
    pos = torch.tensor([c - 1 for c in ctx], dtype=torch.int64, device=dev)
    kin = torch.zeros((n_layers, n_seqs, n_kv, d), dtype=torch.bfloat16, device=dev)
    vin = torch.zeros_like(kin)
    qin = torch.zeros((n_layers, n_seqs, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    gout = torch.zeros((n_layers, n_seqs, n_kv * G, d), dtype=torch.float32, device=dev)
    wss = [H.make_step_workspace(graphd.lay, l, 1, n_seqs, n_kv * G, device=dev)
           for l in range(n_layers)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for l in range(n_layers):
                H.hwkv_decode_step(graphd.cache, l, 1, pos, kin[l:l + 1], vin[l:l + 1],
                                   qin[l:l + 1], scale, wss[l], gout[l:l + 1])
    torch.cuda.synchronize()
    g = synth.gen(616, dev)
    ews = H.make_workspace(eager.lay, 0, n_layers, n_seqs, n_kv * G, device=dev)
    eout = torch.empty_like(gout)
    for step in range(4):
        say("fused graph replay step", step)
        k = synth.randn((n_layers, n_seqs, 1, n_kv, d), torch.bfloat16, g)
        v = synth.randn(k.shape, torch.bfloat16, g)
        q = synth.randn(qin.shape, torch.bfloat16, g, std=scale)
        p = torch.tensor([c - 1 + step for c in ctx], dtype=torch.int64, device=dev)
        H.hwkv_append(eager.cache, 0, n_layers, p, k, v)
        H.hwkv_decode_attn(eager.cache, 0, n_layers, p + 1, q, scale, ews, eout)
        kin.copy_(k[:, :, 0])
        vin.copy_(v[:, :, 0])
        qin.copy_(q)
        pos.copy_(p)
        graph.replay()
        torch.cuda.synchronize()
        _ = (torch.randn(1000, device=dev) * 2).sum().item()  # unrelated eager work
        assert torch.equal(gout, eout), step
        assert torch.equal(graphd.cache.pool, eager.cache.pool), step
        graph.replay()  # same token into the same slot again: idempotent
        torch.cuda.synchronize()
        assert torch.equal(gout, eout), step


def test_stack48_step_full_size():
    """The 48-layer 112K stack (windows from {1K,4K,16K,64K}, seed 0, batch 1):
    the single-launch step and the two-launch step (the split stage appends;
    the benchmark's headline launches) equal the append + split + merge
    launches bit for bit over every output row and the whole pool, the bf16
    output the benchmark writes is those results rounded to bf16, and sampled
    layers match the oracle."""
    H = hw()
    dev = device()
    w = synth.stack_windows(48, 8, 0)
    say("stack48 fused: fill twins")
    e = build_stack_case(w, torch.bfloat16, 128, 3, synth.CTX_112K, 1, seed=103)
    f = build_stack_case(w, torch.bfloat16, 128, 3, synth.CTX_112K, 1, seed=103)
    say("stack48 fused: steps")
    o_e = stack_step(e)
    pos = torch.tensor([synth.CTX_112K], device=dev)
    ws = H.make_step_workspace(f.lay, 0, 48, 1, 24, device=dev)
    o_f = torch.full_like(o_e, float("nan"))
    H.hwkv_decode_step(f.cache, 0, 48, pos, f.k_new, f.v_new, f.q, 1.0 / math.sqrt(128), ws, o_f)
    torch.cuda.synchronize()
    assert torch.equal(o_e, o_f)
    assert torch.equal(e.cache.pool, f.cache.pool)
    say("stack48 two launches: fill and step")
    del e
    torch.cuda.empty_cache()
    t = build_stack_case(w, torch.bfloat16, 128, 3, synth.CTX_112K, 1, seed=103)
    ws2 = H.make_workspace(t.lay, 0, 48, 1, 24, device=dev)
    o_t = torch.full_like(o_e, float("nan"))
    H.hwkv_decode_append_attn(t.cache, 0, 48, pos, t.k_new, t.v_new, t.q, 1.0 / math.sqrt(128),
                              ws2, o_t)
    torch.cuda.synchronize()
    assert torch.equal(o_e, o_t)
    assert torch.equal(t.cache.pool, f.cache.pool)
    # the headline writes bf16: the same results rounded to nearest even
    say("stack48 two launches: bf16 output")
    o16 = torch.empty(o_t.shape, dtype=torch.bfloat16, device=dev)
    H.hwkv_decode_attn(t.cache, 0, 48, pos + 1, t.q, 1.0 / math.sqrt(128), ws2, o16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o_t.to(torch.bfloat16))
    del t
    got = to_host_f64(o_f)
    worst = 0.0
    for l in (0, 17, 47):
        worst = max(worst, row_rel_err(got[l:l + 1], stack_oracle_layer(f, l)))
    say("stack48 fused max row rel err (sampled layers)", worst)
    assert worst <= BF16_TOL
    assert worst <= DECODE_REGRESSION_TOL, worst


def test_stack48_per_layer_split384():
    """The per-layer launch pattern of the benchmark's graph legs on the
    48-layer 112K stack: decode split length 384, one two-launch step
    (appending split + merge) per layer; sampled layers against the oracle."""
    H = hw()
    dev = device()
    w = synth.stack_windows(48, 8, 0)
    say("stack48 per layer split 384: fill")
    c = build_stack_case(w, torch.bfloat16, 128, 3, synth.CTX_112K, 1, seed=103,
                         split_tokens=384)
    assert c.lay.desc().split_tokens == 384
    pos = torch.tensor([synth.CTX_112K], device=dev)
    out = torch.full((48, 1, 24, 128), float("nan"), dtype=torch.float32, device=dev)
    say("stack48 per layer split 384: 48 steps")
    for l in range(48):
        ws = H.make_workspace(c.lay, l, 1, 1, 24, device=dev)
        H.hwkv_decode_append_attn(c.cache, l, 1, pos, c.k_new[l:l + 1].contiguous(),
                                  c.v_new[l:l + 1].contiguous(), c.q[l:l + 1].contiguous(),
                                  1.0 / math.sqrt(128), ws, out[l:l + 1])
    torch.cuda.synchronize()
    got = to_host_f64(out)
    assert np.all(np.isfinite(got))
    worst = 0.0
    for l in (0, 5, 17, 31, 47):
        worst = max(worst, row_rel_err(got[l:l + 1], stack_oracle_layer(c, l)))
    say("stack48 per layer split 384 max row rel err (sampled layers)", worst)
    assert worst <= BF16_TOL
    assert worst <= DECODE_REGRESSION_TOL, worst
