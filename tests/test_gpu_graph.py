"""HIP-graph capture of the decode path: the per-layer append + split + merge
launches are captured once and replayed step after step (positions in device
scalars updated by a fill kernel outside the graph, new tokens copied into the
captured inputs), with eager work and synchronisations between replays.
Every replay must equal the same step run eagerly on an identical twin cache,
bit for bit."""
import math

import torch
import pytest

import synth
from _gpu_common import build_decode_case, device, hw, say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_steps():
    H = hw()
    dev = device()
    windows = [[64, 1000, 17], [300, 16, 2048], [5, 700, 128]]
    ctx = [2500, 90]
    n_layers, n_kv, G, d = 3, 3, 2, 128
    eager = build_decode_case(windows, torch.bfloat16, d, G, ctx, seed=501, split_tokens=256)
    graphd = build_decode_case(windows, torch.bfloat16, d, G, ctx, seed=501, split_tokens=256)
    n_seqs = len(ctx)
    scale = 1.0 / math.sqrt(d)

    # captured inputs of the graph
    pos = torch.tensor([c - 1 for c in ctx], dtype=torch.int64, device=dev)
    cl = torch.tensor(ctx, dtype=torch.int64, device=dev)
    kin = torch.zeros((n_layers, n_seqs, 1, n_kv, d), dtype=torch.bfloat16, device=dev)
    vin = torch.zeros_like(kin)
    qin = torch.zeros((n_layers, n_seqs, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    gout = torch.zeros((n_layers, n_seqs, n_kv * G, d), dtype=torch.float32, device=dev)
    wss = [H.make_workspace(graphd.lay, l, 1, n_seqs, n_kv * G, device=dev)
           for l in range(n_layers)]
    ks = [kin[l:l + 1] for l in range(n_layers)]
    vs = [vin[l:l + 1] for l in range(n_layers)]
    qs = [qin[l:l + 1] for l in range(n_layers)]
    outs = [gout[l:l + 1] for l in range(n_layers)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for l in range(n_layers):
                H.hwkv_append(graphd.cache, l, 1, pos, ks[l], vs[l])
                H.hwkv_decode_attn(graphd.cache, l, 1, cl, qs[l], scale, wss[l], outs[l])
    torch.cuda.synchronize()
    # capture does not execute: the twin caches are still identical here

    g = synth.gen(502, dev)
    ews = H.make_workspace(eager.lay, 0, n_layers, n_seqs, n_kv * G, device=dev)
    eout = torch.empty_like(gout)
    for step in range(4):
        say("graph replay step", step)
        k = synth.randn(kin.shape, torch.bfloat16, g)
        v = synth.randn(kin.shape, torch.bfloat16, g)
        q = synth.randn(qin.shape, torch.bfloat16, g, std=1.0 / math.sqrt(d))
        p = torch.tensor([c - 1 + step for c in ctx], dtype=torch.int64, device=dev)
        # eager step on the twin
        H.hwkv_append(eager.cache, 0, n_layers, p, k, v)
        H.hwkv_decode_attn(eager.cache, 0, n_layers, p + 1, q, scale, ews, eout)
        # graph step: new inputs into the captured buffers, then replay
        kin.copy_(k)
        vin.copy_(v)
        qin.copy_(q)
        pos.copy_(p)
        cl.copy_(p + 1)
        graph.replay()
        torch.cuda.synchronize()
        _ = (torch.randn(1000, device=dev) * 2).sum().item()  # unrelated eager work
        assert torch.equal(gout, eout), step
        # replaying the same step again is idempotent (same token, same slot)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gout, eout), step
