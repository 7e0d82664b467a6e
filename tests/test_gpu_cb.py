"""Continuous decode batch on the GPU, sampled against the oracle.

32 sequences with contexts uniform in [4K, 160K] plus one sequence per
window level starting 100 tokens before its window edge (so that 256 steps
cross the edge and wrap the ring), 48 layers with the stack's windows, 256
decode steps of append + attention, each step one appending split launch
(which also writes every sequence's new token) and one merge launch for all
layers and sequences: the launch pattern of the continuous-batch benchmark.
The benchmark writes bf16 outputs; at each checkpoint a non-appending
decode of the same state with bf16 output must equal the step's fp32 output
rounded to bf16, bit for bit.

The pool starts filled with N(0,1) bf16 values (synthetic input); by the
ring placement every slot of a head's ring then holds the token of one of
the last C positions before the start.  For sampled heads the oracle's own
layout and ring-slot functions read that initial window back from the pool,
append the tokens the steps add, and decode at checkpoint steps."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_common import BF16_TOL, DECODE_REGRESSION_TOL, device, hw, row_rel_err, say

pytestmark = pytest.mark.gpu

N_STEPS = 256
CHECKPOINTS = (0, 1, 127, 255)


def _initial_rows(pool, ids, nb, off, b, hi, positions, d):
    """K and V rows (bf16 bits) of `positions` of head `hi` of table row b,
    located with the oracle's ring placement."""
    rows_k, rows_v = [], []
    for t in positions:
        j, row = oracle.ring_slot(int(t), 16, int(nb[hi]))
        blk = int(ids[b, off[hi] + j])
        rows_k.append((blk * 2 + 0) * 16 + row)
        rows_v.append((blk * 2 + 1) * 16 + row)
    pv = pool.view(torch.bfloat16).view(-1, d)
    idx_k = torch.tensor(rows_k, dtype=torch.int64, device=pool.device)
    idx_v = torch.tensor(rows_v, dtype=torch.int64, device=pool.device)
    return synth.to_raw(pv[idx_k]), synth.to_raw(pv[idx_v])


def test_continuous_batch_sampled():
    H = hw()
    dev = device()
    n_layers, n_kv, G, d = 48, 8, 3, 128
    windows = synth.stack_windows(n_layers, n_kv, 0)
    L0 = [int(x) for x in synth.cb_contexts()] + [w - 100 for w in synth.WINDOW_LEVELS]
    n_seqs = len(L0)
    say("cb: layout + pool fill for", n_seqs, "sequences")
    lay = H.hwkv_layout_create(windows, 16, d, torch.bfloat16)
    cache = H.make_cache(lay, n_seqs, device=dev)
    synth.fill_normal(cache.pool, 104, progress=True)
    torch.cuda.synchronize()
    nb, off, bps = oracle.layout(windows, 16)
    ids = cache.block_ids.cpu().numpy()

    # samples: two heads of each window level on the edge-crossing sequences,
    # plus random (sequence, layer, head) triples of the uniform batch
    rng = np.random.default_rng(11)
    samples = []
    for e, wl in enumerate(synth.WINDOW_LEVELS):
        ls, hs = np.nonzero(windows == wl)
        for k in rng.choice(len(ls), 2, replace=False):
            samples.append((32 + e, int(ls[k]), int(hs[k])))
    for _ in range(16):
        samples.append((int(rng.integers(0, 32)), int(rng.integers(0, n_layers)),
                        int(rng.integers(0, n_kv))))

    init = {}
    for (b, l, h) in samples:
        hi = l * n_kv + h
        C = int(nb[hi]) * 16
        n0 = min(C, L0[b])
        pos = range(L0[b] - n0, L0[b])
        init[(b, l, h)] = (L0[b] - n0,) + _initial_rows(cache.pool, ids, nb, off, b, hi, pos, d)

    L0_t = torch.tensor(L0, dtype=torch.int64, device=dev)
    ws = H.make_workspace(lay, 0, n_layers, n_seqs, n_kv * G, device=dev)
    out = torch.empty((n_layers, n_seqs, n_kv * G, d), dtype=torch.float32, device=dev)
    out16 = torch.empty((n_layers, n_seqs, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    g = synth.gen(108, dev)
    sb = torch.tensor([s[0] for s in samples], device=dev)
    sl = torch.tensor([s[1] for s in samples], device=dev)
    shh = torch.tensor([s[2] for s in samples], device=dev)
    k_rec, v_rec, q_rec, o_rec = [], [], [], {}
    say("cb: running", N_STEPS, "steps")
    for i in range(N_STEPS):
        kn = synth.randn((n_layers, n_seqs, 1, n_kv, d), torch.bfloat16, g)
        vn = synth.randn((n_layers, n_seqs, 1, n_kv, d), torch.bfloat16, g)
        q = synth.randn((n_layers, n_seqs, n_kv * G, d), torch.bfloat16, g,
                        std=1.0 / math.sqrt(d))
        H.hwkv_decode_append_attn(cache, 0, n_layers, L0_t + i, kn, vn, q, 1.0 / math.sqrt(d),
                                  ws, out)
        k_rec.append(kn[sl, sb, 0, shh].clone())
        v_rec.append(vn[sl, sb, 0, shh].clone())
        qg = q.view(n_layers, n_seqs, n_kv, G, d)
        q_rec.append(qg[sl, sb, shh].clone())
        if i in CHECKPOINTS:
            o_rec[i] = out.view(n_layers, n_seqs, n_kv, G, d)[sl, sb, shh].clone()
            H.hwkv_decode_attn(cache, 0, n_layers, L0_t + i + 1, q, 1.0 / math.sqrt(d), ws, out16)
            assert torch.equal(out16, out.to(torch.bfloat16)), i
    torch.cuda.synchronize()
    say("cb: oracle on", len(samples), "heads x", len(CHECKPOINTS), "checkpoints")
    k_rec = synth.to_raw(torch.stack(k_rec))  # [steps][samples][d]
    v_rec = synth.to_raw(torch.stack(v_rec))
    q_rec = synth.to_raw(torch.stack(q_rec))  # [steps][samples][G][d]
    worst = 0.0
    for si, (b, l, h) in enumerate(samples):
        base, k0, v0 = init[(b, l, h)]
        for i in CHECKPOINTS:
            kh = np.concatenate([k0, k_rec[:i + 1, si]])[None, None, :, None, :]
            vh = np.concatenate([v0, v_rec[:i + 1, si]])[None, None, :, None, :]
            ref = oracle.decode(np.array([[windows[l, h]]]), [L0[b] + i + 1],
                                q_rec[i, si][None, None], kh, vh, [base], 1.0 / math.sqrt(d))
            got = o_rec[i][si].double().cpu().numpy()
            worst = max(worst, row_rel_err(got, ref[0, 0]))
    say("cb: max row rel err", worst)
    assert worst <= BF16_TOL
    assert worst <= DECODE_REGRESSION_TOL, worst
