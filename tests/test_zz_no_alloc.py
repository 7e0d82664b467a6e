"""hwkv_decode_append_attn_static, the entry point for callers that cannot
allocate device memory: the split records live in the library's static
scratch instead of a caller workspace.  Its results must be those of
hwkv_decode_append_attn bit for bit (same kernels, same order), on two calls
in a row where the second is smaller than the first (the scratch keeps the
first call's records; nothing of them may leak into the second)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_common import (BF16_TOL, DECODE_REGRESSION_TOL, build_decode_case, device, hw,
                         oracle_decode, row_rel_err, say, to_host_f64)

pytestmark = pytest.mark.gpu

WINDOWS = [[64, 1000, 300], [5000, 16, 2048], [700, 4096, 1], [33, 100, 9000]]
CTX = [9100, 4000, 700]


def _twin(seed):
    return build_decode_case(WINDOWS, torch.bfloat16, 128, 3, CTX, seed=seed, split_tokens=512,
                             chunk=1500)


def test_static_scratch_entry_matches_the_workspace_entry():
    H = hw()
    dev = device()
    say("no-alloc entry: build twins")
    a, b = _twin(701), _twin(701)
    n_layers, n_q, d = 4, 9, 128
    scale = 1.0 / math.sqrt(d)

    # call 1: every layer, all three sequences
    say("no-alloc entry: call 1 (4 layers x 3 sequences)")
    pos = torch.tensor([c - 1 for c in CTX], device=dev)
    ws = H.make_workspace(a.lay, 0, n_layers, 3, n_q, device=dev)
    out_a = torch.full((n_layers, 3, n_q, d), float("nan"), device=dev)
    out_b = torch.full_like(out_a, float("nan"))
    H.hwkv_decode_append_attn(a.cache, 0, n_layers, pos, a.k_new, a.v_new, a.q, scale, ws, out_a)
    H.hwkv_decode_append_attn_static(b.cache, 0, n_layers, pos, b.k_new, b.v_new, b.q, scale,
                                     out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(a.cache.pool, b.cache.pool)
    err = row_rel_err(to_host_f64(out_b), oracle_decode(b))
    say("no-alloc entry: call 1 max row rel err", err)
    assert err <= BF16_TOL and err <= DECODE_REGRESSION_TOL

    # call 2, smaller: layers 1..2, two sequences through seq_slots, the next
    # token of each, bf16 output
    say("no-alloc entry: call 2 (2 layers x 2 sequences)")
    slots = torch.tensor([2, 0], dtype=torch.int32, device=dev)
    pos2 = torch.tensor([CTX[2], CTX[0]], device=dev)
    g = synth.gen(702, dev)
    k2 = synth.randn((2, 2, 1, 3, d), torch.bfloat16, g)
    v2 = synth.randn((2, 2, 1, 3, d), torch.bfloat16, g)
    q2 = synth.randn((2, 2, n_q, d), torch.bfloat16, g, std=1.0 / math.sqrt(d))
    ws2 = H.make_workspace(a.lay, 1, 2, 2, n_q, device=dev)
    o2a = torch.full((2, 2, n_q, d), float("nan"), dtype=torch.bfloat16, device=dev)
    o2b = torch.full_like(o2a, float("nan"))
    H.hwkv_decode_append_attn(a.cache, 1, 2, pos2, k2, v2, q2, scale, ws2, o2a, seq_slots=slots)
    H.hwkv_decode_append_attn_static(b.cache, 1, 2, pos2, k2, v2, q2, scale, o2b,
                                     seq_slots=slots)
    torch.cuda.synchronize()
    assert torch.equal(o2a, o2b)
    assert torch.equal(a.cache.pool, b.cache.pool)
    assert torch.all(torch.isfinite(o2b.float()))
    # and against the oracle: history + the call-1 token + the call-2 token
    sl = [2, 0]
    n_tok = [CTX[s] - b.base[s] for s in sl]  # stored tokens per sequence so far
    kh = np.zeros((2, 2, max(n_tok) + 1, 3, d), b.k_hist.dtype)
    vh = np.zeros_like(kh)
    for i, s in enumerate(sl):
        kh[:, i, :n_tok[i]] = b.k_hist[1:3, s, :n_tok[i]]
        vh[:, i, :n_tok[i]] = b.v_hist[1:3, s, :n_tok[i]]
        kh[:, i, n_tok[i]] = synth.to_raw(k2[:, i, 0])
        vh[:, i, n_tok[i]] = synth.to_raw(v2[:, i, 0])
    ref = oracle.decode(b.windows[1:3], [CTX[2] + 1, CTX[0] + 1], synth.to_raw(q2), kh, vh,
                        [b.base[2], b.base[0]], scale)
    ref16 = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    got = to_host_f64(o2b)
    assert np.abs(got - ref16).max() <= np.abs(ref).max() * 2 ** -7
