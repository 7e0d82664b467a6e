"""Pins of the CPU oracle against facts it does not compute itself.

Each test ties one oracle function to something outside it: values worked out
by hand from the HeadWiseKV pages (tests/golden/, each with its citation), the
full-cache growth law, torch's scaled_dot_product_attention in float64 (a
library routine that shares no code with the oracle), closed forms,
invariants, and brute force on tiny inputs.  A plausible slip anywhere in the
oracle -- a dropped scale, a sign, a window off by one, a transposed head map,
a wrong ring modulus, a missing factor 2 -- fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _t(shape, seed, dtype=torch.float32, std=1.0):
    return synth.randn(shape, dtype, synth.gen(seed), std)


def _f64(t: torch.Tensor) -> torch.Tensor:
    # torch's own widening, independent of the oracle's bf16 decoding
    return t.to(torch.float64)


# --------------------------------------------------------------------------
# layout and memory estimate
# --------------------------------------------------------------------------

def test_blocks_per_head_match_policy_yaml(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "policy_yaml_layers.json")))
    bs = g["block_size"]
    for layer in g["layers"]:
        got = [oracle.blocks(w, bs) for w in layer["kv_head_windows"]]
        assert got == layer["blocks_per_head"]
    w = np.array([layer["kv_head_windows"] for layer in g["layers"]])
    nb, off, bps = oracle.layout(w, bs)
    assert bps == g["two_layer_blocks_per_seq"]
    assert int(off[8]) == g["layers"][0]["blocks"]
    assert list(nb[:8]) == g["layers"][0]["blocks_per_head"]


def test_mem_estimate_policy_yaml(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "policy_yaml_layers.json")))
    for layer in g["layers"]:
        w = np.array([layer["kv_head_windows"]])
        got = oracle.mem_estimate(w, g["block_size"], g["head_dim"], g["elem_bytes"], 1)
        assert got == layer["bytes_per_seq"]
    w0 = np.array([g["layers"][0]["kv_head_windows"]])
    assert oracle.mem_estimate(w0, 16, 128, 2, 8) == g["layer0_eight_seqs_bytes"]


def test_blocks_ceil_hand_values():
    cases = {(1, 16): 1, (15, 16): 1, (16, 16): 1, (17, 16): 2, (32, 16): 2,
             (33, 16): 3, (100, 16): 7, (1000, 64): 16, (65536, 16): 4096, (5, 1): 5}
    for (w, bs), nb in cases.items():
        assert oracle.blocks(w, bs) == nb, (w, bs)


def test_mem_estimate_reduces_to_full_cache_growth_law(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "full_cache_growth.json")))
    for c in g["cases"]:
        w = np.full((c["n_layers"], c["num_heads"]), c["seq_len"], np.int32)
        got = oracle.mem_estimate(w, 16, c["head_dim"], c["elem_bytes"], 1)
        assert got == c["bytes"], c


def test_mem_estimate_rounds_windows_up_to_whole_blocks():
    # w=17 needs 2 blocks of 16 rows, w=1 one block: 3 blocks of
    # 16 rows x 64 dims x (K+V) x 4 bytes = 3 x 8192 bytes (worked by hand)
    assert oracle.mem_estimate(np.array([[17, 1]]), 16, 64, 4, 1) == 24576
    assert oracle.mem_estimate(np.array([[17, 1]]), 16, 64, 4, 5) == 5 * 24576


def test_layout_offsets_partition_each_table_row():
    rng = np.random.default_rng(7)
    w = rng.integers(1, 300, size=(5, 3)).astype(np.int32)
    nb, off, bps = oracle.layout(w, 16)
    assert off[0] == 0 and off[-1] == bps
    assert np.array_equal(np.diff(off), nb.astype(np.int64))
    assert np.all(nb >= 1) and np.all(nb.astype(np.int64) * 16 >= w.reshape(-1))
    assert np.all((nb.astype(np.int64) - 1) * 16 < w.reshape(-1))
    table = oracle.default_table(4, bps)
    assert np.array_equal(np.sort(table.reshape(-1)), np.arange(4 * bps))


# --------------------------------------------------------------------------
# ring placement and append
# --------------------------------------------------------------------------

def test_ring_slot_hand_values():
    # bs=16, 3 blocks: t=37 is in logical block 2, row 5; t=48 wraps to ring
    # block 0 (3 mod 3), row 0; t=100 -> logical block 6 -> ring block 0, row 4
    assert oracle.ring_slot(37, 16, 3) == (2, 5)
    assert oracle.ring_slot(48, 16, 3) == (0, 0)
    assert oracle.ring_slot(100, 16, 3) == (0, 4)
    assert oracle.ring_slot(0, 16, 1) == (0, 0)


@pytest.mark.parametrize("bs,nb", [(4, 1), (4, 3), (16, 5)])
def test_ring_slots_cover_every_slot_once(bs, nb):
    C = bs * nb
    for start in (0, 7, 123):
        seen = set()
        for t in range(start, start + C):
            j, row = oracle.ring_slot(t, bs, nb)
            assert 0 <= j < nb and 0 <= row < bs
            seen.add(j * bs + row)
            assert oracle.ring_slot(t + C, bs, nb) == (j, row)
        assert seen == set(range(C))


def _pool_row(pool, table, head_off, nblocks, slot, hi, t, kv, bs, d, eb):
    """Read one stored row back with the block-table arithmetic written out
    here (row t of head hi lives in ring block (t//bs) % nblocks[hi])."""
    blk = table[slot, head_off[hi] + (t // bs) % nblocks[hi]]
    off = ((blk * 2 + kv) * bs + t % bs) * d * eb
    return pool[off:off + d * eb]


def test_append_equals_token_by_token_last_writer_wins():
    """Chunked appends (including chunks longer than the ring) leave the pool
    exactly as writing every token one at a time, in order, would."""
    bs, d = 4, 8
    windows = np.array([[3, 8], [13, 1]], np.int32)
    n_layers, n_kv = windows.shape
    nb, off, bps = oracle.layout(windows, bs)
    n_seqs = 2
    rng = np.random.default_rng(3)
    table = rng.permutation(n_seqs * bps).astype(np.int32).reshape(n_seqs, bps)
    n_tok = 41
    k = rng.standard_normal((n_layers, n_seqs, n_tok, n_kv, d)).astype(np.float32)
    v = rng.standard_normal((n_layers, n_seqs, n_tok, n_kv, d)).astype(np.float32)
    init = rng.integers(0, 256, size=n_seqs * bps * 2 * bs * d * 4).astype(np.uint8)

    ref = init.copy()  # token-by-token replay
    for t in range(n_tok):
        oracle.append(ref, table, windows, bs, d, 0, [t] * n_seqs,
                      k[:, :, t:t + 1], v[:, :, t:t + 1])
    for chunks in ([41], [1, 40], [17, 24], [5, 5, 5, 26], [30, 11]):
        pool = init.copy()
        t0 = 0
        for c in chunks:
            oracle.append(pool, table, windows, bs, d, 0, [t0] * n_seqs,
                          k[:, :, t0:t0 + c], v[:, :, t0:t0 + c])
            t0 += c
        assert np.array_equal(pool, ref), chunks

    # and the replay itself holds, for every head, the newest C tokens
    for l in range(n_layers):
        for b in range(n_seqs):
            for h in range(n_kv):
                hi = l * n_kv + h
                C = nb[hi] * bs
                for t in range(max(0, n_tok - C), n_tok):
                    got = _pool_row(ref, table, off, nb, b, hi, t, 0, bs, d, 4)
                    assert np.array_equal(got.view(np.float32), k[l, b, t, h])
                    got = _pool_row(ref, table, off, nb, b, hi, t, 1, bs, d, 4)
                    assert np.array_equal(got.view(np.float32), v[l, b, t, h])


def test_append_leaves_other_bytes_untouched():
    bs, d = 4, 4
    windows = np.array([[5, 2]], np.int32)
    nb, off, bps = oracle.layout(windows, bs)
    table = oracle.default_table(3, bps)
    init = np.random.default_rng(1).integers(0, 256, 3 * bps * 2 * bs * d * 4).astype(np.uint8)
    pool = init.copy()
    k = np.ones((1, 1, 1, 2, d), np.float32)
    oracle.append(pool, table, windows, bs, d, 0, [6], k, 2 * k, seq_slots=[1])
    changed = np.nonzero(pool != init)[0]
    # exactly 2 heads x (K row + V row) x 16 bytes may change, all in slot 1
    assert changed.size <= 4 * d * 4
    lo, hi = bps * 2 * bs * d * 4, 2 * bps * 2 * bs * d * 4
    assert changed.min() >= lo and changed.max() < hi


# --------------------------------------------------------------------------
# decode attention
# --------------------------------------------------------------------------

def _sdpa_decode(q, k_hist, v_hist, L, windows=None, scale=None):
    """torch SDPA (float64) for one (layer, seq): q [n_q, d], k/v [T, n_kv, d]
    holding positions [0, T); attends [max(0, L-w), L) per kv head."""
    n_q, d = q.shape
    n_kv = k_hist.shape[1]
    G = n_q // n_kv
    qq = q.reshape(1, n_q, 1, d)
    kk = k_hist[:L].permute(1, 0, 2).reshape(1, n_kv, L, d)
    vv = v_hist[:L].permute(1, 0, 2).reshape(1, n_kv, L, d)
    mask = None
    if windows is not None:
        pos = torch.arange(L)
        mask = torch.zeros(1, n_q, 1, L, dtype=torch.bool)
        for i in range(n_q):
            mask[0, i, 0] = pos >= L - int(windows[i // G])
    o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, enable_gqa=True, scale=scale)
    return o.reshape(n_q, d)


def _decode_case(dtype, n_layers, n_seqs, n_kv, G, d, T, seed):
    q = _t((n_layers, n_seqs, n_kv * G, d), seed, dtype, std=1.0 / math.sqrt(d))
    k = _t((n_layers, n_seqs, T, n_kv, d), seed + 1, dtype)
    v = _t((n_layers, n_seqs, T, n_kv, d), seed + 2, dtype)
    return q, k, v


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_decode_full_window_is_full_attention(dtype):
    n_layers, n_seqs, n_kv, G, d, T = 2, 2, 2, 3, 64, 150
    q, k, v = _decode_case(dtype, n_layers, n_seqs, n_kv, G, d, T, 11)
    L = [150, 97]
    windows = np.array([[150, 10 ** 6], [4096, 151]], np.int32)  # all >= L
    scale = 1.0 / math.sqrt(d)
    got = oracle.decode(windows, L, synth.to_raw(q), synth.to_raw(k), synth.to_raw(v),
                        [0, 0], scale)
    for l in range(n_layers):
        for b in range(n_seqs):
            ref = _sdpa_decode(_f64(q[l, b]), _f64(k[l, b]), _f64(v[l, b]), L[b])
            assert np.abs(got[l, b] - ref.numpy()).max() <= 1e-12


@pytest.mark.parametrize("d", [32, 256])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_decode_window_is_band_masked_attention(dtype, d):
    n_layers, n_seqs, n_kv, G, T = 2, 3, 4, 2, 200
    q, k, v = _decode_case(dtype, n_layers, n_seqs, n_kv, G, d, T, 21)
    L = [200, 64, 129]
    windows = np.array([[1, 7, 64, 100], [33, 128, 2, 500]], np.int32)
    scale = 1.0 / math.sqrt(d)
    got = oracle.decode(windows, L, synth.to_raw(q), synth.to_raw(k), synth.to_raw(v),
                        [0] * n_seqs, scale)
    for l in range(n_layers):
        for b in range(n_seqs):
            ref = _sdpa_decode(_f64(q[l, b]), _f64(k[l, b]), _f64(v[l, b]), L[b], windows[l])
            assert np.abs(got[l, b] - ref.numpy()).max() <= 1e-12


def test_widening_of_every_16_bit_pattern_matches_the_libraries():
    """The oracle decodes stored bf16 and fp16 bits itself (from the formats'
    definitions); numpy's float16 and torch's bfloat16 conversions are
    independent implementations of the same formats."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = bits.view(np.float16)
    got = oracle.widen(f16)
    ref = f16.astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))  # -0.0 stays -0.0
    got = oracle.widen(bits)  # uint16 carries bf16 bits
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_decode_scale_is_applied():
    # with a non-default scale the oracle must still match SDPA's `scale`
    q, k, v = _decode_case(torch.float32, 1, 1, 1, 1, 16, 40, 5)
    got = oracle.decode(np.array([[25]]), [40], synth.to_raw(q), synth.to_raw(k),
                        synth.to_raw(v), [0], 0.7)
    mask = torch.zeros(1, 1, 1, 40, dtype=torch.bool)
    mask[..., 15:] = True
    ref = F.scaled_dot_product_attention(
        _f64(q[0, 0]).reshape(1, 1, 1, 16), _f64(k[0, 0]).permute(1, 0, 2).reshape(1, 1, 40, 16),
        _f64(v[0, 0]).permute(1, 0, 2).reshape(1, 1, 40, 16), attn_mask=mask, scale=0.7)
    assert np.abs(got[0, 0, 0] - ref.reshape(16).numpy()).max() <= 1e-12


def test_decode_residency_equals_masked_full_cache():
    n_layers, n_seqs, n_kv, G, d, T = 3, 2, 2, 2, 16, 300
    q, k, v = _decode_case(torch.bfloat16, n_layers, n_seqs, n_kv, G, d, T, 31)
    windows = np.array([[1, 16], [17, 299], [300, 64]], np.int32)
    L = [300, 171]
    args = (synth.to_raw(q), synth.to_raw(k), synth.to_raw(v), [0, 0], 0.25)
    a = oracle.decode(windows, L, *args)
    b = oracle.decode(windows, L, *args, masked=True)
    assert np.abs(a - b).max() <= 1e-12


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_decode_w1_returns_newest_v_exactly(dtype):
    q, k, v = _decode_case(dtype, 1, 2, 2, 3, 64, 50, 41)
    L = [50, 9]
    got = oracle.decode(np.array([[1, 1]]), L, synth.to_raw(q), synth.to_raw(k),
                        synth.to_raw(v), [0, 0], 0.125)
    vv = synth.raw_to_f64(synth.to_raw(v))
    for b in range(2):
        for i in range(6):
            assert np.array_equal(got[0, b, i], vv[0, b, L[b] - 1, i // 3])


def test_decode_needle_pins_the_window_edge():
    d, T, w = 32, 120, 40
    g = synth.gen(51)
    q = torch.randn(d, generator=g, dtype=torch.float64) / math.sqrt(d)
    k = 0.01 * torch.randn(T, 1, d, generator=g, dtype=torch.float64)
    v = torch.randn(T, 1, d, generator=g, dtype=torch.float64)
    scale = 1.0 / math.sqrt(d)
    needle_k = q / q.norm() * (60.0 / scale / q.norm())  # score exactly 60
    L = T

    def run(pos, key):
        kk = k.clone()
        kk[pos, 0] = key
        raw = lambda x: x.to(torch.float32).numpy()  # noqa: E731
        return oracle.decode(np.array([[w]]), [L],
                             raw(q.reshape(1, 1, 1, d)), raw(kk.reshape(1, 1, T, 1, d)),
                             raw(v.reshape(1, 1, T, 1, d)), [0], scale)[0, 0, 0]

    v32 = v.to(torch.float32).to(torch.float64).numpy()
    for pos in (L - w, L - 1, L - w // 2):  # inside: the needle dominates
        o = run(pos, needle_k)
        assert np.abs(o - v32[pos, 0]).max() < 1e-12
    # just outside: the output does not depend on that key at all
    o_out = run(L - w - 1, needle_k)
    o_zero = run(L - w - 1, torch.zeros(d, dtype=torch.float64))
    assert np.array_equal(o_out, o_zero)
    assert np.abs(o_out - v32[L - w - 1, 0]).max() > 0.1


def test_decode_equal_keys_give_window_mean_and_constant_v_is_returned():
    d, T, w, L = 16, 90, 33, 80
    g = synth.gen(61)
    q = torch.randn(1, 1, 2, d, generator=g)
    k = torch.randn(1, 1, 1, 1, d, generator=g).expand(1, 1, T, 1, d).contiguous()
    v = torch.randn(1, 1, T, 1, d, generator=g)
    got = oracle.decode(np.array([[w]]), [L], q.numpy(), k.numpy(), v.numpy(), [0], 0.3)
    mean = v[0, 0, L - w:L, 0].to(torch.float64).mean(0).numpy()
    assert np.abs(got[0, 0, 0] - mean).max() <= 1e-13
    assert np.abs(got[0, 0, 1] - mean).max() <= 1e-13
    kr = torch.randn(1, 1, T, 1, d, generator=g)
    vc = torch.randn(1, 1, 1, 1, d, generator=g).expand(1, 1, T, 1, d).contiguous()
    got = oracle.decode(np.array([[w]]), [L], q.numpy(), kr.numpy(), vc.numpy(), [0], 0.3)
    assert np.abs(got[0, 0, 0] - vc[0, 0, 0, 0].double().numpy()).max() <= 1e-14


def test_decode_gqa_identical_queries_give_identical_outputs():
    q, k, v = _decode_case(torch.bfloat16, 1, 1, 2, 3, 32, 70, 71)
    q[0, 0, 4] = q[0, 0, 3]  # heads 3 and 4 share kv head 1
    got = oracle.decode(np.array([[20, 60]]), [70], synth.to_raw(q), synth.to_raw(k),
                        synth.to_raw(v), [0], 0.2)
    assert np.array_equal(got[0, 0, 3], got[0, 0, 4])
    assert not np.array_equal(got[0, 0, 2], got[0, 0, 3])


def test_decode_depends_only_on_window_content_not_position():
    d, w = 16, 24
    q, k, v = _decode_case(torch.bfloat16, 1, 1, 1, 2, d, w, 81)
    outs = []
    for base in (0, 5, 1000, 123456):
        # same w tokens placed at [base, base+w); history given from `base`
        L = base + w
        outs.append(oracle.decode(np.array([[w]]), [L], synth.to_raw(q), synth.to_raw(k),
                                  synth.to_raw(v), [base], 0.25))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_decode_rejects_history_that_misses_the_window():
    q, k, v = _decode_case(torch.float32, 1, 1, 1, 1, 8, 10, 3)
    with pytest.raises(ValueError):
        oracle.decode(np.array([[11]]), [12], q.numpy(), k.numpy(), v.numpy(), [2], 1.0)


def _brute_decode(q, k, v, L, w, scale):
    """numpy twin written independently: loop over positions, float64."""
    lo = max(0, L - w)
    s = np.array([scale * float(np.dot(q, k[t])) for t in range(lo, L)])
    p = np.exp(s - s.max())
    return (p[:, None] * v[lo:L]).sum(0) / p.sum()


def test_decode_brute_force_tiny():
    rng = np.random.default_rng(91)
    for trial in range(20):
        n_kv, G, d = rng.integers(1, 4), rng.integers(1, 4), rng.integers(1, 9)
        T = int(rng.integers(1, 40))
        L = int(rng.integers(1, T + 1))
        w = rng.integers(1, 50, size=(1, n_kv)).astype(np.int32)
        q = rng.standard_normal((1, 1, n_kv * G, d)).astype(np.float32)
        k = rng.standard_normal((1, 1, T, n_kv, d)).astype(np.float32)
        v = rng.standard_normal((1, 1, T, n_kv, d)).astype(np.float32)
        got = oracle.decode(w, [L], q, k, v, [0], 0.5)
        for i in range(n_kv * G):
            h = i // G
            ref = _brute_decode(q[0, 0, i].astype(np.float64), k[0, 0, :, h].astype(np.float64),
                                v[0, 0, :, h].astype(np.float64), L, int(w[0, h]), 0.5)
            assert np.abs(got[0, 0, i] - ref).max() <= 1e-12


def test_decode_through_the_pool_equals_decode_from_history():
    """Append a token stream with the append model, read each head's window
    back from the pool bytes, and attend: same result as the logical history
    (residency materialised, not masked)."""
    bs, d, G = 4, 8, 2
    windows = np.array([[5, 12, 1], [9, 4, 30]], np.int32)
    n_layers, n_kv = windows.shape
    nb, off, bps = oracle.layout(windows, bs)
    n_seqs, n_tok = 2, 37
    rng = np.random.default_rng(17)
    table = rng.permutation(n_seqs * bps).astype(np.int32).reshape(n_seqs, bps)
    k = rng.standard_normal((n_layers, n_seqs, n_tok, n_kv, d)).astype(np.float32)
    v = rng.standard_normal((n_layers, n_seqs, n_tok, n_kv, d)).astype(np.float32)
    q = rng.standard_normal((n_layers, n_seqs, n_kv * G, d)).astype(np.float32)
    pool = np.zeros(n_seqs * bps * 2 * bs * d * 4, np.uint8)
    for t0, c in ((0, 10), (10, 1), (11, 26)):
        oracle.append(pool, table, windows, bs, d, 0, [t0] * n_seqs,
                      k[:, :, t0:t0 + c], v[:, :, t0:t0 + c])
    ref = oracle.decode(windows, [n_tok] * n_seqs, q, k, v, [0] * n_seqs, 0.3)
    W = int(windows.max())
    base = n_tok - W
    kh = np.zeros((n_layers, n_seqs, W, n_kv, d), np.float32)
    vh = np.zeros_like(kh)
    for l in range(n_layers):
        for b in range(n_seqs):
            for h in range(n_kv):
                hi = l * n_kv + h
                for t in range(max(base, n_tok - int(windows[l, h])), n_tok):
                    kh[l, b, t - base, h] = _pool_row(pool, table, off, nb, b, hi, t, 0, bs, d, 4).view(np.float32)
                    vh[l, b, t - base, h] = _pool_row(pool, table, off, nb, b, hi, t, 1, bs, d, 4).view(np.float32)
    got = oracle.decode(windows, [n_tok] * n_seqs, q, kh, vh, [base] * n_seqs, 0.3)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# chunked prefill
# --------------------------------------------------------------------------

def _prefill_case(dtype, n_seqs, n_kv, G, d, P, n, seed):
    q = _t((n_seqs, n, n_kv * G, d), seed, dtype, std=1.0 / math.sqrt(d))
    kc = _t((n_seqs, n, n_kv, d), seed + 1, dtype)
    vc = _t((n_seqs, n, n_kv, d), seed + 2, dtype)
    kh = _t((n_seqs, P, n_kv, d), seed + 3, dtype)
    vh = _t((n_seqs, P, n_kv, d), seed + 4, dtype)
    return q, kc, vc, kh, vh


def _raw(*ts):
    return [synth.to_raw(t) for t in ts]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_prefill_full_window_is_causal_attention(dtype):
    n_seqs, n_kv, G, d, P, n = 2, 2, 2, 32, 45, 30
    q, kc, vc, kh, vh = _prefill_case(dtype, n_seqs, n_kv, G, d, P, n, 101)
    scale = 1.0 / math.sqrt(d)
    got = oracle.prefill([P + n, 10 ** 5], [P] * n_seqs, *_raw(q, kc, vc, kh, vh),
                         [0] * n_seqs, scale)
    for b in range(n_seqs):
        # full sequence [0, P+n): queries for the first P rows are dummies;
        # torch's is_causal (square) mask is the plain causal definition
        k_all = torch.cat([_f64(kh[b]), _f64(kc[b])]).permute(1, 0, 2).unsqueeze(0)
        v_all = torch.cat([_f64(vh[b]), _f64(vc[b])]).permute(1, 0, 2).unsqueeze(0)
        q_all = torch.cat([torch.zeros(P, n_kv * G, d, dtype=torch.float64), _f64(q[b])])
        o = F.scaled_dot_product_attention(q_all.permute(1, 0, 2).unsqueeze(0), k_all, v_all,
                                           is_causal=True, enable_gqa=True)
        ref = o[0].permute(1, 0, 2)[P:].numpy()
        assert np.abs(got[b] - ref).max() <= 1e-12


@pytest.mark.parametrize("d", [16, 256])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_prefill_window_is_band_masked_attention(dtype, d):
    n_seqs, n_kv, G, P, n = 2, 3, 2, 50, 40
    q, kc, vc, kh, vh = _prefill_case(dtype, n_seqs, n_kv, G, d, P, n, 111)
    windows = [1, 17, 64]
    pos0 = [50, 0]
    scale = 0.3
    got = oracle.prefill(windows, pos0, *_raw(q, kc, vc, kh, vh), [0, 0], scale)
    for b in range(n_seqs):
        Pb = pos0[b]
        k_all = torch.cat([_f64(kh[b, :Pb]), _f64(kc[b])]).permute(1, 0, 2).unsqueeze(0)
        v_all = torch.cat([_f64(vh[b, :Pb]), _f64(vc[b])]).permute(1, 0, 2).unsqueeze(0)
        Lk = Pb + n
        mask = torch.zeros(1, n_kv * G, n, Lk, dtype=torch.bool)
        t = torch.arange(Lk)
        for i in range(n_kv * G):
            for r in range(n):
                p = Pb + r
                mask[0, i, r] = (t <= p) & (t > p - windows[i // G])
        o = F.scaled_dot_product_attention(_f64(q[b]).permute(1, 0, 2).unsqueeze(0), k_all, v_all,
                                           attn_mask=mask, scale=scale, enable_gqa=True)
        ref = o[0].permute(1, 0, 2).numpy()
        assert np.abs(got[b] - ref).max() <= 1e-12


def test_prefill_chunk_size_invariance():
    n_kv, G, d, P, n = 2, 2, 16, 60, 48
    q, kc, vc, kh, vh = _prefill_case(torch.bfloat16, 1, n_kv, G, d, P, n, 121)
    windows = [20, 100]
    q, kc, vc, kh, vh = _raw(q, kc, vc, kh, vh)
    whole = oracle.prefill(windows, [P], q, kc, vc, kh, vh, [0], 0.25)
    for n1 in (1, 17, 47):
        a = oracle.prefill(windows, [P], q[:, :n1], kc[:, :n1], vc[:, :n1], kh, vh, [0], 0.25)
        kh2 = np.concatenate([kh, kc[:, :n1]], axis=1)
        vh2 = np.concatenate([vh, vc[:, :n1]], axis=1)
        b = oracle.prefill(windows, [P + n1], q[:, n1:], kc[:, n1:], vc[:, n1:], kh2, vh2,
                           [0], 0.25)
        assert np.abs(np.concatenate([a, b], axis=1) - whole).max() <= 1e-13


def test_prefill_last_row_equals_decode():
    n_kv, G, d, P, n = 2, 3, 32, 70, 25
    q, kc, vc, kh, vh = _prefill_case(torch.bfloat16, 1, n_kv, G, d, P, n, 131)
    windows = np.array([[9, 64]], np.int32)
    q, kc, vc, kh, vh = _raw(q, kc, vc, kh, vh)
    pf = oracle.prefill(windows[0], [P], q, kc, vc, kh, vh, [0], 0.2, rows=[n - 1])
    k_all = np.concatenate([kh, kc], axis=1)[None]
    v_all = np.concatenate([vh, vc], axis=1)[None]
    dec = oracle.decode(windows, [P + n], q[None, :, n - 1], k_all, v_all, [0], 0.2)
    assert np.abs(pf[0, 0] - dec[0, 0]).max() <= 1e-13


def test_prefill_row_subset_matches_all_rows():
    q, kc, vc, kh, vh = _raw(*_prefill_case(torch.float32, 2, 1, 2, 8, 20, 16, 141))
    whole = oracle.prefill([7], [20, 3], q, kc, vc, kh, vh, [0, 0], 0.5)
    some = oracle.prefill([7], [20, 3], q, kc, vc, kh, vh, [0, 0], 0.5, rows=[15, 0, 6])
    assert np.array_equal(some, whole[:, [15, 0, 6]])


def test_large_logits_stay_finite_and_match_sdpa():
    """Scores in the hundreds: a softmax without the max shift overflows."""
    d, T, L = 16, 60, 60
    g = synth.gen(151)
    q = (40.0 * torch.randn(1, 1, 2, d, generator=g))
    k = torch.randn(1, 1, T, 1, d, generator=g)
    v = torch.randn(1, 1, T, 1, d, generator=g)
    got = oracle.decode(np.array([[33]]), [L], q.numpy(), k.numpy(), v.numpy(), [0], 1.0)
    assert np.all(np.isfinite(got))
    ref = _sdpa_decode(_f64(q[0, 0]), _f64(k[0, 0]), _f64(v[0, 0]), L, [33], scale=1.0)
    assert np.abs(got[0, 0] - ref.numpy()).max() <= 1e-12 * max(1.0, np.abs(ref.numpy()).max())
    qp = 40.0 * torch.randn(1, 8, 2, d, generator=g)
    kc = torch.randn(1, 8, 1, d, generator=g)
    vc = torch.randn(1, 8, 1, d, generator=g)
    pf = oracle.prefill([5], [T], qp.numpy(), kc.numpy(), vc.numpy(), k[0].numpy(), v[0].numpy(),
                        [0], 1.0)
    assert np.all(np.isfinite(pf))
