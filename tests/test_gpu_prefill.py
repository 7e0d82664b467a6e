"""Chunked-prefill parity on the GPU against the fp64 oracle.

Row metric as for decode: max|o - r| / max|r| <= 2e-3 per output row (bf16
cache, fp32 output).  Covers ragged chunk ends, P = 0 (no history), windows
shorter and longer than the chunk, all GQA group sizes, d = 64, 128 and 256,
chunk-size invariance, last row == decode, the 161K-context configuration on
sampled rows, and both precisions of the P.V product: P in fp16 (the
default entry, with its fall-back for V values outside fp16's range) and P
split into two bf16 products (hwkv_prefill_attn_exact)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_common import (BF16_TOL, DECODE_REGRESSION_TOL, device, hw, row_rel_err, say,
                         to_host_f64)

pytestmark = pytest.mark.gpu


class PrefillCase:
    def __init__(self, windows, d, G, pos0, n, seed, hist_keep=None, out_dtype=torch.float32,
                 split_chunks=None, dtype=torch.bfloat16, block_size=16, block_ids=None,
                 v_edit=None):
        """v_edit(v, b, p0): edits, in place, a V tensor [..., rows, n_kv, d]
        whose rows hold positions p0, p0 + 1, ... of sequence b (None for the
        chunk, which holds every sequence: v[b] starts at pos0[b])."""
        H = hw()
        dev = device()
        self.windows = np.asarray(windows, np.int32)
        n_kv = self.windows.shape[0]
        self.n_kv, self.G, self.d, self.n = n_kv, G, d, n
        self.pos0 = list(pos0)
        n_seqs = len(pos0)
        self.lay = H.hwkv_layout_create(self.windows[None, :], block_size, d, dtype)
        self.cache = H.make_cache(self.lay, n_seqs, device=dev, fill=0xFF, block_ids=block_ids)
        # the fast entry's workspace, filled with NaN bit patterns: rows the
        # call reads are always written first
        self.ws = H.make_prefill_workspace(self.lay, 0, n_seqs, n, device=dev)
        self.ws.fill_(0xFF)
        g = synth.gen(seed, dev)
        bs = block_size
        cap = int(((self.windows.astype(np.int64) + bs - 1) // bs * bs).max())
        keep = cap if hist_keep is None else hist_keep
        self.hbase = [max(0, p - keep) for p in pos0]
        Th = max(max(p - hb for p, hb in zip(pos0, self.hbase)), 1)
        self.Th = Th
        raw_dt = np.float16 if dtype == torch.float16 else np.uint16
        self.k_hist = np.zeros((n_seqs, Th, n_kv, d), raw_dt)
        self.v_hist = np.zeros_like(self.k_hist)
        for b in range(n_seqs):
            nh = pos0[b] - self.hbase[b]
            if nh == 0:
                continue
            kh = synth.randn((1, 1, nh, n_kv, d), dtype, g)
            vh = synth.randn((1, 1, nh, n_kv, d), dtype, g)
            if v_edit is not None:
                v_edit(vh[0, 0], b, self.hbase[b])
            self.k_hist[b, :nh] = synth.to_raw(kh[0, 0])
            self.v_hist[b, :nh] = synth.to_raw(vh[0, 0])
            H.hwkv_append(self.cache, 0, 1, torch.tensor([self.hbase[b]], device=dev), kh, vh,
                          seq_slots=torch.tensor([b], dtype=torch.int32, device=dev))
        self.q = synth.randn((n_seqs, n, n_kv * G, d), dtype, g, std=1.0 / math.sqrt(d))
        self.k = synth.randn((n_seqs, n, n_kv, d), dtype, g)
        self.v = synth.randn((n_seqs, n, n_kv, d), dtype, g)
        if v_edit is not None:
            for b in range(n_seqs):
                v_edit(self.v[b], b, pos0[b])
        torch.cuda.synchronize()

    def run(self, out_dtype=torch.float32, scale=None, exact=False):
        H = hw()
        dev = device()
        out = torch.full((len(self.pos0), self.n, self.n_kv * self.G, self.d), float("nan"),
                         dtype=out_dtype, device=dev)
        s = 1.0 / math.sqrt(self.d) if scale is None else scale
        self.call(torch.tensor(self.pos0, device=dev), out, s, exact=exact)
        torch.cuda.synchronize()
        return out

    def call(self, pos0, out, scale, exact=False, seq_slots=None, cache=None):
        """One call of the fast (default) or the exact entry on this case's q, k, v."""
        H = hw()
        cache = self.cache if cache is None else cache
        if exact:
            H.hwkv_prefill_attn_exact(cache, 0, pos0, self.q, self.k, self.v, out, scale,
                                      seq_slots=seq_slots)
        else:
            H.hwkv_prefill_attn(cache, 0, pos0, self.q, self.k, self.v, self.ws, out, scale,
                                seq_slots=seq_slots)

    def oracle(self, rows=None, scale=None):
        s = 1.0 / math.sqrt(self.d) if scale is None else scale
        return oracle.prefill(self.windows, self.pos0, synth.to_raw(self.q), synth.to_raw(self.k),
                              synth.to_raw(self.v), self.k_hist, self.v_hist, self.hbase, s,
                              rows=rows)


def _check(got, ref):
    assert np.all(np.isfinite(got))
    err = row_rel_err(got, ref)
    say("max row rel err", err)
    assert err <= BF16_TOL, err


def test_small_ragged_with_and_without_history():
    say("prefill small ragged")
    c = PrefillCase([1, 17, 64, 100], 128, 3, [50, 0], 77, seed=401)
    _check(to_host_f64(c.run()), c.oracle())


@pytest.mark.parametrize("d,G", [(128, 1), (128, 2), (128, 4), (64, 3), (64, 6), (64, 8),
                                 (128, 8)])
def test_instances(d, G):
    say("prefill instance", d, G)
    c = PrefillCase([33, 700], d, G, [1000, 40, 3], 96, seed=402)
    _check(to_host_f64(c.run()), c.oracle())


def test_windows_longer_than_history_and_chunk_boundaries():
    # windows reaching past position 0, chunk starting mid-block, long chunk
    say("prefill long windows")
    c = PrefillCase([2000, 16, 300, 4096], 128, 3, [123, 1711], 300, seed=403)
    _check(to_host_f64(c.run()), c.oracle())


def test_bf16_output_and_scale():
    say("prefill bf16 out")
    c = PrefillCase([64, 130], 128, 2, [500], 64, seed=404)
    got = to_host_f64(c.run(out_dtype=torch.bfloat16, scale=0.07))
    ref = c.oracle(scale=0.07)
    ref_b = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.abs(got - ref_b).max() <= np.abs(ref).max() * 2 ** -7


def test_f16_output():
    """fp16 outputs: the oracle rounded to binary16 (nearest even), within half
    a binary16 ulp of the largest output plus the kernel's own error (the
    exact variant's fp32 result carries ~1e-5 of the row maximum, so
    element-wise ulps of small entries are not a fair measure)."""
    say("prefill f16 out")
    c = PrefillCase([64, 130, 2000], 128, 2, [500, 0], 100, seed=409)
    got = c.run(out_dtype=torch.float16, exact=True).cpu().numpy().astype(np.float64)
    ref = c.oracle()
    ref16 = ref.astype(np.float16).astype(np.float64)
    assert np.abs(got - ref16).max() <= np.abs(ref).max() * 2 ** -10


def test_f16_output_default_entry():
    """The default entry (P in fp16 for the P.V product) with fp16 outputs,
    against the oracle at the gate: the fp16-P error (3-4.5e-4 of the row
    maximum, measured) plus the output rounding (at most half a binary16 ulp,
    2^-11 of the row maximum) stay well inside 2e-3."""
    say("prefill f16 out, default entry")
    c = PrefillCase([64, 130, 2000], 128, 2, [500, 0], 100, seed=409)
    _check(to_host_f64(c.run(out_dtype=torch.float16)), c.oracle())
    c16 = PrefillCase([64, 130, 2000], 128, 2, [500, 0], 100, seed=410, dtype=torch.float16)
    _check(to_host_f64(c16.run(out_dtype=torch.float16)), c16.oracle())


def test_workspace_rules():
    """fp16 caches need no workspace (a null one is accepted and the result is
    that of a call with one); bf16 caches refuse a null or short workspace
    before launching anything, and a larger one changes nothing."""
    H = hw()
    dev = device()
    say("prefill workspace rules")
    c16 = PrefillCase([64, 130, 2000], 128, 2, [500, 0], 100, seed=411, dtype=torch.float16)
    assert H.hwkv_prefill_workspace_bytes(c16.lay, 0, 2, 100) == 0
    with_ws = c16.run()
    pos = torch.tensor(c16.pos0, device=dev)
    out = torch.full_like(with_ws, float("nan"))
    H.hwkv_prefill_attn(c16.cache, 0, pos, c16.q, c16.k, c16.v, None, out, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(out, with_ws)
    c = PrefillCase([64, 700], 128, 3, [500, 40], 33, seed=412)
    good = c.run()
    need = H.hwkv_prefill_workspace_bytes(c.lay, 0, 2, 33)
    assert need == 2 * ((63 + 33) + (699 + 33)) * 256
    pos = torch.tensor(c.pos0, device=dev)
    out = torch.zeros_like(good)
    for ws, status in ((None, "HWKV_ERR_INVALID_ARG"), (c.ws[:need - 256], "HWKV_ERR_CAPACITY")):
        with pytest.raises(H.HwkvError) as e:
            H.hwkv_prefill_attn(c.cache, 0, pos, c.q, c.k, c.v, ws, out, 1 / math.sqrt(128))
        assert e.value.status_name == status
    torch.cuda.synchronize()
    assert torch.all(out == 0)  # nothing was launched
    big = H._alloc_aligned(need + (1 << 20), dev)
    big.fill_(0x7F)
    H.hwkv_prefill_attn(c.cache, 0, pos, c.q, c.k, c.v, big, out, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(out, good)


def test_many_sequences():
    """260 sequences x 8 KV heads (2080 (sequence, kv head) pairs: the V
    pre-pass gives each pair one workgroup), ragged positions, every row of
    every sequence against the oracle."""
    say("prefill many sequences")
    rng = np.random.default_rng(9)
    pos0 = [int(x) for x in rng.integers(0, 700, 260)]
    c = PrefillCase([16, 64, 100, 300, 33, 1, 257, 200], 128, 3, pos0, 40, seed=413)
    _check(to_host_f64(c.run()), c.oracle())


def test_chunk_size_invariance_and_last_row_equals_decode():
    """Prefill n rows at once == prefill n1, append n1, prefill the rest; the
    last row equals a decode step at L = P + n after appending the chunk.
    Run on the exact variant (~1e-5): with P rounded to fp16 the rounding
    depends on each workgroup's running maximum, which the chunking moves, so
    the default entry agrees only to its own error (checked at the gate)."""
    H = hw()
    dev = device()
    windows = [40, 500, 96]
    P, n, n1 = 700, 160, 70
    say("prefill chunk invariance")
    whole = PrefillCase(windows, 128, 3, [P], n, seed=405)
    o_all = whole.run(exact=True)
    o_fast = whole.run()
    assert row_rel_err(to_host_f64(o_fast), to_host_f64(o_all)) <= BF16_TOL
    two = PrefillCase(windows, 128, 3, [P], n, seed=405)
    q, k, v = two.q, two.k, two.v
    out1 = torch.empty((1, n1, 9, 128), dtype=torch.float32, device=dev)
    H.hwkv_prefill_attn_exact(two.cache, 0, torch.tensor([P], device=dev),
                              q[:, :n1].contiguous(), k[:, :n1].contiguous(),
                              v[:, :n1].contiguous(), out1, 1 / math.sqrt(128))
    H.hwkv_append(two.cache, 0, 1, torch.tensor([P], device=dev), k[None, :, :n1].contiguous(),
                  v[None, :, :n1].contiguous())
    out2 = torch.empty((1, n - n1, 9, 128), dtype=torch.float32, device=dev)
    H.hwkv_prefill_attn_exact(two.cache, 0, torch.tensor([P + n1], device=dev),
                              q[:, n1:].contiguous(), k[:, n1:].contiguous(),
                              v[:, n1:].contiguous(), out2, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    o_two = torch.cat([out1, out2], dim=1)
    assert row_rel_err(to_host_f64(o_two), to_host_f64(o_all)) <= 1e-5
    # decode at L = P + n over the appended chunk, for the last query row
    H.hwkv_append(two.cache, 0, 1, torch.tensor([P + n1], device=dev),
                  k[None, :, n1:].contiguous(), v[None, :, n1:].contiguous())
    ws = H.make_workspace(two.lay, 0, 1, 1, 9, device=dev)
    dec = torch.empty((1, 1, 9, 128), dtype=torch.float32, device=dev)
    H.hwkv_decode_attn(two.cache, 0, 1, torch.tensor([P + n], device=dev),
                       q[None, :, n - 1].contiguous(), 1 / math.sqrt(128), ws, dec)
    torch.cuda.synchronize()
    assert row_rel_err(to_host_f64(dec[0, 0]), to_host_f64(o_all[0, n - 1])) <= 1e-5


def test_prefill_config_161k_then_append_and_decode():
    """4 sequences at 161K context, one 2048-token chunk, windows of the
    printed policy's layer 0 (up to 65536): sampled rows (first, last, tile
    and window edges, random) of every head against the oracle; then the
    chunk is appended and decode steps follow (the appending split, two
    launches per step), every head checked against the oracle over the
    logical stream history + chunk + new tokens."""
    H = hw()
    dev = device()
    P, n, n_kv, G, d = synth.CTX_161K, 2048, 8, 3, 128
    say("prefill 161K config: fill")
    c = PrefillCase(list(synth.YAML_LAYER0), d, G, [P] * 4, n, seed=105)
    say("prefill 161K config: run")
    out32 = c.run()
    got = to_host_f64(out32)
    # the benchmark's launch writes bf16: the same fp32 results rounded to
    # nearest even, bit for bit
    say("prefill 161K config: bf16 output")
    out16 = c.run(out_dtype=torch.bfloat16)
    assert torch.equal(out16, out32.to(torch.bfloat16))
    del out16, out32
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 1, 31, 32, 63, 64, 1023, 1024, 2046, 2047] +
                      list(rng.integers(0, 2048, 14))))
    say("prefill 161K config: oracle on", len(rows), "rows")
    ref = c.oracle(rows=rows)
    _check(got[:, rows], ref)

    say("prefill 161K config: append the chunk, decode")
    pos0 = torch.tensor(c.pos0, device=dev)
    H.hwkv_append(c.cache, 0, 1, pos0, c.k[None], c.v[None])
    steps = 3
    g = synth.gen(1051, dev)
    kd = synth.randn((steps, 1, 4, 1, n_kv, d), torch.bfloat16, g)
    vd = synth.randn((steps, 1, 4, 1, n_kv, d), torch.bfloat16, g)
    qd = synth.randn((steps, 1, 4, n_kv * G, d), torch.bfloat16, g, std=1.0 / math.sqrt(d))
    ws = H.make_workspace(c.lay, 0, 1, 4, n_kv * G, device=dev)
    outs = []
    for i in range(steps):
        out = torch.full((1, 4, n_kv * G, d), float("nan"), dtype=torch.float32, device=dev)
        H.hwkv_decode_append_attn(c.cache, 0, 1, pos0 + n + i, kd[i], vd[i], qd[i],
                                  1.0 / math.sqrt(d), ws, out)
        outs.append(out)
    torch.cuda.synchronize()
    # logical stream of every sequence from the history base on
    k_all = np.concatenate([c.k_hist, synth.to_raw(c.k), synth.to_raw(kd[:, 0, :, 0]
                                                                      ).transpose(1, 0, 2, 3)],
                           axis=1)[None]
    v_all = np.concatenate([c.v_hist, synth.to_raw(c.v), synth.to_raw(vd[:, 0, :, 0]
                                                                      ).transpose(1, 0, 2, 3)],
                           axis=1)[None]
    worst = 0.0
    for i in range(steps):
        L = P + n + i + 1
        ref = oracle.decode(c.windows[None, :], [L] * 4, synth.to_raw(qd[i]), k_all, v_all,
                            c.hbase, 1.0 / math.sqrt(d))
        o = to_host_f64(outs[i])
        assert np.all(np.isfinite(o))
        worst = max(worst, row_rel_err(o, ref))
    say("161K decode after prefill: max row rel err", worst)
    assert worst <= BF16_TOL
    assert worst <= DECODE_REGRESSION_TOL, worst


def test_prefill_config_161k_head_dim256():
    """The 161K chunk at head_dim 256 (the configuration the benchmark's
    mixed-stack leg times: 4 sequences, 2048 rows at P = 164,864, layer-0
    windows up to 65536, 8 KV x 3 query heads, default entry): sampled rows
    of every head against the oracle; the bf16 output the benchmark writes
    equals the fp32 results rounded to nearest even."""
    P, n, G, d = synth.CTX_161K, 2048, 3, 256
    say("prefill 161K head_dim 256: fill")
    c = PrefillCase(list(synth.YAML_LAYER0), d, G, [P] * 4, n, seed=106)
    say("prefill 161K head_dim 256: run")
    out32 = c.run()
    got = to_host_f64(out32)
    out16 = c.run(out_dtype=torch.bfloat16)
    assert torch.equal(out16, out32.to(torch.bfloat16))
    del out16, out32
    rng = np.random.default_rng(8)
    rows = sorted(set([0, 1, 31, 32, 63, 64, 1023, 1024, 2046, 2047] +
                      list(rng.integers(0, 2048, 10))))
    say("prefill 161K head_dim 256: oracle on", len(rows), "rows")
    _check(got[:, rows], c.oracle(rows=rows))


@pytest.mark.parametrize("d,G", [(128, 3), (64, 2), (128, 8)])
def test_f16_instances(d, G):
    """fp16 cache: fp16 MFMA tiles, P rounded once to fp16 for the PV product."""
    say("prefill f16", d, G)
    c = PrefillCase([300, 17, 2048, 64][:2 if G == 8 else 4], d, G, [1000, 0, 77], 333, seed=711,
                    dtype=torch.float16)
    _check(to_host_f64(c.run()), c.oracle())


@pytest.mark.parametrize("bs,dtype", [(32, torch.bfloat16), (64, torch.float16),
                                      (256, torch.bfloat16)])
def test_other_block_sizes_with_permuted_ids(bs, dtype):
    """Cache blocks of 32..256 tokens (each 64-key tile gathers its 16-key
    slices from the blocks that hold them), permuted block ids, history that
    wraps the rings; bit-identical to 16-token blocks."""
    windows = [4096, 1000, 65, 300]
    say("prefill block size", bs, dtype)
    H = hw()
    lay = H.hwkv_layout_create(np.array([windows], np.int32), bs, 128, dtype)
    bps = lay.desc().blocks_per_seq
    perm = np.random.default_rng(bs).permutation(2 * bps).astype(np.int32).reshape(2, bps)
    c = PrefillCase(windows, 128, 3, [9000, 130], 400, seed=712, dtype=dtype, block_size=bs,
                    block_ids=perm)
    out = c.run()
    _check(to_host_f64(out), c.oracle())
    c16 = PrefillCase(windows, 128, 3, [9000, 130], 400, seed=712, dtype=dtype, block_size=16)
    assert torch.equal(out, c16.run())


@pytest.mark.parametrize("G,dtype", [(1, torch.bfloat16), (2, torch.float16), (3, torch.bfloat16),
                                     (4, torch.float16), (6, torch.bfloat16), (8, torch.float16)])
def test_head_dim_256(G, dtype):
    """head_dim 256 (32 KiB K/V tiles, one wave per SIMD): ragged chunk end,
    no history, windows shorter and longer than the chunk."""
    say("prefill head_dim 256", G, dtype)
    c = PrefillCase([33, 700, 4096, 1], 256, G, [1000, 40, 0], 150, seed=430 + G, dtype=dtype)
    _check(to_host_f64(c.run()), c.oracle())


def test_head_dim_256_block_sizes_bitwise():
    """head_dim 256 with 64-token blocks and permuted ids equals 16-token
    blocks bit for bit, and matches the oracle."""
    windows = [2048, 300, 65]  # the longest a multiple of 64: both caches draw the same history
    say("prefill head_dim 256 block size 64")
    H = hw()
    lay = H.hwkv_layout_create(np.array([windows], np.int32), 64, 256, torch.bfloat16)
    bps = lay.desc().blocks_per_seq
    perm = np.random.default_rng(64).permutation(2 * bps).astype(np.int32).reshape(2, bps)
    c = PrefillCase(windows, 256, 2, [3000, 70], 200, seed=440, block_size=64, block_ids=perm)
    out = c.run()
    _check(to_host_f64(out), c.oracle())
    c16 = PrefillCase(windows, 256, 2, [3000, 70], 200, seed=440, block_size=16)
    assert torch.equal(out, c16.run())


EXACT_TOL = 1e-4  # P split into bf16 high part + bf16 remainder: ~16 significant bits


@pytest.mark.parametrize("d,G", [(128, 3), (64, 4), (256, 2)])
def test_exact_variant_and_fp16_p_error(d, G):
    """Both P.V precisions against the oracle on one case: the exact variant
    within 1e-4 (measured ~1e-5), the default (P in fp16) within the gate."""
    say("prefill exact vs fp16 P", d, G)
    c = PrefillCase([2000, 16, 300, 4096], d, G, [1234, 5000], 200, seed=450 + d)
    ref = c.oracle()
    err_x = row_rel_err(to_host_f64(c.run(exact=True)), ref)
    err_f = row_rel_err(to_host_f64(c.run()), ref)
    say("exact", err_x, "fp16 P", err_f)
    assert err_x <= EXACT_TOL
    assert err_f <= BF16_TOL


@pytest.mark.parametrize("d", [128, 64, 256])
def test_v_beyond_fp16_range_falls_back_to_exact(d):
    """V elements of +-2^20 (finite in bf16, beyond fp16's 65504) in the
    history and in the chunk: the fp16 pass of every workgroup that reads them
    turns non-finite, so those rows are redone exactly; all rows
    match the oracle, and the rows that attend to the large values equal the
    exact variant bit for bit (the fast pass marks every row whose result is
    non-finite, and the second pass recomputes exactly those)."""
    big = 2.0 ** 20
    P, n = 3000, 130
    hist_pos, chunk_row = P - 5, 10

    def edit(v, b, p0):
        if b != 0:
            return
        if p0 < P:  # history rows
            v[hist_pos - p0, 0, 3] = big
        else:       # chunk rows
            v[chunk_row, 1, d - 7] = -big

    say("prefill V beyond fp16 range", d)
    c = PrefillCase([64, 500, 16, 2000], d, 3, [P, 700], n, seed=460, v_edit=edit)
    out = c.run()
    got = to_host_f64(out)
    _check(got, c.oracle())
    exact = c.run(exact=True)
    # kv head 0 (window 64) reads the history value in rows r <= 58 (position
    # P + r - 63 <= hist_pos); kv head 1 (window 500) reads the chunk value in
    # every row r >= chunk_row
    assert torch.equal(out[0, :59, 0:3], exact[0, :59, 0:3])
    assert torch.equal(out[0, chunk_row:, 3:6], exact[0, chunk_row:, 3:6])


@pytest.mark.parametrize("d", [128, 64, 256])
def test_tiny_v_falls_back_to_exact(d):
    """V of kv head 1 scaled by 2^-20 (|v| ~ 1e-6: normal in bf16, subnormal
    in fp16): its outputs are far below 2^-12 of their softmax sums, so its
    rows are redone exactly (bit for bit the exact variant) while the other heads keep
    the fp16 pass; every row matches the oracle."""
    def edit(v, b, p0):
        v[..., 1, :] *= 2.0 ** -20

    say("prefill tiny V", d)
    c = PrefillCase([300, 2000, 64], d, 2, [1500, 40], 96, seed=470, v_edit=edit)
    out = c.run()
    _check(to_host_f64(out), c.oracle())
    exact = c.run(exact=True)
    assert torch.equal(out[:, :, 2:4], exact[:, :, 2:4])


@pytest.mark.parametrize("n,pos0", [(1, [0, 5, 4096]), (2, [1, 17, 300]), (33, [0, 64, 1000])])
def test_tiny_chunks(n, pos0):
    """Chunks of 1, 2 and 33 rows (one workgroup, mostly idle waves; a single
    row at P = 0 attends to itself only), both precisions."""
    say("prefill tiny chunk", n, pos0)
    c = PrefillCase([1, 100, 2000], 128, 3, pos0, n, seed=480 + n)
    ref = c.oracle()
    _check(to_host_f64(c.run()), ref)
    assert row_rel_err(to_host_f64(c.run(exact=True)), ref) <= EXACT_TOL


def test_prefill_graph_replays_match_eager():
    """Both prefill entries captured in one HIP graph (a workgroup of the
    default entry redoes its rows exactly when it meets the V value beyond
    fp16's range): three replays, with eager work and synchronisations in
    between, each bit-identical to the eager calls."""
    H = hw()
    dev = device()
    big = 2.0 ** 20

    def edit(v, b, p0):
        if b == 0 and p0 < 900:
            v[900 - 3 - p0, 1, 5] = big

    say("prefill graph replays")
    c = PrefillCase([64, 500, 2000], 128, 3, [900, 40], 130, seed=490, v_edit=edit)
    pos = torch.tensor(c.pos0, device=dev)
    shape = (len(c.pos0), c.n, c.n_kv * c.G, c.d)
    o_fast = torch.zeros(shape, dtype=torch.float32, device=dev)
    o_exact = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    scale = 1.0 / math.sqrt(c.d)

    def calls():
        c.call(pos, o_fast, scale)
        c.call(pos, o_exact, scale, exact=True)

    calls()
    torch.cuda.synchronize()
    want_fast, want_exact = o_fast.clone(), o_exact.clone()
    _check(to_host_f64(want_fast), c.oracle())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()  # warm the launch path on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(3):
        o_fast.fill_(float("nan"))
        o_exact.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_fast, want_fast), rep
        assert torch.equal(o_exact, want_exact), rep


def test_invalid_slot_and_negative_position_give_nan_rows():
    """A slot outside the block table, or pos0 < 0, makes that sequence's rows
    NaN (nothing outside the table or pool is read); the other sequences'
    rows are bit-identical to a call with valid arguments."""
    H = hw()
    dev = device()
    say("prefill invalid slot / position")
    c = PrefillCase([64, 700], 128, 3, [500, 300, 900], 40, seed=495)
    good = c.run()
    scale = 1.0 / math.sqrt(c.d)
    for slots, pos0, bad in (([0, 7, 2], c.pos0, 1), ([0, 1, 2], [500, -3, 900], 1),
                             ([-1, 1, 2], c.pos0, 0)):
        out = torch.zeros_like(good)
        c.call(torch.tensor(pos0, device=dev), out, scale,
               seq_slots=torch.tensor(slots, dtype=torch.int32, device=dev))
        torch.cuda.synchronize()
        assert torch.all(torch.isnan(out[bad])), (slots, pos0)
        for b in range(3):
            if b != bad:
                assert torch.equal(out[b], good[b]), (slots, pos0, b)
