"""Bad device values on the GPU: the one behaviour every kernel shares.

Device arrays are the caller's contract.  The kernels never let a bad value
steer a memory access, and they turn each one into a visible result:
  - a block id outside the pool: append skips the rows that map to it; an
    attention query row whose window holds a key stored in that block is
    NaN (decode: every query head of that (sequence, kv head); prefill:
    exactly the chunk rows whose window reaches the block's keys);
  - a meta blob of another layout behind a view that claims this layout:
    append writes nothing; attention writes NaN over its whole output.
Every row not named above must be bit-identical to a call with good
values."""
import math

import pytest
import torch

from _gpu_common import build_decode_case, device, hw, run_decode_step, say
from test_gpu_prefill import PrefillCase

pytestmark = pytest.mark.gpu


def _head_off(lay):
    return [int(x) for x in hw().hwkv_layout_query(lay)[3]]


def _pool_blocks(cache):
    return cache.pool.numel() // cache.layout.desc().block_bytes


def test_decode_block_id_outside_the_pool_gives_nan_for_its_head():
    H = hw()
    dev = device()
    w = [64, 300]
    G = 2
    ctx = [400, 400, 40]
    say("decode: block id outside the pool")
    c = build_decode_case([w], torch.bfloat16, 128, G, ctx, seed=601)
    good = run_decode_step(c)  # appends token ctx - 1, then decodes
    off = _head_off(c.lay)
    nb1 = (w[1] + 15) // 16
    blocks = _pool_blocks(c.cache)
    tbl = c.cache.block_ids
    # seq 0, kv head 1: the block holding position 300 (inside [100, 400))
    tbl[0, off[1] + (300 // 16) % nb1] = blocks + 3
    # seq 1, kv head 0: a negative id on the block of position 380
    tbl[1, off[0] + (380 // 16) % 4] = -1
    # seq 2 (context 40 < both windows), kv head 1: ring block 10 would hold
    # positions 160..175, which do not exist yet: it is never read
    tbl[2, off[1] + 10] = blocks
    torch.cuda.synchronize()
    n_q = 2 * G
    ws = H.make_workspace(c.lay, 0, 1, 3, n_q, device=dev)
    scale = 1.0 / math.sqrt(128)
    for mode in ("attn", "append_attn", "step"):
        say("decode bad id, path", mode)
        out = torch.zeros((1, 3, n_q, 128), dtype=torch.float32, device=dev)
        if mode == "attn":
            H.hwkv_decode_attn(c.cache, 0, 1, torch.tensor(ctx, device=dev), c.q, scale, ws, out)
        else:
            # re-appends token ctx - 1 (same bits) on the way
            pos = torch.tensor([x - 1 for x in ctx], device=dev)
            if mode == "append_attn":
                H.hwkv_decode_append_attn(c.cache, 0, 1, pos, c.k_new, c.v_new, c.q, scale, ws,
                                          out)
            else:
                sws = H.make_step_workspace(c.lay, 0, 1, 3, n_q, device=dev)
                H.hwkv_decode_step(c.cache, 0, 1, pos, c.k_new, c.v_new, c.q, scale, sws, out)
        torch.cuda.synchronize()
        nan = torch.isnan(out[0])
        want = torch.zeros_like(nan)
        want[0, G:2 * G] = True  # seq 0, query heads of kv head 1
        want[1, 0:G] = True      # seq 1, query heads of kv head 0
        assert torch.equal(nan.all(dim=-1), want.any(dim=-1)), mode
        assert torch.equal(nan.any(dim=-1), want.any(dim=-1)), mode
        keep = ~want
        assert torch.equal(out[0][keep], good[0][keep]), mode


def test_append_skips_rows_of_a_block_id_outside_the_pool():
    H = hw()
    dev = device()
    say("append: block id outside the pool")
    lay = H.hwkv_layout_create([[48, 16]], 16, 64, torch.float32)
    cache = H.make_cache(lay, 1, device=dev, fill=0x11)
    off = _head_off(lay)
    cache.block_ids[0, off[0] + 1] = _pool_blocks(cache)  # positions 16..31 of head 0
    before = cache.pool.clone()
    k = torch.randn((1, 1, 48, 2, 64), device=dev)
    v = torch.randn_like(k)
    H.hwkv_append(cache, 0, 1, torch.tensor([0], device=dev), k, v)
    torch.cuda.synchronize()
    pool = cache.pool.view(torch.float32).view(-1, 2, 16, 64)  # [block][K|V][row][d]
    ids = cache.block_ids[0].tolist()
    # head 0: ring blocks 0 and 2 written, block 1 (bad id) skipped
    for j, t0 in ((0, 0), (2, 32)):
        assert torch.equal(pool[ids[off[0] + j], 0], k[0, 0, t0:t0 + 16, 0])
        assert torch.equal(pool[ids[off[0] + j], 1], v[0, 0, t0:t0 + 16, 0])
    # head 1 (one block) keeps the newest 16 tokens
    assert torch.equal(pool[ids[off[1]], 0], k[0, 0, 32:48, 1])
    # nothing else changed: the pool outside those blocks is as before
    written = {ids[off[0]], ids[off[0] + 2], ids[off[1]]}
    bb = lay.desc().block_bytes
    for blk in range(_pool_blocks(cache)):
        if blk not in written:
            assert torch.equal(cache.pool[blk * bb:(blk + 1) * bb], before[blk * bb:(blk + 1) * bb])


def test_prefill_block_id_outside_the_pool_gives_nan_rows_that_reach_it():
    H = hw()
    dev = device()
    say("prefill: block id outside the pool")
    w = [64, 700]
    c = PrefillCase(w, 128, 3, [500, 300, 900], 40, seed=602)
    scale = 1.0 / math.sqrt(128)
    want_good = {"fast": c.run(), "exact": c.run(exact=True)}
    off = _head_off(c.lay)
    nb1 = (w[1] + 15) // 16
    # seq 2 (P = 900), kv head 1 (w = 700): history keys 208..223.  Row r
    # (position 900 + r) reaches back to 201 + r, so rows 0..22 read them.
    c.cache.block_ids[2, off[1] + (208 // 16) % nb1] = _pool_blocks(c.cache) + 7
    # seq 0 (P = 500), kv head 0 (w = 64): keys 448..463; row r reaches back
    # to 437 + r, so rows 0..26 read them
    c.cache.block_ids[0, off[0] + (448 // 16) % 4] = -5
    torch.cuda.synchronize()
    for name in ("fast", "exact"):
        say("prefill bad id, entry", name)
        out = torch.zeros_like(want_good[name])
        c.call(torch.tensor(c.pos0, device=dev), out, scale, exact=name == "exact")
        torch.cuda.synchronize()
        nan = torch.isnan(out)
        want = torch.zeros(nan.shape[:3], dtype=torch.bool, device=dev)
        want[2, :23, 3:6] = True
        want[0, :27, 0:3] = True
        assert torch.equal(nan.all(dim=-1), want), name
        assert torch.equal(nan.any(dim=-1), want), name
        assert torch.equal(out[~want], want_good[name][~want]), name


def _lying_cache(H, cache, other_layout):
    """A view that pairs this cache's pool and table with the meta blob of
    another layout while claiming the cache's own fingerprint, so the host
    check passes and only the kernels' own comparison can catch it."""
    meta_host = H.hwkv_meta_fill(other_layout)
    meta = H._alloc_aligned(meta_host.size, cache.pool.device)
    meta.copy_(torch.from_numpy(meta_host))
    return H.Cache(cache.layout, cache.pool, cache.block_ids, meta, cache.meta_fingerprint)


def test_foreign_meta_blob_decode_and_append():
    H = hw()
    dev = device()
    say("foreign meta blob: decode and append")
    c = build_decode_case([[64, 300]], torch.bfloat16, 128, 3, [400, 120], seed=603)
    other = H.hwkv_layout_create([[64, 301]], 16, 128, torch.bfloat16)  # same geometry
    assert other.desc().meta_bytes == c.lay.desc().meta_bytes
    bad = _lying_cache(H, c.cache, other)
    pos = torch.tensor([399, 119], device=dev)
    before = c.cache.pool.clone()
    H.hwkv_append(bad, 0, 1, pos, c.k_new, c.v_new)
    torch.cuda.synchronize()
    assert torch.equal(c.cache.pool, before)
    ws = H.make_workspace(c.lay, 0, 1, 2, 6, device=dev)
    sws = H.make_step_workspace(c.lay, 0, 1, 2, 6, device=dev)
    scale = 1.0 / math.sqrt(128)
    for mode, out_dtype in (("attn", torch.float32), ("append_attn", torch.bfloat16),
                            ("step", torch.float16)):
        say("foreign meta, path", mode)
        out = torch.zeros((1, 2, 6, 128), dtype=out_dtype, device=dev)
        if mode == "attn":
            H.hwkv_decode_attn(bad, 0, 1, pos + 1, c.q, scale, ws, out)
        elif mode == "append_attn":
            H.hwkv_decode_append_attn(bad, 0, 1, pos, c.k_new, c.v_new, c.q, scale, ws, out)
        else:
            H.hwkv_decode_step(bad, 0, 1, pos, c.k_new, c.v_new, c.q, scale, sws, out)
        torch.cuda.synchronize()
        assert torch.all(torch.isnan(out.float())), mode
        assert torch.equal(c.cache.pool, before), mode  # the appending paths wrote nothing


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_foreign_meta_blob_prefill(out_dtype):
    H = hw()
    dev = device()
    say("foreign meta blob: prefill", out_dtype)
    c = PrefillCase([64, 700], 128, 3, [500, 0], 77, seed=604)
    other = H.hwkv_layout_create([[64, 701]], 16, 128, torch.bfloat16)
    bad = _lying_cache(H, c.cache, other)
    for exact in (False, True):
        out = torch.zeros((2, 77, 6, 128), dtype=out_dtype, device=dev)
        c.call(torch.tensor(c.pos0, device=dev), out, 1.0 / math.sqrt(128), exact=exact, cache=bad)
        torch.cuda.synchronize()
        assert torch.all(torch.isnan(out.float()))


def test_merge_accepts_more_batch_entries_than_table_rows():
    """Several batch entries reading one slot (seq_slots): the split stage
    reads the table through the slots and the merge stage reads only the
    workspace, so a batch larger than the table is valid end to end."""
    H = hw()
    dev = device()
    say("batch larger than the table")
    c = build_decode_case([[64, 300]], torch.bfloat16, 128, 2, [400], seed=605)
    good = run_decode_step(c)
    n = 3
    q = c.q.expand(1, n, 4, 128).contiguous()
    ws = H.make_workspace(c.lay, 0, 1, n, 4, device=dev)
    out = torch.zeros((1, n, 4, 128), dtype=torch.float32, device=dev)
    H.hwkv_decode_attn(c.cache, 0, 1, torch.tensor([400] * n, device=dev), q,
                       1.0 / math.sqrt(128), ws, out,
                       seq_slots=torch.zeros(n, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    for b in range(n):
        assert torch.equal(out[0, b], good[0, 0]), b
