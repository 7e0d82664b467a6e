"""Append parity on the GPU: after scripted sequences of hwkv_append calls the
whole pool must be byte-identical to the oracle's append model applied to the
same initial bytes (bit copies, so the bar is exact equality)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_common import device, hw, say

pytestmark = pytest.mark.gpu


def _run_script(windows, dtype, d, n_seqs, table_rows, script, seed, slots=None, perm=False,
                layer_begin=0, n_layers=None, block_size=16):
    H = hw()
    dev = device()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    windows = np.asarray(windows, np.int32)
    L_all, n_kv = windows.shape
    n_layers = L_all - layer_begin if n_layers is None else n_layers
    lay = H.hwkv_layout_create(windows, block_size, d, dtype)
    bps = lay.desc().blocks_per_seq
    rng = np.random.default_rng(seed)
    ids = (rng.permutation(table_rows * bps) if perm else np.arange(table_rows * bps))
    ids = ids.astype(np.int32).reshape(table_rows, bps)
    cache = H.make_cache(lay, table_rows, device=dev, block_ids=ids)
    init = rng.integers(0, 256, size=cache.pool.numel(), dtype=np.uint8)
    cache.pool.copy_(torch.from_numpy(init))
    ref = init.copy()
    g = synth.gen(seed, dev)
    slot_t = None if slots is None else torch.tensor(slots, dtype=torch.int32, device=dev)
    for step, (pos0, n_new) in enumerate(script):
        say("append", dtype, d, windows.tolist()[:2], "step", step, "pos0", pos0, "n", n_new)
        k = synth.randn((n_layers, n_seqs, n_new, n_kv, d), tdt, g)
        v = synth.randn((n_layers, n_seqs, n_new, n_kv, d), tdt, g)
        p = torch.tensor(pos0, dtype=torch.int64, device=dev)
        H.hwkv_append(cache, layer_begin, n_layers, p, k, v, seq_slots=slot_t)
        oracle.append(ref, ids, windows, block_size, d, layer_begin, pos0, synth.to_raw(k),
                      synth.to_raw(v), seq_slots=slots)
        torch.cuda.synchronize()
        got = cache.pool.cpu().numpy()
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, "step %d: %d bytes differ, first at %d" % (step, bad.size, bad[0])


def test_tiny_config_one_append_then_one_token():
    # 1 layer, w=[32,128], fp32, d=64: 256 tokens in one call (longer than
    # both rings), then the decode step's token 256
    _run_script([[32, 128]], "f32", 64, 1, 1, [([0], 256), ([256], 1)], seed=201)


def test_bf16_ragged_windows_chunks_and_wraparound():
    windows = [[1, 15, 16, 17, 100, 512, 513, 2000], [48, 7, 1024, 33, 64, 65, 1, 300]]
    script = [([0, 5, 1000], 1), ([1, 6, 1001], 15), ([16, 21, 1016], 17),
              ([33, 38, 1033], 700), ([733, 738, 1733], 2500), ([3233, 3238, 4233], 3)]
    _run_script(windows, "bf16", 128, 3, 3, script, seed=202)


def test_permuted_table_seq_slots_and_layer_range():
    windows = [[64, 20], [5, 130], [1000, 16], [17, 1]]
    script = [([0, 100], 50), ([50, 150], 90), ([140, 240], 1), ([141, 241], 333)]
    _run_script(windows, "bf16", 64, 2, 5, script, seed=203, slots=[4, 1], perm=True,
                layer_begin=1, n_layers=2)


def test_rows_wider_than_a_workgroup():
    # 12 KV heads of fp32 d=128: a token row of all heads is 384 16-byte
    # chunks, more than a workgroup's threads, so each thread walks several
    # chunks of one token; chunks longer than some rings, wraparound
    windows = [[16, 31, 129, 1, 64, 200, 17, 33, 1000, 2, 48, 65],
               [7, 300, 16, 90, 1, 513, 40, 8, 65, 129, 1000, 3]]
    script = [([0, 3], 1), ([1, 4], 70), ([71, 74], 300), ([371, 374], 1100), ([1471, 1474], 5)]
    _run_script(windows, "f32", 128, 2, 2, script, seed=205)


def test_f32_d128_many_sequences():
    windows = [[16, 31, 129]]
    script = [([int(x) for x in np.arange(9) * 7], 40), ([int(x) for x in np.arange(9) * 7 + 40], 1)]
    _run_script(windows, "f32", 128, 9, 9, script, seed=204, perm=True)


@pytest.mark.parametrize("block_size", [32, 64, 48, 1])
def test_other_block_sizes(block_size):
    """The append is a bit copy for any block size: ring block (t / bs) % nb,
    row t % bs."""
    windows = [[1, 15, 64, 65, 100, 512], [33, 7, 1024, 200, 64, 2]]
    script = [([0, 5], 1), ([1, 6], 40), ([41, 46], 129), ([170, 175], 1100), ([1270, 1275], 3)]
    _run_script(windows, "bf16", 64, 2, 3, script, seed=206 + block_size, perm=True,
                block_size=block_size)


def test_invalid_device_values_are_skipped_not_faulted():
    """A slot outside the table and a negative position skip their rows; a
    block id outside the pool is skipped too.  Everything else is written."""
    H = hw()
    dev = device()
    windows = np.array([[32, 48]], np.int32)
    lay = H.hwkv_layout_create(windows, 16, 64, "bf16")
    bps = lay.desc().blocks_per_seq
    ids = np.arange(2 * bps, dtype=np.int32).reshape(2, bps)
    bad_ids = ids.copy()
    bad_ids[1, 0] = 1 << 30  # outside the pool
    cache = H.make_cache(lay, 2, device=dev, block_ids=bad_ids)
    init = np.random.default_rng(9).integers(0, 256, cache.pool.numel(), dtype=np.uint8)
    cache.pool.copy_(torch.from_numpy(init))
    g = synth.gen(205, dev)
    k = synth.randn((1, 4, 40, 2, 64), torch.bfloat16, g)
    v = synth.randn((1, 4, 40, 2, 64), torch.bfloat16, g)
    # batch entries: 0 -> slot 0 ok; 1 -> slot 7 (outside); 2 -> pos0 < 0; 3 -> slot 1
    slots = torch.tensor([0, 7, 0, 1], dtype=torch.int32, device=dev)
    pos = torch.tensor([3, 3, -5, 10], dtype=torch.int64, device=dev)
    say("append invalid device values")
    H.hwkv_append(cache, 0, 1, pos, k, v, seq_slots=slots)
    torch.cuda.synchronize()
    got = cache.pool.cpu().numpy()
    # expected: entries 0 and 3 only; entry 3's writes that would land in the
    # out-of-pool block (ring block 0 of head 0 of row 1) are dropped
    ref = init.copy()
    kr, vr = synth.to_raw(k), synth.to_raw(v)
    oracle.append(ref, ids, windows, 16, 64, 0, [3], kr[:, 0:1], vr[:, 0:1], seq_slots=[0])
    ref2 = ref.copy()
    oracle.append(ref2, ids, windows, 16, 64, 0, [10], kr[:, 3:4], vr[:, 3:4], seq_slots=[1])
    blk = int(ids[1, 0])
    bb = lay.desc().block_bytes
    ref2[blk * bb:(blk + 1) * bb] = ref[blk * bb:(blk + 1) * bb]
    assert np.array_equal(got, ref2)
