"""Host half of the C ABI, on the CPU: the library loads, exports every symbol
its header declares, and its layout arithmetic is bit-exact against the
oracle.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

hw = pytest.importorskip("head_windowed_kv_amd", reason="libhwkv.so not built")

CONFIG_WINDOWS = {
    "tiny": np.array([[32, 128]], np.int32),
    "single_layer": np.array([synth.YAML_LAYER0], np.int32),
    "stack48": synth.stack_windows(48, 8, 0),
    "yaml_two_layers": np.array([synth.YAML_LAYER0, synth.YAML_LAYER1], np.int32),
}


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "hwkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hwkv_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hw.LIB_PATH)
    declared = _declared_symbols()
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(hw.EXPORTED) == declared


def test_abi_version():
    # 2: hwkv_cache carries the fingerprint of its meta blob
    assert hw.hwkv_abi_version() == hw.ABI_VERSION == 3
    text = open(os.path.join(ROOT, "include", "hwkv.h")).read()
    assert re.search(r"#define HWKV_ABI_VERSION %du\b" % hw.ABI_VERSION, text)


@pytest.mark.parametrize("name", sorted(CONFIG_WINDOWS))
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_layout_and_estimate_bit_exact_vs_oracle(name, dtype, d):
    w = CONFIG_WINDOWS[name]
    lay = hw.hwkv_layout_create(w, 16, d, dtype)
    desc, w_out, nb, off = hw.hwkv_layout_query(lay)
    onb, ooff, obps = oracle.layout(w, 16)
    assert np.array_equal(w_out, w)
    assert np.array_equal(nb.reshape(-1), onb)
    assert np.array_equal(off, ooff)
    assert desc.blocks_per_seq == obps
    eb = 2 if dtype == "bf16" else 4
    assert desc.block_bytes == 2 * 16 * d * eb
    for n in (1, 3, 32):
        assert hw.hwkv_mem_estimate(lay, n) == oracle.mem_estimate(w, 16, d, eb, n)
    assert np.array_equal(hw.hwkv_table_fill(lay, 3), oracle.default_table(3, obps))


def test_stack48_seed0_numbers():
    """The 48-layer synthetic stack: level counts and exact pool bytes."""
    w = synth.stack_windows(48, 8, 0)
    counts = {lv: int((w == lv).sum()) for lv in synth.WINDOW_LEVELS}
    assert counts == {1024: 79, 4096: 98, 16384: 114, 65536: 93}
    assert int(w.sum()) == 8444928
    lay = hw.hwkv_layout_create(w, 16, 128, "bf16")
    assert hw.hwkv_mem_estimate(lay, 1) == 4323803136
    assert hw.hwkv_mem_estimate(lay, 32) == 138361700352


def test_random_windows_bit_exact():
    rng = np.random.default_rng(5)
    for _ in range(20):
        nl, nh = rng.integers(1, 6), rng.integers(1, 9)
        w = rng.integers(1, 70000, size=(nl, nh)).astype(np.int32)
        w[rng.random(w.shape) < 0.2] = 1
        lay = hw.hwkv_layout_create(w, 16, 128, "bf16", split_tokens=int(rng.choice([16, 256, 512])))
        desc, _, nb, off = hw.hwkv_layout_query(lay)
        onb, ooff, obps = oracle.layout(w, 16)
        assert np.array_equal(nb.reshape(-1), onb) and np.array_equal(off, ooff)
        assert hw.hwkv_mem_estimate(lay, 7) == oracle.mem_estimate(w, 16, 128, 2, 7)
        splits = -(-w.astype(np.int64) // desc.split_tokens)
        assert desc.n_work == int(splits.sum())
        assert desc.max_window == int(w.max())


def test_workspace_bytes():
    w = np.array([[1024, 4096], [100, 1]], np.int32)
    lay = hw.hwkv_layout_create(w, 16, 128, "bf16", split_tokens=512)
    # splits: 2 + 8 + 1 + 1 = 12 items; record = 3*(128+2) = 390 -> 392 floats
    assert hw.hwkv_workspace_bytes(lay, 0, 2, 5, 6) == 12 * 392 * 4 * 5
    assert hw.hwkv_workspace_bytes(lay, 1, 1, 1, 6) == 2 * 392 * 4
    assert hw.hwkv_workspace_bytes(lay, 0, 1, 1, 2) == 10 * 132 * 4


def test_prefill_workspace_bytes():
    """bf16 caches: one fp16 V row of head_dim values per key of
    [P - w + 1, P + n_chunk), per (sequence, kv head); other dtypes: none."""
    w = np.array([[64, 700], [1, 4096]], np.int32)
    lay = hw.hwkv_layout_create(w, 16, 128, "bf16")
    assert hw.hwkv_prefill_workspace_bytes(lay, 0, 3, 40) == 3 * ((63 + 40) + (699 + 40)) * 256
    assert hw.hwkv_prefill_workspace_bytes(lay, 1, 1, 1) == (1 + 4096) * 256
    for dt in ("f16", "f32"):
        lay16 = hw.hwkv_layout_create(w, 16, 64, dt)
        assert hw.hwkv_prefill_workspace_bytes(lay16, 1, 8, 2048) == 0
    for args in ((2, 1, 1), (-1, 1, 1), (0, 0, 1), (0, 1, 0)):
        with pytest.raises(hw.HwkvError) as e:
            hw.hwkv_prefill_workspace_bytes(lay, *args)
        assert e.value.status_name == "HWKV_ERR_INVALID_ARG", args
    # one head's rows reach 2^31 bytes (d = 128: 2^23 rows of 256 bytes)
    big = hw.hwkv_layout_create([[(1 << 23) - 100, 16]], 16, 128, "bf16")
    assert hw.hwkv_prefill_workspace_bytes(big, 0, 1, 100) == ((1 << 23) - 1 + 15 + 100) * 256
    with pytest.raises(hw.HwkvError) as e:
        hw.hwkv_prefill_workspace_bytes(big, 0, 1, 101)
    assert e.value.status_name == "HWKV_ERR_UNSUPPORTED"
    assert "hwkv_prefill_attn_exact" in str(e.value)


def test_prefill_workspace_errors_before_launch():
    """A missing, misaligned or short prefill workspace is refused on the
    host; the exact entry takes none."""
    lay = hw.hwkv_layout_create([[64, 700]], 16, 128, "bf16")
    cv = _fake_cache(lay, hw.hwkv_mem_estimate(lay, 2), 2)
    P = lambda mib: ctypes.c_void_p(mib << 20)  # noqa: E731
    need = hw.hwkv_prefill_workspace_bytes(lay, 0, 2, 40)

    def call(ws, nbytes):
        return hw.STATUS_NAMES[hw._lib.hwkv_prefill_attn(
            lay.handle, ctypes.byref(cv), 0, 2, None, P(10), 40, 6, P(9), P(5), P(6), ws, nbytes,
            P(11), 0, 0.1, None)]

    assert call(None, need) == "HWKV_ERR_INVALID_ARG"
    assert call(ctypes.c_void_p((8 << 20) + 16), need) == "HWKV_ERR_MISALIGNED"
    assert call(P(8), need - 1) == "HWKV_ERR_CAPACITY"
    assert "need %d" % need in hw.hwkv_last_error()
    big = hw.hwkv_layout_create([[(1 << 23) - 100, 16]], 16, 128, "bf16")
    cvb = _fake_cache(big, hw.hwkv_mem_estimate(big, 1), 1)
    st = hw._lib.hwkv_prefill_attn(big.handle, ctypes.byref(cvb), 0, 1, None, P(10), 101, 2,
                                   P(9), P(5), P(6), P(8), 1 << 40, P(11), 0, 0.1, None)
    assert hw.STATUS_NAMES[st] == "HWKV_ERR_UNSUPPORTED"


def test_meta_blob_header():
    lay = hw.hwkv_layout_create(CONFIG_WINDOWS["tiny"], 16, 64, "f32")
    meta = hw.hwkv_meta_fill(lay)
    desc = lay.desc()
    assert meta.size == desc.meta_bytes and meta.size % 256 == 0
    assert int(meta[:4].view(np.uint32)[0]) == 0x564B5748
    assert int(meta[4:8].view(np.uint32)[0]) == hw.ABI_VERSION == hw.hwkv_abi_version()
    assert int(meta[8:16].view(np.uint64)[0]) == desc.fingerprint
    assert hw.hwkv_meta_fingerprint(meta) == desc.fingerprint


def test_meta_fingerprint_rejects_other_blobs():
    lay = hw.hwkv_layout_create(CONFIG_WINDOWS["tiny"], 16, 64, "f32")
    meta = hw.hwkv_meta_fill(lay)
    with pytest.raises(hw.HwkvError) as e:
        hw.hwkv_meta_fingerprint(meta[:32])
    assert e.value.status_name == "HWKV_ERR_INVALID_ARG"
    junk = meta.copy()
    junk[:4] = 0
    with pytest.raises(hw.HwkvError) as e:
        hw.hwkv_meta_fingerprint(junk)
    assert e.value.status_name == "HWKV_ERR_ABI_MISMATCH"
    old = meta.copy()
    old[4:8] = np.array([hw.ABI_VERSION - 1], np.uint32).view(np.uint8)
    with pytest.raises(hw.HwkvError) as e:
        hw.hwkv_meta_fingerprint(old)
    assert e.value.status_name == "HWKV_ERR_ABI_MISMATCH"
    assert "ABI version %d" % (hw.ABI_VERSION - 1) in str(e.value)


def test_fingerprint_tracks_every_parameter():
    base = hw.hwkv_layout_create([[32, 128]], 16, 64, "f32").desc().fingerprint
    others = [hw.hwkv_layout_create([[32, 129]], 16, 64, "f32"),
              hw.hwkv_layout_create([[32, 128]], 16, 128, "f32"),
              hw.hwkv_layout_create([[32, 128]], 16, 64, "bf16"),
              hw.hwkv_layout_create([[32, 128]], 16, 64, "f32", split_tokens=32),
              hw.hwkv_layout_create([[32], [128]], 16, 64, "f32")]
    fps = {o.desc().fingerprint for o in others}
    assert base not in fps and len(fps) == len(others)


@pytest.mark.parametrize("args,status", [
    (([[0, 4]], 16, 128, "bf16"), "HWKV_ERR_INVALID_ARG"),
    (([[-5]], 16, 128, "bf16"), "HWKV_ERR_INVALID_ARG"),
    (([[16]], 0, 128, "bf16"), "HWKV_ERR_INVALID_ARG"),
    (([[16]], 2048, 128, "bf16"), "HWKV_ERR_INVALID_ARG"),
    (([[16]], 16, 0, "bf16"), "HWKV_ERR_INVALID_ARG"),
    (([[16]], 16, 1025, "bf16"), "HWKV_ERR_INVALID_ARG"),
    (([[16]], 16, 128, "bf16", 24), "HWKV_ERR_INVALID_ARG"),
    (([[16]], 32, 128, "bf16", 48), "HWKV_ERR_INVALID_ARG"),
    (([[16]], 16, 128, "bf16", 4096), "HWKV_ERR_INVALID_ARG"),
])
def test_layout_create_errors(args, status):
    with pytest.raises(hw.HwkvError) as e:
        hw.hwkv_layout_create(*args)
    assert e.value.status_name == status


@pytest.mark.parametrize("bs,d,dt", [(32, 128, "bf16"), (64, 256, "f16"), (48, 96, "f32"),
                                     (1, 8, "bf16"), (1024, 1024, "f32")])
def test_any_block_size_head_dim_and_dtype_can_be_described(bs, d, dt):
    """A layout is a host description: sizes without a kernel still get exact
    block counts and estimates (equal to the oracle's)."""
    w = np.array([[1, 47, 1000], [4096, 65, 3]], np.int32)
    lay = hw.hwkv_layout_create(w, bs, d, dt)
    desc, _, nb, off = hw.hwkv_layout_query(lay)
    ref_nb, ref_off, ref_bps = oracle.layout(w, bs)
    assert np.array_equal(nb.reshape(-1), ref_nb) and np.array_equal(off, ref_off)
    eb = {"bf16": 2, "f16": 2, "f32": 4}[dt]
    for n in (0, 1, 7):
        assert hw.hwkv_mem_estimate(lay, n) == oracle.mem_estimate(w, bs, d, eb, n)
    # default decode split: the largest multiple of the block size <= 1024
    assert desc.split_tokens == max(1, 1024 // bs) * bs


def _unsupported_calls(lay, group):
    """Status of append / decode / prefill on a fake cache view.  Each call
    also carries one invalid argument that is checked after the kernel check
    (n_new = 0, scale = inf, n_chunk = 0), so every call fails validation and
    nothing is ever launched: UNSUPPORTED if no kernel exists, else
    INVALID_ARG."""
    cv = _fake_cache(lay, hw.hwkv_mem_estimate(lay, 1), 1)
    p = [ctypes.c_void_p(x << 20) for x in range(4, 13)]
    n_q = lay.desc().n_kv_heads * group
    ws_bytes = 1 << 30
    st_app = hw._lib.hwkv_append(lay.handle, ctypes.byref(cv), 0, 1, 1, None, p[0], 0, p[1], p[2],
                                 None)
    st_dec = hw._lib.hwkv_decode_attn(lay.handle, ctypes.byref(cv), 0, 1, 1, None, p[0], n_q,
                                      p[3], float("inf"), ctypes.c_void_p(256 << 20), ws_bytes,
                                      p[4], 0, None)
    st_pf = hw._lib.hwkv_prefill_attn(lay.handle, ctypes.byref(cv), 0, 1, None, p[0], 0, n_q,
                                      p[3], p[1], p[2], ctypes.c_void_p(256 << 20), ws_bytes,
                                      p[4], 0, 0.1, None)
    st_pfx = hw._lib.hwkv_prefill_attn_exact(lay.handle, ctypes.byref(cv), 0, 1, None, p[0], 0,
                                             n_q, p[3], p[1], p[2], p[4], 0, 0.1, None)
    assert st_pfx == st_pf  # the exact variant validates the same way
    return [hw.STATUS_NAMES[x] for x in (st_app, st_dec, st_pf)]


@pytest.mark.parametrize("bs,d,dt,want", [
    (32, 128, "bf16", ["ok", "ok", "ok"]),
    (16, 128, "f16", ["ok", "ok", "ok"]),
    (16, 128, "f32", ["ok", "ok", "HWKV_ERR_UNSUPPORTED"]),
    (48, 128, "bf16", ["ok", "HWKV_ERR_UNSUPPORTED", "HWKV_ERR_UNSUPPORTED"]),
    (512, 64, "bf16", ["ok", "HWKV_ERR_UNSUPPORTED", "HWKV_ERR_UNSUPPORTED"]),
    (16, 96, "bf16", ["ok", "HWKV_ERR_UNSUPPORTED", "HWKV_ERR_UNSUPPORTED"]),
    (16, 256, "bf16", ["ok", "ok", "ok"]),
    (64, 256, "f16", ["ok", "ok", "ok"]),
    (16, 256, "f32", ["ok", "HWKV_ERR_UNSUPPORTED", "HWKV_ERR_UNSUPPORTED"]),
    (16, 4, "bf16", ["HWKV_ERR_UNSUPPORTED", "HWKV_ERR_UNSUPPORTED", "HWKV_ERR_UNSUPPORTED"]),
])
def test_device_calls_without_a_kernel_are_rejected_before_launch(bs, d, dt, want):
    lay = hw.hwkv_layout_create([[64, 16]], bs, d, dt)
    got = _unsupported_calls(lay, 3)
    for g, w in zip(got, want):
        assert g == ("HWKV_ERR_INVALID_ARG" if w == "ok" else w)


@pytest.mark.parametrize("d,group,want", [
    (256, 4, ["ok", "ok", "ok"]),
    (256, 6, ["ok", "ok", "ok"]),
    (256, 5, ["ok", "HWKV_ERR_UNSUPPORTED", "HWKV_ERR_UNSUPPORTED"]),
    (128, 8, ["ok", "ok", "ok"]),
    (128, 5, ["ok", "HWKV_ERR_UNSUPPORTED", "HWKV_ERR_UNSUPPORTED"]),
])
def test_group_sizes_without_a_kernel_are_rejected_before_launch(d, group, want):
    lay = hw.hwkv_layout_create([[64, 16]], 16, d, "bf16")
    got = _unsupported_calls(lay, group)
    for g, w in zip(got, want):
        assert g == ("HWKV_ERR_INVALID_ARG" if w == "ok" else w)


def test_capacity_check_matches_a_walk_over_rows_and_heads():
    """The first head whose blocks do not fit, found by walking sequence rows
    and heads in allocation order (brute force over the oracle's layout)."""
    w = np.array([synth.YAML_LAYER0, synth.YAML_LAYER1, [16, 1, 33, 5000, 7, 64, 1024, 3]],
                 np.int32)
    lay = hw.hwkv_layout_create(w, 16, 128, "bf16")
    bb = lay.desc().block_bytes
    nb, off, bps = oracle.layout(w, 16)
    rng = np.random.default_rng(5)
    n_seqs = 3
    for avail in list(rng.integers(0, n_seqs * bps, 40)) + [0, bps - 1, bps, n_seqs * bps - 1]:
        pool = int(avail) * bb + int(rng.integers(0, bb))
        got = hw.hwkv_capacity_check(lay, n_seqs, pool)
        # brute force: blocks end at row*bps + off[i] + nb[i]
        want = None
        for row in range(n_seqs):
            for i in range(len(nb)):
                if row * bps + off[i] + nb[i] > avail:
                    want = (row, i // 8, i % 8)
                    break
            if want:
                break
        assert (got[:3] if got else None) == want, avail
        if got:
            assert got[3].startswith("KV cache block allocation failed at layer %d, head %d"
                                     % (want[1], want[2]))
    assert hw.hwkv_capacity_check(lay, n_seqs, n_seqs * bps * bb) is None


def test_table_fill_overflow_is_reported():
    lay = hw.hwkv_layout_create([[65536] * 8], 16, 128, "bf16")
    with pytest.raises(hw.HwkvError) as e:
        hw.hwkv_table_fill(lay, 100000)
    assert e.value.status_name == "HWKV_ERR_OVERFLOW"


def _fake_cache(lay, pool_bytes, rows, pool_ptr=1 << 20, fingerprint=None):
    # device pointers are never dereferenced: validation fails first
    fp = lay.desc().fingerprint if fingerprint is None else fingerprint
    return hw.hwkv_cache(pool_ptr, pool_bytes, 2 << 20, rows, 3 << 20, fp)


def _every_device_call(lay, cv, scale=0.1, n_q=4, with_scale_only=False):
    """Status of every device entry point on cache view cv with fake device
    pointers, in the order of the header.  Callers make sure that every call
    fails validation: a call that passed would launch a kernel on them.
    with_scale_only: only the attention calls (which take a scale)."""
    P = lambda mib: ctypes.c_void_p(mib << 20)  # noqa: E731
    L = hw._lib
    h = lay.handle
    c = ctypes.byref(cv)
    big = 1 << 40
    head = [] if with_scale_only else [
        L.hwkv_append(h, c, 0, 1, 1, None, P(4), 1, P(5), P(6), None)]
    mid = [] if with_scale_only else [
        L.hwkv_decode_merge(h, c, 0, 1, 1, P(10), n_q, P(8), big, P(11), 0, None)]
    return head + [
        L.hwkv_decode_split(h, c, 0, 1, 1, None, P(10), n_q, P(9), scale, P(8), big, None),
    ] + mid + [
        L.hwkv_decode_attn(h, c, 0, 1, 1, None, P(10), n_q, P(9), scale, P(8), big, P(11), 0,
                           None),
        L.hwkv_decode_split_append(h, c, 0, 1, 1, None, P(10), P(5), P(6), n_q, P(9), scale, P(8),
                                   big, None),
        L.hwkv_decode_append_attn(h, c, 0, 1, 1, None, P(10), P(5), P(6), n_q, P(9), scale, P(8),
                                  big, P(11), 0, None),
        L.hwkv_decode_step(h, c, 0, 1, 1, None, P(10), P(5), P(6), n_q, P(9), scale, P(8), big,
                           P(11), 0, None),
        L.hwkv_prefill_attn(h, c, 0, 1, None, P(10), 7, n_q, P(9), P(5), P(6), P(8), big, P(11),
                            0, scale, None),
        L.hwkv_prefill_attn_exact(h, c, 0, 1, None, P(10), 7, n_q, P(9), P(5), P(6), P(11), 0,
                                  scale, None),
    ]


def test_cache_of_another_layout_is_rejected_before_launch():
    """Kernel-ABI check (page "KV Cache Management in Hybrid Attention LLMs",
    4.2): a cache view whose blob was written for another layout (here one
    window differs by one token) is refused by every device call, on the host,
    before anything is enqueued."""
    a = hw.hwkv_layout_create([[32, 128]], 16, 64, "bf16")
    b = hw.hwkv_layout_create([[32, 129]], 16, 64, "bf16")
    fa, fb = a.desc().fingerprint, b.desc().fingerprint
    assert fa != fb
    cv = _fake_cache(b, hw.hwkv_mem_estimate(b, 1), 1, fingerprint=fa)
    got = _every_device_call(b, cv)
    assert [hw.STATUS_NAMES[s] for s in got] == ["HWKV_ERR_ABI_MISMATCH"] * len(got)
    msg = hw.hwkv_last_error()
    assert "%016x" % fa in msg and "%016x" % fb in msg
    # the blob's own fingerprint, read back from a host copy, is what a
    # caller puts in the view; the same calls then get past this check and
    # stop at the next one (a pool one byte short of the estimate)
    cv_ok = _fake_cache(b, hw.hwkv_mem_estimate(b, 1) - 1, 1,
                        fingerprint=hw.hwkv_meta_fingerprint(hw.hwkv_meta_fill(b)))
    got = _every_device_call(b, cv_ok)
    assert [hw.STATUS_NAMES[s] for s in got] == ["HWKV_ERR_CAPACITY"] * len(got)


@pytest.mark.parametrize("scale", [0.0, -0.0, -0.125, float("nan"), float("inf"),
                                   float("-inf")])
def test_non_positive_or_non_finite_scale_is_rejected(scale):
    lay = hw.hwkv_layout_create([[32, 128]], 16, 64, "bf16")
    cv = _fake_cache(lay, hw.hwkv_mem_estimate(lay, 1), 1)
    got = _every_device_call(lay, cv, scale=scale, with_scale_only=True)
    assert [hw.STATUS_NAMES[s] for s in got] == ["HWKV_ERR_INVALID_ARG"] * 7
    assert "scale must be finite and > 0" in hw.hwkv_last_error()


def test_capacity_error_names_layer_and_head():
    w = np.array([synth.YAML_LAYER0, synth.YAML_LAYER1], np.int32)
    lay = hw.hwkv_layout_create(w, 16, 128, "bf16")
    need = hw.hwkv_mem_estimate(lay, 2)
    bb = lay.desc().block_bytes
    # room for row 0 and the first 18944 + 100 blocks of row 1: row 1 stops in
    # layer 1, head 0 (offset 18944, 64 blocks) -> head 1 (offset 19008) fails
    avail_blocks = lay.desc().blocks_per_seq + 18944 + 100
    cv = _fake_cache(lay, avail_blocks * bb, 2)
    pos = ctypes.c_void_p(4 << 20)
    st = hw._lib.hwkv_append(lay.handle, ctypes.byref(cv), 0, 1, 1, None, pos, 1,
                             ctypes.c_void_p(5 << 20), ctypes.c_void_p(6 << 20), None)
    assert hw.STATUS_NAMES[st] == "HWKV_ERR_CAPACITY"
    msg = hw.hwkv_last_error()
    assert "KV cache block allocation failed at layer 1, head 1" in msg
    assert str(need) in msg


def test_misaligned_pool_is_rejected_before_launch():
    lay = hw.hwkv_layout_create([[32, 128]], 16, 64, "f32")
    cv = _fake_cache(lay, hw.hwkv_mem_estimate(lay, 1), 1, pool_ptr=(1 << 20) + 64)
    st = hw._lib.hwkv_append(lay.handle, ctypes.byref(cv), 0, 1, 1, None, ctypes.c_void_p(4 << 20),
                             1, ctypes.c_void_p(5 << 20), ctypes.c_void_p(6 << 20), None)
    assert hw.STATUS_NAMES[st] == "HWKV_ERR_MISALIGNED"


def test_decode_argument_errors_before_launch():
    lay = hw.hwkv_layout_create([[32, 128]], 16, 64, "f32")
    cv = _fake_cache(lay, hw.hwkv_mem_estimate(lay, 1), 1)
    ws = ctypes.c_void_p(8 << 20)
    q = ctypes.c_void_p(9 << 20)
    ctx = ctypes.c_void_p(10 << 20)
    out = ctypes.c_void_p(11 << 20)
    need = hw.hwkv_workspace_bytes(lay, 0, 1, 1, 4)
    f = hw._lib.hwkv_decode_attn
    # n_q_heads not a multiple of n_kv_heads
    assert f(lay.handle, ctypes.byref(cv), 0, 1, 1, None, ctx, 3, q, 0.1, ws, need, out, 0,
             None) == 1
    # workspace too small
    assert f(lay.handle, ctypes.byref(cv), 0, 1, 1, None, ctx, 4, q, 0.1, ws, need - 4, out, 0,
             None) == 4
    # layer range outside the layout
    assert f(lay.handle, ctypes.byref(cv), 0, 2, 1, None, ctx, 4, q, 0.1, ws, need, out, 0,
             None) == 1
    # more sequences than table rows without seq_slots
    assert f(lay.handle, ctypes.byref(cv), 0, 1, 2, None, ctx, 4, q, 0.1, ws, need, out, 0,
             None) == 1
    # unsupported GQA group (5)
    lay5 = hw.hwkv_layout_create([[32]], 16, 64, "f32")
    cv5 = _fake_cache(lay5, hw.hwkv_mem_estimate(lay5, 1), 1)
    assert f(lay5.handle, ctypes.byref(cv5), 0, 1, 1, None, ctx, 5, q, 0.1, ws, 1 << 20, out, 0,
             None) == 2
    # non-finite scale
    assert f(lay.handle, ctypes.byref(cv), 0, 1, 1, None, ctx, 4, q, float("inf"), ws, need, out,
             0, None) == 1
    # batch sizes outside [1, 65535] (the sequences are a grid dimension)
    slots = ctypes.c_void_p(12 << 20)
    for n_seqs in (0, -1, 65536):
        assert f(lay.handle, ctypes.byref(cv), 0, 1, n_seqs, slots, ctx, 4, q, 0.1, ws, 1 << 40,
                 out, 0, None) == 1, n_seqs
        assert "n_seqs" in hw.hwkv_last_error()
    lay_p = hw.hwkv_layout_create([[32, 128]], 16, 128, "bf16")
    cvp = _fake_cache(lay_p, hw.hwkv_mem_estimate(lay_p, 1), 1)
    for n_seqs in (0, 65536):
        assert hw._lib.hwkv_prefill_attn(lay_p.handle, ctypes.byref(cvp), 0, n_seqs, slots, ctx,
                                         7, 4, q, ctypes.c_void_p(5 << 20),
                                         ctypes.c_void_p(6 << 20), ws, 1 << 40, out, 0, 0.1,
                                         None) == 1, n_seqs


def test_static_scratch_entry_refuses_calls_beyond_its_array():
    """hwkv_decode_append_attn_static (callers that cannot allocate) keeps its
    split records in a static array of HWKV_STATIC_SCRATCH_BYTES: the 48-layer
    112K stack fits 5 sequences per call; 6 are refused on the host, before
    any device is touched."""
    text = open(os.path.join(ROOT, "include", "hwkv.h")).read()
    m = re.search(r"#define HWKV_STATIC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == hw.STATIC_SCRATCH_BYTES
    lay = hw.hwkv_layout_create(CONFIG_WINDOWS["stack48"], 16, 128, "bf16")
    assert hw.hwkv_workspace_bytes(lay, 0, 48, 5, 24) <= hw.STATIC_SCRATCH_BYTES
    assert hw.hwkv_workspace_bytes(lay, 0, 48, 6, 24) > hw.STATIC_SCRATCH_BYTES
    cv = _fake_cache(lay, hw.hwkv_mem_estimate(lay, 6), 6)
    P = lambda mib: ctypes.c_void_p(mib << 20)  # noqa: E731
    st = hw._lib.hwkv_decode_append_attn_static(lay.handle, ctypes.byref(cv), 0, 48, 6, None,
                                                P(10), P(5), P(6), 24, P(9), 0.1, P(11), 0, None)
    assert hw.STATUS_NAMES[st] == "HWKV_ERR_CAPACITY"
    assert "static scratch holds %d" % hw.STATIC_SCRATCH_BYTES in hw.hwkv_last_error()
