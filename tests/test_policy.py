"""Policy documents and the mem-estimate command (host only).

Pins: the two window vectors printed in the write-up's policy example with
their hand-worked block counts and bytes (tests/golden/); the oracle's exact
estimate for the 48-layer stack; a brute-force walk for the first head that
does not fit a budget; schema errors named by layer."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synth

hw = pytest.importorskip("head_windowed_kv_amd", reason="libhwkv.so not built")
from head_windowed_kv_amd import policy as P  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIXTURE = os.path.join(ROOT, "tests", "golden", "headwise-kv-config.yaml")


def _golden():
    with open(os.path.join(ROOT, "tests", "golden", "policy_yaml_layers.json")) as f:
        return json.load(f)


def test_printed_policy_loads_with_its_windows_and_budget():
    pol = P.load_policy(FIXTURE)
    g = _golden()
    assert pol.model_name == "Qwen3.6-27B" and pol.budget_gb == 48.0
    assert pol.windows.shape == (2, 8)
    for l, layer in enumerate(g["layers"]):
        assert pol.windows[l].tolist() == layer["kv_head_windows"]


def test_printed_policy_estimate_matches_hand_worked_values():
    g = _golden()
    pol = P.load_policy(FIXTURE)
    est = P.estimate(pol, n_seqs=1, block_size=g["block_size"], head_dim=g["head_dim"],
                     dtype="bf16")
    assert est.head_blocks.tolist() == [x["blocks_per_head"] for x in g["layers"]]
    assert est.blocks_per_seq == g["two_layer_blocks_per_seq"]
    assert est.layer_bytes_per_seq.tolist() == [x["bytes_per_seq"] for x in g["layers"]]
    assert est.total_bytes == sum(x["bytes_per_seq"] for x in g["layers"])
    assert est.fits  # 277 MB against 48 GB
    one = P.estimate(P.Policy(pol.windows[:1]), n_seqs=8)
    assert one.total_bytes == g["layer0_eight_seqs_bytes"]


def test_stack48_policy_round_trip_and_estimate():
    w = synth.stack_windows(48, 8, 0)
    pol = P.Policy(w, "stack48", 48.0)
    back = P.parse_policy(P.policy_to_yaml(pol))
    assert np.array_equal(back.windows, w) and back.model_name == "stack48"
    assert back.budget_gb == 48.0
    for n in (1, 32):
        est = P.estimate(back, n_seqs=n)
        assert est.total_bytes == oracle.mem_estimate(w, 16, 128, 2, n)
    assert P.estimate(back, 1).total_bytes == 4323803136


@pytest.mark.parametrize("n_seqs", [1, 11, 12, 40])
def test_budget_names_the_first_head_that_does_not_fit(n_seqs):
    w = synth.stack_windows(48, 8, 0)
    pol = P.Policy(w, None, 48.0)
    est = P.estimate(pol, n_seqs=n_seqs)
    budget = 48 * 10 ** 9
    nb, off, bps = oracle.layout(w, 16)
    bb = 16 * 128 * 2 * 2
    avail = budget // bb
    want = None
    for row in range(n_seqs):
        for i in range(len(nb)):
            if row * bps + off[i] + nb[i] > avail:
                want = (row, i // 8, i % 8)
                break
        if want:
            break
    assert (est.first_unfit[:3] if est.first_unfit else None) == want
    assert est.fits == (oracle.mem_estimate(w, 16, 128, 2, n_seqs) <= budget)


@pytest.mark.parametrize("doc,msg", [
    ("per_layer_policies: []", "non-empty"),
    ("per_layer_policies:\n- layer_id: 1\n  kv_head_windows: [16]", "missing [0]"),
    ("per_layer_policies:\n- layer_id: 0\n  kv_head_windows: [16]\n"
     "- layer_id: 0\n  kv_head_windows: [16]", "twice"),
    ("per_layer_policies:\n- layer_id: 0\n  kv_head_windows: [16, 32]\n"
     "- layer_id: 1\n  kv_head_windows: [16]", "layer 1 has 1 kv heads"),
    ("per_layer_policies:\n- layer_id: 0\n  kv_head_windows: [16, 0]", "layer 0, head 1"),
    ("per_layer_policies:\n- layer_id: 0\n  kv_head_windows: [16, 4.5]", "not an integer"),
    ("per_layer_policies:\n- layer_id: 0\n  kv_head_windows: [16]\nbudget_gb: -1", "budget_gb"),
    ("[1, 2]", "mapping"),
    ("per_layer_policies: [: bad", "not valid YAML"),
])
def test_schema_errors(doc, msg):
    with pytest.raises(P.PolicyError) as e:
        P.parse_policy(doc)
    assert msg in str(e.value)


def test_layer_order_in_the_file_does_not_matter():
    a = P.parse_policy("per_layer_policies:\n- layer_id: 1\n  kv_head_windows: [7, 9]\n"
                       "- layer_id: 0\n  kv_head_windows: [1, 3]")
    assert a.windows.tolist() == [[1, 3], [7, 9]]


def test_sizes():
    assert P.parse_size("48g") == 48 * 10 ** 9
    assert P.parse_size("48GiB") == 48 << 30
    assert P.parse_size("1.5t") == 1_500_000_000_000
    assert P.parse_size(123) == 123
    with pytest.raises(ValueError):
        P.parse_size("12 parsecs")


def _cli(*args):
    return subprocess.run([sys.executable, "-m", "head_windowed_kv_amd.mem_estimate", *args],
                          cwd=ROOT, capture_output=True, text=True, timeout=120)


def test_cli_fits_and_reports_exact_bytes():
    r = _cli("--config", FIXTURE, "--n-seqs", "8", "--json", "--context", "112k")
    assert r.returncode == 0, r.stderr
    out = json.loads(r.stdout)
    g = _golden()
    per_seq = sum(x["bytes_per_seq"] for x in g["layers"])
    assert out["bytes_per_seq"] == per_seq and out["total_bytes"] == 8 * per_seq
    assert out["rows_within_budget"] == 48 * 10 ** 9 // per_seq
    # a full cache of 112K tokens for 2 layers x 8 heads: the growth law
    # seq_len x heads x head_dim x 2 (K and V) x 2 bytes, per layer
    assert out["full_cache_bytes"] == 8 * 2 * 114688 * 8 * 128 * 2 * 2


def test_cli_over_budget_names_layer_and_head(tmp_path):
    r = _cli("--config", FIXTURE, "--n-seqs", "200", "--budget", "0.3g")
    assert r.returncode == 3, r.stdout + r.stderr
    # 0.3e9 B = 36621 blocks of 8 KiB: row 0 takes 33856, row 1 has 2765 left,
    # which ends inside layer 0, head 4 (blocks 2560..6655 of the row)
    assert "KV cache block allocation failed at layer 0, head 4: sequence row 1" in r.stdout
    bad = tmp_path / "bad.yaml"
    bad.write_text("per_layer_policies:\n- layer_id: 3\n  kv_head_windows: [1]\n")
    r = _cli("--config", str(bad))
    assert r.returncode == 2 and "missing" in r.stderr
