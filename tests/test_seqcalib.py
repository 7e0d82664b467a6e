"""SeqCalib policy search (host only).

Pins: a hand-worked three-layer example (including the budget running out,
which the write-up's listing leaves undefined and this search reports), a
conditional distortion worked by hand, brute-force enumeration (with an
unconstrained budget the greedy choice is the global optimum; with a tight one
it can differ from it, since the search commits layer by layer), the layer
costs against the hand-worked block formula of the printed policy, the
per-layer choice rule as an invariant on random tables, and the command's
policy file read back by the policy loader."""
import itertools
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import synth

hw = pytest.importorskip("head_windowed_kv_amd", reason="libhwkv.so not built")
from head_windowed_kv_amd import policy as P  # noqa: E402
from head_windowed_kv_amd import seqcalib as S  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# three candidates with costs 1, 2, 4 units
CANDS = [(1,), (2,), (4,)]
UNIT_COST = {(1,): 1, (2,): 2, (4,): 4}
TABLE = [[5.0, 3.0, 1.0], [6.0, 2.0, 1.0], [9.0, 4.0, 0.0]]


def _run(table, budget):
    idx = {c: j for j, c in enumerate(CANDS)}
    return S.seqcalib(len(table), CANDS, lambda l, w, ch: table[l][idx[w]], budget,
                      cost=lambda l, w: UNIT_COST[w])


def test_hand_worked_greedy():
    # budget 7: layer 0 takes (4,) [d 1, 3 left], layer 1 (2,) [d 2, 1 left],
    # layer 2 only (1,) fits [d 9]: total distortion 12, cost 7
    r = _run(TABLE, 7)
    assert r.windows.tolist() == [[4], [2], [1]]
    assert r.costs == [4, 2, 1] and r.remaining == [3, 1, 0]
    assert r.total_distortion == 12.0
    # the global optimum under the same budget is lower (5 + 2 + 0 = 7 at
    # (1,), (2,), (4,)): the search commits layer by layer
    best = min((sum(TABLE[l][j] for l, j in enumerate(js)), js)
               for js in itertools.product(range(3), repeat=3)
               if sum(UNIT_COST[CANDS[j]] for j in js) <= 7)
    assert best == (7.0, (0, 1, 2))


def test_budget_running_out_is_reported_with_the_layer():
    with pytest.raises(S.InfeasibleBudget) as e:
        _run(TABLE, 6)  # (4,), then (2,): nothing left for layer 2
    assert e.value.layer == 2 and e.value.remaining == 0 and e.value.cheapest == 1
    with pytest.raises(S.InfeasibleBudget) as e:
        _run(TABLE, 0)
    assert e.value.layer == 0


def test_conditional_distortion_hand_worked():
    # layer 1 is cheap to compress only if layer 0 kept its long window
    def dist(layer, w, chosen):
        if layer == 0:
            return {(1,): 3.0, (2,): 2.0, (4,): 1.0}[w]
        long0 = chosen[0] == (4,)
        return {(1,): 0.5 if long0 else 9.0, (2,): 1.0, (4,): 1.5}[w]
    r = S.seqcalib(2, CANDS, dist, 5, cost=lambda l, w: UNIT_COST[w])
    assert r.windows.tolist() == [[4], [1]] and r.total_distortion == 1.5
    r = S.seqcalib(2, CANDS, dist, 3, cost=lambda l, w: UNIT_COST[w])
    # layer 0 can only afford (2,) [1 left]; layer 1 then sees 9.0 for (1,)
    assert r.windows.tolist() == [[2], [1]] and r.distortions == [2.0, 9.0]


def test_candidates_may_depend_on_the_layers_below():
    calls = []

    def cands(layer, chosen):
        calls.append((layer, list(chosen)))
        return CANDS if layer == 0 else [w for w in CANDS if w <= chosen[-1]]
    r = S.seqcalib(3, cands, lambda l, w, ch: -w[0], 100, cost=lambda l, w: UNIT_COST[w])
    assert r.windows.tolist() == [[4], [4], [4]]
    assert calls == [(0, []), (1, [(4,)]), (2, [(4,), (4,)])]


def test_unconstrained_budget_is_the_global_optimum_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(20):
        table = rng.random((3, 3)).tolist()
        r = _run(table, 10 ** 9)
        best = min(itertools.product(range(3), repeat=3),
                   key=lambda js: sum(table[l][j] for l, j in enumerate(js)))
        assert r.windows.tolist() == [[CANDS[j][0]] for j in best]


def test_choice_rule_invariant_on_random_tables():
    """Each layer's choice is a least-distortion candidate among those that
    fit the budget left by the layers below; the total never exceeds B."""
    rng = np.random.default_rng(4)
    for trial in range(50):
        table = rng.integers(0, 5, (4, 3)).astype(float).tolist()
        budget = int(rng.integers(4, 16))
        try:
            r = _run(table, budget)
        except S.InfeasibleBudget as e:
            assert min(UNIT_COST.values()) > e.remaining
            continue
        assert r.total_cost <= budget
        left = budget
        for l, w in enumerate(map(tuple, r.windows.tolist())):
            fit = [j for j, c in enumerate(CANDS) if UNIT_COST[c] <= left]
            assert table[l][CANDS.index(w)] == min(table[l][j] for j in fit)
            left -= UNIT_COST[w]


def test_layer_cost_is_the_block_formula_of_the_printed_policy(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "policy_yaml_layers.json")))
    for layer in g["layers"]:
        assert S.layer_cost(layer["kv_head_windows"]) == layer["bytes_per_seq"]
        assert S.layer_cost(layer["kv_head_windows"], n_seqs=3) == 3 * layer["bytes_per_seq"]


def test_levels_search_on_a_small_stack():
    cands = S.candidate_vectors(synth.WINDOW_LEVELS, 2)
    assert len(cands) == 16
    # distortion falls with the total window: every layer takes the largest
    # vector that fits what is left
    dist = lambda l, w, ch: (l + 1) / (1.0 + sum(w) / 1024.0)  # noqa: E731
    top = S.layer_cost((65536, 65536))
    r = S.seqcalib(4, cands, dist, 4 * top)
    assert r.windows.tolist() == [[65536, 65536]] * 4 and r.total_cost == 4 * top
    # one byte less: the last layer gets the next largest vector (the two of
    # equal total keep the earlier one)
    r = S.seqcalib(4, cands, dist, 4 * top - 1)
    assert r.windows.tolist() == [[65536, 65536]] * 3 + [[16384, 65536]]
    assert r.total_cost == sum(S.layer_cost(w) for w in r.windows.tolist()) <= 4 * top - 1
    with pytest.raises(ValueError):
        S.candidate_vectors(synth.WINDOW_LEVELS, 8, max_vectors=1000)


def test_command_writes_a_policy_the_loader_reads(tmp_path):
    doc = {"model_name": "toy", "candidates": [[1024, 4096], [4096, 16384], [65536, 65536]],
           "distortion": [[3.0, 2.0, 1.0], [5.0, 1.0, 0.0], [1.0, 1.0, 1.0]]}
    tab = tmp_path / "d.json"
    tab.write_text(json.dumps(doc))
    out = tmp_path / "policy.yaml"
    # budget: 65536-pair costs 2 * 65536 * 512 B = 64 MiB per layer
    budget = S.layer_cost((65536, 65536)) + S.layer_cost((4096, 16384)) + \
        S.layer_cost((1024, 4096))
    r = subprocess.run([sys.executable, "-m", "head_windowed_kv_amd.seqcalib", "--table",
                        str(tab), "--budget", str(budget), "--out", str(out)], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    pol = P.load_policy(str(out))
    assert pol.model_name == "toy"
    # layer 0 takes the longest pair (d 1.0), layer 1 the middle one (d 1.0),
    # layer 2 the first that fits what is left (ties keep the earlier one)
    assert pol.windows.tolist() == [[65536, 65536], [4096, 16384], [1024, 4096]]
    r = subprocess.run([sys.executable, "-m", "head_windowed_kv_amd.seqcalib", "--table",
                        str(tab), "--budget", "1000"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 3 and "layer 0" in r.stderr
