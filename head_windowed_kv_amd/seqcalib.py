"""SeqCalib: per-head window policy search in execution order, under a budget.

The HeadWiseKV write-up (KnoAI), section 核心技术 1, poses the choice of one
window vector w_i per layer (one window per physical KV head, from discrete
levels such as 1024 / 4096 / 16384 / 65536) as

    minimise  sum_i D_i(w_i)   subject to   sum_i R_i(w_i) <= B,

with D_i a distortion measured on the model and R_i the memory of layer i.
SeqCalib walks the layers in execution order; for layer i it scores every
candidate vector with a distortion that may depend on the vectors already
chosen for the layers below, and keeps the least distorting candidate whose
memory still fits the remaining budget, then charges that memory.

This module is that search.  Distortions need the model and calibration data,
which are the caller's: pass a callable ``distortion(layer, w, chosen)`` or a
table of unconditional values.  R_i is the exact memory of layer i's blocks
(ceil(w/bs) blocks per head, K and V, times the number of sequence rows),
asked of the C library through a one-layer layout.  When no candidate of a
layer fits what is left, the write-up's listing would go on with no window;
here that is an error naming the layer.
"""
from __future__ import annotations

import itertools
import json
import sys
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence

import numpy as np

from . import hwkv_layout_create, hwkv_mem_estimate
from .policy import Policy, parse_size, policy_to_yaml


class InfeasibleBudget(ValueError):
    """No candidate of a layer fits the budget left after the layers below."""

    def __init__(self, layer: int, remaining: int, cheapest: int):
        super().__init__("SeqCalib: no window vector of layer %d fits the remaining budget of %d "
                         "bytes (its cheapest candidate needs %d)" % (layer, remaining, cheapest))
        self.layer, self.remaining, self.cheapest = layer, remaining, cheapest


def layer_cost(w: Sequence[int], block_size: int = 16, head_dim: int = 128, dtype="bf16",
               n_seqs: int = 1) -> int:
    """R_i(w): exact bytes of one layer's K/V blocks for n_seqs rows."""
    lay = hwkv_layout_create(np.asarray([list(w)], np.int32), block_size, head_dim, dtype)
    return hwkv_mem_estimate(lay, n_seqs)


def candidate_vectors(levels: Sequence[int], n_kv_heads: int,
                      max_vectors: Optional[int] = None) -> List[tuple]:
    """Every per-head vector over the levels (levels ** n_kv_heads of them)."""
    n = len(levels) ** n_kv_heads
    if max_vectors is not None and n > max_vectors:
        raise ValueError("%d candidate vectors exceed the limit of %d" % (n, max_vectors))
    return [tuple(int(x) for x in v) for v in itertools.product(levels, repeat=n_kv_heads)]


@dataclass
class SeqCalibResult:
    windows: np.ndarray               # int32 [n_layers][n_kv_heads]
    costs: List[int]                  # R_i of the chosen vectors, bytes
    distortions: List[float]          # D_i of the chosen vectors
    remaining: List[int] = field(default_factory=list)  # budget left after each layer

    @property
    def total_cost(self) -> int:
        return int(sum(self.costs))

    @property
    def total_distortion(self) -> float:
        return float(sum(self.distortions))

    def policy(self, model_name: Optional[str] = None,
               budget_gb: Optional[float] = None) -> Policy:
        return Policy(self.windows.copy(), model_name, budget_gb)


def seqcalib(n_layers: int, candidates, distortion: Callable, budget: int,
             cost: Optional[Callable] = None) -> SeqCalibResult:
    """Greedy search in execution order.

    candidates: a list of window vectors shared by all layers, or a
        callable ``candidates(layer, chosen)`` returning the feasible vectors
        of a layer given the vectors chosen below it.
    distortion: ``distortion(layer, w, chosen) -> float``, chosen being the
        list of vectors of layers 0..layer-1.
    budget: total bytes B.
    cost: ``cost(layer, w) -> bytes``; default layer_cost(w) (bs 16, d 128,
        bf16, one sequence row).
    Ties in distortion keep the earlier candidate.
    """
    if cost is None:
        def cost(layer, w):
            return layer_cost(w)
    remaining = int(budget)
    chosen: List[tuple] = []
    costs, dists, rem = [], [], []
    for layer in range(n_layers):
        cands = candidates(layer, list(chosen)) if callable(candidates) else candidates
        best, best_d, best_c, cheapest = None, float("inf"), None, None
        for w in cands:
            w = tuple(int(x) for x in w)
            c = int(cost(layer, w))
            cheapest = c if cheapest is None else min(cheapest, c)
            if c > remaining:
                continue
            d = float(distortion(layer, w, list(chosen)))
            if d < best_d:
                best, best_d, best_c = w, d, c
        if best is None:
            raise InfeasibleBudget(layer, remaining, -1 if cheapest is None else cheapest)
        chosen.append(best)
        costs.append(best_c)
        dists.append(best_d)
        remaining -= best_c
        rem.append(remaining)
    return SeqCalibResult(np.array(chosen, np.int32), costs, dists, rem)


def seqcalib_table(candidates: Sequence[Sequence[int]], table, budget: int,
                   block_size: int = 16, head_dim: int = 128, dtype="bf16",
                   n_seqs: int = 1) -> SeqCalibResult:
    """SeqCalib with unconditional distortions: table[layer][j] is D_i of
    candidates[j]."""
    cands = [tuple(int(x) for x in c) for c in candidates]
    index = {c: j for j, c in enumerate(cands)}
    tab = [list(map(float, row)) for row in table]
    for i, row in enumerate(tab):
        if len(row) != len(cands):
            raise ValueError("distortion row %d has %d values for %d candidates"
                             % (i, len(row), len(cands)))
    costs = {c: layer_cost(c, block_size, head_dim, dtype, n_seqs) for c in cands}
    return seqcalib(len(tab), cands, lambda layer, w, chosen: tab[layer][index[w]], budget,
                    cost=lambda layer, w: costs[w])


def main(argv=None) -> int:
    """python -m head_windowed_kv_amd.seqcalib --table distortions.json --budget 48g
    [--n-seqs N] [--block-size 16] [--head-dim 128] [--dtype bf16] [--out policy.yaml]

    distortions.json: {"candidates": [[w_0, ..., w_{H-1}], ...],
                       "distortion": [[D_0(c_0), D_0(c_1), ...], ...]  (one row per layer),
                       "model_name": optional}
    Writes the chosen policy in the policy-file schema (stdout or --out)."""
    import argparse
    p = argparse.ArgumentParser(prog="python -m head_windowed_kv_amd.seqcalib")
    p.add_argument("--table", required=True)
    p.add_argument("--budget", required=True)
    p.add_argument("--n-seqs", type=int, default=1)
    p.add_argument("--block-size", type=int, default=16)
    p.add_argument("--head-dim", type=int, default=128)
    p.add_argument("--dtype", default="bf16", choices=("bf16", "f16", "f32"))
    p.add_argument("--out", default=None)
    a = p.parse_args(argv)
    with open(a.table, encoding="utf-8") as f:
        doc = json.load(f)
    budget = parse_size(a.budget)
    try:
        res = seqcalib_table(doc["candidates"], doc["distortion"], budget, a.block_size,
                             a.head_dim, a.dtype, a.n_seqs)
    except InfeasibleBudget as e:
        print("error: %s" % e, file=sys.stderr)
        return 3
    text = policy_to_yaml(res.policy(doc.get("model_name"), budget / 1e9))
    if a.out:
        with open(a.out, "w", encoding="utf-8") as f:
            f.write(text)
    else:
        sys.stdout.write(text)
    print("total cost %d bytes of %d, total distortion %.6g"
          % (res.total_cost, budget, res.total_distortion), file=sys.stderr)
    return 0


if __name__ == "__main__":
    sys.exit(main())
