"""Exact KV-cache footprint of a per-head window policy, before serving.

    python -m head_windowed_kv_amd.mem_estimate --config policy.yaml \\
        [--n-seqs N] [--block-size 16] [--head-dim 128] [--dtype bf16] \\
        [--budget 48g] [--context 112k] [--per-head] [--json]

The HeadWiseKV write-up (核心技术 2) computes the footprint of a policy file
before the server starts; its operations table plans the memory budget with
a command-line calculator and names the failing (layer, head) when an
allocation does not fit.  This command does both from the library's exact
estimate: it prints the pool bytes for N sequence rows (K and V blocks,
ceil(w / block_size) blocks per head), the per-layer split, how many rows fit
the budget and, if N rows do not, the first head whose blocks would fail.
With --context it also prints the footprint of a full cache of that length
for comparison.  Exit status: 0 fits (or no budget given), 3 over budget,
2 invalid policy or arguments.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

from . import hwkv_layout_create, hwkv_mem_estimate
from .policy import GB, GIB, PolicyError, estimate, load_policy, parse_size


def _tokens(text: str) -> int:
    """'112k' -> 114688 (K read as 1024 tokens), '4096' -> 4096."""
    t = text.strip().lower()
    if t.endswith("k"):
        return int(round(float(t[:-1]) * 1024))
    return int(t)


def _fmt(b: int) -> str:
    return "%d B (%.3f GB, %.3f GiB)" % (b, b / GB, b / GIB)


def main(argv=None) -> int:
    p = argparse.ArgumentParser(prog="python -m head_windowed_kv_amd.mem_estimate",
                                description=__doc__.split("\n\n")[1])
    p.add_argument("--config", required=True, help="policy YAML (per_layer_policies)")
    p.add_argument("--n-seqs", type=int, default=1, help="sequence rows of the pool")
    p.add_argument("--block-size", type=int, default=16)
    p.add_argument("--head-dim", type=int, default=128)
    p.add_argument("--dtype", default="bf16", choices=("bf16", "f16", "f32"))
    p.add_argument("--budget", default=None,
                   help="pool budget, e.g. 48g (10^9 B), 48gib (2^30 B) or bytes; default: the "
                        "policy's budget_gb")
    p.add_argument("--context", default=None, help="context length for a full-cache comparison")
    p.add_argument("--per-head", action="store_true", help="list every head's blocks")
    p.add_argument("--json", action="store_true", help="one JSON object instead of text")
    a = p.parse_args(argv)
    try:
        pol = load_policy(a.config)
        budget = parse_size(a.budget) if a.budget is not None else None
        est = estimate(pol, a.n_seqs, a.block_size, a.head_dim, a.dtype, budget)
    except (PolicyError, ValueError, OSError) as e:
        print("error: %s" % e, file=sys.stderr)
        return 2
    per_seq = est.blocks_per_seq * est.block_bytes
    rows_fit = None
    if est.budget_bytes is not None and per_seq > 0:
        rows_fit = est.budget_bytes // per_seq
    full = None
    if a.context is not None:
        ctx = _tokens(a.context)
        full_lay = hwkv_layout_create(np.full(pol.windows.shape, ctx, np.int32), a.block_size,
                                      a.head_dim, a.dtype)
        full = hwkv_mem_estimate(full_lay, a.n_seqs)
    res = {"config": a.config, "model_name": pol.model_name, "layers": pol.n_layers,
           "kv_heads": pol.n_kv_heads, "block_size": a.block_size, "head_dim": a.head_dim,
           "dtype": a.dtype, "n_seqs": a.n_seqs, "block_bytes": est.block_bytes,
           "blocks_per_seq": est.blocks_per_seq, "bytes_per_seq": per_seq,
           "total_bytes": est.total_bytes, "budget_bytes": est.budget_bytes,
           "rows_within_budget": rows_fit, "fits": est.fits,
           "layer_bytes_per_seq": [int(x) for x in est.layer_bytes_per_seq]}
    if est.first_unfit is not None:
        row, layer, head, msg = est.first_unfit
        res["first_unfit"] = {"seq_row": row, "layer": layer, "head": head, "message": msg}
    if full is not None:
        res["full_cache_context"] = _tokens(a.context)
        res["full_cache_bytes"] = full
        res["resident_fraction"] = est.total_bytes / full if full else None
    if a.per_head:
        res["head_blocks"] = est.head_blocks.tolist()
    if a.json:
        print(json.dumps(res))
    else:
        print("policy %s%s: %d layers x %d kv heads, block_size %d, head_dim %d, %s"
              % (a.config, " (%s)" % pol.model_name if pol.model_name else "", pol.n_layers,
                 pol.n_kv_heads, a.block_size, a.head_dim, a.dtype))
        print("per sequence row: %d blocks x %d B = %s" % (est.blocks_per_seq, est.block_bytes,
                                                         _fmt(per_seq)))
        print("pool for %d row(s): %s" % (a.n_seqs, _fmt(est.total_bytes)))
        if full is not None:
            print("full cache at %d tokens: %s; resident fraction %.4f"
                  % (res["full_cache_context"], _fmt(full), res["resident_fraction"] or 0.0))
        for l, b in enumerate(est.layer_bytes_per_seq):
            line = "  layer %3d: %12d B per row" % (l, b)
            if a.per_head:
                line += "  blocks %s" % est.head_blocks[l].tolist()
            print(line)
        if est.budget_bytes is not None:
            print("budget %s: %d row(s) fit" % (_fmt(est.budget_bytes), rows_fit))
            if est.first_unfit is not None:
                print(est.first_unfit[3])
    return 0 if est.fits else 3


if __name__ == "__main__":
    sys.exit(main())
