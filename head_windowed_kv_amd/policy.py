"""Per-head window policies: the policy file, its layout and its exact footprint.

The HeadWiseKV write-up (KnoAI), section 核心技术 2 "Grouped-Cache Runtime",
describes the policy a serving engine loads: a YAML document with the model
name, a global budget (``budget_gb``) and ``per_layer_policies``, one entry per
layer with its ``layer_id`` and a ``kv_head_windows`` vector (one window per
physical KV head).  Each head's block table holds ceil(window / block_size)
blocks, so the footprint is exact before the server starts; the write-up's
operations table adds that a policy change needs a restart and that an
allocation failure names the (layer, head) in the policy.

This module parses and validates such a document (``yaml.safe_load`` only: a
policy file executes nothing), writes one back, and asks the C library for the
layout, the exact estimate and the capacity check; it does no cache arithmetic
of its own beyond summing the library's per-head block counts for display.
"""
from __future__ import annotations

import io
import re
from dataclasses import dataclass
from typing import Optional, Union

import numpy as np

from . import (Layout, hwkv_capacity_check, hwkv_layout_create, hwkv_layout_query,
               hwkv_mem_estimate)

#: bytes per "GB" of ``budget_gb`` and of a "g"/"gb" size suffix: read as the
#: SI gigabyte; "gib" selects 2^30 explicitly
GB = 10 ** 9
GIB = 1 << 30


class PolicyError(ValueError):
    """A policy document that does not describe a valid per-head layout."""


@dataclass(frozen=True)
class Policy:
    windows: np.ndarray                 # int32 [n_layers][n_kv_heads], layer-major
    model_name: Optional[str] = None
    budget_gb: Optional[float] = None

    @property
    def n_layers(self) -> int:
        return int(self.windows.shape[0])

    @property
    def n_kv_heads(self) -> int:
        return int(self.windows.shape[1])

    def budget_bytes(self) -> Optional[int]:
        return None if self.budget_gb is None else int(round(self.budget_gb * GB))


def _int_window(x, where: str) -> int:
    if isinstance(x, bool) or not isinstance(x, (int, np.integer)):
        raise PolicyError("%s: window %r is not an integer" % (where, x))
    if x < 1 or x > 2 ** 31 - 1:
        raise PolicyError("%s: window %d outside [1, 2^31-1]" % (where, x))
    return int(x)


def policy_from_dict(doc) -> Policy:
    """Validate a parsed policy document (a mapping)."""
    if not isinstance(doc, dict):
        raise PolicyError("a policy document must be a mapping")
    layers = doc.get("per_layer_policies")
    if not isinstance(layers, list) or not layers:
        raise PolicyError("per_layer_policies must be a non-empty list")
    by_id = {}
    for n, entry in enumerate(layers):
        if not isinstance(entry, dict):
            raise PolicyError("per_layer_policies[%d] is not a mapping" % n)
        lid = entry.get("layer_id")
        if isinstance(lid, bool) or not isinstance(lid, (int, np.integer)) or lid < 0:
            raise PolicyError("per_layer_policies[%d]: layer_id must be an integer >= 0" % n)
        if lid in by_id:
            raise PolicyError("layer_id %d appears twice" % lid)
        w = entry.get("kv_head_windows")
        if not isinstance(w, list) or not w:
            raise PolicyError("layer %d: kv_head_windows must be a non-empty list" % lid)
        by_id[int(lid)] = [_int_window(x, "layer %d, head %d" % (lid, h)) for h, x in enumerate(w)]
    n_layers = len(by_id)
    missing = sorted(set(range(n_layers)) - set(by_id))
    if missing:
        raise PolicyError("layer_id values must be 0..%d; missing %s" % (n_layers - 1, missing))
    n_kv = len(by_id[0])
    for lid in range(n_layers):
        if len(by_id[lid]) != n_kv:
            raise PolicyError("layer %d has %d kv heads, layer 0 has %d"
                              % (lid, len(by_id[lid]), n_kv))
    budget = doc.get("budget_gb")
    if budget is not None:
        if isinstance(budget, bool) or not isinstance(budget, (int, float)) or not budget > 0:
            raise PolicyError("budget_gb must be a positive number")
        budget = float(budget)
    name = doc.get("model_name")
    if name is not None and not isinstance(name, str):
        raise PolicyError("model_name must be a string")
    windows = np.array([by_id[l] for l in range(n_layers)], dtype=np.int32)
    return Policy(windows, name, budget)


def parse_policy(text: str) -> Policy:
    import yaml
    try:
        doc = yaml.safe_load(io.StringIO(text))
    except yaml.YAMLError as e:
        raise PolicyError("not valid YAML: %s" % e) from None
    return policy_from_dict(doc)


def load_policy(path: str) -> Policy:
    with open(path, encoding="utf-8") as f:
        return parse_policy(f.read())


def policy_to_yaml(policy: Policy) -> str:
    """The policy as a YAML document of the same schema (one flow list per
    layer), which parse_policy reads back to the same windows."""
    out = []
    if policy.model_name is not None:
        out.append("model_name: %s" % _yaml_str(policy.model_name))
    if policy.budget_gb is not None:
        out.append("budget_gb: %r" % float(policy.budget_gb))
    out.append("per_layer_policies:")
    for l in range(policy.n_layers):
        out.append("- layer_id: %d" % l)
        out.append("  kv_head_windows: [%s]" % ", ".join(str(int(x)) for x in policy.windows[l]))
    return "\n".join(out) + "\n"


def _yaml_str(s: str) -> str:
    return '"%s"' % s.replace("\\", "\\\\").replace('"', '\\"')


def parse_size(text: Union[str, int, float]) -> int:
    """Bytes from '48g', '48gb', '48GiB', '512m', '1.5t' or a plain number of
    bytes.  g/gb/t/m are SI (10^9, 10^12, 10^6); gib/tib/mib are binary."""
    if isinstance(text, (int, float)):
        return int(text)
    m = re.fullmatch(r"\s*([0-9]*\.?[0-9]+)\s*([a-zA-Z]*)\s*", text)
    if not m:
        raise ValueError("cannot read a size from %r" % text)
    unit = m.group(2).lower()
    mult = {"": 1, "b": 1, "k": 10 ** 3, "kb": 10 ** 3, "m": 10 ** 6, "mb": 10 ** 6, "g": GB,
            "gb": GB, "t": 10 ** 12, "tb": 10 ** 12, "kib": 1 << 10, "mib": 1 << 20,
            "gib": GIB, "tib": 1 << 40}.get(unit)
    if mult is None:
        raise ValueError("unknown size unit %r" % m.group(2))
    return int(round(float(m.group(1)) * mult))


def layout_for(policy: Policy, block_size: int = 16, head_dim: int = 128, dtype="bf16",
               split_tokens: int = 0) -> Layout:
    return hwkv_layout_create(policy.windows, block_size, head_dim, dtype, split_tokens)


@dataclass
class Estimate:
    n_seqs: int
    block_size: int
    head_dim: int
    block_bytes: int
    blocks_per_seq: int
    total_bytes: int                   # hwkv_mem_estimate(n_seqs)
    layer_bytes_per_seq: np.ndarray    # int64 [n_layers]
    head_blocks: np.ndarray            # int32 [n_layers][n_kv_heads]
    budget_bytes: Optional[int] = None
    first_unfit: Optional[tuple] = None  # (seq_row, layer, head, message)

    @property
    def fits(self) -> bool:
        return self.first_unfit is None


def estimate(policy: Policy, n_seqs: int = 1, block_size: int = 16, head_dim: int = 128,
             dtype="bf16", budget_bytes: Optional[int] = None) -> Estimate:
    """Exact footprint of n_seqs sequence rows under the policy, and, with a
    budget (default: the document's budget_gb), the first (row, layer, head)
    whose blocks would not fit in it."""
    lay = layout_for(policy, block_size, head_dim, dtype)
    desc, _, nb, _ = hwkv_layout_query(lay)
    total = hwkv_mem_estimate(lay, n_seqs)
    if budget_bytes is None:
        budget_bytes = policy.budget_bytes()
    unfit = None
    if budget_bytes is not None:
        unfit = hwkv_capacity_check(lay, n_seqs, budget_bytes)
    layer_bytes = nb.astype(np.int64).sum(axis=1) * int(desc.block_bytes)
    return Estimate(n_seqs, block_size, head_dim, int(desc.block_bytes), int(desc.blocks_per_seq),
                    total, layer_bytes, nb, budget_bytes, unfit)
