#!/usr/bin/env python3
"""Benchmark of the per-head windowed KV decode step on one MI355X.

Workload (default): 48 layers x 8 KV heads (24 query heads, GQA group 3),
head_dim 128, bf16, block_size 16, per-head windows drawn from
{1024, 4096, 16384, 65536} with weights 0.2/0.3/0.3/0.2 (numpy seed 0),
context 112K (114,688 tokens), batch 1.  One step = append of the new token
for all 48 layers + decode attention (split + merge) over exactly the last
w_h tokens of every head, one launch of each kernel for the whole stack.
Inputs are synthetic N(0,1) K/V and N(0,1/128) q, resident in HBM before the
timed region starts.

Prints one JSON line.  Extra legs: `roofline` (the split kernel, timed with
HIP events on its own stream), `cpu_baseline` (the fp64 CPU oracle on a
bounded sample of the same step) and `per_layer_graph` (48 per-layer launch
triplets captured in one HIP graph).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
METRIC = "decode tokens/s + effective KV-read GB/s (% of HBM peak), per-head-window attn"
KV_BYTES_PER_TOK_HEAD = 512  # K + V row: 2 x 128 x bf16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=50,
                   help="untimed steps first; the first few dozen steps after the cache fill "
                        "run up to 6%% slower than the steady state")
    p.add_argument("--split-tokens", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--graph-split-tokens", type=int, default=384,
                   help="decode split length of the second per-layer graph variant (384 is "
                        "the fastest per-layer split measured from 128 to 1024)")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--prefill-only", action="store_true",
                   help="run only the 161K chunked-prefill leg (e.g. under rocprofv3 --pmc)")
    p.add_argument("--no-mixed", action="store_true",
                   help="skip the mixed-stack leg (fp16 / 64-token blocks, hybrid SWA + "
                        "global stack, head_dim 256 prefill) and the GQA-group leg")
    p.add_argument("--mixed-only", action="store_true",
                   help="run only the mixed-stack and GQA-group legs (e.g. under rocprofv3)")
    p.add_argument("--single-layer-only", action="store_true",
                   help="run only the one-layer, 8-sequence, 32K-context decode leg (e.g. "
                        "under rocprofv3)")
    p.add_argument("--config", choices=("stack48", "cb"), default="stack48",
                   help="stack48: the 48-layer 112K decode step (default, the headline line); "
                        "cb: the 32-sequence continuous batch, 256 steps (138 GB pool)")
    p.add_argument("--cb-steps", type=int, default=256)
    p.add_argument("--no-cb", action="store_true",
                   help="skip the continuous-batch leg of the default run")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--counter-pass", action="store_true",
                   help="short run for a rocprofv3 --pmc pass: a few steps plus one probe "
                        "copy of known size (the counters' calibration)")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) "
                        "into profiles/decode_split_stack48_counters.json (with --config cb: "
                        "decode_split_cb_counters.json) and exit")
    return p.parse_args()


def code_tokens(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed, so
    that a hash of it changes with the code, not with its comments or
    layout (string and character literals are kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":  # literal: copy through its closing quote
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha() -> str:
    """Hash of the decode kernel's code (decode.hip and the shared header,
    comments and layout ignored): committed counter summaries are reported
    only while it matches the one they were taken on."""
    h = hashlib.sha256()
    for f in ("decode.hip", "hwkv_internal.h"):
        with open(os.path.join(ROOT, "head_windowed_kv_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


COUNTER_FILES = {"stack48": "decode_split_stack48_counters.json",
                 "cb": "decode_split_cb_counters.json"}
COUNTER_COMMANDS = {
    "stack48": "python -u bench.py --counter-pass --steps 3 --warmup 2",
    "cb": "python -u bench.py --config cb --counter-pass --cb-steps 4"}


def load_traffic(split_tokens: int, workload: str = "stack48"):
    """HBM traffic of one split launch from committed rocprofv3 counter runs,
    valid only while the kernel source and split size are the ones the
    counters were taken on."""
    path = os.path.join(ROOT, "profiles", COUNTER_FILES[workload])
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha() or \
            rec.get("split_tokens") != split_tokens:
        return None
    return rec.get("traffic_bytes_per_launch")


PROBE_COPY_BYTES = 1 << 30
# decode split length of the one-layer, 8-sequence, 32K leg: the fastest for
# that workload in a sweep of 1024-2048 tokens (its 672 streaming workgroups
# then fit the 768 resident slots at once: 0.116-0.120 ms against 0.121-0.126
# at the default 1024)
SINGLE_LAYER_SPLIT = 2048


def probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "head_windowed_kv_amd", "libhwkv_probe.so"))
    lib.hwkv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_void_p]
    lib.hwkv_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                    ctypes.c_int, ctypes.c_void_p]
    return lib


def read_ceiling(torch, buf, reps=24):
    """Practical HBM read bandwidth: a plain streaming read over `buf`, the
    median of `reps` reads at each of two grid sizes."""
    import ctypes
    lib = probe_lib()
    s = torch.cuda.current_stream()
    out = torch.zeros(4, dtype=torch.uint8, device=buf.device)
    n = buf.numel() // 16 * 16
    best = 0.0
    for grid in (2048, 16384):
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            rc = lib.hwkv_probe_read(ctypes.c_void_p(buf.data_ptr()), n,
                                     ctypes.c_void_p(out.data_ptr()), grid,
                                     ctypes.c_void_p(s.cuda_stream))
            e1.record(s)
            torch.cuda.synchronize()
            assert rc == 0
            ts.append(e0.elapsed_time(e1))
        best = max(best, n / (sorted(ts)[len(ts) // 2] / 1e3) / 1e9)
    return best


def probe_copy_once(torch, dev):
    import ctypes
    lib = probe_lib()
    src = torch.ones(PROBE_COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    s = torch.cuda.current_stream()
    rc = lib.hwkv_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                             PROBE_COPY_BYTES, 4096, ctypes.c_void_p(s.cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0


def _pmc_rows(folder, counter):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc output folder
    (CSV or SQLite)."""
    import csv
    import glob
    import sqlite3
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if rows:
        return rows
    for f in glob.glob(os.path.join(folder, "**", "*.db"), recursive=True):
        con = sqlite3.connect(f)
        q = ("select k.name, p.value from pmc_events p join kernels k on p.event_id = k.id "
             "where p.counter_name = ?")
        try:
            rows += [(n, float(v)) for n, v in con.execute(q, (counter,))]
        except sqlite3.Error:
            cols = [c[1] for c in con.execute("pragma table_info(counters_collection)")]
            name_col = "kernel_name" if "kernel_name" in cols else "name"
            q = "select %s, value from counters_collection where counter_name = ?" % name_col
            rows += [(n, float(v)) for n, v in con.execute(q, (counter,))]
    return rows


def summarize_counters(fetch_dir, write_dir, split_tokens, workload="stack48"):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the split kernel, each
    scaled by what the same counter reads for the probe copy of known size;
    workload: the 48-layer headline step (stack48) or the continuous batch
    (cb), whose counter passes each run the probe copy too."""
    import head_windowed_kv_amd as H
    import synth
    lay = H.hwkv_layout_create(synth.stack_windows(48, 8, 0), 16, 128, "bf16", split_tokens)
    out = {"kernel_source_sha": kernel_source_sha(), "probe_copy_bytes": PROBE_COPY_BYTES,
           "split_tokens": lay.desc().split_tokens, "workload": workload,
           "command": "rocprofv3 --pmc <COUNTER> --output-format csv -d <dir> -o run -- " +
                      COUNTER_COMMANDS[workload]}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(folder, counter)
        split = [v for n, v in rows if "decode_split_kernel" in n]
        copy = [v for n, v in rows if "probe_copy_kernel" in n]
        if not split or not copy:
            raise SystemExit("no %s rows for the split or the probe copy in %s" % (counter, folder))
        split_kib = sorted(split)[len(split) // 2]
        copy_kib = copy[-1]
        scale = PROBE_COPY_BYTES / (copy_kib * 1024.0)
        out[counter] = {"split_kib_per_dispatch": split_kib, "probe_copy_kib": copy_kib,
                        "scale": round(scale, 4), "split_bytes_scaled": split_kib * 1024 * scale,
                        "dispatches": len(split)}
    out["traffic_bytes_per_launch"] = (out["FETCH_SIZE"]["split_bytes_scaled"] +
                                       out["WRITE_SIZE"]["split_bytes_scaled"])
    path = os.path.join(ROOT, "profiles", COUNTER_FILES[workload])
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    args = parse()
    # A full pass of Python's cyclic garbage collector over the ~170K objects
    # torch and numpy hold pauses the host for 30-40 ms; inside a timed region
    # the GPU then runs dry (one such pass turned a 0.7 ms step average into
    # 2.4 ms).  Collect once here and keep the collector off for the run.
    gc.collect()
    gc.disable()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.split_tokens, args.config)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.config == "cb":
        cb_run(args)
        return
    if args.prefill_only:
        import torch

        import head_windowed_kv_amd as H
        import synth
        torch.cuda.set_device(0)
        print(json.dumps({"prefill_161k": prefill_leg(H, torch, synth)}), flush=True)
        return
    if args.mixed_only:
        import torch

        import head_windowed_kv_amd as H
        import synth
        torch.cuda.set_device(0)
        print(json.dumps({"mixed_stacks": mixed_leg(H, torch, synth),
                          "gqa_groups": gqa_leg(H, torch, synth)}), flush=True)
        return
    if args.single_layer_only:
        import torch

        import head_windowed_kv_amd as H
        import synth
        torch.cuda.set_device(0)
        print(json.dumps({"single_layer_8seqs_ctx32k": single_layer_leg(
            H, torch, synth, split_tokens=SINGLE_LAYER_SPLIT)}), flush=True)
        return

    import numpy as np
    import torch

    import head_windowed_kv_amd as H
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    n_layers, n_kv, G, d, bs = 48, 8, 3, 128, 16
    L0 = synth.CTX_112K
    n_seqs = 1
    windows = synth.stack_windows(n_layers, n_kv, 0)
    lay = H.hwkv_layout_create(windows, bs, d, torch.bfloat16, args.split_tokens)
    desc = lay.desc()
    cache = H.make_cache(lay, n_seqs, device=dev)
    cap = int(((windows.astype(np.int64) + bs - 1) // bs * bs).max())
    n_hist = min(L0, cap)

    # ---- fill: per layer, the last n_hist positions before L0 ----
    t_fill = time.time()
    pos_hist = torch.full((n_seqs,), L0 - n_hist, dtype=torch.int64, device=dev)
    for l in range(n_layers):
        g = synth.gen(103 * 100003 + l, dev)
        k = synth.randn((1, n_seqs, n_hist, n_kv, d), torch.bfloat16, g)
        v = synth.randn((1, n_seqs, n_hist, n_kv, d), torch.bfloat16, g)
        H.hwkv_append(cache, l, 1, pos_hist, k, v)
        del k, v
    torch.cuda.synchronize()
    t_fill = time.time() - t_fill

    # warmup steps, the timed steps, then as many again for the split-kernel
    # timing pass (the token stream continues through all of them)
    n_steps = args.warmup + 2 * args.steps
    g = synth.gen(104, dev)
    q = synth.randn((n_layers, n_seqs, n_kv * G, d), torch.bfloat16, g, std=1.0 / math.sqrt(d))
    k_new = synth.randn((n_steps, n_layers, n_seqs, 1, n_kv, d), torch.bfloat16, g)
    v_new = synth.randn((n_steps, n_layers, n_seqs, 1, n_kv, d), torch.bfloat16, g)
    pos = [torch.full((n_seqs,), L0 + i, dtype=torch.int64, device=dev) for i in range(n_steps)]
    ctx = [torch.full((n_seqs,), L0 + i + 1, dtype=torch.int64, device=dev)
           for i in range(n_steps)]
    ws = H.make_workspace(lay, 0, n_layers, n_seqs, n_kv * G, device=dev)
    out = torch.empty((n_layers, n_seqs, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream()

    # algorithmic K/V bytes of one decode step: every head reads min(w, L) rows
    def step_bytes(L):
        return float(np.minimum(windows.astype(np.int64), L).sum()) * KV_BYTES_PER_TOK_HEAD

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    # one step = the split stage, which also appends each layer's new token,
    # then the merge stage (hwkv_decode_append_attn as its two stage calls, so
    # that the split kernel can be timed on its own)
    def run_step(i, evp=None):
        if evp is not None:
            evp[0].record(stream)
        H.hwkv_decode_split_append(cache, 0, n_layers, pos[i], k_new[i], v_new[i], q, scale, ws,
                                   stream=stream)
        if evp is not None:
            evp[1].record(stream)
        H.hwkv_decode_merge(cache, 0, n_layers, ctx[i], ws, out, stream=stream)

    # The first warmup step loads the library's kernels (~30 ms with the GPU
    # idle); a sustained load after such an idle gap runs ~5-15% slow for the
    # next ~20 steps while the clocks settle.  The practical read ceiling (a
    # plain streaming read over the same pool, ~50 ms) is measured right
    # after that first step, so the settling happens inside it and the timed
    # steps see the steady state.
    run_step(0)
    torch.cuda.synchronize()
    ceiling = read_ceiling(torch, cache.pool)
    for i in range(1, args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    if args.counter_pass:
        for j in range(args.steps):
            run_step(args.warmup + j)
        probe_copy_once(torch, dev)
        print(json.dumps({"counter_pass": True, "steps": args.steps}), flush=True)
        return
    # the timed region: K consecutive steps, nothing recorded between them
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for j in range(args.steps):
        run_step(args.warmup + j)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    # the split kernel's own duration, from a separate pass of K more steps
    # with HIP events around each split launch on the stream it runs on
    for j in range(args.steps):
        run_step(args.warmup + args.steps + j, ev[j])
    torch.cuda.synchronize()
    split_ms = [a.elapsed_time(b) for a, b in ev]
    split_avg_ms = sum(split_ms) / len(split_ms)
    bytes_step = step_bytes(L0 + args.warmup + 1)
    tok_per_s = n_seqs * args.steps / (total_ms / 1e3)
    kv_gbps = bytes_step / (ms_per_step / 1e3) / 1e9
    split_gbps = bytes_step / (split_avg_ms / 1e3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(tok_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "stack48_ctx112k_decode_step",
            "layers": n_layers, "kv_heads": n_kv, "q_heads": n_kv * G, "head_dim": d,
            "block_size": bs, "context": L0, "batch": n_seqs,
            "windows": "per (layer, head) from {1024,4096,16384,65536} p=.2/.3/.3/.2, "
                       "numpy default_rng(0)",
            "split_tokens": desc.split_tokens,
            "launch": "one split launch (which also appends the new token) + one merge launch "
                      "for all 48 layers",
        },
        "kv_read_bytes_per_step": bytes_step,
        "kv_read_gbps": round(kv_gbps, 1),
        "kv_read_frac_of_peak": round(kv_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_split_kernel<bf16, d128, G3, append>",
            "achieved": round(split_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(split_gbps / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(desc.split_tokens),
            "traffic_source": "committed rocprofv3 --pmc counters (FETCH_SIZE, WRITE_SIZE per "
                              "dispatch, scaled by the probe copy of known size) in "
                              "profiles/decode_split_stack48_counters.json; reported only while "
                              "the kernel source hash and split length match (else null)",
            "avg_launch_ms": round(split_avg_ms, 4),
            "avg_launch_timing": "HIP events around each split launch, in a pass of %d steps "
                                 "after the timed region" % args.steps,
            "algorithmic_bytes_per_launch": bytes_step,
        },
        "fill_seconds": round(t_fill, 2),
    }
    result["practical_read_ceiling_gbps"] = round(ceiling, 1)
    result["roofline"]["frac_of_practical_ceiling"] = round(split_gbps / ceiling, 4)

    result["three_launch_step"] = three_launch_leg(H, torch, cache, q, k_new, v_new,
                                                   L0 + n_steps, n_seqs, args.steps, step_bytes,
                                                   scale, ws, out)
    result["two_launch_step_repeat"] = fused_leg(H, torch, cache, lay, q, k_new, v_new,
                                                 L0 + n_steps + 16, n_seqs, n_kv, G, d,
                                                 args.steps, step_bytes, two_launch=True)
    result["single_launch_step"] = fused_leg(H, torch, cache, lay, q, k_new, v_new,
                                             L0 + n_steps + 32, n_seqs, n_kv, G, d, args.steps,
                                             step_bytes)
    if not args.no_graph:
        for mode in ("three_launches", "append_in_split", "single_launch"):
            for st in (desc.split_tokens, args.graph_split_tokens):
                key = "per_layer_graph_%s_split%d" % (mode, st)
                glay = lay if st == desc.split_tokens else \
                    H.hwkv_layout_create(windows, bs, d, torch.bfloat16, st)
                result[key] = per_layer_graph(H, torch, cache, glay, windows, q, k_new, v_new,
                                              L0 + n_steps + 64, n_seqs, n_kv, G, d, step_bytes,
                                              mode)
    if not args.no_prefill:
        del cache, ws  # the decode pool is not needed any more
        torch.cuda.empty_cache()
        result["prefill_161k"] = prefill_leg(H, torch, synth)
        torch.cuda.empty_cache()
        result["single_layer_8seqs_ctx32k"] = single_layer_leg(H, torch, synth,
                                                               split_tokens=SINGLE_LAYER_SPLIT)
        torch.cuda.empty_cache()
        if not args.no_mixed:
            result["mixed_stacks"] = mixed_leg(H, torch, synth)
            torch.cuda.empty_cache()
            result["gqa_groups"] = gqa_leg(H, torch, synth)
    if not args.no_cb:
        torch.cuda.empty_cache()
        result["continuous_batch_32seq"] = cb_leg(args, H, torch, synth)
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(windows, L0, n_kv, G, d, args.cpu_seconds,
                                              tok_per_s, result.get("prefill_161k"))
    print(json.dumps(result), flush=True)


def cb_run(args):
    """`--config cb`: the continuous batch as the JSON line itself."""
    import torch

    import head_windowed_kv_amd as H
    import synth
    torch.cuda.set_device(0)
    leg = cb_leg(args, H, torch, synth)
    if args.counter_pass:  # the counters' calibration, as in the headline's counter pass
        probe_copy_once(torch, torch.device("cuda", 0))
    res = {"metric": METRIC, "value": leg["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
           "steps": leg["steps"], "warmup": 2, "ms_per_step": leg["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": leg["config"],
           "kv_read_gbps": leg["kv_read_gbps"], "kv_read_frac_of_peak": leg["kv_read_frac_of_peak"],
           "roofline": leg["roofline"], "fill_seconds": leg["fill_seconds"]}
    print(json.dumps(res), flush=True)


def cb_leg(args, H, torch, synth):
    """Continuous batch: 32 sequences with contexts uniform in [4K, 160K],
    the 48-layer stack's windows, 256 decode steps of append + attention
    (hwkv_decode_append_attn: the split stage appends each sequence's new
    token, then the merge), one launch of each kernel per step for all
    layers and sequences.  Then a pass of 16 more steps with HIP events
    around each split launch gives the split kernel's roofline."""
    import numpy as np

    dev = torch.device("cuda", 0)
    n_layers, n_kv, G, d = 48, 8, 3, 128
    windows = synth.stack_windows(n_layers, n_kv, 0)
    L0 = synth.cb_contexts()
    n_seqs = len(L0)
    lay = H.hwkv_layout_create(windows, 16, d, torch.bfloat16, args.split_tokens)
    t = time.time()
    cache = H.make_cache(lay, n_seqs, device=dev)
    pool_bytes = cache.pool.numel()
    synth.fill_normal(cache.pool, 104, progress=True)
    torch.cuda.synchronize()
    t_fill = time.time() - t
    g = synth.gen(107, dev)
    q = synth.randn((n_layers, n_seqs, n_kv * G, d), torch.bfloat16, g, std=1.0 / math.sqrt(d))
    ws = H.make_workspace(lay, 0, n_layers, n_seqs, n_kv * G, device=dev)
    out = torch.empty((n_layers, n_seqs, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    L0_t = torch.tensor(L0, dtype=torch.int64, device=dev)
    n_steps = args.cb_steps
    kn = synth.randn((n_layers, n_seqs, 1, n_kv, d), torch.bfloat16, g)
    vn = synth.randn((n_layers, n_seqs, 1, n_kv, d), torch.bfloat16, g)
    n_roof = 16
    pos = [L0_t + i for i in range(n_steps + 2 + n_roof)]
    ctx = [p + 1 for p in pos]
    scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream()

    def step(i):  # append + attention: the split stage appends, then the merge
        H.hwkv_decode_append_attn(cache, 0, n_layers, pos[i], kn, vn, q, scale, ws, out)

    step(0)
    step(1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(n_steps):
        step(2 + i)
    e1.record(s)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    w64 = windows.astype(np.int64).reshape(-1)

    def bytes_at(L):  # K/V bytes every head of every sequence reads at contexts L
        return float(np.minimum(w64[None, :], np.asarray(L)[:, None]).sum()) * \
            KV_BYTES_PER_TOK_HEAD
    kv_bytes = sum(bytes_at(L0 + 3 + i) for i in range(n_steps))
    # split-kernel pass: the two stage calls of the same step, events around the split
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_roof)]
    roof_bytes = 0.0
    for j in range(n_roof):
        i = 2 + n_steps + j
        ev[j][0].record(s)
        H.hwkv_decode_split_append(cache, 0, n_layers, pos[i], kn, vn, q, scale, ws)
        ev[j][1].record(s)
        H.hwkv_decode_merge(cache, 0, n_layers, ctx[i], ws, out)
        roof_bytes += bytes_at(L0 + i + 1)
    torch.cuda.synchronize()
    split_ms = sum(a.elapsed_time(b) for a, b in ev) / n_roof
    split_gbps = roof_bytes / n_roof / (split_ms / 1e3) / 1e9
    del cache
    return {"workload": "continuous_batch_32seq_ctx4k_160k_stack48",
            "config": {"workload": "continuous_batch_32seq_ctx4k_160k_stack48",
                       "layers": n_layers, "kv_heads": n_kv, "q_heads": n_kv * G,
                       "head_dim": d, "block_size": 16, "batch": n_seqs,
                       "contexts": "uniform integers in [4096, 163840], numpy default_rng(1)",
                       "split_tokens": lay.desc().split_tokens, "pool_bytes": pool_bytes},
            "steps": n_steps, "ms_per_step": round(total_ms / n_steps, 4),
            "tokens_per_s": round(n_seqs * n_steps / (total_ms / 1e3), 2),
            "kv_read_bytes_total": kv_bytes,
            "kv_read_gbps": round(kv_bytes / (total_ms / 1e3) / 1e9, 1),
            "kv_read_frac_of_peak": round(kv_bytes / (total_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "launch": "hwkv_decode_append_attn per step: appending split + merge for all 48 "
                      "layers and 32 sequences",
            "roofline": {"bound": "hbm", "kernel": "decode_split_kernel<bf16, d128, G3, append>",
                         "achieved": round(split_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(split_gbps / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic(lay.desc().split_tokens, "cb"),
                         "traffic_source": "committed rocprofv3 --pmc counters (FETCH_SIZE, "
                                           "WRITE_SIZE per dispatch, scaled by the probe copy "
                                           "of known size) in profiles/"
                                           "decode_split_cb_counters.json; reported only while "
                                           "the kernel source hash and split length match "
                                           "(else null)",
                         "avg_launch_ms": round(split_ms, 4),
                         "algorithmic_bytes_per_launch": roof_bytes / n_roof,
                         "avg_launch_timing": "HIP events around each split launch, %d steps "
                                              "after the timed ones" % n_roof},
            "fill_seconds": round(t_fill, 1)}


def gemm_reference_tflops(torch, n=16384, reps=5):
    """Practical bf16 matrix-core rate on this machine: a plain n x n x n bf16
    GEMM from the vendor library (torch.matmul), timed with HIP events.  A
    reference point for the prefill's MFMA fraction (the way the streaming
    read probe is one for decode), not part of the measured path."""
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(2):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return 2.0 * n ** 3 / (ms / 1e3) / 1e12


def prefill_leg(H, torch, synth):
    """Chunked prefill at 161K context: 4 sequences, 8 KV heads x 3, d=128,
    bf16, windows of the printed policy's layer 0 (4096 x2, 16384 x2, 65536
    x4), one 2048-token chunk at P = 164,864; then the chunk is appended and
    128 decode steps follow.  Prefill attention is timed alone (it only reads
    the cache, so replays are identical); the append and the decode steps
    are timed separately."""
    import numpy as np
    dev = torch.device("cuda", 0)
    n_seqs, n_kv, G, d, n = 4, 8, 3, 128, 2048
    P = synth.CTX_161K
    w = np.array([synth.YAML_LAYER0], np.int32)
    lay = H.hwkv_layout_create(w, 16, d, torch.bfloat16)
    cache = H.make_cache(lay, n_seqs, device=dev)
    cap = int(((w.astype(np.int64) + 15) // 16 * 16).max())
    for b in range(n_seqs):  # history: the last `cap` positions before P
        g = synth.gen(105 * 100003 + b, dev)
        kh = synth.randn((1, 1, cap, n_kv, d), torch.bfloat16, g)
        vh = synth.randn((1, 1, cap, n_kv, d), torch.bfloat16, g)
        H.hwkv_append(cache, 0, 1, torch.tensor([P - cap], device=dev), kh, vh,
                      seq_slots=torch.tensor([b], dtype=torch.int32, device=dev))
        del kh, vh
    g = synth.gen(106, dev)
    q = synth.randn((n_seqs, n, n_kv * G, d), torch.bfloat16, g, std=1.0 / math.sqrt(d))
    k = synth.randn((n_seqs, n, n_kv, d), torch.bfloat16, g)
    v = synth.randn((n_seqs, n, n_kv, d), torch.bfloat16, g)
    out = torch.empty((n_seqs, n, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    pos = torch.full((n_seqs,), P, dtype=torch.int64, device=dev)
    scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream()
    # the default entry's workspace: the fp16 copy of the V rows it reads
    pws = H.make_prefill_workspace(lay, 0, n_seqs, n, device=dev)
    pws_bytes = int(pws.numel())

    def fast(*a):
        H.hwkv_prefill_attn(*a[:6], pws, *a[6:])

    def median_ms(fn, reps=10):
        for _ in range(2):
            fn(cache, 0, pos, q, k, v, out, scale)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn(cache, 0, pos, q, k, v, out, scale)
            e1.record(s)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]
    # P in fp16 (the default entry) and P split into two bf16 products
    exact_ms = median_ms(H.hwkv_prefill_attn_exact, 5)
    pf_ms = median_ms(fast)
    # algorithmic flops: per query row and query head, 4 d flops per key in
    # its window [p-w+1, p] (QK^T and PV, 2 flops per multiply-add)
    keys = 0
    for wh in w[0]:
        for r in range(n):
            keys += min(int(wh), P + r + 1)
    flop = 4.0 * d * G * keys * n_seqs
    # the chunk append: the first call writes the chunk (timed alone, with its
    # one-off host costs); repeats write the same bytes to the same slots.
    # Each repeat is queued behind a short spin kernel that holds the stream
    # while the host enqueues the first event, the call and the second event,
    # so the event pair brackets the GPU work alone (the call's host work
    # takes longer than its kernel)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    H.hwkv_append(cache, 0, 1, pos, k[None], v[None])
    e1.record(s)
    torch.cuda.synchronize()
    append_first_ms = e0.elapsed_time(e1)
    append_ts = []
    spin = getattr(torch.cuda, "_sleep", None)  # torch's spin kernel (bounded by a cycle count)
    for _ in range(12):
        if spin is not None:
            spin(2_000_000)
        e0.record(s)
        H.hwkv_append(cache, 0, 1, pos, k[None], v[None])
        e1.record(s)
        torch.cuda.synchronize()
        append_ts.append(e0.elapsed_time(e1))
    append_ms = sorted(append_ts[2:])[5]
    # every chunk token is read and written (the chunk is shorter than every window)
    assert n <= int(w.min())
    append_bytes = 2.0 * n_seqs * n * n_kv * KV_BYTES_PER_TOK_HEAD
    # 128 decode steps after the chunk (two untimed ones first: the first
    # calls after the prefill carry one-off host and launch costs)
    n_dec, n_warm = 128, 2
    kd = synth.randn((n_warm + n_dec, 1, n_seqs, 1, n_kv, d), torch.bfloat16, g)
    vd = synth.randn((n_warm + n_dec, 1, n_seqs, 1, n_kv, d), torch.bfloat16, g)
    qd = synth.randn((n_warm + n_dec, 1, n_seqs, n_kv * G, d), torch.bfloat16, g,
                     std=1.0 / math.sqrt(d))
    posd = [torch.full((n_seqs,), P + n + i, dtype=torch.int64, device=dev)
            for i in range(n_warm + n_dec)]
    ws = H.make_workspace(lay, 0, 1, n_seqs, n_kv * G, device=dev)
    od = torch.empty((1, n_seqs, n_kv * G, d), dtype=torch.bfloat16, device=dev)

    def dec_step(i):  # the appending split (it writes the new token) + the merge
        H.hwkv_decode_append_attn(cache, 0, 1, posd[i], kd[i], vd[i], qd[i], scale, ws, od)
    for i in range(n_warm):
        dec_step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(n_warm, n_warm + n_dec):
        dec_step(i)
    e1.record(s)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / n_dec
    dec_bytes = float(np.minimum(w.astype(np.int64), P + n + n_warm).sum()) * n_seqs * \
        KV_BYTES_PER_TOK_HEAD
    del cache, pws
    torch.cuda.empty_cache()
    gemm_tf = gemm_reference_tflops(torch)
    return {"workload": "4 seqs x 1 layer, 2048-token chunk at P=164864, windows 4096x2/16384x2/"
                        "65536x4, 8x3 heads, d=128, bf16",
            "prefill_ms": round(pf_ms, 4), "prefill_flop": flop,
            "prefill_tflops": round(flop / (pf_ms / 1e3) / 1e12, 1),
            "mfma_frac_of_bf16_peak": round(flop / (pf_ms / 1e3) / 2.5e15, 4),
            "gemm_reference_tflops": round(gemm_tf, 1),
            "frac_of_gemm_reference": round(flop / (pf_ms / 1e3) / 1e12 / gemm_tf, 4),
            "prefill_tokens_per_s": round(n_seqs * n / (pf_ms / 1e3), 1),
            "p_in_pv_product": "fp16 (V copied to fp16 by a pre-pass; exact re-run of rows out "
                               "of range)",
            "prefill_workspace_bytes": pws_bytes,
            "prefill_exact_ms": round(exact_ms, 4),
            "prefill_exact_tflops": round(flop / (exact_ms / 1e3) / 1e12, 1),
            "chunk_append_ms": round(append_ms, 4),
            "chunk_append_first_call_ms": round(append_first_ms, 4),
            "chunk_append_gbps": round(append_bytes / (append_ms / 1e3) / 1e9, 1),
            "chunk_append_timing": ("median of 10 repeats, each queued behind a spin kernel so "
                                    "that the events bracket GPU time only") if spin is not None
                                   else "median of 10 repeats (events include the call's host work)",
            "decode_step_ms": round(dec_ms, 4),
            "decode_tokens_per_s": round(n_seqs / (dec_ms / 1e3), 1),
            "decode_kv_read_gbps": round(dec_bytes / (dec_ms / 1e3) / 1e9, 1),
            "decode_steps": n_dec,
            "decode_launch": "hwkv_decode_append_attn: appending split + merge per step"}


def per_layer_graph(H, torch, cache, lay, windows, q, k_new, v_new, L, n_seqs, n_kv, G, d,
                    step_bytes, mode="three_launches"):
    """The model-realistic launch pattern: per layer append -> split -> merge
    (each layer's q only exists after the previous layer), 144 launches
    captured once in a HIP graph and replayed; positions live in device
    scalars updated by a fill kernel outside the graph.  mode
    "append_in_split": hwkv_decode_append_attn per layer (96 launches);
    "single_launch": hwkv_decode_step per layer (48 launches).  `lay` may
    differ from the cache's layout in its decode split length only (same
    windows, so the same pool geometry); its own meta blob is used."""
    dev = q.device
    n_layers = windows.shape[0]
    if lay is not cache.layout:
        meta_host = H.hwkv_meta_fill(lay)
        meta = H._alloc_aligned(meta_host.size, dev)
        meta.copy_(torch.from_numpy(meta_host))
        cache = H.Cache(lay, cache.pool, cache.block_ids, meta,
                        H.hwkv_meta_fingerprint(meta_host))
    pos = torch.full((n_seqs,), L, dtype=torch.int64, device=dev)
    ctx = torch.full((n_seqs,), L + 1, dtype=torch.int64, device=dev)
    mk = H.make_step_workspace if mode == "single_launch" else H.make_workspace
    wss = [mk(lay, l, 1, n_seqs, n_kv * G, device=dev) for l in range(n_layers)]
    out = torch.empty((n_layers, n_seqs, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    kn = k_new[0].clone()
    vn = v_new[0].clone()
    qs = [q[l:l + 1].contiguous() for l in range(n_layers)]
    kns = [kn[l:l + 1].contiguous() for l in range(n_layers)]
    vns = [vn[l:l + 1].contiguous() for l in range(n_layers)]
    outs = [out[l:l + 1] for l in range(n_layers)]
    scale = 1.0 / math.sqrt(d)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    def layer_step(l):
        if mode == "single_launch":
            H.hwkv_decode_step(cache, l, 1, pos, kns[l], vns[l], qs[l], scale, wss[l], outs[l])
        elif mode == "append_in_split":
            H.hwkv_decode_append_attn(cache, l, 1, pos, kns[l], vns[l], qs[l], scale, wss[l],
                                      outs[l])
        else:
            H.hwkv_append(cache, l, 1, pos, kns[l], vns[l])
            H.hwkv_decode_attn(cache, l, 1, ctx, qs[l], scale, wss[l], outs[l])

    with torch.cuda.stream(side):
        for l in range(n_layers):  # warm the launch path once, eagerly
            layer_step(l)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for l in range(n_layers):
                layer_step(l)
    torch.cuda.synchronize()
    n_rep = 20
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(n_rep + 3):
        pos.fill_(L + 1 + i)
        ctx.fill_(L + 2 + i)
        e0.record(s)
        graph.replay()
        e1.record(s)
        torch.cuda.synchronize()
        if i >= 3:
            times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    b = step_bytes(L + 2)
    return {"ms_per_step_median": round(ms, 4), "tokens_per_s": round(n_seqs / (ms / 1e3), 2),
            "kv_read_gbps": round(b / (ms / 1e3) / 1e9, 1),
            "launches_per_step": {"single_launch": 1, "append_in_split": 2}.get(mode, 3) * n_layers,
            "replays": n_rep,
            "split_tokens": lay.desc().split_tokens}


def stack_decode_time(H, torch, synth, windows, dtype, block_size, L0, steps=20, n_warm=10,
                      seed=0, G=3, d=128):
    """One decode step per call over a whole stack (batch 1): the appending
    split + merge for all layers (hwkv_decode_append_attn, bf16 outputs),
    after filling each layer with the last min(L0, capacity) positions of
    N(0,1) history; `n_warm` untimed steps, then `steps` timed as one block.
    G query heads per KV head, head_dim d."""
    import numpy as np
    dev = torch.device("cuda", 0)
    windows = np.asarray(windows, np.int32)
    n_layers, n_kv = windows.shape
    lay = H.hwkv_layout_create(windows, block_size, d, dtype)
    cache = H.make_cache(lay, 1, device=dev)
    cap = int(((windows.astype(np.int64) + block_size - 1) // block_size * block_size).max())
    n_hist = min(L0, cap)
    pos_hist = torch.full((1,), L0 - n_hist, dtype=torch.int64, device=dev)
    for l in range(n_layers):
        g = synth.gen(seed * 100003 + l, dev)
        k = synth.randn((1, 1, n_hist, n_kv, d), dtype, g)
        v = synth.randn((1, 1, n_hist, n_kv, d), dtype, g)
        H.hwkv_append(cache, l, 1, pos_hist, k, v)
        del k, v
    g = synth.gen(seed + 1, dev)
    n = steps + n_warm
    q = synth.randn((n_layers, 1, n_kv * G, d), dtype, g, std=1.0 / math.sqrt(d))
    kn = synth.randn((n, n_layers, 1, 1, n_kv, d), dtype, g)
    vn = synth.randn((n, n_layers, 1, 1, n_kv, d), dtype, g)
    pos = [torch.full((1,), L0 + i, dtype=torch.int64, device=dev) for i in range(n)]
    ws = H.make_workspace(lay, 0, n_layers, 1, n_kv * G, device=dev)
    out = torch.empty((n_layers, 1, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / math.sqrt(d)
    for i in range(n_warm):
        H.hwkv_decode_append_attn(cache, 0, n_layers, pos[i], kn[i], vn[i], q, scale, ws, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_warm, n):
        H.hwkv_decode_append_attn(cache, 0, n_layers, pos[i], kn[i], vn[i], q, scale, ws, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    b = float(np.minimum(windows.astype(np.int64), L0 + n_warm + steps // 2).sum()) * 4 * d
    del cache, ws
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(1.0 / (ms / 1e3), 1),
            "kv_read_bytes_per_step": b, "kv_read_gbps": round(b / (ms / 1e3) / 1e9, 1),
            "kv_read_frac_of_peak": round(b / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "steps": steps, "split_tokens": lay.desc().split_tokens}


def prefill_time(H, torch, synth, d, reps=10):
    """hwkv_prefill_attn alone on the 161K chunk of prefill_leg (4 sequences,
    8 KV x 3 heads, bf16, printed layer-0 windows, 2048-token chunk at
    P = 164,864) at head dimension d."""
    import numpy as np
    dev = torch.device("cuda", 0)
    n_seqs, n_kv, G, n = 4, 8, 3, 2048
    P = synth.CTX_161K
    w = np.array([synth.YAML_LAYER0], np.int32)
    lay = H.hwkv_layout_create(w, 16, d, torch.bfloat16)
    cache = H.make_cache(lay, n_seqs, device=dev)
    cap = int(((w.astype(np.int64) + 15) // 16 * 16).max())
    for b in range(n_seqs):
        g = synth.gen(105 * 100003 + b, dev)
        kh = synth.randn((1, 1, cap, n_kv, d), torch.bfloat16, g)
        vh = synth.randn((1, 1, cap, n_kv, d), torch.bfloat16, g)
        H.hwkv_append(cache, 0, 1, torch.tensor([P - cap], device=dev), kh, vh,
                      seq_slots=torch.tensor([b], dtype=torch.int32, device=dev))
        del kh, vh
    g = synth.gen(106, dev)
    q = synth.randn((n_seqs, n, n_kv * G, d), torch.bfloat16, g, std=1.0 / math.sqrt(d))
    k = synth.randn((n_seqs, n, n_kv, d), torch.bfloat16, g)
    v = synth.randn((n_seqs, n, n_kv, d), torch.bfloat16, g)
    out = torch.empty((n_seqs, n, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    pos = torch.full((n_seqs,), P, dtype=torch.int64, device=dev)
    pws = H.make_prefill_workspace(lay, 0, n_seqs, n, device=dev)
    for _ in range(2):
        H.hwkv_prefill_attn(cache, 0, pos, q, k, v, pws, out, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        H.hwkv_prefill_attn(cache, 0, pos, q, k, v, pws, out, 1.0 / math.sqrt(d))
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts)[len(ts) // 2]
    keys = sum(min(int(wh), P + r + 1) for wh in w[0] for r in range(n))
    flop = 4.0 * d * G * keys * n_seqs
    del cache, pws
    torch.cuda.empty_cache()
    return {"head_dim": d, "prefill_ms": round(ms, 4), "prefill_flop": flop,
            "prefill_tflops": round(flop / (ms / 1e3) / 1e12, 1),
            "mfma_frac_of_bf16_peak": round(flop / (ms / 1e3) / 2.5e15, 4)}


def mixed_leg(H, torch, synth):
    """Mixed stacks through the same entry points (the 48-layer stacks at
    context 112K, batch 1, one appending split + merge per step for all
    layers): the headline's windows on an fp16 cache in 64-token blocks, and
    a hybrid stack of sliding-window layers (every head 4096 tokens) with
    every fourth layer a per-head global layer; then the 161K chunked prefill
    at head_dim 256."""
    L0 = synth.CTX_112K
    res = {"stack48_f16_block64": stack_decode_time(
               H, torch, synth, synth.stack_windows(48, 8, 0), torch.float16, 64, L0, seed=111),
           "hybrid48_swa4096_every4th_global": stack_decode_time(
               H, torch, synth, synth.hybrid_windows(48, 8, 4096, 4, 0), torch.bfloat16, 16, L0,
               seed=112),
           "prefill_161k_head_dim256": prefill_time(H, torch, synth, 256)}
    res["stack48_f16_block64"]["workload"] = (
        "48 layers x 8x3 heads, d=128, fp16, block size 64, windows of the headline (seed 0), "
        "context 112K, batch 1")
    res["hybrid48_swa4096_every4th_global"]["workload"] = (
        "48 layers x 8x3 heads, d=128, bf16, bs 16: layers 3, 7, ..., 47 per-head windows of the "
        "headline draw, all others every head 4096 (sliding window), context 112K, batch 1")
    res["prefill_161k_head_dim256"]["workload"] = (
        "the 161K chunk of prefill_161k (4 seqs, 2048 rows at P=164864, layer-0 windows, 8x3 "
        "heads, bf16) at head_dim 256")
    return res


def gqa_leg(H, torch, synth):
    """The headline's 48-layer stack (windows of seed 0, context 112K,
    batch 1, bf16, 16-token blocks) with larger GQA groups: 8 query heads
    per KV head at head_dim 128 and 256, 4 at head_dim 128."""
    L0 = synth.CTX_112K
    res = {}
    for G, d in ((4, 128), (8, 128), (8, 256)):
        r = stack_decode_time(H, torch, synth, synth.stack_windows(48, 8, 0), torch.bfloat16, 16,
                              L0, seed=113, G=G, d=d)
        r["workload"] = ("48 layers x 8 KV heads x %d query heads each, d=%d, bf16, windows of "
                         "the headline (seed 0), context 112K, batch 1" % (G, d))
        res["stack48_g%d_d%d" % (G, d)] = r
    return res


def single_layer_leg(H, torch, synth, steps=50, split_tokens=0):
    """One global layer at batch 8: 8 KV heads x 3, d=128, bf16, windows of
    the printed policy's layer 0 (4096 x2, 16384 x2, 65536 x4), context
    32,768 per sequence (so the 64K heads read all 32,768 tokens).  A step
    appends each sequence's new token and attends (appending split + merge,
    two launches); contexts advance by one per step; 10 untimed steps, then
    `steps` timed ones."""
    import numpy as np
    dev = torch.device("cuda", 0)
    n_seqs, n_kv, G, d, L0 = 8, 8, 3, 128, 32768
    w = np.array([synth.YAML_LAYER0], np.int32)
    lay = H.hwkv_layout_create(w, 16, d, torch.bfloat16, split_tokens)
    cache = H.make_cache(lay, n_seqs, device=dev)
    g = synth.gen(102, dev)
    for b in range(n_seqs):
        kh = synth.randn((1, 1, L0, n_kv, d), torch.bfloat16, g)
        vh = synth.randn((1, 1, L0, n_kv, d), torch.bfloat16, g)
        H.hwkv_append(cache, 0, 1, torch.tensor([0], device=dev), kh, vh,
                      seq_slots=torch.tensor([b], dtype=torch.int32, device=dev))
        del kh, vh
    q = synth.randn((1, n_seqs, n_kv * G, d), torch.bfloat16, g, std=1.0 / math.sqrt(d))
    n_warm = 10
    kn = synth.randn((steps + n_warm, 1, n_seqs, n_kv, d), torch.bfloat16, g)
    vn = synth.randn((steps + n_warm, 1, n_seqs, n_kv, d), torch.bfloat16, g)
    pos = [torch.full((n_seqs,), L0 + i, dtype=torch.int64, device=dev)
           for i in range(steps + n_warm)]
    ws = H.make_workspace(lay, 0, 1, n_seqs, n_kv * G, device=dev)
    out = torch.empty((1, n_seqs, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream()
    for i in range(n_warm):
        H.hwkv_decode_append_attn(cache, 0, 1, pos[i], kn[i], vn[i], q, scale, ws, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(n_warm, steps + n_warm):
        H.hwkv_decode_append_attn(cache, 0, 1, pos[i], kn[i], vn[i], q, scale, ws, out)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tok_heads = float(np.minimum(w.astype(np.int64), L0 + n_warm + steps // 2).sum()) * n_seqs
    b = tok_heads * KV_BYTES_PER_TOK_HEAD
    return {"workload": "1 layer, 8 seqs at context 32768, windows 4096x2/16384x2/65536x4, "
                        "8x3 heads, d=128, bf16",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(n_seqs / (ms / 1e3), 1),
            "kv_read_bytes_per_step": b, "kv_read_gbps": round(b / (ms / 1e3) / 1e9, 1),
            "kv_read_frac_of_peak": round(b / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "launches_per_step": 2, "steps": steps, "split_tokens": lay.desc().split_tokens}


def three_launch_leg(H, torch, cache, q, k_new, v_new, L, n_seqs, steps, step_bytes, scale, ws,
                     out):
    """The step as three launches for all 48 layers: hwkv_append of the new
    token, then hwkv_decode_attn (split + merge)."""
    dev = q.device
    n_layers = q.shape[0]
    pos = [torch.full((n_seqs,), L + i, dtype=torch.int64, device=dev) for i in range(steps + 3)]
    ctx = [p + 1 for p in pos]
    s = torch.cuda.current_stream()

    def step(i):
        H.hwkv_append(cache, 0, n_layers, pos[i], k_new[i % len(k_new)], v_new[i % len(v_new)])
        H.hwkv_decode_attn(cache, 0, n_layers, ctx[i], q, scale, ws, out)
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(steps):
        step(3 + i)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    b = step_bytes(L + 3)
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(n_seqs / (ms / 1e3), 2),
            "kv_read_gbps": round(b / (ms / 1e3) / 1e9, 1),
            "kv_read_frac_of_peak": round(b / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "launches_per_step": 3, "steps": steps}


def fused_leg(H, torch, cache, lay, q, k_new, v_new, L, n_seqs, n_kv, G, d, steps, step_bytes,
              two_launch=False):
    """The same decode step as one hwkv_decode_step launch for all 48 layers
    (append, split and merge fused), or, with two_launch, as
    hwkv_decode_append_attn (the split stage appends, then the merge), timed
    with HIP events over `steps` consecutive steps that continue the token
    stream."""
    dev = q.device
    n_layers = q.shape[0]
    mk = H.make_workspace if two_launch else H.make_step_workspace
    fn = H.hwkv_decode_append_attn if two_launch else H.hwkv_decode_step
    ws = mk(lay, 0, n_layers, n_seqs, n_kv * G, device=dev)
    out = torch.empty((n_layers, n_seqs, n_kv * G, d), dtype=torch.bfloat16, device=dev)
    pos = [torch.full((n_seqs,), L + i, dtype=torch.int64, device=dev) for i in range(steps + 3)]
    scale = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream()
    for i in range(3):
        fn(cache, 0, n_layers, pos[i], k_new[i % len(k_new)], v_new[i % len(v_new)], q, scale,
           ws, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(steps):
        fn(cache, 0, n_layers, pos[3 + i], k_new[i % len(k_new)], v_new[i % len(v_new)], q,
           scale, ws, out)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    b = step_bytes(L + 3)
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(n_seqs / (ms / 1e3), 2),
            "kv_read_gbps": round(b / (ms / 1e3) / 1e9, 1),
            "kv_read_frac_of_peak": round(b / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "launches_per_step": 2 if two_launch else 1, "steps": steps}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(windows, L, n_kv, G, d, target_s, gpu_tok_s, gpu_prefill=None):
    """The fp64 oracle, as it is, on the host cores.

    - All threads: one decode step of the whole 48-layer stack, each layer's
      oracle call repeated until the layers together have taken about
      target_s; the step time is the sum over layers of the mean call time.
    - One thread: the same calls, layer by layer until ~target_s / 2 has
      passed, the step time extrapolated by K/V bytes (labelled).
    - The 161K chunked prefill: 16 evenly spaced chunk rows of each
      (sequence, kv head) on all threads, extrapolated by the row count to
      the 2048-row chunk (labelled).
    - The continuous batch: the all-thread step time scaled by the batch's
      K/V bytes per step (labelled)."""
    import numpy as np
    import torch

    import oracle
    import synth

    n_layers = windows.shape[0]
    threads = oracle.threads()
    total_bytes = float(np.minimum(windows.astype(np.int64), L).sum()) * KV_BYTES_PER_TOK_HEAD
    layer_bytes = np.minimum(windows.astype(np.int64), L).sum(axis=1) * KV_BYTES_PER_TOK_HEAD
    inputs = {}

    def layer_inputs(l):
        if l not in inputs:
            W = int(windows[l].max())
            g = synth.gen(9000 + l)
            q = synth.randn((1, 1, n_kv * G, d), torch.bfloat16, g, std=1.0 / math.sqrt(d))
            k = synth.randn((1, 1, W, n_kv, d), torch.bfloat16, g)
            v = synth.randn((1, 1, W, n_kv, d), torch.bfloat16, g)
            inputs[l] = (W, synth.to_raw(q), synth.to_raw(k), synth.to_raw(v))
        return inputs[l]

    def call(l):
        W, qr, kr, vr = layer_inputs(l)
        t = time.time()
        oracle.decode(windows[l:l + 1], [L], qr, kr, vr, [L - W], 1.0 / math.sqrt(d))
        return time.time() - t

    spent = step_s = 0.0
    calls = 0
    per_layer_s = target_s / n_layers
    for l in range(n_layers):
        layer_s, reps = 0.0, 0
        while reps == 0 or layer_s < per_layer_s:
            layer_s += call(l)
            reps += 1
        spent += layer_s
        step_s += layer_s / reps
        calls += reps
        inputs.pop(l, None)
    res = {"value": round(1.0 / step_s, 4), "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": "the full 48-layer decode step (%.2f GB of K/V), %d oracle calls of one "
                     "layer each on %d threads, %.1f s in total; step time = sum over layers "
                     "of the mean call time" % (total_bytes / 1e9, calls, threads, spent),
           "host_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
           "kv_read_gbps": round(total_bytes / step_s / 1e9, 3),
           "gpu_over_cpu": round(gpu_tok_s * step_s, 1)}

    # one thread: layers in order until about half the budget is spent
    oracle.set_threads(1)
    try:
        t1, b1, used = 0.0, 0.0, 0
        for l in range(n_layers):
            t1 += call(l)
            b1 += float(layer_bytes[l])
            used += 1
            inputs.pop(l, None)
            if t1 >= target_s / 2:
                break
    finally:
        oracle.set_threads(threads)
    step_1t = t1 * total_bytes / b1
    res["one_thread"] = {"tokens_per_s": round(1.0 / step_1t, 5),
                         "step_s_extrapolated": round(step_1t, 2),
                         "sample": "layers 0-%d of the step (%.2f of %.2f GB) on 1 thread in "
                                   "%.1f s, extrapolated by K/V bytes" %
                                   (used - 1, b1 / 1e9, total_bytes / 1e9, t1)}

    # the 161K chunked prefill on sampled rows
    n_seqs, n, P = 4, 2048, synth.CTX_161K
    wl = np.array(synth.YAML_LAYER0, np.int32)
    cap = int(((wl.astype(np.int64) + 15) // 16 * 16).max())
    g = synth.gen(9100)
    dev = torch.device("cuda", 0) if torch.cuda.is_available() else torch.device("cpu")
    gd = synth.gen(9100, dev)
    kh = synth.to_raw(synth.randn((n_seqs, cap, n_kv, d), torch.bfloat16, gd))
    vh = synth.to_raw(synth.randn((n_seqs, cap, n_kv, d), torch.bfloat16, gd))
    qc = synth.to_raw(synth.randn((n_seqs, n, n_kv * G, d), torch.bfloat16, g,
                                  std=1.0 / math.sqrt(d)))
    kc = synth.to_raw(synth.randn((n_seqs, n, n_kv, d), torch.bfloat16, g))
    vc = synth.to_raw(synth.randn((n_seqs, n, n_kv, d), torch.bfloat16, g))
    rows = np.linspace(0, n - 1, 16).astype(np.int64)
    t = time.time()
    oracle.prefill(wl, [P] * n_seqs, qc, kc, vc, kh, vh, [P - cap] * n_seqs,
                   1.0 / math.sqrt(d), rows=rows)
    t_rows = time.time() - t
    chunk_s = t_rows * n / rows.size
    pf = {"chunk_step_s_extrapolated": round(chunk_s, 2),
          "tokens_per_s": round(n_seqs * n / chunk_s, 2),
          "sample": "16 evenly spaced rows of the 2048-row chunk, all 4 sequences and 24 "
                    "query heads, on %d threads in %.1f s, extrapolated by the row count"
                    % (threads, t_rows)}
    if gpu_prefill:
        pf["gpu_over_cpu"] = round(chunk_s / (gpu_prefill["prefill_ms"] / 1e3), 1)
    res["prefill_161k"] = pf
    del kh, vh, qc, kc, vc

    # the continuous batch: same 48-layer stack, 32 contexts in [4K, 160K]
    Lcb = synth.cb_contexts()
    w64 = windows.astype(np.int64).reshape(-1)
    cb_bytes = float(np.minimum(w64[None, :], Lcb[:, None]).sum()) * KV_BYTES_PER_TOK_HEAD
    cb_step_s = step_s * cb_bytes / total_bytes
    res["continuous_batch"] = {"tokens_per_s": round(len(Lcb) / cb_step_s, 4),
                               "sample": "extrapolated from the all-thread 48-layer step by K/V "
                                         "bytes per step (%.1f GB)" % (cb_bytes / 1e9)}
    return res


if __name__ == "__main__":
    main()
