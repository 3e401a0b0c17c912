#!/usr/bin/env python3
"""Decode-step benchmark of the LoopKV quantized decode path on one MI355X.

A step is one decode pass over every (loop, layer) cell of the workload's
plan for the whole batch (after appending the step's new token to every
stored cell when the workload appends).  Inputs are resident in HBM before
timing starts.  Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload lean-16k]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lean-16k")
    ap.add_argument("--tau", type=float, default=None, help="one tau for every cell (sweeps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-samples", type=int, default=8, help="(cell, sequence) oracle samples")
    ap.add_argument("--report", default=None, help="also write a detailed JSON report here")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from loop_aware_quantized_amd import abi, runner
    from loop_aware_quantized_amd import inputs as wl

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    abi.lib()  # fail loudly if the HIP library is missing

    w = wl.WORKLOADS[args.workload]
    kinds, taus = wl.make_plan(w)
    if args.tau is not None:
        taus = wl.with_tau(taus, args.tau)
    n_steps = args.warmup + args.steps + 2
    extra = w.append_tokens * n_steps
    t_setup = time.time()
    st = runner.CacheState(w, dev, kinds, taus, extra_tokens=extra)
    R, L, B, H, D = w.loops, w.layers, w.batch, w.heads, w.head_dim
    log(f"[bench] {w.name}: B={B} R={R} L={L} H={H} D={D} P={w.page} stored cells={len(st.stored)} "
        f"pool pages={st.num_pages}")
    for i, (r, l) in enumerate(st.stored):
        st.prefill_cell(r, l)
        if i % 8 == 7:
            torch.cuda.synchronize()
            log(f"[bench] prefilled {i + 1}/{len(st.stored)} cells ({time.time() - t_setup:.1f} s)")
    torch.cuda.synchronize()
    queries = {(r, l): wl.cell_query(w, st.cell_index(r, l), dev)[1]
               for r in range(R) for l in range(L)}
    new_kv = {}
    if w.append_tokens:
        for (r, l) in st.stored:
            new_kv[(r, l)] = wl.append_kv(w, st.cell_index(r, l), 0, w.append_tokens, dev)
    lens0 = st.lens0.astype(np.int64)
    lens_dev = [torch.from_numpy((lens0 + s * w.append_tokens).astype(np.int32)).to(dev)
                for s in range(n_steps + 1)]
    out = torch.empty(B, H, D, dtype=torch.float32, device=dev)
    opts = abi.make_opts(st.workspace)
    cells_order = [(r, l) for r in range(R) for l in range(L)]
    batches = [st.batch(lens_dev[s]) for s in range(n_steps + 1)]
    log(f"[bench] setup {time.time() - t_setup:.1f} s")

    step_idx = [0]

    def step(counters=None):
        s = step_idx[0]
        if w.append_tokens:
            app = abi.make_batch(lens_dev[s], st.block_tables, st.max_seq_len)
            for (r, l) in st.stored:
                k, v = new_kv[(r, l)]
                abi.loopkv_append(st.plan, st.cells, r, l, app, w.append_tokens, k, v)
        bt = batches[s + 1] if w.append_tokens else batches[0]
        o = opts if counters is None else abi.make_opts(st.workspace, counters=counters)
        for (r, l) in cells_order:
            abi.loopkv_decode(st.plan, st.cells, r, l, bt, queries[(r, l)], out, o)
        step_idx[0] += 1

    def lens_of_step(s):
        return lens0 + (s + 1) * w.append_tokens if w.append_tokens else lens0

    # ---- warmup, then timed steps (whole-step events)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    first_timed = step_idx[0]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step")

    # ---- per-kernel pass: library events around every launch of one step
    abi.loopkv_profile_enable(True)
    for c in (abi.KERNEL_SPLIT, abi.KERNEL_MERGE, abi.KERNEL_APPEND):
        abi.loopkv_profile_collect(c)
    prof_step = step_idx[0]
    step()
    torch.cuda.synchronize()
    kstats = {name: abi.loopkv_profile_collect(c) for name, c in
              (("split", abi.KERNEL_SPLIT), ("merge", abi.KERNEL_MERGE), ("append", abi.KERNEL_APPEND))}
    abi.loopkv_profile_enable(False)

    # ---- counters pass: flagged token-heads (low-plane bytes actually read)
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    cnt_step = step_idx[0]
    step(counters=cnt)
    torch.cuda.synchronize()
    flagged, lo_bytes = (int(x) for x in cnt.cpu().tolist())

    # ---- byte accounting (plan-required bytes, counted once)
    def src_kind(r, l):
        return int(kinds[R - 1, l]) if kinds[r, l] == wl.KIND_REUSE else int(kinds[r, l])

    def split_bytes(lens):
        tok = int(lens.sum())
        tot = 0
        for (r, l) in cells_order:
            per = runner.required_bytes_per_token_head(src_kind(r, l), D)
            if src_kind(r, l) == wl.KIND_Q4 and taus[r, l] == 0.0:
                per += D // 4     # tau = 0: every low-plane row is required
            tot += tok * H * per
        return tot

    pages = int(((lens_of_step(first_timed) + w.page - 1) // w.page).sum())
    per_cell_fixed = B * H * (2 * D + 4 * D) + 4 * pages          # q, out, page tables
    timed_tokens = sum(int(lens_of_step(s).sum()) for s in range(first_timed, first_timed + args.steps))
    kv_tokens = timed_tokens * R * L
    value = kv_tokens / (total_ms / 1e3)
    lens_t = lens_of_step(first_timed)
    # lo_bytes: low-plane rows fetched in one full step (counters, all cells and heads)
    step_bytes = split_bytes(lens_t) + lo_bytes + R * L * per_cell_fixed
    step_gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    lens_p = lens_of_step(prof_step)
    n_split, split_ms = kstats["split"]
    split_alg = split_bytes(lens_p)
    achieved = split_alg / (split_ms / 1e3) / 1e9 if split_ms > 0 else 0.0
    stored_bytes = sum(st.plan.pool_bytes(r, l, st.num_pages) for (r, l) in st.stored)
    q4_cells = [c for c in st.stored if kinds[c] == wl.KIND_Q4]
    all_q4_bytes = (len(cells_order) * st.plan.pool_bytes(*q4_cells[0], st.num_pages)
                    if q4_cells else None)

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, st, kinds, taus, args.cpu_samples, dev)

    res = {
        "metric": "decode-attn KV tokens/s + achieved HBM GB/s vs peak, Ouro-1.4B shape, 16K ctx",
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) bf16 K/V with outlier channels and heavy tokens)",
        "config": {"workload": w.name, "batch": B, "loops": R, "layers": L, "heads": H,
                   "head_dim": D, "page": w.page, "context": int(lens_t.max()),
                   "tau": "per-cell plan" if args.tau is None else args.tau,
                   "append_tokens_per_step": w.append_tokens},
        "hbm_gbs_required": step_gbs,
        "hbm_frac_required": step_gbs / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None, "launches": n_split,
                     "avg_launch_us": split_ms * 1e3 / max(n_split, 1),
                     "alg_bytes_per_launch": split_alg / max(n_split, 1)},
        "kernels_ms_per_step": {k: v[1] for k, v in kstats.items()},
        "lo_plane": {"flagged_token_heads": flagged, "lo_bytes_read": lo_bytes,
                     "lo_bytes_stored_q4_sources": int(sum(
                         int(lens_of_step(cnt_step).sum()) * H * D // 4
                         for (r, l) in cells_order if src_kind(r, l) == wl.KIND_Q4))},
        "storage": {"stored_bytes": stored_bytes, "all_4bit_bytes": all_q4_bytes},
        "cpu_baseline": cpu,
    }
    if args.report:
        with open(args.report, "w") as f:
            json.dump(res, f, indent=2)
    print(json.dumps(res), flush=True)


def cpu_baseline(w, st, kinds, taus, n_samples, dev):
    """Time oracle.attention.decode on (cell, sequence) samples (cache build excluded)."""
    import oracle.attention as oa
    import oracle.cache as oc
    from loop_aware_quantized_amd import inputs as wl
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    R, L = w.loops, w.layers
    rng = np.random.default_rng(12345)
    # cover 4-bit, 2-bit, reuse->4-bit and reuse->2-bit cells
    groups = {}
    for r in range(R):
        for l in range(L):
            k = int(kinds[r, l])
            src = int(kinds[R - 1, l]) if k == wl.KIND_REUSE else k
            groups.setdefault((k == wl.KIND_REUSE, src), []).append((r, l))
    picks = []
    keys = sorted(groups)
    i = 0
    while len(picks) < n_samples and keys:
        g = groups[keys[i % len(keys)]]
        picks.append(g[rng.integers(len(g))])
        i += 1
    t_total, tokens = 0.0, 0
    for (r, l) in picks:
        sr, sl = oa.resolve_source(kinds, r, l)
        b = int(rng.integers(w.batch))
        T = int(st.lens0[b])
        K, V = wl.cell_kv(w, st.cell_index(sr, sl), T, dev, b, b + 1)
        kb, vb = wl.bf16_bits(K[0]), wl.bf16_bits(V[0])
        del K, V
        cache = oc.build_cell_cache(kb, vb, int(kinds[sr, sl]))
        qb = wl.bf16_bits(wl.cell_query(w, st.cell_index(r, l), dev)[1])[b]
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                oa.decode(cache, qb, float(taus[r, l]))
                t_total += time.perf_counter() - t0
        else:
            t0 = time.perf_counter()
            oa.decode(cache, qb, float(taus[r, l]))
            t_total += time.perf_counter() - t0
        tokens += T
        log(f"[bench] oracle sample cell ({r},{l}) seq {b}: T={T} cumulative {t_total:.1f} s")
    return {"value": tokens / t_total, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(picks)} (cell, sequence) decodes of {w.name}, all {w.heads} heads, "
                      f"{tokens} KV tokens, cache build excluded, numpy single thread",
            "seconds": t_total}


if __name__ == "__main__":
    main()
