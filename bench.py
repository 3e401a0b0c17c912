#!/usr/bin/env python3
"""Decode-step benchmark of the LoopKV quantized decode path on one MI355X.

A step is one decode pass over every (loop, layer) cell of the workload's
plan for the whole batch, after appending the step's new token to every
stored cell when the workload appends.  Inputs are resident in HBM before
timing starts.  Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload lean-16k]
                    [--tau T | --tau-sweep] [--num-splits S] [--report FILE]
"""
from __future__ import annotations

import argparse
import json
import math
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth
METRIC = "decode-attn KV tokens/s + achieved HBM GB/s vs peak, Ouro-1.4B shape, 16K ctx"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lean-16k")
    ap.add_argument("--tau", type=float, default=None, help="one tau for every cell")
    ap.add_argument("--tau-sweep", action="store_true",
                    help="time the workload at every tau of its sweep (one prefill)")
    ap.add_argument("--num-splits", type=int, default=0, help="splits per (sequence, head); 0 = auto")
    ap.add_argument("--graph", action="store_true",
                    help="replay each timed step as one captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-samples", type=int, default=0,
                    help="oracle samples: (cell, sequence) decodes, or (layer, loop, sequence) for the joint-code "
                         "workloads; 0 = 64 (about 35 s of single-core work over the workers), or 40 for joint codes")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="oracle worker processes (capped by the host's cores); 16 is one GPU's share of a box")
    ap.add_argument("--extra", default="ragged-16k,lean-16k-p16,ouro1.4b-4k,ouro2.6b-32k,loopvq-16k",
                    help="comma-separated workloads also timed (no oracle) and reported under 'extra'")
    ap.add_argument("--report", default=None, help="also write the JSON result to this file")
    ap.add_argument("--planner", action="store_true",
                    help="only time the offline plan search (host) and exit")
    ap.add_argument("--probe-sizes", action="store_true",
                    help="only print the read probe's bandwidth at several launch sizes and exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="GIB",
                    help="only run 3 plain device copies of GIB GiB (counter calibration) and exit")
    return ap.parse_args()


def probe_sizes():
    """Read-probe bandwidth per launch size (how much one launch of a given
    size can stream), one JSON line per size."""
    import torch
    from loop_aware_quantized_amd import abi
    big = torch.empty(8 << 30, dtype=torch.uint8, device="cuda")
    # 50 / 67 MB and 805 / 1074 MB: what one 4K and one 16K decode read (2-bit / 4-bit source)
    for mb in (50, 67, 256, 512, 805, 1074, 2048, 4096, 8192):
        n = mb * 10**6 // 4096 * 4096
        reps = max(3, min(50, (8 << 30) // n))
        abi.loopkv_read_probe(big[:n])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            off = (r * n) % ((8 << 30) - n + 1)
            off -= off % 4096
            abi.loopkv_read_probe(big[off:off + n])    # a different window each time
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        print(json.dumps({"probe_mb": mb, "us_per_launch": round(us, 1),
                          "tb_per_s": round(n / (us * 1e-6) / 1e12, 3)}), flush=True)


def planner_report():
    """Time the offline plan search on the synthetic damage tables of the
    4 x 24 and 4 x 48 workloads; one JSON line each."""
    from loop_aware_quantized_amd import abi
    from loop_aware_quantized_amd import inputs as wl
    for name in ("planned-16k", "ouro2.6b-32k"):
        w = wl.WORKLOADS[name]
        d = wl.synthetic_damage(w)
        db, sb = wl.planner_budgets(w)
        reps, t0 = 5, time.perf_counter()
        for _ in range(reps):
            kinds, (reads, store, dmg) = abi.loopkv_plan_optimize(d, db, sb)
        ms = (time.perf_counter() - t0) * 1e3 / reps
        print(json.dumps({"planner": name, "cells": w.loops * w.layers, "ms": round(ms, 2),
                          "damage_budget": db, "storage_budget_units": sb, "reads_units": reads,
                          "storage_units": store, "damage": dmg,
                          "kinds": {k: int((kinds == v).sum()) for k, v in
                                    (("q4", wl.KIND_Q4), ("q2", wl.KIND_Q2), ("reuse", wl.KIND_REUSE))}}),
              flush=True)


def copy_probe(gib):
    """A plain copy kernel of known size, for scaling HBM traffic counters."""
    import torch
    src = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": gib << 30, "copies": 3}), flush=True)


class Bench:
    """Prefilled cache state of one workload plus the timed decode step."""

    def __init__(self, args, w, kinds, taus, n_points):
        import torch
        from loop_aware_quantized_amd import abi, runner
        from loop_aware_quantized_amd import inputs as wl
        self.torch, self.abi, self.runner, self.wl = torch, abi, runner, wl
        self.args, self.w = args, w
        self.kinds, self.taus = kinds, taus
        dev = torch.device("cuda", 0)
        self.dev = dev
        # warmup + timed steps + a profiled pass of as many steps + a counters step
        self.steps_per_point = args.warmup + 2 * args.steps + 2
        extra = w.append_tokens * self.steps_per_point * n_points
        t0 = time.time()
        st = runner.CacheState(w, dev, kinds, taus, extra_tokens=extra)
        self.st = st
        log(f"[bench] {w.name}: B={w.batch} R={w.loops} L={w.layers} H={w.heads} D={w.head_dim} "
            f"P={w.page} stored cells={len(st.stored)} pool pages={st.num_pages}")
        for i, (r, l) in enumerate(st.stored):
            st.prefill_cell(r, l)
            if i % 8 == 7:
                torch.cuda.synchronize()
                log(f"[bench] prefilled {i + 1}/{len(st.stored)} cells ({time.time() - t0:.1f} s)")
        torch.cuda.synchronize()
        R, L = w.loops, w.layers
        self.order = [(r, l) for r in range(R) for l in range(L)]
        self.queries = {c: wl.cell_query(w, st.cell_index(*c), dev)[1] for c in self.order}
        self.new_kv = {c: wl.append_kv(w, st.cell_index(*c), 0, w.append_tokens, dev)
                       for c in st.stored} if w.append_tokens else {}
        self.lens0 = st.lens0.astype(np.int64)
        total_steps = self.steps_per_point * n_points
        self.lens_dev = [torch.from_numpy((self.lens0 + s * w.append_tokens).astype(np.int32)).to(dev)
                         for s in range(total_steps + 1)]
        self.out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=dev)
        self.lens_app_buf = torch.empty_like(self.lens_dev[0])
        self.lens_dec_buf = torch.empty_like(self.lens_dev[0])
        self.graph = None
        self.step_idx = 0
        log(f"[bench] setup {time.time() - t0:.1f} s")

    def set_tau(self, tau):
        self.taus = self.wl.with_tau(self.taus, tau)
        w = self.w
        self.st.taus = self.taus
        self.st.plan = self.abi.Plan(self.abi.plan_blob(w.loops, w.layers, w.heads, w.head_dim, w.page,
                                                        self.kinds, self.taus))

    def lens_of(self, s):
        return self.lens0 + (s + 1) * self.w.append_tokens if self.w.append_tokens else self.lens0

    def launch_step(self, lens_app, lens_dec, sum_dec, counters=None):
        """Enqueue one step: append to every stored cell, then decode every cell."""
        abi, st, w = self.abi, self.st, self.w
        if w.append_tokens:
            app = abi.make_batch(lens_app, st.block_tables, st.max_seq_len)
            for c in st.stored:
                k, v = self.new_kv[c]
                abi.loopkv_append(st.plan, st.cells, c[0], c[1], app, w.append_tokens, k, v)
        bt = st.batch(lens_dec, sum_seq_lens=sum_dec)
        o = abi.make_opts(st.workspace, counters=counters, num_splits=self.args.num_splits)
        for (r, l) in self.order:
            abi.loopkv_decode(st.plan, st.cells, r, l, bt, self.queries[(r, l)], self.out, o)

    def step_lens(self, s):
        """(lengths before the append, lengths attended) device tensors of step s."""
        if self.w.append_tokens:
            return self.lens_dev[s], self.lens_dev[s + 1]
        return self.lens_dev[0], self.lens_dev[0]

    def step(self, counters=None, eager=False):
        s = self.step_idx
        if self.graph is not None and counters is None and not eager:
            # the captured step reads its lengths from two fixed buffers
            la, ld = self.step_lens(s)
            self.lens_app_buf.copy_(la)
            self.lens_dec_buf.copy_(ld)
            self.graph.replay()
        else:
            la, ld = self.step_lens(s)
            self.launch_step(la, ld, int(self.lens_of(s).sum()), counters)
        self.step_idx += 1

    def capture(self):
        """Record one step (all appends and decodes) as a HIP graph."""
        torch = self.torch
        self.graph = None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.launch_step(self.lens_app_buf, self.lens_dec_buf, int(self.lens_of(self.step_idx).sum()))
        torch.cuda.synchronize()
        self.graph = g

    def src_kind(self, r, l):
        R = self.w.loops
        return int(self.kinds[R - 1, l]) if self.kinds[r, l] == self.wl.KIND_REUSE else int(self.kinds[r, l])

    def split_bytes(self, lens):
        """Plan-required bytes the split pass reads for one step."""
        D, H = self.w.head_dim, self.w.heads
        tok = int(lens.sum())
        tot = 0
        for (r, l) in self.order:
            per = self.runner.required_bytes_per_token_head(self.src_kind(r, l), D)
            if self.src_kind(r, l) == self.wl.KIND_Q4 and self.taus[r, l] == 0.0:
                per += D // 4     # tau = 0: every low-plane row is required
            tot += tok * H * per
        return tot

    def timed_steps(self, n, hook):
        """n steps between events on the launch stream; with hook, the library
        stamps every kernel's own start and end (hipExtLaunchKernel events).
        Returns (first step index, events, per-class (launches, ms))."""
        torch, abi = self.torch, self.abi
        classes = (("split", abi.KERNEL_SPLIT), ("merge", abi.KERNEL_MERGE), ("append", abi.KERNEL_APPEND))
        if hook:
            abi.loopkv_profile_enable(True)
            for _, c in classes:
                abi.loopkv_profile_collect(c)
        first = self.step_idx
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        evs[0].record()
        for i in range(n):
            self.step(eager=hook)
            evs[i + 1].record()
        torch.cuda.synchronize()
        kst = None
        if hook:
            kst = {name: abi.loopkv_profile_collect(c) for name, c in classes}
            abi.loopkv_profile_enable(False)
        return first, evs, kst

    def run_point(self):
        """Warmup, the timed steps, a profiled pass of as many steps (every
        kernel's own start/end stamped), and a counters step."""
        torch, abi, args, w = self.torch, self.abi, self.args, self.w
        self.graph = None
        for _ in range(args.warmup):
            self.step()
        torch.cuda.synchronize()
        if args.graph:
            self.capture()
        # the timed steps run unprofiled: stamping a launch's start and end
        # costs a few microseconds between launches
        first, evs, _ = self.timed_steps(args.steps, hook=False)
        prof_first, evs2, kst = self.timed_steps(args.steps, hook=True)
        profiled_ms = evs2[0].elapsed_time(evs2[-1]) / args.steps
        total_ms = evs[0].elapsed_time(evs[-1])
        ms_per_step = total_ms / args.steps
        self.step_spread = step_spread(evs)
        # low-plane rows actually fetched (library counters)
        cnt = torch.zeros(2, dtype=torch.int64, device=self.dev)
        cnt_step = self.step_idx
        self.step(counters=cnt)
        torch.cuda.synchronize()
        flagged, lo_bytes = (int(x) for x in cnt.cpu().tolist())

        B, H, D, R, L = w.batch, w.heads, w.head_dim, w.loops, w.layers
        lens_t = self.lens_of(first)
        pages = int(((lens_t + w.page - 1) // w.page).sum())
        fixed = R * L * (B * H * (2 * D + 4 * D) + 4 * pages)       # q, out, page tables
        timed_tokens = sum(int(self.lens_of(s).sum()) for s in range(first, first + args.steps))
        value = timed_tokens * R * L / (total_ms / 1e3)
        # tau = 0 cells read their low planes inside the split pass (counted in
        # split_bytes); the counters report those rows too, so count only the
        # rows gathered for the other cells
        dense_lo = sum(int(self.lens_of(cnt_step).sum()) * H * D // 4 for (r, l) in self.order
                       if self.src_kind(r, l) == self.wl.KIND_Q4 and self.taus[r, l] == 0.0)
        step_bytes = self.split_bytes(lens_t) + (lo_bytes - dense_lo) + fixed
        step_gbs = step_bytes / (ms_per_step / 1e3) / 1e9
        n_split, split_ms = kst["split"]
        split_alg = sum(self.split_bytes(self.lens_of(s)) for s in range(prof_first, prof_first + args.steps))
        achieved = split_alg / (split_ms / 1e3) / 1e9 if split_ms > 0 else 0.0
        lo_stored = sum(int(self.lens_of(cnt_step).sum()) * H * D // 4
                        for (r, l) in self.order if self.src_kind(r, l) == self.wl.KIND_Q4)
        return {
            "value": value, "ms_per_step": ms_per_step, "step_ms": self.step_spread,
            "hbm_gbs_required": step_gbs, "bytes_required_per_step": step_bytes,
            "split": {"launches": n_split, "ms": split_ms, "alg_bytes": split_alg, "achieved_gbs": achieved},
            "kernels_ms_per_step": {k: v[1] / args.steps for k, v in kst.items()},
            "ms_per_step_profiled": profiled_ms,
            "lo_plane": {"flagged_token_heads": flagged, "lo_bytes_read": lo_bytes,
                         "lo_bytes_stored_4bit_sources": lo_stored,
                         "fraction_read": lo_bytes / lo_stored if lo_stored else None},
            "context": int(lens_t.max()),
        }

    def read_probe_gbs(self, gib=8, reps=5):
        """Measured streaming-read bandwidth (library probe kernel)."""
        torch, abi = self.torch, self.abi
        buf = torch.empty(gib << 30, dtype=torch.uint8, device=self.dev)
        abi.loopkv_read_probe(buf)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            abi.loopkv_read_probe(buf)
        e1.record()
        torch.cuda.synchronize()
        gbs = reps * buf.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
        del buf
        torch.cuda.empty_cache()
        return gbs


def recorded_traffic(workload: str):
    """Per-launch HBM traffic of the split kernel from the committed rocprofv3
    counter summary, or None when it is absent, for another workload, or
    taken from kernel sources that have changed since."""
    import hashlib
    import os
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"decode_split_traffic_{workload.replace('-', '').replace('.', '')}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        h = hashlib.sha256()
        for src in rec["sources"]:
            h.update(open(os.path.join(root, src), "rb").read())
    except (IndexError, KeyError, ValueError, OSError):
        return None
    if h.hexdigest()[:16] != rec.get("source_sha256_16"):
        return None
    return rec.get("traffic_bytes_per_launch_avg")


def _oracle_worker(job):
    """Worker process of the CPU baseline: build the oracle caches of its
    samples (not timed), wait for every worker, then time the decodes
    single-threaded.  Returns (start, end, per-sample seconds, tokens)."""
    import oracle.attention as oa
    import oracle.cache as oc
    samples, barrier = job["samples"], _BARRIER
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        limit = None
    caches = [oc.build_cell_cache(s["kb"], s["vb"], s["kind"]) for s in samples]
    barrier.wait()
    t0 = time.time()
    per = []
    for s, c in zip(samples, caches):
        a = time.perf_counter()
        oa.decode(c, s["qb"], s["tau"])
        per.append(time.perf_counter() - a)
    t1 = time.time()
    del limit
    return t0, t1, per, sum(s["T"] for s in samples)


_BARRIER = None


def _init_worker(barrier):
    global _BARRIER
    _BARRIER = barrier


def cpu_baseline(w, st, kinds, taus, n_samples, dev, workers):
    """Time oracle.attention.decode on (cell, sequence) samples on the host
    cores: `workers` single-threaded processes run at once (cache build
    excluded); the rate is the samples' tokens over the wall time from the
    first worker's start to the last one's end."""
    import multiprocessing as mp
    import os
    from concurrent.futures import ProcessPoolExecutor
    import oracle.attention as oa
    from loop_aware_quantized_amd import inputs as wl
    R, L = w.loops, w.layers
    rng = np.random.default_rng(12345)
    # cover 4-bit, 2-bit, reuse->4-bit and reuse->2-bit cells
    groups = {}
    for r in range(R):
        for l in range(L):
            k = int(kinds[r, l])
            src = int(kinds[R - 1, l]) if k == wl.KIND_REUSE else k
            groups.setdefault((k == wl.KIND_REUSE, src), []).append((r, l))
    keys = sorted(groups)
    picks = [groups[keys[i % len(keys)]][rng.integers(len(groups[keys[i % len(keys)]]))]
             for i in range(n_samples)]
    samples = []
    for (r, l) in picks:
        sr, sl = oa.resolve_source(kinds, r, l)
        b = int(rng.integers(w.batch))
        T = int(st.lens0[b])
        K, V = wl.cell_kv(w, st.cell_index(sr, sl), T, dev, b, b + 1)
        samples.append({"kb": wl.bf16_bits(K[0]), "vb": wl.bf16_bits(V[0]), "kind": int(kinds[sr, sl]),
                        "qb": wl.bf16_bits(wl.cell_query(w, st.cell_index(r, l), dev)[1])[b],
                        "tau": float(taus[r, l]), "T": T})
        del K, V
    workers = max(1, min(workers, os.cpu_count() or 1, len(samples)))
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(workers)
    jobs = [{"samples": samples[i::workers]} for i in range(workers)]
    log(f"[bench] oracle baseline: {len(samples)} (cell, sequence) decodes on {workers} worker processes")
    with ProcessPoolExecutor(workers, mp_context=ctx, initializer=_init_worker, initargs=(barrier,)) as ex:
        res = list(ex.map(_oracle_worker, jobs))
    wall = max(r[1] for r in res) - min(r[0] for r in res)
    per = [x for r in res for x in r[2]]
    tokens = sum(r[3] for r in res)
    log(f"[bench] oracle baseline: {tokens} KV tokens in {wall:.1f} s wall, {sum(per):.1f} s of decode work")
    return {"value": tokens / wall, "unit": "KV tokens/s", "cores": workers, "kind": "oracle",
            "host_cpu_count": os.cpu_count(),
            "sample": f"{len(samples)} (cell, sequence) decodes of {w.name}, all {w.heads} heads, {tokens} KV "
                      f"tokens, cache build excluded; {workers} single-threaded worker processes at once",
            "seconds": wall, "single_core_value": tokens / sum(per)}


def vq_main(args, w):
    """Bench of a LoopVQ-style workload, printed as the JSON line."""
    res = vq_run(args, w, with_cpu=not args.no_cpu_baseline)
    line = json.dumps(res)
    if args.report:
        with open(args.report, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


def vq_run(args, w, with_cpu):
    """Bench of a LoopVQ-style workload: per step, every layer codes one
    appended token (all loops jointly) and every (loop, layer) cell decodes."""
    import torch
    from loop_aware_quantized_amd import abi, runner
    from loop_aware_quantized_amd import inputs as wl
    dev = torch.device("cuda", 0)
    steps_total = args.warmup + args.steps + 1
    t0 = time.time()
    st = runner.VqState(w, dev, extra_tokens=w.append_tokens * steps_total)
    for l in st.layers:
        st.prefill_layer(l)
        if l % 8 == 7:
            torch.cuda.synchronize()
            log(f"[bench] {w.name}: prefilled {l + 1}/{w.layers} layers ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    R, L, B, H, D = w.loops, w.layers, w.batch, w.heads, w.head_dim
    queries = {(r, l): wl.vq_query(w, l, r, dev) for r in range(R) for l in range(L)}
    new_kv = {l: wl.vq_append_kv(w, l, 0, w.append_tokens, dev) for l in range(L)} if w.append_tokens else {}
    lens0 = st.lens0.astype(np.int64)
    lens_dev = [torch.from_numpy((lens0 + s * w.append_tokens).astype(np.int32)).to(dev)
                for s in range(steps_total + 1)]
    out = torch.empty(B, H, D, dtype=torch.float32, device=dev)
    state = {"s": 0}

    def lens_of(s):
        return lens0 + (s + 1) * w.append_tokens

    def step():
        s = state["s"]
        if w.append_tokens:
            for l in range(L):
                st.append(l, *new_kv[l], lens_dev[s])
        ld = lens_dev[s + 1] if w.append_tokens else lens_dev[0]
        for r in range(R):
            for l in range(L):
                st.decode(l, r, queries[(r, l)], out, lens=ld)
        state["s"] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    first = state["s"]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    spread = step_spread(evs)
    abi.loopkv_profile_enable(True)
    for c in (abi.KERNEL_SPLIT, abi.KERNEL_MERGE, abi.KERNEL_APPEND):
        abi.loopkv_profile_collect(c)
    prof = state["s"]
    step()
    torch.cuda.synchronize()
    kst = {n: abi.loopkv_profile_collect(c) for n, c in
           (("split", abi.KERNEL_SPLIT), ("merge", abi.KERNEL_MERGE), ("append", abi.KERNEL_APPEND))}
    abi.loopkv_profile_enable(False)
    tokens = sum(int(lens_of(s).sum()) for s in range(first, first + args.steps)) / args.steps
    per_th = 2 * (D // 4)                           # key + value index bytes per token-head
    step_bytes = R * L * (tokens * H * per_th + B * H * 6 * D)
    split_bytes = R * L * int(lens_of(prof).sum()) * H * per_th
    n_split, split_ms = kst["split"]
    achieved = split_bytes / (split_ms / 1e3) / 1e9
    stored = L * abi.vq_pool_bytes(st.dims, st.num_pages)
    cpu = vq_cpu_baseline(w, st, queries, n_samples=args.cpu_samples or 40) if with_cpu else None
    res = {
        "metric": METRIC, "value": tokens * R * L / (ms / 1e3), "unit": "KV tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "arithmetic": "1-byte joint codes; fp16 codewords widened to f32; scores, softmax and accumulation in f32",
        "data": "synthetic (seeded loop-redundant bf16 K/V, synthetic codebooks)",
        "config": {"workload": w.name, "batch": B, "loops": R, "layers": L, "heads": H, "head_dim": D,
                   "page": w.page, "context": int(lens_of(first).max()), "bits_per_element": 8 / (4 * R),
                   "append_tokens_per_step": w.append_tokens},
        "hbm_gbs_required": step_bytes / (ms / 1e3) / 1e9,
        "roofline": {"bound": "hbm", "kernel": "vq_split_kernel", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "launches": n_split, "avg_launch_us": split_ms * 1e3 / max(n_split, 1)},
        "kernels_ms_per_step": {k: v[1] for k, v in kst.items()},
        "step_ms": spread,
        "storage": {"stored_bytes": stored},
        "cpu_baseline": cpu,
    }
    del st
    torch.cuda.empty_cache()
    return res


def vq_cpu_baseline(w, st, queries, n_samples):
    """Time oracle.loopvq (codeword lookup + float64 attention, all heads) on
    (layer, loop, sequence) samples of a joint-code workload; the index bytes
    are copied from the GPU pool first and that copy is not timed."""
    import oracle.loopvq as ov
    from loop_aware_quantized_amd import inputs as wl
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    rng = np.random.default_rng(54321)
    t_total, tokens = 0.0, 0
    for _ in range(n_samples):
        l, r, b = int(rng.integers(w.layers)), int(rng.integers(w.loops)), int(rng.integers(w.batch))
        T = int(st.lens0[b])
        ki, vi = st.pool_indices(l, b, T)
        cbk, cbv = (wl.vq_joint_codebook(c) for c in st.codebooks[l])
        q = (wl.bf16_bits(queries[(r, l)])[b].astype(np.uint32) << 16).view(np.float32).astype(np.float64)

        def run():
            for h in range(w.heads):
                ov.attend(q[h], ov.decode_loop(ki[:, h].astype(np.int64), cbk, r),
                          ov.decode_loop(vi[:, h].astype(np.int64), cbv, r))

        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                run()
                t_total += time.perf_counter() - t0
        else:
            t0 = time.perf_counter()
            run()
            t_total += time.perf_counter() - t0
        tokens += T
        log(f"[bench] oracle sample layer {l} loop {r} seq {b}: T={T} cumulative {t_total:.1f} s")
    return {"value": tokens / t_total, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_samples} (layer, loop, sequence) decodes of {w.name}, all {w.heads} heads, "
                      f"{tokens} KV tokens, index copy excluded, numpy single thread",
            "seconds": t_total}


def step_spread(evs):
    """Median, p10 and p90 of the per-step durations between consecutive
    events (ms); the events were recorded between steps on the timed stream."""
    import numpy as np
    d = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(len(evs) - 1)])
    return {"median": float(np.median(d)), "p10": float(np.percentile(d, 10)),
            "p90": float(np.percentile(d, 90))}


def sweep_report(points):
    """Bytes read and bandwidth at each point of a tau sweep."""
    return [{"tau": p["tau"], "ms_per_step": p["ms_per_step"],
             "kv_tokens_per_s": p["value"],
             "bytes_required_per_step": p["bytes_required_per_step"],
             "hbm_gbs_required": p["hbm_gbs_required"],
             "split_achieved_gbs": p["split"]["achieved_gbs"],
             "split_frac": p["split"]["achieved_gbs"] / HBM_PEAK_GBS,
             "lo_bytes_read": p["lo_plane"]["lo_bytes_read"],
             "lo_fraction_read": p["lo_plane"]["fraction_read"]} for p in points]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.probe_sizes:
        probe_sizes()
        return
    if args.planner:
        planner_report()
        return
    import torch
    from loop_aware_quantized_amd import abi
    from loop_aware_quantized_amd import inputs as wl
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    torch.cuda.set_device(0)
    abi.lib()  # fail loudly if the HIP library is missing

    if args.workload in wl.VQ_WORKLOADS:
        vq_main(args, wl.VQ_WORKLOADS[args.workload])
        return
    w = wl.WORKLOADS[args.workload]
    kinds, taus = wl.make_plan(w)
    if args.tau is not None:
        taus = wl.with_tau(taus, args.tau)
    sweep = list(w.tau_sweep) if args.tau_sweep else [None]
    bench = Bench(args, w, kinds, taus, len(sweep))
    peak = bench.read_probe_gbs()
    log(f"[bench] measured stream-read peak {peak:.0f} GB/s")

    points = []
    for tau in sweep:
        if tau is not None:
            bench.set_tau(tau)
        r = bench.run_point()
        r["tau"] = "plan" if tau is None else ("inf" if math.isinf(tau) else tau)
        log(f"[bench] tau={r['tau']}: {r['ms_per_step']:.3f} ms/step, split {r['split']['achieved_gbs']:.0f} GB/s")
        points.append(r)
    # primary point: the workload's own plan taus (first point when not sweeping)
    primary = points[0]
    if args.tau_sweep:
        own = float(w.taus[0])
        primary = next(p for p in points if p["tau"] != "inf" and float(p["tau"]) == own)
        bench.set_tau(own)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, bench.st, kinds, bench.taus, args.cpu_samples or 64, bench.dev, args.cpu_workers)

    st = bench.st
    q4_cells = [c for c in st.stored if kinds[c] == wl.KIND_Q4]
    stored_bytes = sum(st.plan.pool_bytes(r, l, st.num_pages) for (r, l) in st.stored)
    all_q4_bytes = (w.loops * w.layers * st.plan.pool_bytes(*q4_cells[0], st.num_pages)
                    if q4_cells else None)
    sp = primary["split"]
    # the split pass's kernel: the streamed variant where the cell's layout is streamed
    hint = int(bench.lens_of(0).sum())
    streamed = {bool(bench.abi.loopkv_decode_layout(st.plan, r, l, w.batch, st.max_seq_len, hint,
                                                     args.num_splits)[0]) for (r, l) in bench.order}
    split_kernel = "+".join(k for k, on in (("decode_split_kernel", False in streamed),
                                            ("decode_stream_kernel", True in streamed)) if on)
    del bench, st
    torch.cuda.empty_cache()
    extra = {}
    for name in [x for x in args.extra.split(",") if x and x != w.name]:
        if name in wl.VQ_WORKLOADS:
            r = vq_run(args, wl.VQ_WORKLOADS[name], with_cpu=False)
            extra[name] = {"ms_per_step": r["ms_per_step"], "kv_tokens_per_s": r["value"],
                           "hbm_gbs_required": r["hbm_gbs_required"], "page": r["config"]["page"],
                           "batch": r["config"]["batch"], "context": r["config"]["context"],
                           "bits_per_element": r["config"]["bits_per_element"],
                           "split_roofline": {k: r["roofline"][k] for k in ("kernel", "achieved", "frac",
                                                                            "avg_launch_us", "launches")},
                           "kernels_ms_per_step": r["kernels_ms_per_step"], "storage": r["storage"]}
            log(f"[bench] extra {name}: {r['ms_per_step']:.3f} ms/step, "
                f"{r['roofline']['kernel']} {r['roofline']['achieved']:.0f} GB/s")
            torch.cuda.empty_cache()
            continue
        ew = wl.WORKLOADS[name]
        ek, et = wl.make_plan(ew)
        # a workload with a tau sweep runs every point; its entry is the
        # point at the workload's own plan tau, the sweep listed beside it
        esweep = list(ew.tau_sweep) or [None]
        eb = Bench(args, ew, ek, et, len(esweep))
        epoints = []
        for tau in esweep:
            if tau is not None:
                eb.set_tau(tau)
            r = eb.run_point()
            r["tau"] = "plan" if tau is None else ("inf" if math.isinf(tau) else tau)
            esp = r["split"]
            log(f"[bench] extra {name} tau={r['tau']}: {r['ms_per_step']:.3f} ms/step, "
                f"split {esp['achieved_gbs']:.0f} GB/s")
            epoints.append(r)
        r = epoints[0]
        if ew.tau_sweep:
            own = float(ew.taus[0])
            r = next(p for p in epoints if p["tau"] != "inf" and float(p["tau"]) == own)
        esp = r["split"]
        extra[name] = {"ms_per_step": r["ms_per_step"], "kv_tokens_per_s": r["value"],
                       "hbm_gbs_required": r["hbm_gbs_required"], "page": ew.page, "batch": ew.batch,
                       "context": r["context"], "tau": r["tau"],
                       "split_roofline": {"achieved": esp["achieved_gbs"], "frac": esp["achieved_gbs"] / HBM_PEAK_GBS,
                                          "avg_launch_us": esp["ms"] * 1e3 / max(esp["launches"], 1),
                                          "launches": esp["launches"]},
                       "kernels_ms_per_step": r["kernels_ms_per_step"], "lo_plane": r["lo_plane"]}
        if ew.tau_sweep:
            extra[name]["tau_sweep"] = sweep_report(epoints)
        del eb
        torch.cuda.empty_cache()
    res = {
        "metric": METRIC,
        "value": primary["value"],
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": primary["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "arithmetic": ("2/4-bit codes; scores and softmax in f32; value weights rounded to f16 (kept in its "
                       "normal range) in f32-accumulated dot products"),
        "data": "synthetic (seeded N(0,1) bf16 K/V with outlier channels and heavy tokens)",
        "config": {"workload": w.name, "batch": w.batch, "loops": w.loops, "layers": w.layers,
                   "heads": w.heads, "head_dim": w.head_dim, "page": w.page,
                   "context": primary["context"], "tau": primary["tau"],
                   "append_tokens_per_step": w.append_tokens,
                   "step_launch": "hip_graph" if args.graph else "eager"},
        "hbm_gbs_required": primary["hbm_gbs_required"],
        "hbm_frac_required": primary["hbm_gbs_required"] / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": split_kernel, "achieved": sp["achieved_gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": sp["achieved_gbs"] / HBM_PEAK_GBS,
                     "traffic": recorded_traffic(w.name), "traffic_unit": "bytes per launch",
                     "launches": sp["launches"],
                     "avg_launch_us": sp["ms"] * 1e3 / max(sp["launches"], 1),
                     "alg_bytes_per_launch": sp["alg_bytes"] / max(sp["launches"], 1),
                     "measured_read_peak": peak,
                     "frac_of_measured_read_peak": sp["achieved_gbs"] / peak},
        "kernels_ms_per_step": primary["kernels_ms_per_step"],
        "step_ms": primary["step_ms"],
        "ms_per_step_profiled_pass": primary["ms_per_step_profiled"],
        "lo_plane": primary["lo_plane"],
        "storage": {"stored_bytes": stored_bytes, "all_4bit_bytes": all_q4_bytes,
                    "saving_vs_all_4bit": (1 - stored_bytes / all_q4_bytes) if all_q4_bytes else None},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    if args.tau_sweep:
        res["tau_sweep"] = sweep_report(points)
    line = json.dumps(res)
    if args.report:
        with open(args.report, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


if __name__ == "__main__":
    main()
