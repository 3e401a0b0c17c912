"""Seeded synthetic inputs for the LoopKV decode path.

This module draws random numbers and builds shapes, plans, lengths and page
tables.  It holds none of the method's arithmetic (no quantization, no
attention); both the HIP path and the CPU oracle receive exactly what it
produces.

Workloads stand in for the Ouro model shapes of the LoopKV abstract
("LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers",
概要: Ouro-1.4B served at up to a 16K-token length) and for Ouro-2.6B (named
on the LoopVQ page).  Values: keys and values N(0,1) in bf16, four outlier key
channels per head scaled by 10, a few "heavy" tokens whose keys are
0.5*q_raw + N(0,1) noise so that they draw strong attention, and queries
q = bf16(q_raw / sqrt(head_dim)) with q_raw ~ N(0,1).  All transforms are done
in fp32 and rounded once to bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KIND_Q4, KIND_Q2, KIND_REUSE = 0, 1, 2

# purposes of seeded streams
_P_PLAN, _P_TAU, _P_LENS, _P_PAGES, _P_KV, _P_APPEND, _P_DAMAGE = range(7)


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                      # stable id used in seeds
    batch: int
    loops: int
    layers: int
    heads: int
    head_dim: int
    page: int
    ctx: int                      # fixed context, or the maximum of a ragged draw
    ctx_min: int | None = None    # ragged: lengths uniform in [ctx_min, ctx]
    shuffle_pages: bool = False
    heavy_frac: float = 0.01      # Bernoulli fraction of heavy tokens
    heavy_count: int | None = None  # exact heavy tokens per (sequence, head)
    plan: str = "random"          # "tiny" | "random" | "lean" | "kivi4" | "planned"
    taus: tuple = (0.01,)         # "random": per-cell draw; else one tau for all cells
    append_tokens: int = 0        # tokens appended per stored cell in one step
    tau_sweep: tuple = field(default=())
    value_scale: float = 1.0      # prefill values are N(0, value_scale^2)

    @property
    def cells(self) -> int:
        return self.loops * self.layers


WORKLOADS = {
    # tiny: 1 sequence, 2 loops x 2 layers, 2 heads of 64, 256 tokens
    "tiny": Workload("tiny", 0, batch=1, loops=2, layers=2, heads=2, head_dim=64, page=16,
                     ctx=256, heavy_count=3, plan="tiny", taus=(0.02,)),
    # Ouro-1.4B-like: 4 loops x 24 layers, 16 heads of 128, batch 8, 4K context
    "ouro1.4b-4k": Workload("ouro1.4b-4k", 1, batch=8, loops=4, layers=24, heads=16,
                            head_dim=128, page=32, ctx=4096, plan="random",
                            taus=(0.005, 0.01, 0.02)),
    # memory-lean plan at a 16K context, batch 32, one appended token per step
    "lean-16k": Workload("lean-16k", 2, batch=32, loops=4, layers=24, heads=16, head_dim=128,
                         page=32, ctx=16384, plan="lean", taus=(0.01,), append_tokens=1),
    # ragged batch of 64, lengths U[512, 16384], 16-token pages, shuffled tables
    "ragged-16k": Workload("ragged-16k", 3, batch=64, loops=4, layers=24, heads=16,
                           head_dim=128, page=16, ctx=16384, ctx_min=512, shuffle_pages=True,
                           heavy_frac=0.005, plan="random", taus=(0.005,)),
    # lean-16k's shape, plan and data over 16-token pages (two pages per key group)
    "lean-16k-p16": Workload("lean-16k-p16", 2, batch=32, loops=4, layers=24, heads=16, head_dim=128,
                             page=16, ctx=16384, plan="lean", taus=(0.01,), append_tokens=1),
    # KIVI-4-style baseline on the lean-16k shape and data: every cell stored
    # at 4 bits, no reuse, tau = 0 (every low plane read)
    "kivi4-16k": Workload("kivi4-16k", 2, batch=32, loops=4, layers=24, heads=16, head_dim=128,
                          page=32, ctx=16384, plan="kivi4", taus=(0.0,), append_tokens=1),
    # lean-16k's shape and data with the plan found by the offline planner on
    # a synthetic damage table (storage within 48.75% of all-4-bit, the lean
    # plan's share; damage within half of the all-2-bit plan's)
    "planned-16k": Workload("planned-16k", 2, batch=32, loops=4, layers=24, heads=16, head_dim=128,
                            page=32, ctx=16384, plan="planned", taus=(0.01,), append_tokens=1),
    # Ouro-2.6B-like: 4 loops x 48 layers, batch 16, 32K context, tau sweep
    "ouro2.6b-32k": Workload("ouro2.6b-32k", 4, batch=16, loops=4, layers=48, heads=16,
                             head_dim=128, page=32, ctx=32768, plan="lean", taus=(0.01,),
                             tau_sweep=(0.0, 0.002, 0.01, 0.05, math.inf)),
}


def seed_of(w: Workload, purpose: int, *key: int) -> int:
    ss = np.random.SeedSequence(0, spawn_key=(w.wid, purpose) + tuple(int(k) for k in key))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def np_rng(w: Workload, purpose: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(seed_of(w, purpose, *key))


# ----------------------------------------------------------------------------
# plans
# ----------------------------------------------------------------------------

# per-loop (4-bit, 2-bit, reuse) counts of the memory-lean plan over 24 layers:
# later loops get more reuse and 2-bit cells; 24 / 38 / 34 of 96 cells
# (25% / 40% / 35%); the final loop cannot reuse itself.
_LEAN_COUNTS_24 = ((14, 4, 6), (6, 8, 10), (2, 4, 18), (2, 22, 0))


def make_plan(w: Workload):
    """(kinds [R][L] int, taus [R][L] float) of a workload, seeded."""
    R, L = w.loops, w.layers
    kinds = np.zeros((R, L), np.int64)
    if w.plan == "tiny":
        # one cell each of 4-bit, 2-bit, reuse and 4-bit, listed layer by layer
        # so that the reuse cell is not in the final loop
        kinds[0, 0], kinds[1, 0], kinds[0, 1], kinds[1, 1] = KIND_Q4, KIND_Q2, KIND_REUSE, KIND_Q4
    elif w.plan == "random":
        # 40% 4-bit, 35% 2-bit, 25% reuse; reuse only in loops 0 .. R-2
        rng = np_rng(w, _P_PLAN)
        n = R * L
        n_reuse = int(round(0.25 * n))
        n_q4 = int(round(0.40 * n))
        early = np.arange((R - 1) * L)
        reuse = rng.choice(early, n_reuse, replace=False)
        rest = np.setdiff1d(np.arange(n), reuse)
        rest = rng.permutation(rest)
        flat = np.full(n, KIND_Q2)
        flat[reuse] = KIND_REUSE
        flat[rest[:n_q4]] = KIND_Q4
        kinds = flat.reshape(R, L)
    elif w.plan == "lean":
        if R != 4 or L % 24:
            raise ValueError("the memory-lean plan is defined for 4 loops and 24k layers")
        mult = L // 24
        rng = np_rng(w, _P_PLAN)
        for r in range(R):
            q4, q2, ru = (c * mult for c in _LEAN_COUNTS_24[r])
            row = np.array([KIND_Q4] * q4 + [KIND_Q2] * q2 + [KIND_REUSE] * ru)
            kinds[r] = row[rng.permutation(L)]
    elif w.plan == "kivi4":
        kinds[:] = KIND_Q4
    elif w.plan == "planned":
        from . import abi
        kinds, _ = abi.loopkv_plan_optimize(synthetic_damage(w), *planner_budgets(w))
    else:
        raise ValueError(w.plan)
    if w.plan == "random" and len(w.taus) > 1:
        taus = np_rng(w, _P_TAU).choice(np.asarray(w.taus, np.float64), size=(R, L))
    else:
        taus = np.full((R, L), float(w.taus[0]))
    return kinds, taus


def synthetic_damage(w: Workload) -> np.ndarray:
    """Seeded stand-in for a per-cell damage profile, float64 [R][L][4]:
    (4-bit, 2-bit, reuse of a 4-bit final cell, reuse of a 2-bit one).

    No profile of a real model exists here (it needs Ouro weights and data);
    the table only has the properties the LoopKV abstract states: damage
    varies across (loop, layer) cells, and sharing damage varies by cell
    with later loops tolerating sharing better.  A cell's quantization
    sensitivity s is log-normal (sigma 0.5); 2-bit damage is s and 4-bit
    damage s/25 (a 4-bit step is a fifth of a 2-bit one; squared error goes
    with the step squared).  Sharing damage is log-normal (sigma 0.5) times
    (R-1-r)/(R-1); a reuse cell also sees its source's quantization.
    """
    R, L = w.loops, w.layers
    rng = np_rng(w, _P_DAMAGE)
    sens = np.exp(rng.normal(0.0, 0.5, (R, L)))
    share = np.exp(rng.normal(0.0, 0.5, (R, L))) * ((R - 1 - np.arange(R)) / max(R - 1, 1))[:, None]
    d = np.empty((R, L, 4))
    d[..., 0] = sens / 25.0
    d[..., 1] = sens
    d[..., 2] = share + sens / 25.0
    d[..., 3] = share + sens
    return d


def planner_budgets(w: Workload):
    """(damage budget, storage budget in 32-byte units per token-head) of a
    planned workload: half the all-2-bit plan's damage, 48.75% of the
    all-4-bit plan's storage (the share the memory-lean plan stores)."""
    d = synthetic_damage(w)
    return 0.5 * float(d[..., 1].sum()), int(0.4875 * 5 * w.loops * w.layers)


def with_tau(taus, tau: float):
    """The same plan with one tau for every cell (tau sweeps)."""
    return np.full_like(np.asarray(taus, np.float64), float(tau))


# ----------------------------------------------------------------------------
# lengths and page tables
# ----------------------------------------------------------------------------

def make_lengths(w: Workload) -> np.ndarray:
    if w.ctx_min is None:
        return np.full(w.batch, w.ctx, np.int32)
    rng = np_rng(w, _P_LENS)
    return rng.integers(w.ctx_min, w.ctx + 1, size=w.batch).astype(np.int32)


def make_block_tables(w: Workload, capacity, extra_pages: int = 0):
    """Page tables for per-sequence token capacities.

    Returns (table int32 [B][max_pages], num_pages).  Sequences own disjoint
    physical pages; a shuffled workload draws them as a random permutation of
    the pool, otherwise they are contiguous and in order.  Unused entries are
    0 (never dereferenced).  ``extra_pages`` spare pages end the pool, which
    holds at least one page (the library takes no empty pool, even for a
    batch of empty sequences).
    """
    capacity = np.asarray(capacity, np.int64)
    pages = (capacity + w.page - 1) // w.page
    total = max(1, int(pages.sum()) + int(extra_pages))
    max_pages = int(max(1, pages.max()))
    phys = np.arange(total, dtype=np.int64)
    if w.shuffle_pages:
        phys = np_rng(w, _P_PAGES).permutation(total)
    table = np.zeros((w.batch, max_pages), np.int32)
    pos = 0
    for b in range(w.batch):
        n = int(pages[b])
        table[b, :n] = phys[pos:pos + n]
        pos += n
    return table, total


# ----------------------------------------------------------------------------
# keys, values, queries (torch, on any device)
# ----------------------------------------------------------------------------

def _gen(w: Workload, device, purpose: int, *key: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(w, purpose, *key))
    return g


def cell_query(w: Workload, cell: int, device, step: int = 0):
    """(q_raw fp32 [B][H][D], q bf16 [B][H][D]) of a cell's query at a step."""
    import torch
    g = _gen(w, device, _P_KV, cell, 0, step)
    qraw = torch.randn(w.batch, w.heads, w.head_dim, generator=g, device=device)
    q = (qraw / math.sqrt(w.head_dim)).to(torch.bfloat16)
    return qraw, q


def outlier_scale(w: Workload, cell: int, device):
    """[H][D] fp32 multipliers: 10 on 4 distinct key channels per head, else 1."""
    import torch
    g = _gen(w, device, _P_KV, cell, 1)
    order = torch.rand(w.heads, w.head_dim, generator=g, device=device).argsort(dim=-1)
    mult = torch.ones(w.heads, w.head_dim, device=device)
    mult.scatter_(1, order[:, :4], 10.0)
    return mult


def cell_kv(w: Workload, cell: int, tokens: int, device, b0: int = 0, b1: int | None = None):
    """Prefill keys and values of a stored cell: bf16 [b1-b0][tokens][H][D].

    Heavy tokens use the cell's step-0 query; outliers multiply every key.
    Sequences are drawn independently, so a batch slice [b0, b1) reproduces
    the same values as the full batch.
    """
    import torch
    b1 = w.batch if b1 is None else b1
    qraw, _ = cell_query(w, cell, device)
    mult = outlier_scale(w, cell, device)
    H, D = w.heads, w.head_dim
    ks, vs = [], []
    for b in range(b0, b1):
        g = _gen(w, device, _P_KV, cell, 2, b)
        K = torch.randn(tokens, H, D, generator=g, device=device)
        if w.heavy_count is not None:
            order = torch.rand(H, tokens, generator=g, device=device).argsort(dim=-1)
            heavy = torch.zeros(H, tokens, dtype=torch.bool, device=device)
            heavy.scatter_(1, order[:, : w.heavy_count], True)
            heavy = heavy.t()
        else:
            heavy = torch.rand(tokens, H, generator=g, device=device) < w.heavy_frac
        K = torch.where(heavy[..., None], 0.5 * qraw[b][None] + K, K)
        K = K * mult[None]
        V = torch.randn(tokens, H, D, generator=g, device=device) * w.value_scale
        ks.append(K.to(torch.bfloat16))
        vs.append(V.to(torch.bfloat16))
    return torch.stack(ks), torch.stack(vs)


def append_kv(w: Workload, cell: int, step: int, n_new: int, device):
    """Keys/values of n_new appended tokens (no heavy tokens), bf16 [B][n_new][H][D]."""
    import torch
    g = _gen(w, device, _P_APPEND, cell, step)
    mult = outlier_scale(w, cell, device)
    K = torch.randn(w.batch, n_new, w.heads, w.head_dim, generator=g, device=device) * mult
    V = torch.randn(w.batch, n_new, w.heads, w.head_dim, generator=g, device=device)
    return K.to(torch.bfloat16), V.to(torch.bfloat16)


def bf16_bits(t) -> np.ndarray:
    """bf16 torch tensor -> numpy uint16 bit patterns (host copy)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# joint vector quantization across loop steps (LoopVQ-style workloads)
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class VqWorkload:
    name: str
    wid: int
    batch: int
    loops: int
    layers: int
    heads: int
    head_dim: int
    page: int
    ctx: int
    append_tokens: int = 0
    loop_noise: float = 0.25      # per-loop deviation from the shared vector

    # the fields make_block_tables reads
    ctx_min = None
    shuffle_pages = False


VQ_WORKLOADS = {
    "loopvq-tiny": VqWorkload("loopvq-tiny", 10, batch=2, loops=4, layers=2, heads=2, head_dim=64, page=16,
                              ctx=300),
    # the lean-16k model shape and batch: 4 loops x 24 layers, 16 heads of 128,
    # 32 sequences of 16K tokens, one token appended per step
    "loopvq-16k": VqWorkload("loopvq-16k", 11, batch=32, loops=4, layers=24, heads=16, head_dim=128, page=32,
                             ctx=16384, append_tokens=1),
}


def vq_codebooks(w: VqWorkload, layer: int, device):
    """(keys, values) codebooks of one layer in the library's layout, fp16
    [R][256][D/4][4]: loop r's 4 channels of codeword c of group j.

    Codebook training is out of scope; the codewords are draws from the
    same loop-redundant model as the data: a shared 4-vector per group plus
    loop_noise * N(0, 1) per loop.
    """
    import torch
    G, R = w.head_dim // 4, w.loops
    out = []
    for kv in range(2):
        g = _gen(w, device, _P_KV, layer, 100 + kv)
        base = torch.randn(G, 256, 1, 4, generator=g, device=device)
        cw = base + w.loop_noise * torch.randn(G, 256, R, 4, generator=g, device=device)
        out.append(cw.permute(2, 1, 0, 3).to(torch.float16).contiguous())
    return out[0], out[1]


def vq_joint_codebook(cb):
    """Library codebook [R][256][G][4] -> joint codewords [G][256][4R]
    (loop r's channels at positions 4r .. 4r+3), as a host float64 array."""
    import numpy as np
    a = cb.float().cpu().numpy().astype(np.float64)
    R, C, G, _ = a.shape
    return a.transpose(2, 1, 0, 3).reshape(G, C, 4 * R)


def vq_kv(w: VqWorkload, layer: int, b: int, t0: int, t1: int, device):
    """Keys and values of tokens [t0, t1) of sequence b, all loops:
    bf16 [R][1][t1 - t0][H][D] each (loop-redundant: shared + noise)."""
    import torch
    n = t1 - t0
    out = []
    for kv in range(2):
        g = _gen(w, device, _P_KV, layer, 200 + kv, b, t0)
        base = torch.randn(1, 1, n, w.heads, w.head_dim, generator=g, device=device)
        x = base + w.loop_noise * torch.randn(w.loops, 1, n, w.heads, w.head_dim, generator=g, device=device)
        out.append(x.to(torch.bfloat16).contiguous())
    return out[0], out[1]


def vq_append_kv(w: VqWorkload, layer: int, step: int, n_new: int, device):
    """Keys and values of n_new appended tokens of every sequence: bf16 [R][B][n_new][H][D]."""
    import torch
    out = []
    for kv in range(2):
        g = _gen(w, device, _P_APPEND, layer, 300 + kv, step)
        base = torch.randn(1, w.batch, n_new, w.heads, w.head_dim, generator=g, device=device)
        x = base + w.loop_noise * torch.randn(w.loops, w.batch, n_new, w.heads, w.head_dim, generator=g,
                                               device=device)
        out.append(x.to(torch.bfloat16).contiguous())
    return out[0], out[1]


def vq_query(w: VqWorkload, layer: int, loop: int, device):
    """bf16 [B][H][D] query of one (loop, layer): N(0, 1) / sqrt(D)."""
    import torch
    g = _gen(w, device, _P_KV, layer, 400 + loop)
    q = torch.randn(w.batch, w.heads, w.head_dim, generator=g, device=device) / math.sqrt(w.head_dim)
    return q.to(torch.bfloat16)
