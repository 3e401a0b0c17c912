"""Plan search by exhaustive enumeration (small grids only).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source
------
LoopKV abstract ("LoopKV: Loop-Aware KV Cache Compression for Serving
Looped Transformers", 概要): the model's output damage is close to the sum
of the damages measured cell by cell; per cell, a profile taken once and
offline selects 4-bit codes, 2-bit codes or borrowing the last loop's
cache, and the plan is the one with the fewest bytes read whose predicted
damage and storage stay within given limits.

Readings where the pages are silent:
* a plan's damage is the sum of its cells' damages; a cell's damage is the
  profiled value of its kind, and for a reuse cell the value for the format
  its source (the final loop's cell of the layer) is stored in;
* reads and storage are counted per token-head in 32-byte units at
  head_dim 128: a decode of a 4-bit source reads both key planes, the high
  value plane and the metadata (4 units), a 2-bit source 3 units; a reuse
  cell reads its source; a stored 4-bit cell holds four planes + metadata
  (5 units), a 2-bit cell 3, a reuse cell nothing;
* among plans within both budgets the chosen one has least reads, then least
  damage, then least storage.

Pins (tests/test_planner.py): hand-computed one-layer cases in
tests/golden/planner_cases.txt, and closed forms (unbounded budgets give the
all-reuse plan over 2-bit final cells; a zero damage budget with zero 4-bit
damages gives the all-4-bit plan).
"""
from __future__ import annotations

import itertools

import numpy as np

Q4, Q2, REUSE = 0, 1, 2
READ = {Q4: 4, Q2: 3}
STORE = {Q4: 5, Q2: 3}


def plan_cost(kinds, damage):
    """(reads, storage, damage) of a plan kinds[R][L] under damage[R][L][4]."""
    R, L = kinds.shape
    reads = store = 0
    dmg = 0.0
    for l in range(L):
        src = int(kinds[R - 1, l])
        if src == REUSE:
            raise ValueError("the final loop cannot reuse itself")
        for r in range(R):
            k = int(kinds[r, l])
            if k == REUSE:
                reads += READ[src]
                dmg += float(damage[r, l, 2 if src == Q4 else 3])
            else:
                reads += READ[k]
                store += STORE[k]
                dmg += float(damage[r, l, 0 if k == Q4 else 1])
    return reads, store, dmg


def all_plans(R, L):
    """Every valid plan of an R x L grid (reuse never in the final loop)."""
    per_cell = [[Q4, Q2, REUSE] if r < R - 1 else [Q4, Q2] for r in range(R) for _ in range(L)]
    for flat in itertools.product(*per_cell):
        yield np.array(flat, np.int64).reshape(R, L)


def optimize(damage, damage_budget, storage_budget, rel=1e-12):
    """Brute-force optimum: (kinds, (reads, storage, damage)) or None.

    Damages that differ by less than ``rel`` (relative) count as equal, so
    the order of summation does not pick the winner.
    """
    damage = np.asarray(damage, np.float64)
    R, L = damage.shape[:2]
    best = None
    for kinds in all_plans(R, L):
        rd, st, dm = plan_cost(kinds, damage)
        if dm > damage_budget * (1 + rel) or st > storage_budget:
            continue
        if best is None:
            best = (kinds, (rd, st, dm))
            continue
        brd, bst, bdm = best[1]
        tol = rel * max(abs(bdm), 1e-300)
        if rd < brd or (rd == brd and (dm < bdm - tol or (abs(dm - bdm) <= tol and st < bst))):
            best = (kinds, (rd, st, dm))
    return best
