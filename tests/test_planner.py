"""Offline plan search: the library's exact search against the brute-force
oracle, and the oracle against hand-computed cases and closed forms."""
import os
import time

import numpy as np
import pytest

from loop_aware_quantized_amd import abi
from loop_aware_quantized_amd import inputs as wl
from oracle import planner as op

Q4, Q2, RU = wl.KIND_Q4, wl.KIND_Q2, wl.KIND_REUSE
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "planner_cases.txt")
NAMES = {"Q4": Q4, "Q2": Q2, "RU": RU}

# the golden file's one-layer, two-loop damage table
GOLDEN_DAMAGE = np.array([[[0.1, 1.0, 0.3, 1.5]], [[0.2, 2.0, 0.0, 0.0]]])


def _golden_cases():
    for line in open(GOLDEN):
        if not line.startswith("case "):
            continue
        lhs, rhs = line[5:].split("->")
        db, sb = lhs.split()
        rhs = rhs.split()
        if rhs == ["none"]:
            yield float(db), int(sb), None
        else:
            yield float(db), int(sb), ([NAMES[rhs[0]], NAMES[rhs[1]]], int(rhs[2]), int(rhs[3]), float(rhs[4]))


@pytest.mark.parametrize("case", list(_golden_cases()))
def test_oracle_golden(case):
    db, sb, want = case
    got = op.optimize(GOLDEN_DAMAGE, db, sb)
    if want is None:
        assert got is None
        return
    kinds, (rd, st, dm) = got
    assert kinds[:, 0].tolist() == want[0]
    assert (rd, st) == (want[1], want[2]) and abs(dm - want[3]) < 1e-12


@pytest.mark.parametrize("case", list(_golden_cases()))
def test_library_golden(case):
    db, sb, want = case
    if want is None:
        with pytest.raises(abi.LoopKVError) as e:
            abi.loopkv_plan_optimize(GOLDEN_DAMAGE, db, sb)
        assert e.value.code == abi.E_PLAN
        return
    kinds, (rd, st, dm) = abi.loopkv_plan_optimize(GOLDEN_DAMAGE, db, sb)
    assert kinds[:, 0].tolist() == want[0]
    assert (rd, st) == (want[1], want[2]) and abs(dm - want[3]) < 1e-12


def test_oracle_closed_forms():
    rng = np.random.default_rng(1)
    d = rng.uniform(0.1, 1.0, (3, 2, 4))
    # unbounded budgets, reuse of a 2-bit cell free of damage: every
    # non-final cell reuses a 2-bit final cell (3 units of reads each, the
    # least possible; no other plan with those reads has less damage)
    d[..., 3] = 0.0
    kinds, (rd, st, _) = op.optimize(d, 1e9, 10 ** 9)
    assert rd == 3 * 6 and st == 3 * 2
    assert np.all(kinds[-1] == Q2) and np.all(kinds[:-1] == RU)
    # zero damage budget, zero 4-bit damage: everything stored at 4 bits
    d0 = d.copy()
    d0[..., 0] = 0.0
    kinds, (rd, st, dm) = op.optimize(d0, 0.0, 10 ** 9)
    assert np.all(kinds == Q4) and (rd, st, dm) == (4 * 6, 5 * 6, 0.0)


@pytest.mark.parametrize("R,L", [(1, 3), (2, 1), (2, 3), (3, 2), (4, 1)])
def test_library_matches_brute_force(R, L):
    rng = np.random.default_rng(100 * R + L)
    n_feasible = 0
    for trial in range(12):
        d = rng.exponential(1.0, (R, L, 4))
        lo = op.plan_cost(np.full((R, L), Q4), d)[2]
        hi = op.plan_cost(np.full((R, L), Q2), d)[2]
        db = float(rng.uniform(0.5 * min(lo, hi), 1.2 * max(lo, hi)))
        sb = int(rng.integers(3 * L, 5 * R * L + 1))
        want = op.optimize(d, db, sb)
        if want is None:
            with pytest.raises(abi.LoopKVError):
                abi.loopkv_plan_optimize(d, db, sb)
            continue
        n_feasible += 1
        kinds, (rd, st, dm) = abi.loopkv_plan_optimize(d, db, sb)
        assert (rd, st) == want[1][:2]
        assert abs(dm - want[1][2]) <= 1e-9 * max(1.0, abs(dm))
        assert op.plan_cost(kinds, d)[:2] == (rd, st)
        assert not np.any(kinds[-1] == RU)
    assert n_feasible > 0


def test_budgets_are_monotone():
    """More budget never costs more reads."""
    d = wl.synthetic_damage(wl.WORKLOADS["lean-16k"])
    last = None
    for frac in (0.2, 0.3, 0.5, 0.8, 1.0):
        db = frac * float(d[..., 1].sum())
        try:
            _, (rd, st, dm) = abi.loopkv_plan_optimize(d, db, 10 ** 9)
        except abi.LoopKVError:
            continue
        assert dm <= db * (1 + 1e-12)
        if last is not None:
            assert rd <= last
        last = rd
    assert last is not None


def test_planner_beats_lean_plan_at_its_budgets():
    """Given the hand-made memory-lean plan's own damage and storage as
    budgets, the search finds a plan that reads no more."""
    w = wl.WORKLOADS["lean-16k"]
    d = wl.synthetic_damage(w)
    lean, _ = wl.make_plan(w)
    rd, st, dm = op.plan_cost(lean, d)
    kinds, (rd2, st2, dm2) = abi.loopkv_plan_optimize(d, dm, st)
    assert rd2 <= rd and st2 <= st and dm2 <= dm * (1 + 1e-12)
    assert op.plan_cost(kinds, d)[:2] == (rd2, st2)


def test_planned_workload_plan():
    """The planned workload's plan is valid, within both budgets, and found
    in well under a second for 4 x 48 cells."""
    for name in ("planned-16k",):
        w = wl.WORKLOADS[name]
        t0 = time.perf_counter()
        kinds, taus = wl.make_plan(w)
        assert time.perf_counter() - t0 < 2.0
        assert kinds.shape == (w.loops, w.layers) and not np.any(kinds[-1] == RU)
        d = wl.synthetic_damage(w)
        rd, st, dm = op.plan_cost(kinds, d)
        db, sb = wl.planner_budgets(w)
        assert dm <= db * (1 + 1e-12) and st <= sb
    d = wl.synthetic_damage(wl.WORKLOADS["ouro2.6b-32k"])
    t0 = time.perf_counter()
    abi.loopkv_plan_optimize(d, float(d[..., 1].sum()) * 0.4, 10 ** 9)
    assert time.perf_counter() - t0 < 2.0
