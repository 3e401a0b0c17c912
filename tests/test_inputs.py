"""Host logic of the seeded synthetic workloads: plans, lengths, page tables,
and the storage a plan needs (computed by the library's host functions)."""
import math

import numpy as np
import pytest

from loop_aware_quantized_amd import abi
from loop_aware_quantized_amd import inputs as wl

Q4, Q2, RU = wl.KIND_Q4, wl.KIND_Q2, wl.KIND_REUSE


def _counts(row):
    return tuple(int((row == k).sum()) for k in (Q4, Q2, RU))


def test_tiny_plan_is_layer_major():
    kinds, taus = wl.make_plan(wl.WORKLOADS["tiny"])
    assert kinds.tolist() == [[Q4, RU], [Q2, Q4]]
    assert np.all(taus == 0.02)


def test_random_plan_fractions_and_reuse_placement():
    w = wl.WORKLOADS["ouro1.4b-4k"]
    kinds, taus = wl.make_plan(w)
    assert _counts(kinds.ravel()) == (38, 34, 24)
    assert not np.any(kinds[-1] == RU), "reuse only in loops 0 .. R-2"
    assert set(np.unique(taus)) <= {0.005, 0.01, 0.02}
    again, _ = wl.make_plan(w)
    assert np.array_equal(kinds, again), "plans are seeded"


@pytest.mark.parametrize("name,mult", [("lean-16k", 1), ("ouro2.6b-32k", 2)])
def test_lean_plan_counts_per_loop(name, mult):
    kinds, taus = wl.make_plan(wl.WORKLOADS[name])
    want = [(14, 4, 6), (6, 8, 10), (2, 4, 18), (2, 22, 0)]
    for r in range(4):
        assert _counts(kinds[r]) == tuple(c * mult for c in want[r])
    assert np.all(taus == 0.01)


def test_kivi4_plan():
    kinds, taus = wl.make_plan(wl.WORKLOADS["kivi4-16k"])
    assert np.all(kinds == Q4) and np.all(taus == 0.0)


def test_ragged_lengths_and_shuffled_tables():
    w = wl.WORKLOADS["ragged-16k"]
    lens = wl.make_lengths(w)
    assert lens.shape == (64,) and lens.min() >= 512 and lens.max() <= 16384
    table, num_pages = wl.make_block_tables(w, lens)
    pages = (lens + 15) // 16
    assert num_pages == pages.sum()
    used = np.concatenate([table[b, :pages[b]] for b in range(w.batch)])
    assert np.array_equal(np.sort(used), np.arange(num_pages)), "a permutation of the pool"
    assert not np.array_equal(used, np.arange(num_pages)), "shuffled"


def _stored_bytes(w, kinds, tokens_per_seq):
    p = abi.Plan(abi.plan_blob(w.loops, w.layers, w.heads, w.head_dim, w.page, kinds,
                               np.zeros(kinds.shape)))
    pages = w.batch * -(-tokens_per_seq // w.page)
    return sum(p.pool_bytes(r, l, pages) for r in range(w.loops) for l in range(w.layers)
               if kinds[r, l] != RU)


def test_lean_plan_storage_vs_all_4bit():
    """The lean 25/40/35 mix stores 51% fewer bytes than an all-4-bit plan
    (two 2-bit planes of a 4-bit cell vs one of a 2-bit cell, plus shared
    metadata; reuse stores nothing)."""
    w = wl.WORKLOADS["lean-16k"]
    lean, _ = wl.make_plan(w)
    kivi, _ = wl.make_plan(wl.WORKLOADS["kivi4-16k"])
    a, b = _stored_bytes(w, lean, 16385), _stored_bytes(w, kivi, 16385)
    # per token-head: 4-bit 160 B (4 planes of 32 B + 32 B meta), 2-bit 96 B
    per_tok = (24 * 160 + 38 * 96) / (96 * 160)
    assert math.isclose(a / b, per_tok, rel_tol=1e-9)
    assert 0.51 < 1 - a / b < 0.52      # 51.25%
