"""The streamed split layout's host bounds against a replica of the
kernels' range arithmetic (CPU only; no kernel runs).

The host (`loopkv_decode_layout`) reports, for a ragged batch with a
length-sum hint, the grid (waves), the main range length and the records
per (sequence, head).  The replica below restates what the stream and
merge kernels compute from the real lengths: tiles of all pairs laid end to
end (sequence-major, then head), ranges of tpw tiles for the first
main_waves ranges and of tail tiles after, ranges past the grid taken by
the last wave, one partial record per range that meets a pair, and the
first token of each record.  Checked for exact, too small and too large
hints: every tile lands in exactly one record, a pair's records are
numbered 0..n-1 in tile order, n stays within the reported bound, the
merge's first-token formula names each record's first tile, and no
segment is longer than a main range (the kernels size their page-table
slice by it).
"""
import numpy as np
import pytest

from loop_aware_quantized_amd import abi

TILE = 64
SLOTS = 256 * 12          # resident wave slots when no device is visible
TAIL = 16                 # tiles per second-round range


def _plan(H):
    kinds = np.zeros((1, 1), np.int32)
    return abi.Plan(abi.plan_blob(1, 1, H, 128, 32, kinds, np.array([[0.01]])))


def _ranges(tpw, mw, tt):
    rs = lambda w: w * tpw if w < mw else mw * tpw + (w - mw) * tt
    wo = lambda t: t // tpw if t < mw * tpw else mw + (t - mw * tpw) // tt
    return rs, wo


def _check(lens, H, hint):
    B, tm = len(lens), max(lens)
    p = _plan(H)
    streamed, S, ln, waves = abi.loopkv_decode_layout(p, 0, 0, B, tm, hint, 0)
    if not streamed:
        return None
    tpw = ln // TILE
    tt = min(TAIL, tpw)
    # main_waves from the host's rule, tied to the reported grid size
    tiles_ub = H * (-(-hint // TILE) + B)
    mw = min(SLOTS, -(-tiles_ub // tpw))
    assert waves == mw + -(-max(0, tiles_ub - mw * tpw) // tt)
    rs, wo = _ranges(tpw, mw, tt)
    nb = [-(-T // TILE) for T in lens]
    first = np.concatenate([[0], np.cumsum([H * n for n in nb])])
    total = int(first[-1])
    seen = {}
    # the stream kernel: wave w takes range w, the last wave the ranges past the grid
    todo = list(range(waves))
    w = waves
    while rs(w) < total:
        todo.append(w)
        w += 1
    for w in todo:
        t, te = rs(w), min(rs(w + 1), total)
        while t < te:
            b = int(np.searchsorted(first[:B], t, side="right") - 1)
            n = nb[b]
            h = (t - first[b]) // n
            j = t - first[b] - h * n
            seg = min(n - j, te - t)
            assert seg <= tpw
            rec = w - wo(first[b] + h * n)
            assert 0 <= rec < S, (rec, S)
            for jj in range(j, j + seg):
                assert (b, h, jj) not in seen
                seen[(b, h, jj)] = rec
            t += seg
    # the merge: records 0..n-1 of each pair, record r starting at its first tile
    for b in range(B):
        for h in range(H):
            n = nb[b]
            if n == 0:
                continue
            tile0 = int(first[b]) + h * n
            w0 = wo(tile0)
            used = wo(tile0 + n - 1) - w0 + 1
            assert used <= S
            got = {}
            for jj in range(n):
                got.setdefault(seen.pop((b, h, jj)), []).append(jj)
            assert sorted(got) == list(range(used))
            for r, js in got.items():
                assert max(0, rs(w0 + r) - tile0) == min(js)
                assert js == list(range(min(js), max(js) + 1))
    assert not seen
    return waves, S


@pytest.mark.parametrize("scale", [1.0, 0.5, 0.05, 1.3])
def test_streamed_ranges_cover_every_tile_once(scale):
    rng = np.random.default_rng(5)
    hit = 0
    for _ in range(12):
        B = int(rng.integers(2, 120))
        H = int(rng.choice([1, 4, 16]))
        lens = [int(x) for x in rng.integers(1, 12000, B)]
        lens[0] = 12000                     # a ragged batch under its maximum
        hint = max(1, int(sum(lens) * scale))
        if _check(lens, H, hint) is not None:
            hit += 1
    assert hit >= 6, "most draws take the streamed layout"


def test_streamed_layout_of_the_ragged_16k_shape():
    from loop_aware_quantized_amd import inputs as wl
    w = wl.WORKLOADS["ragged-16k"]
    lens = [int(x) for x in wl.make_lengths(w)]
    waves, S = _check(lens, w.heads, sum(lens))
    assert waves > SLOTS and S >= 2


def test_gpu_sweep_covers_every_layout():
    """The seeded GPU parity sweep (tests/test_gpu_sweep.py) decodes in the
    streamed layout, in uniform splits and in a single split per pair, so a
    change of the split choice cannot leave one of them untested there."""
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "gpu_sweep_cases", os.path.join(os.path.dirname(os.path.abspath(__file__)), "test_gpu_sweep.py"))
    sweep = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(sweep)
    seen = {"streamed": 0, "uniform": 0, "one split": 0}
    n_cases = len(sweep.test_random_configuration.pytestmark[0].args[1])
    for case in range(n_cases):
        D, P, H, R, L, B, lens, kinds, taus, o = sweep.draw_case(case)
        plan = abi.Plan(abi.plan_blob(R, L, H, D, P, np.array(kinds), np.array(taus)))
        hint = sum(lens) if o["hint"] else 0
        for r in range(R):
            for l in range(L):
                streamed, S, _, _ = abi.loopkv_decode_layout(plan, r, l, B, max(max(lens), 1), hint,
                                                             o["splits"])
                seen["streamed" if streamed else ("one split" if S == 1 else "uniform")] += 1
    assert all(v >= 5 for v in seen.values()), seen
