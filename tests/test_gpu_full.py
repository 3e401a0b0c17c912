"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic split count, whole batch per call).

For each workload, a few cells covering every source kind (4-bit, 2-bit,
reuse of a 4-bit cell, reuse of a 2-bit cell) are prefilled at full size and
decoded for the whole batch; sampled sequences are compared against the CPU
oracle (pool bytes bit-exact, masks outside the ambiguity band bit-exact,
outputs within 2e-3 of the output's L_inf norm).
"""
import math

import numpy as np
import pytest

from loop_aware_quantized_amd import abi
from loop_aware_quantized_amd import inputs as wl
from loop_aware_quantized_amd import runner
from oracle import attention as oa
from parity_util import check_pool, compare_decode, say, tau_str

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def _pick_cells(kinds):
    """One cell per (reuse?, source kind) class, smallest loop/layer first."""
    R, L = kinds.shape
    picked = {}
    for r in range(R):
        for l in range(L):
            k = int(kinds[r, l])
            src = int(kinds[R - 1, l]) if k == wl.KIND_REUSE else k
            picked.setdefault((k == wl.KIND_REUSE, src), (r, l))
    return sorted(picked.values())


def _sources(kinds, cells):
    return sorted({oa.resolve_source(kinds, r, l) for (r, l) in cells})


def _run(w, seqs, taus=None, append=False, tau_sweep=()):
    kinds, plan_taus = wl.make_plan(w)
    if taus is not None:
        plan_taus = taus
    cells = _pick_cells(kinds)
    srcs = _sources(kinds, cells)
    say(f"{w.name}: cells {cells} sources {srcs} sequences {seqs}")
    st = runner.CacheState(w, DEV, kinds, plan_taus, extra_tokens=1 if append else 0,
                           only_cells=set(srcs))
    kept = {}
    for (r, l) in srcs:
        kept[(r, l)] = st.prefill_cell(r, l, set(seqs))
    lens = st.lens0.copy()
    if append:
        # one appended token per sequence on every source cell, as in a decode step
        lens_dev = torch.from_numpy(lens.astype(np.int32)).to(DEV)
        for (r, l) in srcs:
            k, v = wl.append_kv(w, st.cell_index(r, l), 0, 1, DEV)
            st.append(r, l, k, v, lens_dev)
            kb, vb = wl.bf16_bits(k), wl.bf16_bits(v)
            for b in seqs:
                ok, ov = kept[(r, l)][b]
                kept[(r, l)][b] = (np.concatenate([ok, kb[b]]), np.concatenate([ov, vb[b]]))
        lens = lens + 1
    lens_dev = torch.from_numpy(lens.astype(np.int32)).to(DEV)
    torch.cuda.synchronize()
    for (r, l) in srcs:
        for b in seqs:
            check_pool(st, r, l, b, *kept[(r, l)][b], T=int(lens[b]))
    sweep = tau_sweep or (None,)
    for tau in sweep:
        if tau is not None:
            st.taus = wl.with_tau(plan_taus, tau)
            st.plan = abi.Plan(abi.plan_blob(w.loops, w.layers, w.heads, w.head_dim, w.page,
                                             st.kinds, st.taus))
        for (r, l) in cells:
            q = wl.cell_query(w, st.cell_index(r, l), DEV)[1]
            out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV)
            mask = st.new_mask()
            st.decode(r, l, q, out, mask=mask, lens=lens_dev, sum_seq_lens=int(lens.sum()))
            torch.cuda.synchronize()
            src = oa.resolve_source(st.kinds, r, l)
            s = compare_decode(st, r, l, q, out, mask, kept[src], seqs, lens=lens)
            say(f"  cell ({r},{l}) src {src} kind {st.kinds[src]} tau {tau_str(st.taus[r, l])}: "
                f"rel err {s['rel']:.2e} flagged {s['flagged']} band {s['band']}")
    return st


def test_full_ouro14b_4k():
    _run(wl.WORKLOADS["ouro1.4b-4k"], seqs=[0, 5])


def test_full_lean_16k_with_append():
    _run(wl.WORKLOADS["lean-16k"], seqs=[3, 31], append=True)


def test_full_ragged_16k():
    w = wl.WORKLOADS["ragged-16k"]
    lens = wl.make_lengths(w)
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 17})
    _run(w, seqs=seqs)


def test_full_ouro26b_32k_tau_sweep():
    w = wl.WORKLOADS["ouro2.6b-32k"]
    _run(w, seqs=[2], tau_sweep=w.tau_sweep)


def test_full_kivi4_16k_dense():
    # same shape and data as lean-16k, every cell 4-bit with tau = 0
    _run(wl.WORKLOADS["kivi4-16k"], seqs=[0, 31], append=True)


def test_full_planned_16k():
    # the offline planner's plan on the lean-16k shape and data
    _run(wl.WORKLOADS["planned-16k"], seqs=[1, 30], append=True)
