"""Allocation-free decode (loopkv_decode_noalloc) against loopkv_decode.

Both run the same kernels with the same split layout; the allocation-free
entry point takes its partials and candidate lists from the library's fixed
device scratch instead of a caller workspace.  Two calls in a row (the
second with a smaller batch and shorter sequences, so stale scratch from the
first is present) must give the workspace path's bits, and those outputs
match the oracle.
"""
import math

import numpy as np
import pytest

from loop_aware_quantized_amd import abi
from loop_aware_quantized_amd import inputs as wl
from loop_aware_quantized_amd import runner
from oracle import attention as oa
from parity_util import compare_decode, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"
Q4, Q2, RU = wl.KIND_Q4, wl.KIND_Q2, wl.KIND_REUSE


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(wid, batch, lens, heads):
    w = wl.Workload(f"noalloc-{wid}", wid, batch=batch, loops=2, layers=3, heads=heads, head_dim=128, page=32,
                    ctx=max(lens), heavy_frac=0.01)
    kinds = [[Q4, Q2, RU], [Q4, Q4, Q4]]
    taus = [[0.01, 0.01, 0.005], [0.0, math.inf, 0.02]]
    st = runner.CacheState(w, DEV, kinds, taus, lengths=lens)
    kept = st.prefill({c: set(range(batch)) for c in st.stored})
    torch.cuda.synchronize()
    return st, kept


def _run(st, r, l, noalloc):
    w = st.w
    q = wl.cell_query(w, st.cell_index(r, l), DEV)[1]
    out = torch.full((w.batch, w.heads, w.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    mask = st.new_mask()
    cnt = torch.zeros(2, dtype=torch.int64, device=DEV)
    bt = st.batch(sum_seq_lens=int(st.lens0.sum()))
    if noalloc:
        opts = abi.make_opts(None, mask_bits=mask, counters=cnt)
        abi.loopkv_decode_noalloc(st.plan, st.cells, r, l, bt, q, out, opts)
    else:
        opts = abi.make_opts(st.workspace, mask_bits=mask, counters=cnt)
        abi.loopkv_decode(st.plan, st.cells, r, l, bt, q, out, opts)
    torch.cuda.synchronize()
    return q, out, mask, cnt


def test_noalloc_matches_workspace_decode_on_two_calls():
    # the larger call first, then a smaller one over the same scratch
    cases = [(250, 4, [3000, 2049, 700, 64], 4), (251, 2, [700, 33], 2)]
    for wid, batch, lens, heads in cases:
        st, kept = _case(wid, batch, lens, heads)
        for r in range(2):
            for l in range(3):
                need = abi.loopkv_decode_noalloc_bytes(st.plan, r, l, batch, st.max_seq_len,
                                                       int(st.lens0.sum()), 0)
                assert 0 < need <= abi.NOALLOC_SCRATCH_BYTES
                q, out_w, mask_w, cnt_w = _run(st, r, l, noalloc=False)
                _, out_n, mask_n, cnt_n = _run(st, r, l, noalloc=True)
                assert torch.equal(out_n.view(torch.int32), out_w.view(torch.int32)), (wid, r, l)
                assert torch.equal(mask_n, mask_w), (wid, r, l)
                assert torch.equal(cnt_n, cnt_w), (wid, r, l)
                src = oa.resolve_source(st.kinds, r, l)
                s = compare_decode(st, r, l, q, out_n, mask_n, kept[src], range(batch))
                say(f"  case {wid} cell ({r},{l}): scratch {need} B, bit-identical to the workspace path, "
                    f"rel err {s['rel']:.2e} flagged {s['flagged']}")


def test_noalloc_rejects_a_batch_above_the_scratch():
    """A 16K-token batch of 32 x 16 pairs with a tau mask needs about 70 MB of
    candidate lists: refused with LOOPKV_E_CAPACITY before any launch."""
    R, L, H, D, P = 1, 1, 16, 128, 32
    plan = abi.Plan(abi.plan_blob(R, L, H, D, P, np.array([[Q4]]), np.array([[0.01]])))
    B, T = 32, 16384
    need = abi.loopkv_decode_noalloc_bytes(plan, 0, 0, B, T, B * T, 0)
    assert need > abi.NOALLOC_SCRATCH_BYTES
    pages = B * T // P
    pool = torch.empty(plan.pool_bytes(0, 0, pages), dtype=torch.uint8, device=DEV)
    staging = torch.empty(plan.staging_bytes(0, 0, B), dtype=torch.uint8, device=DEV)
    cells = abi.cell_array(plan, {(0, 0): (pool, staging, pages, B)})
    table = torch.arange(pages, dtype=torch.int32, device=DEV).view(B, T // P)
    lens = torch.full((B,), T, dtype=torch.int32, device=DEV)
    q = torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(B, H, D, dtype=torch.float32, device=DEV)
    with pytest.raises(abi.LoopKVError) as e:
        abi.loopkv_decode_noalloc(plan, cells, 0, 0, abi.make_batch(lens, table, T, sum_seq_lens=B * T), q, out,
                                  abi.make_opts(None))
    assert e.value.code == abi.E_CAPACITY
