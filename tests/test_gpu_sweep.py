"""GPU parity over a seeded random sweep of small configurations.

Each case draws its own shape (head dim, page size, heads, loops, layers,
batch), ragged lengths (with the edge lengths 0, 1, 63, 64 and 65 mixed in),
a plan (reuse only before the final loop), per-cell tau from the fast paths
and the sparse range, page shuffling, heavy-token fraction, split count and
whether the length-sum hint is given, then checks every stored pool byte and
every decoded cell against the oracle (parity bar of tests/parity_util.py).
The draws come from numpy's seeded generator, so a case is reproduced by its
number alone.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from loop_aware_quantized_amd import abi
from loop_aware_quantized_amd import inputs as wl
from loop_aware_quantized_amd import runner
from parity_util import check_pool, compare_decode, say, tau_str

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0) if torch.cuda.is_available() else None
Q4, Q2, RU = wl.KIND_Q4, wl.KIND_Q2, wl.KIND_REUSE
TAUS = [0.0, 1e-3, 5e-3, 0.02, 0.1, math.inf]
EDGE_LENS = [0, 1, 63, 64, 65]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw_case(case: int):
    """Shape, lengths, plan and decode options of sweep case `case`."""
    rng = np.random.default_rng([7, case])
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64]))
    H = int(rng.integers(1, 6))
    R = int(rng.integers(1, 4))
    L = int(rng.integers(1, 4))
    B = int(rng.integers(1, 9))
    lens = [int(x) for x in rng.integers(0, 6001, size=B)]
    for i in range(B):
        if rng.random() < 0.3:
            lens[i] = int(rng.choice(EDGE_LENS))
    kinds = [[int(rng.choice([Q4, Q2, RU] if r < R - 1 else [Q4, Q2])) for _ in range(L)] for r in range(R)]
    taus = [[float(rng.choice(TAUS)) for _ in range(L)] for _ in range(R)]
    opts = dict(shuffle=bool(rng.random() < 0.5), heavy=float(rng.choice([0.0, 0.01, 0.05])),
                splits=int(rng.choice([0, 0, 1, 2, 5])), hint=bool(rng.random() < 0.7))
    return D, P, H, R, L, B, lens, kinds, taus, opts


@pytest.mark.parametrize("case", range(40))
def test_random_configuration(case):
    D, P, H, R, L, B, lens, kinds, taus, o = draw_case(case)
    say(f"sweep case {case}: D={D} P={P} H={H} R={R} L={L} B={B} lens={lens} kinds={kinds} "
        f"taus={[[tau_str(t) for t in row] for row in taus]} {o}")
    w = wl.Workload(f"sweep-{case}", 300 + case, batch=B, loops=R, layers=L, heads=H, head_dim=D, page=P,
                    ctx=max(max(lens), 1), heavy_frac=o["heavy"], shuffle_pages=o["shuffle"])
    st = runner.CacheState(w, DEV, kinds, taus, lengths=lens)
    kept = st.prefill({c: set(range(B)) for c in st.stored})
    torch.cuda.synchronize()
    for (r, l) in st.stored:
        for b in range(B):
            if lens[b] > 0:                  # an empty sequence stores nothing
                check_pool(st, r, l, b, *kept[(r, l)][b])
    for r in range(R):
        for l in range(L):
            q = wl.cell_query(w, st.cell_index(r, l), DEV)[1]
            out = torch.empty(B, H, D, dtype=torch.float32, device=DEV)
            mask = st.new_mask()
            st.decode(r, l, q, out, num_splits=o["splits"], mask=mask,
                      sum_seq_lens=None if o["hint"] else 0)
            torch.cuda.synchronize()
            src = oa.resolve_source(st.kinds, r, l)
            s = compare_decode(st, r, l, q, out, mask, kept[src], range(B))
            say(f"  cell ({r},{l}) src {src} tau {tau_str(taus[r][l])}: rel err {s['rel']:.2e} "
                f"flagged {s['flagged']} band {s['band']}")
            # the allocation-free entry point runs the same kernels and layout:
            # the same bits, whenever the batch fits its fixed scratch
            hint = int(st.lens0.sum()) if o["hint"] else 0
            if abi.loopkv_decode_noalloc_bytes(st.plan, r, l, B, st.max_seq_len, hint, o["splits"]) \
                    <= abi.NOALLOC_SCRATCH_BYTES:
                out2 = torch.full_like(out, float("nan"))
                mask2 = st.new_mask()
                opts = abi.make_opts(None, mask_bits=mask2, num_splits=o["splits"])
                abi.loopkv_decode_noalloc(st.plan, st.cells, r, l, st.batch(sum_seq_lens=hint), q, out2, opts)
                torch.cuda.synchronize()
                assert torch.equal(out, out2) and torch.equal(mask, mask2), (r, l)


def test_all_sequences_empty():
    """A batch whose every sequence is empty decodes to zeros in every mode
    (4-bit sparse, dense and plain, 2-bit, reuse) and sets no mask bit."""
    w = wl.Workload("all-empty", 350, batch=3, loops=2, layers=3, heads=2, head_dim=128, page=16, ctx=1)
    kinds = [[Q4, Q2, RU], [Q4, Q4, Q2]]
    taus = [[0.01, 0.01, 0.0], [0.0, math.inf, 0.02]]
    st = runner.CacheState(w, DEV, kinds, taus, lengths=[0, 0, 0])
    st.prefill({c: set() for c in st.stored})
    for r in range(2):
        for l in range(3):
            q = wl.cell_query(w, st.cell_index(r, l), DEV)[1]
            out = torch.full((3, 2, 128), float("nan"), dtype=torch.float32, device=DEV)
            mask = st.new_mask()
            st.decode(r, l, q, out, mask=mask)
            torch.cuda.synchronize()
            assert torch.count_nonzero(out) == 0, (r, l)
            assert mask.numel() == 0 or torch.count_nonzero(mask) == 0, (r, l)


@pytest.mark.parametrize("case", range(12))
def test_append_random_schedules(case):
    """Random starting lengths per sequence, then a random schedule of
    appends (1 to 70 tokens per call, the same count for every sequence from
    its own length), crossing key groups and pages: every pool byte equals
    the oracle's packing of the whole sequence, and decodes match."""
    rng = np.random.default_rng([13, case])
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64]))
    H = int(rng.integers(1, 4))
    B = int(rng.integers(1, 5))
    start = rng.integers(0, 201, size=B).astype(np.int32)
    steps = [int(rng.choice([1, 1, 1, 2, 5, 31, 32, 33, 70])) for _ in range(int(rng.integers(1, 7)))]
    final = start + sum(steps)
    taus = [[float(rng.choice(TAUS)), float(rng.choice(TAUS))]]
    say(f"append case {case}: D={D} P={P} H={H} B={B} start={start.tolist()} steps={steps}")
    w = wl.Workload(f"append-sweep-{case}", 360 + case, batch=B, loops=1, layers=2, heads=H, head_dim=D, page=P,
                    ctx=int(final.max()), heavy_frac=0.02, shuffle_pages=bool(rng.random() < 0.5))
    st = runner.CacheState(w, DEV, [[Q4, Q2]], taus, lengths=final)
    T = int(final.max())
    kept = {}
    for (r, l) in st.stored:
        K, V = wl.cell_kv(w, st.cell_index(r, l), T, DEV)
        for bi in range(B):
            n0 = int(start[bi])
            if n0:
                lens = torch.zeros(1, dtype=torch.int32, device=DEV)
                batch = abi.make_batch(lens, st.block_tables[bi:bi + 1], st.max_seq_len,
                                       slots=st.slots[bi:bi + 1])
                abi.loopkv_append(st.plan, st.cells, r, l, batch, n0, K[bi:bi + 1, :n0].contiguous(),
                                  V[bi:bi + 1, :n0].contiguous())
        cur = start.copy()
        for n in steps:
            idx = torch.from_numpy((cur[:, None] + np.arange(n)[None, :]).astype(np.int64)).to(DEV)
            kk = torch.stack([K[bi, idx[bi]] for bi in range(B)])
            vv = torch.stack([V[bi, idx[bi]] for bi in range(B)])
            st.append(r, l, kk, vv, torch.from_numpy(cur).to(DEV))
            cur = cur + n
        kept[(r, l)] = {bi: (wl.bf16_bits(K[bi, :int(final[bi])]), wl.bf16_bits(V[bi, :int(final[bi])]))
                        for bi in range(B)}
    torch.cuda.synchronize()
    for (r, l) in st.stored:
        for bi in range(B):
            check_pool(st, r, l, bi, *kept[(r, l)][bi])
    for l in range(2):
        q = wl.cell_query(w, st.cell_index(0, l), DEV)[1]
        out = torch.empty(B, H, D, dtype=torch.float32, device=DEV)
        mask = st.new_mask()
        st.decode(0, l, q, out, mask=mask)
        torch.cuda.synchronize()
        compare_decode(st, 0, l, q, out, mask, kept[(0, l)], range(B))
