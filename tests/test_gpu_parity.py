"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Sizes here span several 64-token tiles, every page size, both head dims,
ragged tails, empty sequences, all three decode modes (tau = 0, finite tau,
tau = +inf), 2-bit cells and reuse cells of both source kinds.
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
Q4, Q2, RU = wl.KIND_Q4, wl.KIND_Q2, wl.KIND_REUSE


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decode(st, r, l, num_splits=0, q=None, sm_scale=1.0):
    w = st.w
    if q is None:
        q = wl.cell_query(w, st.cell_index(r, l), DEV)[1]
    out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV)
    mask = st.new_mask()
    cnt = torch.zeros(2, dtype=torch.int64, device=DEV)
    st.decode(r, l, q, out, num_splits=num_splits, mask=mask, counters=cnt, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return q, out, mask, cnt


def _all_cells(st, kept, seqs, num_splits=0):
    stats = {}
    for r in range(st.w.loops):
        for l in range(st.w.layers):
            q, out, mask, cnt = _decode(st, r, l, num_splits)
            src = oa.resolve_source(st.kinds, r, l)
            s = compare_decode(st, r, l, q, out, mask, kept[src], seqs)
            stats[(r, l)] = s
            say(f"  cell ({r},{l}) src {src} kind {st.kinds[src]} tau {tau_str(st.taus[r, l])}: "
                f"rel err {s['rel']:.2e} flagged {s['flagged']} band {s['band']}")
    return stats


def test_tiny_workload_end_to_end():
    w = wl.WORKLOADS["tiny"]
    st = runner.CacheState(w, DEV)
    kept = st.prefill({c: set(range(w.batch)) for c in st.stored})
    torch.cuda.synchronize()
    for (r, l) in st.stored:
        for b in range(w.batch):
            check_pool(st, r, l, b, *kept[(r, l)][b])
    stats = _all_cells(st, kept, range(w.batch))
    assert sum(s["flagged"] for s in stats.values()) > 0, "tiny workload should flag heavy tokens"


MIXED_KINDS = [[Q4, Q2, RU, RU], [Q4, Q4, Q2, Q4]]
MIXED_TAUS = [[0.01, 0.02, 0.0, 0.005], [0.0, math.inf, 0.01, 0.03]]
MIXED_LENS = [1, 63, 64, 65, 700, 2049]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("P", [16, 32, 64])
def test_mixed_plan_ragged(D, P):
    say(f"mixed plan D={D} P={P}")
    w = wl.Workload(f"mixed-{D}-{P}", 100 + D + P, batch=len(MIXED_LENS), loops=2, layers=4,
                    heads=3, head_dim=D, page=P, ctx=max(MIXED_LENS), heavy_frac=0.01,
                    shuffle_pages=(P == 16))
    st = runner.CacheState(w, DEV, MIXED_KINDS, MIXED_TAUS, lengths=MIXED_LENS)
    kept = st.prefill({c: set(range(w.batch)) for c in st.stored})
    torch.cuda.synchronize()
    for (r, l) in st.stored:
        for b in range(w.batch):
            check_pool(st, r, l, b, *kept[(r, l)][b])
    _all_cells(st, kept, range(w.batch))


def test_empty_and_short_sequences():
    w = wl.Workload("short", 130, batch=4, loops=1, layers=2, heads=2, head_dim=128, page=16,
                    ctx=300, heavy_frac=0.02)
    st = runner.CacheState(w, DEV, [[Q4, Q2]], [[0.01, 0.01]], lengths=[0, 5, 300, 32])
    kept = st.prefill({c: set(range(w.batch)) for c in st.stored})
    torch.cuda.synchronize()
    for l in range(2):
        q, out, mask, _ = _decode(st, 0, l)
        assert torch.all(out[0] == 0)
        compare_decode(st, 0, l, q, out, mask, kept[(0, l)], range(w.batch))


def test_split_counts_and_page_shuffle():
    """num_splits 1 / 3 / auto all match the oracle; shuffled page tables give
    bit-identical outputs to contiguous ones."""
    kinds, taus = [[Q4, Q2]], [[0.005, 0.005]]
    lens = [3000, 4096, 1500]
    outs = {}
    for shuffle in (False, True):
        w = wl.Workload("splits", 140, batch=3, loops=1, layers=2, heads=4, head_dim=128, page=16,
                        ctx=4096, heavy_frac=0.01, shuffle_pages=shuffle)
        st = runner.CacheState(w, DEV, kinds, taus, lengths=lens)
        kept = st.prefill({c: set(range(3)) for c in st.stored})
        for l in range(2):
            for ns in (1, 3, 0):
                q, out, mask, _ = _decode(st, 0, l, num_splits=ns)
                compare_decode(st, 0, l, q, out, mask, kept[(0, l)], range(3))
                outs[(shuffle, l, ns)] = (out.cpu().numpy(), mask.cpu().numpy())
    for l in range(2):
        for ns in (1, 3, 0):
            a, b = outs[(False, l, ns)], outs[(True, l, ns)]
            assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
            assert np.array_equal(a[1], b[1])


@pytest.mark.parametrize("tau", [1e-4, 1e-3])
def test_small_tau_candidate_spill(tau):
    """Thresholds so low that a split's candidates overflow the on-chip
    buffer (one 4096-token split: up to 1/tau survivors) still flag exactly
    the oracle's tokens."""
    w = wl.Workload("spill", 170, batch=2, loops=1, layers=2, heads=2, head_dim=128, page=32,
                    ctx=4096, heavy_frac=0.0)
    st = runner.CacheState(w, DEV, [[Q4, Q4]], [[tau, tau]], lengths=[4096, 3001])
    kept = st.prefill({c: set(range(2)) for c in st.stored})
    for l in range(2):
        for ns in (1, 0):
            q, out, mask, cnt = _decode(st, 0, l, num_splits=ns)
            s = compare_decode(st, 0, l, q, out, mask, kept[(0, l)], range(2))
            say(f"  tau {tau} splits {ns}: rel err {s['rel']:.2e} flagged {s['flagged']} band {s['band']}")
            assert s["flagged"] > 0


@pytest.mark.parametrize("vscale", [1.0, 1e-2, 1e-4, 1e-5])
def test_small_value_magnitudes(vscale):
    """Values of magnitude 1 down to 1e-5 (value scales deep in fp16's
    subnormal range): 4-bit sparse, plain and dense cells and a 2-bit cell,
    with one split and the automatic layout, stay within the 2e-3 bound.
    The split pass's fp16 value weights p * s would lose it below 1e-4
    without the weight exponent it carries."""
    w = wl.Workload(f"vscale-{vscale:g}", 240, batch=3, loops=1, layers=4, heads=4, head_dim=128, page=32,
                    ctx=3000, heavy_frac=0.01, value_scale=vscale)
    st = runner.CacheState(w, DEV, [[Q4, Q4, Q4, Q2]], [[0.01, math.inf, 0.0, 0.01]],
                           lengths=[3000, 1777, 64])
    kept = st.prefill({c: set(range(3)) for c in st.stored})
    worst = 0.0
    for l in range(4):
        for ns in (1, 0):
            q, out, mask, _ = _decode(st, 0, l, num_splits=ns)
            s = compare_decode(st, 0, l, q, out, mask, kept[(0, l)], range(3))
            worst = max(worst, s["rel"])
            say(f"  vscale {vscale:g} layer {l} splits {ns}: rel err {s['rel']:.2e} |o| {s['scale']:.2e} "
                f"flagged {s['flagged']} band {s['band']}")
    assert worst < 1e-3


def test_near_uniform_batch_vs_one_split():
    """16 x 16 (sequence, head) pairs of near-equal length in the automatic
    split layout: every mode matches the oracle, and the outputs match the
    one-split-per-pair layout's."""
    w = wl.Workload("ranked", 190, batch=16, loops=1, layers=3, heads=16, head_dim=128, page=32,
                    ctx=6000, heavy_frac=0.01)
    lens = [6000 - 7 * i for i in range(16)]
    st = runner.CacheState(w, DEV, [[Q4, Q2, Q4]], [[0.01, 0.01, 0.0]], lengths=lens)
    seqs = [0, 15]
    kept = st.prefill({c: set(seqs) for c in st.stored})
    for l in range(3):
        q, out, mask, _ = _decode(st, 0, l)
        s = compare_decode(st, 0, l, q, out, mask, kept[(0, l)], seqs)
        q1, out1, mask1, _ = _decode(st, 0, l, num_splits=1, q=q)
        rel = float((out - out1).abs().max() / out1.abs().max())
        say(f"  layer {l}: rel err {s['rel']:.2e} flagged {s['flagged']}; vs one split {rel:.2e}")
        assert rel < 1e-3


def test_concurrent_streams_own_workspaces():
    """Decodes of three cells (every mode) issued on three streams at once,
    each with its own workspace, output, mask and counters, give the same
    bits as the same decodes one after another on the default stream."""
    w = wl.Workload("streams", 230, batch=4, loops=1, layers=3, heads=4, head_dim=128, page=32,
                    ctx=3000, heavy_frac=0.01)
    st = runner.CacheState(w, DEV, [[Q4, Q2, Q4]], [[0.01, 0.01, 0.0]])
    st.prefill()
    ws_bytes = st.plan.decode_workspace_bytes(w.batch, st.max_seq_len)

    def run(l, stream, ws):
        q = wl.cell_query(w, st.cell_index(0, l), DEV)[1]
        out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV)
        mask = st.new_mask()
        cnt = torch.zeros(2, dtype=torch.int64, device=DEV)
        opts = abi.make_opts(ws, mask_bits=mask, counters=cnt)
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())   # inputs were made on the default stream
        abi.loopkv_decode(st.plan, st.cells, 0, l, st.batch(sum_seq_lens=int(st.lens0.sum())), q, out, opts,
                          stream=stream)
        return out, mask, cnt

    ref = {}
    for l in range(3):
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
        ref[l] = run(l, None, ws)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=DEV) for _ in range(3)]
    torch.cuda.synchronize()
    for rep in range(3):
        got = {l: run(l, streams[l], wss[l]) for l in range(3)}
        torch.cuda.synchronize()
        for l in range(3):
            for a, b in zip(got[l], ref[l]):
                assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                                   b.view(torch.int32) if b.dtype == torch.float32 else b), (rep, l)


@pytest.mark.timeout(300)
def test_long_sequence_few_pairs():
    """A 600K-token sequence over two (sequence, head) pairs: the automatic
    layout would want more than the 2048 splits a pair may have, so splits
    grow instead.  A tau near 1/T flags many tokens (long candidate lists,
    several gather passes).  The oracle side takes about half a minute."""
    lens = [600_003, 1000]
    w = wl.Workload("long", 210, batch=2, loops=1, layers=1, heads=1, head_dim=128, page=64,
                    ctx=max(lens), heavy_frac=0.0)
    st = runner.CacheState(w, DEV, [[Q4]], [[1e-6]], lengths=lens)
    kept = st.prefill({c: {0, 1} for c in st.stored})
    q, out, mask, cnt = _decode(st, 0, 0)
    s = compare_decode(st, 0, 0, q, out, mask, kept[(0, 0)], [0, 1])
    say(f"  rel err {s['rel']:.2e} flagged {s['flagged']} band {s['band']}")
    assert s["flagged"] > 1000


@pytest.mark.parametrize("sm_scale", [0.0883883, 12.0])
def test_sm_scale_flat_and_peaky(sm_scale):
    """Score scales other than 1 in every mode: 1/sqrt(128) (a flat softmax,
    few tokens reach tau) and 12 (a peaky one, a few tokens hold most of the
    weight) match the oracle at the same scale, with one split and with the
    automatic layout."""
    w = wl.Workload("scale", 210, batch=3, loops=2, layers=3, heads=4, head_dim=128, page=32,
                    ctx=2500, heavy_frac=0.01)
    kinds = [[RU, Q2, Q4], [Q4, Q4, Q2]]
    taus = [[0.002, 0.01, 0.01], [0.0, math.inf, 0.01]]
    st = runner.CacheState(w, DEV, kinds, taus, lengths=[2500, 777, 64])
    kept = st.prefill({c: set(range(3)) for c in st.stored})
    flagged = 0
    for r in range(2):
        for l in range(3):
            src = oa.resolve_source(st.kinds, r, l)
            for ns in (1, 0):
                q, out, mask, _ = _decode(st, r, l, num_splits=ns, sm_scale=sm_scale)
                s = compare_decode(st, r, l, q, out, mask, kept[src], range(3), sm_scale=sm_scale)
                flagged += s["flagged"]
                say(f"  scale {sm_scale} cell ({r},{l}) splits {ns}: rel err {s['rel']:.2e} "
                    f"flagged {s['flagged']} band {s['band']}")
    if sm_scale > 1.0:
        assert flagged > 0


def test_max_batch_short_sequences():
    """The largest batch one call takes (65535 sequences, the grids' batch
    dimension) of 40-token sequences: appends and decodes of a 4-bit sparse
    and a 2-bit cell match the oracle on sampled sequences, first and last
    included."""
    B = 65535
    w = wl.Workload("maxbatch", 220, batch=B, loops=1, layers=2, heads=2, head_dim=64, page=16,
                    ctx=40, heavy_frac=0.05)
    T = 40
    st = runner.CacheState(w, DEV, [[Q4, Q2]], [[0.05, 0.05]], lengths=[T] * B)
    seqs = [0, 1, 4097, 32767, B - 2, B - 1]
    # one bulk draw per cell (the per-sequence draws of the workload
    # generator would take minutes at this batch)
    g = torch.Generator(device=DEV)
    g.manual_seed(220)
    kept = {}
    zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
    for l in range(2):
        K = torch.randn(B, T, w.heads, w.head_dim, generator=g, device=DEV).to(torch.bfloat16)
        V = torch.randn(B, T, w.heads, w.head_dim, generator=g, device=DEV).to(torch.bfloat16)
        batch = abi.make_batch(zeros, st.block_tables, st.max_seq_len)
        abi.loopkv_append(st.plan, st.cells, 0, l, batch, T, K, V)
        kept[(0, l)] = {b: (wl.bf16_bits(K[b]), wl.bf16_bits(V[b])) for b in seqs}
        del K, V
    torch.cuda.synchronize()
    for l in range(2):
        for b in seqs:
            check_pool(st, 0, l, b, *kept[(0, l)][b])
        q, out, mask, _ = _decode(st, 0, l)
        s = compare_decode(st, 0, l, q, out, mask, kept[(0, l)], seqs)
        say(f"  layer {l}: rel err {s['rel']:.2e} flagged {s['flagged']} band {s['band']}")
        assert torch.isfinite(out).all()


def test_many_short_ragged_pairs():
    """4096 sequences x 16 heads of 32-128 tokens with the ragged length hint
    (the regime where the ragged rule alone asks for splits longer than any
    sequence): one split per pair, as long as the longest sequence, so the
    candidate lists stay inside the workspace; sampled sequences of a 4-bit
    sparse cell (most tokens are candidates at these lengths) and a 2-bit
    cell match the oracle."""
    B, T, H, D = 4096, 128, 16, 64
    w = wl.Workload("manypairs", 230, batch=B, loops=1, layers=2, heads=H, head_dim=D, page=16,
                    ctx=T, heavy_frac=0.0)
    st = runner.CacheState(w, DEV, [[Q4, Q2]], [[0.01, 0.01]], lengths=[T] * B)
    rng = np.random.default_rng(230)
    # attended lengths are whole key groups, so a prefix of the stored
    # 128-token sequence is exactly the cache of that prefix
    lens_np = (32 * rng.integers(1, 5, size=B)).astype(np.int32)
    lens = torch.from_numpy(lens_np).to(DEV)
    hint = int(lens_np.sum())
    assert st.plan.decode_splits(B, T, hint, 0) == (1, T)
    seqs = sorted({0, 1, 2047, B - 2, B - 1, *rng.choice(B, 5, replace=False).tolist()})
    g = torch.Generator(device=DEV)
    g.manual_seed(230)
    kept = {}
    zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
    for l in range(2):
        K = torch.randn(B, T, H, D, generator=g, device=DEV).to(torch.bfloat16)
        V = torch.randn(B, T, H, D, generator=g, device=DEV).to(torch.bfloat16)
        abi.loopkv_append(st.plan, st.cells, 0, l, abi.make_batch(zeros, st.block_tables, st.max_seq_len),
                          T, K, V)
        kept[(0, l)] = {b: (wl.bf16_bits(K[b]), wl.bf16_bits(V[b])) for b in seqs}
        del K, V
    torch.cuda.synchronize()
    for l in range(2):
        q = wl.cell_query(w, st.cell_index(0, l), DEV)[1]
        out = torch.empty(B, H, D, dtype=torch.float32, device=DEV)
        mask = st.new_mask()
        st.decode(0, l, q, out, mask=mask, lens=lens, sum_seq_lens=hint)
        torch.cuda.synchronize()
        s = compare_decode(st, 0, l, q, out, mask, kept[(0, l)], seqs, lens=lens_np)
        say(f"  layer {l}: rel err {s['rel']:.2e} flagged {s['flagged']} band {s['band']}")
        assert torch.isfinite(out).all()


@pytest.mark.parametrize("hint_scale", [1.0, 0.5, 0.05, 1.45])
def test_streamed_layout_any_length_hint(hint_scale):
    """A ragged batch in the streamed split layout, with the length-sum hint
    exact, too small (tiles past the ranges go to the last wave) and too
    large: every sampled sequence matches the oracle."""
    B, H = 24, 8
    lens = np.random.default_rng(77).integers(100, 6000, B).astype(np.int64)
    lens[3] = 6000
    w = wl.Workload("hint", 195, batch=B, loops=1, layers=2, heads=H, head_dim=128, page=32,
                    ctx=6000, heavy_frac=0.01)
    st = runner.CacheState(w, DEV, [[Q4, Q2]], [[0.01, math.inf]], lengths=list(lens))
    seqs = [0, 3, B - 1]
    kept = st.prefill({c: set(seqs) for c in st.stored})
    hint = max(1, int(lens.sum() * hint_scale))
    streamed, S, ln, waves = abi.loopkv_decode_layout(st.plan, 0, 0, B, 6000, hint, 0)
    assert streamed, "a ragged batch with a length hint takes the streamed layout"
    for l in range(2):
        q = wl.cell_query(w, st.cell_index(0, l), DEV)[1]
        out = torch.empty(B, H, w.head_dim, dtype=torch.float32, device=DEV)
        mask = st.new_mask()
        st.decode(0, l, q, out, mask=mask, sum_seq_lens=hint)
        torch.cuda.synchronize()
        s = compare_decode(st, 0, l, q, out, mask, kept[(0, l)], seqs)
        say(f"  hint x{hint_scale} layer {l}: {waves} waves, {S} records per pair, rel err {s['rel']:.2e}")


@pytest.mark.parametrize("ragged", [False, True])
def test_graph_replay_matches_eager(ragged):
    """Appends and decodes captured in one HIP graph give, on every replay,
    the same bytes as the same calls made eagerly (eager work and
    synchronizations run between the replays), and every replay's outputs
    and masks match the oracle on the sequence as it stands after that
    replay's append.  Ragged: the calls carry a length-sum hint of half the
    real sum, so the streamed layout fixed at capture leaves tiles past its
    grid (taken by the last wave), more of them on every replay."""
    w = wl.Workload("graph", 180, batch=3, loops=2, layers=2, heads=4, head_dim=128, page=16,
                    ctx=700, heavy_frac=0.01)
    kinds, taus = [[Q4, Q2], [Q4, Q4]], [[0.01, 0.01], [0.0, math.inf]]
    n_steps = 4
    lengths = [700, 120, 333] if ragged else None
    st_e = runner.CacheState(w, DEV, kinds, taus, extra_tokens=n_steps, lengths=lengths)
    st_g = runner.CacheState(w, DEV, kinds, taus, extra_tokens=n_steps, lengths=lengths)
    hint = int(st_e.lens0.sum()) // 2 if ragged else 0
    if ragged:
        assert abi.loopkv_decode_layout(st_e.plan, 0, 0, w.batch, st_e.max_seq_len, hint, 0)[0] == 1
    kept = None
    for st in (st_e, st_g):
        for c in st.stored:
            st.pools[c].zero_()     # unwritten bytes compare equal too
        kept = st.prefill({c: set(range(w.batch)) for c in st.stored})
    cells = [(r, l) for r in range(2) for l in range(2)]
    qs = {c: wl.cell_query(w, st_e.cell_index(*c), DEV)[1] for c in cells}
    new = {c: wl.append_kv(w, st_e.cell_index(*c), 0, 1, DEV) for c in st_e.stored}
    new_host = {c: (wl.bf16_bits(k), wl.bf16_bits(v)) for c, (k, v) in new.items()}   # [B][1][H][D]
    lens0 = torch.from_numpy(st_e.lens0.astype(np.int32)).to(DEV)

    def run(st, lens_app, lens_dec, outs, masks):
        app = abi.make_batch(lens_app, st.block_tables, st.max_seq_len)
        for c in st.stored:
            abi.loopkv_append(st.plan, st.cells, c[0], c[1], app, 1, *new[c])
        for i, (r, l) in enumerate(cells):
            st.decode(r, l, qs[(r, l)], outs[i], mask=masks[i], lens=lens_dec, sum_seq_lens=hint)

    def buffers(st):
        return ([torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV) for _ in cells],
                [st.new_mask() for _ in cells])

    la = torch.empty_like(lens0)
    ld = torch.empty_like(lens0)
    outs_g, masks_g = buffers(st_g)
    la.copy_(lens0)
    ld.copy_(lens0 + 1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(st_g, la, ld, outs_g, masks_g)
    torch.cuda.synchronize()
    for step in range(n_steps):
        outs_e, masks_e = buffers(st_e)
        run(st_e, lens0 + step, lens0 + step + 1, outs_e, masks_e)
        torch.cuda.synchronize()
        la.copy_(lens0 + step)
        ld.copy_(lens0 + step + 1)
        g.replay()
        torch.cuda.synchronize()
        for i in range(len(cells)):
            assert torch.equal(outs_g[i].view(torch.int32), outs_e[i].view(torch.int32)), (step, cells[i])
            assert torch.equal(masks_g[i], masks_e[i]), (step, cells[i])
        for c in st_e.stored:
            assert torch.equal(st_g.pools[c], st_e.pools[c]), (step, c)
        # the oracle on each sequence's tokens so far: prefill, then the same
        # appended token once per replay
        host = {c: {b: tuple(np.concatenate([kept[c][b][i]] + [new_host[c][i][b]] * (step + 1))
                             for i in range(2)) for b in range(w.batch)} for c in st_e.stored}
        lens_now = st_e.lens0 + step + 1
        for i, (r, l) in enumerate(cells):
            src = oa.resolve_source(st_g.kinds, r, l)
            compare_decode(st_g, r, l, qs[(r, l)], outs_g[i], masks_g[i], host[src], range(w.batch), lens=lens_now)
        say(f"  replay {step}: {len(cells)} cells bit-identical to eager and within the oracle's bound")


def test_decode_is_deterministic():
    w = wl.Workload("determ", 150, batch=2, loops=1, layers=1, heads=4, head_dim=128, page=32,
                    ctx=5000, heavy_frac=0.01)
    st = runner.CacheState(w, DEV, [[Q4]], [[0.002]])
    st.prefill()
    res = [_decode(st, 0, 0) for _ in range(3)]
    for q, out, mask, cnt in res[1:]:
        assert torch.equal(out.view(torch.int32), res[0][1].view(torch.int32))
        assert torch.equal(mask, res[0][2])
        assert torch.equal(cnt, res[0][3])


def _append_all(st, K, V, schedule):
    """Append K/V [B][T][H][D] following schedule [(t0, t1), ...] (same for all sequences)."""
    for (r, l) in st.stored:
        for (t0, t1) in schedule:
            lens = torch.full((st.w.batch,), t0, dtype=torch.int32, device=DEV)
            st.append(r, l, K[(r, l)][:, t0:t1].contiguous(), V[(r, l)][:, t0:t1].contiguous(), lens)


def test_append_token_by_token_equals_bulk():
    """The cache is a pure function of the sequence: one-token appends, a
    multi-group append and a single bulk append give identical bytes, equal
    to the oracle's packing."""
    T = 100
    w = wl.Workload("append", 160, batch=3, loops=1, layers=2, heads=2, head_dim=128, page=16,
                    ctx=T, heavy_frac=0.01)
    kinds, taus = [[Q4, Q2]], [[0.01, 0.01]]
    a = runner.CacheState(w, DEV, kinds, taus, lengths=[T] * 3)
    b = runner.CacheState(w, DEV, kinds, taus, lengths=[T] * 3)
    K, V = {}, {}
    for (r, l) in a.stored:
        K[(r, l)], V[(r, l)] = wl.cell_kv(w, a.cell_index(r, l), T, DEV)
    _append_all(a, K, V, [(0, T)])
    sched = [(0, 37)] + [(t, t + 1) for t in range(37, 60)] + [(60, T)]
    _append_all(b, K, V, sched)
    torch.cuda.synchronize()
    for (r, l) in a.stored:
        for s in range(3):
            kb, vb = wl.bf16_bits(K[(r, l)][s]), wl.bf16_bits(V[(r, l)][s])
            check_pool(a, r, l, s, kb, vb)
            check_pool(b, r, l, s, kb, vb)


def test_append_ragged_lengths_and_staging():
    """Appends from different starting lengths per sequence, including ones
    that cross key groups, then decode over the result."""
    w = wl.Workload("append-ragged", 170, batch=4, loops=1, layers=2, heads=2, head_dim=64,
                    page=32, ctx=160, heavy_frac=0.02)
    kinds, taus = [[Q4, Q2]], [[0.0, 0.01]]
    start = np.array([0, 31, 33, 64], np.int32)
    steps = [1, 2, 45, 1]
    final = start + sum(steps)
    st = runner.CacheState(w, DEV, kinds, taus, lengths=final)
    T = int(final.max())
    kept = {}
    for (r, l) in st.stored:
        K, V = wl.cell_kv(w, st.cell_index(r, l), T, DEV)
        # per-sequence starting contents: sequence b holds its first start[b] tokens
        for bi in range(w.batch):
            n0 = int(start[bi])
            if n0:
                lens = torch.zeros(1, dtype=torch.int32, device=DEV)
                batch = abi.make_batch(lens, st.block_tables[bi:bi + 1], st.max_seq_len,
                                       slots=st.slots[bi:bi + 1])
                abi.loopkv_append(st.plan, st.cells, r, l, batch, n0, K[bi:bi + 1, :n0].contiguous(),
                                  V[bi:bi + 1, :n0].contiguous())
        cur = start.copy()
        for n in steps:
            lens = torch.from_numpy(cur).to(DEV)
            idx = torch.from_numpy((cur[:, None] + np.arange(n)[None, :]).astype(np.int64)).to(DEV)
            kk = torch.stack([K[bi, idx[bi]] for bi in range(w.batch)])
            vv = torch.stack([V[bi, idx[bi]] for bi in range(w.batch)])
            st.append(r, l, kk, vv, lens)
            cur = cur + n
        kept[(r, l)] = {bi: (wl.bf16_bits(K[bi]), wl.bf16_bits(V[bi])) for bi in range(w.batch)}
    torch.cuda.synchronize()
    for (r, l) in st.stored:
        for bi in range(w.batch):
            check_pool(st, r, l, bi, *kept[(r, l)][bi])
    for l in range(2):
        q, out, mask, _ = _decode(st, 0, l)
        compare_decode(st, 0, l, q, out, mask, kept[(0, l)], range(w.batch))


def test_debug_checks_and_log_lines(capfd, monkeypatch):
    """LOOPKV_LOG=1 prints one line per call (cell, source, mode, split
    layout, required bytes); LOOPKV_DEBUG=1 rejects an out-of-range page-table
    entry and a length above max_seq_len with LOOPKV_E_INVAL before anything
    is launched (the output keeps its sentinel).  The corrupted case decodes
    a 2-bit cell, whose kernels read the pool only through bounds-checked
    buffer loads."""
    w = wl.Workload("debug", 260, batch=2, loops=1, layers=2, heads=2, head_dim=64, page=16, ctx=200,
                    heavy_frac=0.01)
    st = runner.CacheState(w, DEV, [[Q4, Q2]], [[0.01, 0.01]], lengths=[200, 90])
    kept = st.prefill({c: {0, 1} for c in st.stored})
    torch.cuda.synchronize()
    capfd.readouterr()
    monkeypatch.setenv("LOOPKV_LOG", "1")
    q, out, mask, _ = _decode(st, 0, 0)
    err = capfd.readouterr().err
    monkeypatch.delenv("LOOPKV_LOG")
    line = [x for x in err.splitlines() if x.startswith("[loopkv] decode cell (0,0)")]
    assert line and "4-bit sparse-tau" in line[0] and "splits=" in line[0] and "bytes" in line[0], err
    compare_decode(st, 0, 0, q, out, mask, kept[(0, 0)], range(2))

    monkeypatch.setenv("LOOPKV_DEBUG", "1")
    q, out, mask, _ = _decode(st, 0, 1)           # valid tables pass the check
    compare_decode(st, 0, 1, q, out, mask, kept[(0, 1)], range(2))
    bad = st.block_tables.clone()
    bad[1, 2] = st.num_pages                      # one past the pool
    sentinel = torch.full((w.batch, w.heads, w.head_dim), float("nan"), device=DEV)
    opts = abi.make_opts(st.workspace)
    with pytest.raises(abi.LoopKVError) as e:
        abi.loopkv_decode(st.plan, st.cells, 0, 1, abi.make_batch(st.lens, bad, st.max_seq_len), q, sentinel, opts)
    assert e.value.code == abi.E_INVAL and "block_tables[1][2]" in e.value.message
    long_lens = torch.tensor([200, st.max_seq_len + 1], dtype=torch.int32, device=DEV)
    with pytest.raises(abi.LoopKVError) as e:
        abi.loopkv_decode(st.plan, st.cells, 0, 1, abi.make_batch(long_lens, st.block_tables, st.max_seq_len), q,
                          sentinel, opts)
    assert e.value.code == abi.E_INVAL and "seq_lens[1]" in e.value.message
    torch.cuda.synchronize()
    assert torch.isnan(sentinel).all(), "nothing may be launched after a failed check"
    monkeypatch.delenv("LOOPKV_DEBUG")
