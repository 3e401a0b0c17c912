"""GPU parity of the joint loop-step vector quantization path (LoopVQ-style)
against oracle/loopvq.py, through the C ABI.

Bar: every stored index of a compared sequence equals the oracle's nearest
codeword of the raw inputs, or (near-ties decided in fp32) one whose float64
distance is within 1e-5 relative of the least; decoded outputs within 2e-3
of the output's L_inf norm per compared block, the oracle decoding only
indices checked that way.
"""
import numpy as np
import pytest

from loop_aware_quantized_amd import inputs as wl
from loop_aware_quantized_amd import runner
from oracle import loopvq as ov
from parity_util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda"
OUT_TOL = 2e-3


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _sq_distances(x, cb_j):
    """Squared distances [T][256] of joint vectors x [T][J] to one group's
    codewords [256][J], as |x|^2 - 2 x.c + |c|^2 (float64); pinned against
    the oracle's direct definition on sampled tokens in check_indices."""
    return (x * x).sum(-1)[:, None] - 2.0 * (x @ cb_j.T) + (cb_j * cb_j).sum(-1)[None, :]


def check_indices(gpu_idx, x_loops_bits, codebook):
    """Every index of gpu_idx [T][H][G] must name a nearest codeword of the
    raw joint vectors x_loops_bits (uint16 bf16 [R][T][H][D]) within 1e-5
    relative (the GPU decides in fp32).  Returns the exact-match fraction."""
    cb = wl.vq_joint_codebook(codebook)                        # [G][256][4R]
    x = bf16_to_f64(x_loops_bits)
    T, H, G = gpu_idx.shape
    exact = 0
    for h in range(H):
        jv = ov.joint_vectors(x[:, :, h, :])                   # [T][G][4R]
        sample = np.unique(np.linspace(0, T - 1, min(T, 64)).astype(np.int64))
        direct = ov.distances(x[:, sample, h, :], cb)          # [n][G][256]
        for j in range(G):
            d = _sq_distances(jv[:, j], cb[j])
            assert np.allclose(d[sample], direct[:, j], rtol=1e-9, atol=1e-9)
            dmin = d.min(-1)
            got = d[np.arange(T), gpu_idx[:, h, j].astype(np.int64)]
            bad = got > dmin * (1 + 1e-5) + 1e-9
            assert not bad.any(), f"head {h} group {j}: {bad.sum()} indices are not nearest codewords"
            exact += int((gpu_idx[:, h, j] == np.argmin(d, -1)).sum())
    return exact / max(gpu_idx.size, 1)


def compare(st, l, loop, q, out, kv_bits, seqs, lens, sm_scale=1.0):
    """Outputs of the decoded sequences against the oracle.  Every key and
    value index the oracle decodes is first checked against the raw inputs
    kv_bits[b] = (keys, values) bf16 bits [R][T][H][D] of sequence b (once
    per state, layer, sequence and length: decoding other loops reads the
    same indices)."""
    cbk, cbv = (wl.vq_joint_codebook(c) for c in st.codebooks[l])
    qh = bf16_to_f64(wl.bf16_bits(q))
    oh = out.cpu().numpy()
    errs, scale = [], 0.0
    for b in seqs:
        T = int(lens[b])
        ki, vi = st.pool_indices(l, b, T)
        checked = st.__dict__.setdefault("_checked_indices", set())
        if T and (l, b, T) not in checked:
            kb, vb = kv_bits[b]
            assert kb.shape[1] == T and vb.shape[1] == T
            check_indices(ki, kb, st.codebooks[l][0])
            check_indices(vi, vb, st.codebooks[l][1])
            checked.add((l, b, T))
        for h in range(st.w.heads):
            k_hat = ov.decode_loop(ki[:, h].astype(np.int64), cbk, loop)
            v_hat = ov.decode_loop(vi[:, h].astype(np.int64), cbv, loop)
            want = ov.attend(qh[b, h], k_hat, v_hat, sm_scale)
            errs.append(np.abs(oh[b, h] - want).max())
            scale = max(scale, np.abs(want).max())
    err = max(errs)
    assert np.all(np.isfinite(oh))
    assert err <= OUT_TOL * max(scale, 1e-30), f"layer {l} loop {loop}: err {err:.3e} vs {scale:.3e}"
    return err / max(scale, 1e-30)


def test_vq_tiny_end_to_end():
    w = wl.VQ_WORKLOADS["loopvq-tiny"]
    lens = [300, 57]
    st = runner.VqState(w, DEV, lengths=lens)
    for l in st.layers:
        kept = st.prefill_layer(l, keep={0, 1})
        torch.cuda.synchronize()
        for b in (0, 1):
            ki, vi = st.pool_indices(l, b, lens[b])
            fk = check_indices(ki, kept[b][0], st.codebooks[l][0])
            fv = check_indices(vi, kept[b][1], st.codebooks[l][1])
            say(f"  layer {l} seq {b}: exact index matches K {fk:.4f} V {fv:.4f}")
        for loop in range(w.loops):
            q = wl.vq_query(w, l, loop, DEV)
            out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV)
            st.decode(l, loop, q, out)
            torch.cuda.synchronize()
            rel = compare(st, l, loop, q, out, kept, (0, 1), lens)
            say(f"  layer {l} loop {loop}: rel err {rel:.2e}")
            again = torch.empty_like(out)
            st.decode(l, loop, q, again)
            torch.cuda.synchronize()
            assert torch.equal(out, again), "fixed summation order: repeated calls give identical bits"


def test_vq_empty_sequence_and_appends():
    w = wl.VqWorkload("vq-append", 12, batch=3, loops=2, layers=1, heads=2, head_dim=128, page=32, ctx=100)
    lens = np.array([100, 0, 33], np.int32)
    st = runner.VqState(w, DEV, lengths=lens, extra_tokens=5)
    kept = st.prefill_layer(0, keep={0, 1, 2})
    R, H, D = w.loops, w.heads, w.head_dim
    host = {b: list(kept.get(b, (np.zeros((R, 0, H, D), np.uint16),) * 2)) for b in range(3)}
    # five single-token appends to every sequence (raw inputs kept on the host)
    for step in range(5):
        k, v = wl.vq_append_kv(w, 0, step, 1, DEV)
        st.append(0, k, v, torch.from_numpy(lens + step).to(DEV))
        kb, vb = wl.bf16_bits(k), wl.bf16_bits(v)                    # [R][B][1][H][D]
        for b in range(3):
            host[b][0] = np.concatenate([host[b][0], kb[:, b]], axis=1)
            host[b][1] = np.concatenate([host[b][1], vb[:, b]], axis=1)
    lens_now = lens + 5
    torch.cuda.synchronize()
    q = wl.vq_query(w, 0, 1, DEV)
    out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV)
    st.decode(0, 1, q, out, lens=torch.from_numpy(lens_now).to(DEV))
    torch.cuda.synchronize()
    compare(st, 0, 1, q, out, host, (0, 1, 2), lens_now)
    # a zero-length batch entry decodes to zeros
    zero = torch.from_numpy(np.array([0, 0, 0], np.int32)).to(DEV)
    st.decode(0, 0, q, out, lens=zero)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0


def test_vq_16k_sampled():
    w = wl.VQ_WORKLOADS["loopvq-16k"]
    seqs = [0, 31]
    st = runner.VqState(w, DEV, layers=[5])
    kept = st.prefill_layer(5, keep=set(seqs))
    torch.cuda.synchronize()
    for b in seqs:
        ki, vi = st.pool_indices(5, b, w.ctx)
        fk = check_indices(ki, kept[b][0], st.codebooks[5][0])
        fv = check_indices(vi, kept[b][1], st.codebooks[5][1])
        say(f"  seq {b}: exact index matches over all {w.ctx} tokens: K {fk:.5f} V {fv:.5f}")
    for loop in range(w.loops):
        q = wl.vq_query(w, 5, loop, DEV)
        out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV)
        st.decode(5, loop, q, out)
        torch.cuda.synchronize()
        rel = compare(st, 5, loop, q, out, kept, seqs, st.lens0)
        say(f"  loop {loop}: rel err {rel:.2e}")


@pytest.mark.parametrize("loops", [2, 3])
def test_vq_several_splits(loops):
    """Few sequence-heads, so every sequence is cut into several splits
    (merged by the log-sum-exp merge), with a ragged last split."""
    w = wl.VqWorkload(f"vq-splits-{loops}", 13, batch=2, loops=loops, layers=1, heads=2, head_dim=128,
                      page=32, ctx=3000)
    lens = np.array([3000, 1100], np.int32)
    st = runner.VqState(w, DEV, lengths=lens)
    kept = st.prefill_layer(0, keep={0, 1})
    torch.cuda.synchronize()
    for b in (0, 1):
        ki, vi = st.pool_indices(0, b, int(lens[b]))
        assert check_indices(ki, kept[b][0], st.codebooks[0][0]) > 0.99
        assert check_indices(vi, kept[b][1], st.codebooks[0][1]) > 0.99
    for loop in range(loops):
        q = wl.vq_query(w, 0, loop, DEV)
        out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV)
        st.decode(0, loop, q, out)
        torch.cuda.synchronize()
        rel = compare(st, 0, loop, q, out, kept, (0, 1), lens)
        say(f"  loops {loops} loop {loop}: rel err {rel:.2e}")


@pytest.mark.parametrize("sm_scale", [0.05, 30.0])
def test_vq_flat_and_peaky_softmax(sm_scale):
    """A near-uniform softmax and a peaky one whose running maximum rises
    far above the first scores many times along the sequence."""
    w = wl.VqWorkload("vq-scale", 14, batch=2, loops=4, layers=1, heads=2, head_dim=128, page=32, ctx=5000)
    lens = np.array([5000, 700], np.int32)
    st = runner.VqState(w, DEV, lengths=lens)
    kept = st.prefill_layer(0, keep={0, 1})
    torch.cuda.synchronize()
    for loop in (0, 3):
        q = wl.vq_query(w, 0, loop, DEV)
        out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV)
        st.decode(0, loop, q, out, sm_scale=sm_scale)
        torch.cuda.synchronize()
        rel = compare(st, 0, loop, q, out, kept, (0, 1), lens, sm_scale)
        say(f"  scale {sm_scale} loop {loop}: rel err {rel:.2e}")


def test_vq_split_length_cap():
    """Enough sequence-heads to fill the chip with one split each, but
    sequences longer than the longest split: two splits per sequence-head,
    the second one short, merged by the log-sum-exp merge."""
    w = wl.VqWorkload("vq-cap", 15, batch=16, loops=4, layers=1, heads=16, head_dim=128, page=32, ctx=33000)
    st = runner.VqState(w, DEV)
    seqs = (0, 15)
    kept = st.prefill_layer(0, keep=set(seqs))
    torch.cuda.synchronize()
    q = wl.vq_query(w, 0, 2, DEV)
    out = torch.empty(w.batch, w.heads, w.head_dim, dtype=torch.float32, device=DEV)
    st.decode(0, 2, q, out)
    torch.cuda.synchronize()
    rel = compare(st, 0, 2, q, out, kept, seqs, st.lens0)
    say(f"  33000 tokens, 256 sequence-heads: rel err {rel:.2e}")
