"""Pins of the oracle's cell decode (CPU only).

Library special cases (torch scaled_dot_product_attention, float64, CPU):
* tau = 0 equals full 4-bit attention over the dequantized cache;
* tau = +inf equals high-plane-only attention, with each value at the mean
  of the four full reconstructions of its high-plane bucket;
* a 2-bit cell equals plain attention over its dequantized cache.
Invariants: reuse equals the source with the reuse cell's own query and tau;
at most floor(1/tau) flags; masks nested in tau; flag <=> score >= LSE+ln tau.
Brute force: 50-digit mpmath on tiny inputs.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import cache as oc
from oracle import codec


def _bf16_bits(x):
    x = np.asarray(x, np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _make(rng, T, H, D, kind, heavy=0):
    """Random cache with some heavy tokens (keys aligned with the query)."""
    qraw = rng.standard_normal((H, D)).astype(np.float32)
    K = rng.standard_normal((T, H, D)).astype(np.float32)
    if heavy:
        pos = rng.choice(T, heavy, replace=False)
        K[pos] += 0.5 * qraw[None] * 4
    K[:, :, :2] *= 10
    V = rng.standard_normal((T, H, D)).astype(np.float32)
    c = oc.build_cell_cache(_bf16_bits(K), _bf16_bits(V), kind)
    q = _bf16_bits(qraw / math.sqrt(D))
    return c, q


def _sdpa(q_bits, K, V, scale):
    q = torch.from_numpy(codec.bf16_bits_to_f32(q_bits).astype(np.float64))  # [H, D]
    k = torch.from_numpy(K).permute(1, 0, 2)  # [H, T, D]
    v = torch.from_numpy(V).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None, :, None, :], k[None], v[None], scale=scale)
    return o[0, :, 0, :].numpy()


def _mid_by_enumeration(c):
    """Mean of the four full reconstructions (lo = 0..3) of each value's bucket."""
    hi = (c.v_codes >> 2).astype(np.uint8)
    T, H, D = c.v_codes.shape
    j = np.arange(D) // 32
    s = c.v_scale[:, :, j].astype(np.float64)
    z = c.v_zero[:, :, j].astype(np.float64)
    acc = np.zeros((T, H, D))
    for lo in range(4):
        acc += codec.dequantize(codec.join_planes(hi, np.full_like(hi, lo)), s, z)
    return acc / 4


@pytest.mark.parametrize("sm_scale", [1.0, 0.37])
def test_tau_zero_is_full_4bit_attention(sm_scale):
    rng = np.random.default_rng(11)
    c, q = _make(rng, 200, 3, 64, oc.KIND_Q4, heavy=4)
    r = oa.decode(c, q, 0.0, sm_scale)
    assert r["flags"].all()
    ref = _sdpa(q, oa.dequant_keys(c), oa.dequant_values_full(c), sm_scale)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_tau_inf_is_high_plane_attention():
    rng = np.random.default_rng(12)
    c, q = _make(rng, 150, 2, 64, oc.KIND_Q4, heavy=3)
    r = oa.decode(c, q, math.inf)
    assert not r["flags"].any()
    ref = _sdpa(q, oa.dequant_keys(c), _mid_by_enumeration(c), 1.0)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_midpoint_is_bucket_mean():
    rng = np.random.default_rng(13)
    c, _ = _make(rng, 40, 2, 64, oc.KIND_Q4)
    np.testing.assert_allclose(oa.dequant_values_mid(c), _mid_by_enumeration(c),
                               rtol=0, atol=1e-12)


def test_two_bit_cell_is_plain_attention():
    rng = np.random.default_rng(14)
    c, q = _make(rng, 97, 2, 128, oc.KIND_Q2, heavy=2)
    for tau in (0.0, 0.01, math.inf):
        r = oa.decode(c, q, tau)
        assert not r["flags"].any()
        ref = _sdpa(q, oa.dequant_keys(c), oa.dequant_values_full(c), 1.0)
        np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_keys_dequantized_within_half_step():
    rng = np.random.default_rng(15)
    qraw = rng.standard_normal((2, 64)).astype(np.float32)
    K = rng.standard_normal((70, 2, 64)).astype(np.float32)
    kb = _bf16_bits(K)
    c = oc.build_cell_cache(kb, _bf16_bits(K), oc.KIND_Q4)
    Kh = oa.dequant_keys(c)
    s = c.k_scale[np.arange(70) // 32].astype(np.float64)
    assert np.all(np.abs(Kh - codec.bf16_bits_to_f32(kb)) <= s * (0.5 + 2 ** -20))


def test_mask_invariants():
    rng = np.random.default_rng(16)
    c, q = _make(rng, 500, 4, 64, oc.KIND_Q4, heavy=6)
    prev = None
    for tau in (0.0, 1e-4, 0.002, 0.01, 0.05, 0.3, 1.0, math.inf):
        r = oa.decode(c, q, tau)
        f = r["flags"]
        if tau > 0 and math.isfinite(tau):
            assert np.all(f.sum(axis=1) <= math.floor(1 / tau))
            # flag <=> score >= LSE + ln tau (away from rounding)
            thr = r["lse"][:, None] + math.log(tau)
            away = np.abs(r["score"] - thr) > 1e-9
            assert np.array_equal(f[away], (r["score"] >= thr)[away])
        if prev is not None:
            assert np.all(f <= prev)  # larger tau flags a subset
        prev = f


def test_reuse_equals_source_with_own_query():
    rng = np.random.default_rng(17)
    R, L = 3, 2
    kinds = np.array([[oc.KIND_REUSE, oc.KIND_Q4],
                      [oc.KIND_Q2, oc.KIND_REUSE],
                      [oc.KIND_Q4, oc.KIND_Q2]])
    assert oa.resolve_source(kinds, 0, 0) == (2, 0)
    assert oa.resolve_source(kinds, 1, 1) == (2, 1)
    assert oa.resolve_source(kinds, 0, 1) == (0, 1)
    with pytest.raises(ValueError):
        oa.resolve_source(np.array([[oc.KIND_Q4], [oc.KIND_REUSE]]), 1, 0)
    src, q_own = _make(rng, 120, 2, 64, oc.KIND_Q4, heavy=2)
    _, q_src = _make(rng, 120, 2, 64, oc.KIND_Q4, heavy=2)
    a = oa.decode(src, q_own, 0.02)
    b = oa.decode(src, q_src, 0.02)
    assert not np.allclose(a["out"], b["out"])  # own query matters


def test_empty_sequence_gives_zero():
    c = oc.CellCache(oc.KIND_Q4, np.zeros((0, 2, 64), np.uint8), np.zeros((0, 2, 64), np.float16),
                     np.zeros((0, 2, 64), np.float16), np.zeros((0, 2, 64), np.uint8),
                     np.zeros((0, 2, 2), np.float16), np.zeros((0, 2, 2), np.float16))
    r = oa.decode(c, np.zeros((2, 64), np.uint16), 0.01)
    assert np.array_equal(r["out"], np.zeros((2, 64)))


@pytest.mark.parametrize("kind", [oc.KIND_Q4, oc.KIND_Q2])
def test_mpmath_brute_force_tiny(kind):
    """Tiny cells recomputed element by element at 50 digits."""
    mpmath.mp.dps = 50
    rng = np.random.default_rng(18 + kind)
    T, H, D = 6, 1, 32
    c, q = _make(rng, T, H, D, kind, heavy=1)
    qf = codec.bf16_bits_to_f32(q)
    for tau in (0.0, 0.15, math.inf):
        r = oa.decode(c, q, tau, sm_scale=0.5)
        sc = []
        for t in range(T):
            acc = mpmath.mpf(0)
            for d in range(D):
                kv = (mpmath.mpf(int(c.k_codes[t, 0, d])) * mpmath.mpf(float(c.k_scale[0, 0, d]))
                      + mpmath.mpf(float(c.k_zero[0, 0, d])))
                acc += mpmath.mpf(float(qf[0, d])) * kv
            sc.append(acc / 2)
        m = max(sc)
        e = [mpmath.e ** (s - m) for s in sc]
        tot = sum(e)
        p = [x / tot for x in e]
        out = []
        for d in range(D):
            acc = mpmath.mpf(0)
            for t in range(T):
                code = int(c.v_codes[t, 0, d])
                s = mpmath.mpf(float(c.v_scale[t, 0, d // 32]))
                z = mpmath.mpf(float(c.v_zero[t, 0, d // 32]))
                if kind == oc.KIND_Q4 and not (p[t] >= tau):
                    v = (4 * (code >> 2) + mpmath.mpf(3) / 2) * s + z
                else:
                    v = code * s + z
                acc += p[t] * v
            out.append(float(acc))
        flags = [bool(pt >= tau) if kind == oc.KIND_Q4 else False for pt in p]
        assert r["flags"][0].tolist() == flags
        np.testing.assert_allclose(r["out"][0], np.array(out), rtol=1e-13, atol=1e-13)


def test_ambiguity_band_closed_form():
    """The band where either mask decision is accepted is |p - tau| <= 1e-3 tau
    (a threshold on a computed float cannot be exact at the boundary): weights
    5e-4 tau away are inside, 2e-3 tau away outside, on both sides; tau = 0
    and tau = +inf (no threshold to be near) have an empty band."""
    for tau in (1e-4, 0.005, 0.02, 0.5):
        inside = np.array([tau * (1 - 5e-4), tau, tau * (1 + 5e-4), tau * (1 - 9.9e-4), tau * (1 + 9.9e-4)])
        outside = np.array([tau * (1 - 2e-3), tau * (1 + 2e-3), tau * 0.5, tau * 1.5, 0.0, 1.0])
        assert oa.ambiguity_band(inside, tau).all(), tau
        assert not oa.ambiguity_band(outside, tau).any(), tau
    p = np.array([0.0, 1e-9, 0.3, 1.0])
    assert not oa.ambiguity_band(p, 0.0).any()
    assert not oa.ambiguity_band(p, math.inf).any()


def test_ambiguity_band_is_rare_at_workload_shapes():
    """On a realistic (sequence, head) set the band holds a tiny share of the
    flagged tokens, which is what lets the GPU parity checks bound it."""
    rng = np.random.default_rng(11)
    c, q = _make(rng, 4096, 8, 64, oc.KIND_Q4, heavy=40)
    for tau in (0.002, 0.01):
        r = oa.decode(c, q, tau)
        band = oa.ambiguity_band(r["p"], tau)
        assert r["flags"].sum() > 20
        assert band.sum() <= 2 + r["flags"].sum() // 50, (tau, band.sum(), r["flags"].sum())
