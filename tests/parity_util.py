"""Comparison helpers for the GPU parity tests (test infrastructure).

The GPU side runs only through the C ABI (loop_aware_quantized_amd.runner);
the reference side is the CPU oracle.  Both get the same seeded inputs.

Parity bar:
* pools: bit-exact on every defined byte;
* tau masks: bit-exact outside the ambiguity band |p - tau| <= 1e-3 tau,
  where either decision is correct; the band may hold at most
  16 + flagged/50 token-heads per comparison;
* outputs: after the oracle adopts the GPU's decisions inside the band,
  max |o_gpu - o_oracle| <= 2e-3 * max |o_oracle| over the compared
  [sequence, head, channel] block of one cell.
"""
from __future__ import annotations

import math
import sys

import numpy as np

from oracle import attention as oa
from oracle import cache as oc
from loop_aware_quantized_amd import inputs as wl

OUT_TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_pool_pages(state, r, l, b, T):
    """Host copy [H, pages, HB] of the physical pages holding sequence b's first T tokens."""
    import torch
    reg_hb = state.plan.head_block_bytes(r, l)
    H = state.w.heads
    n = -(-T // state.w.page)
    pages = state.table_np[b, :n].astype(np.int64)
    pool = state.pools[(r, l)].view(H, state.num_pages, reg_hb)
    idx = torch.from_numpy(pages).to(pool.device)
    return pool.index_select(1, idx).cpu().numpy()


def check_pool(state, r, l, b, k_bits, v_bits, T=None):
    """GPU pool bytes of (cell, sequence) vs the oracle's packing, defined bytes only."""
    T = int(state.lens0[b]) if T is None else T
    if T == 0:
        return 0
    kind = int(state.kinds[r, l])
    cache = oc.build_cell_cache(k_bits[:T], v_bits[:T], kind)
    n = -(-T // state.w.page)
    ref, defined = oc.pack_pool(cache, state.w.page, np.arange(n), n)
    got = gpu_pool_pages(state, r, l, b, T)
    bad = (ref != got) & defined
    if bad.any():
        h, p, o = np.argwhere(bad)[0]
        raise AssertionError(f"pool mismatch cell ({r},{l}) seq {b}: {bad.sum()} bytes; first at "
                             f"head {h} page {p} offset {o}: gpu {got[h, p, o]} oracle {ref[h, p, o]}")
    return int(defined.sum())


_CACHE = {}


def _cell_cache(k_bits, v_bits, T, kind):
    """Oracle cache of a sequence prefix, memoized on the host arrays' identity."""
    key = (id(k_bits), id(v_bits), T, kind)
    hit = _CACHE.get(key)
    if hit is None or hit[0] is not k_bits or hit[1] is not v_bits:
        if len(_CACHE) > 16:
            _CACHE.clear()
        hit = (k_bits, v_bits, oc.build_cell_cache(k_bits[:T], v_bits[:T], kind))
        _CACHE[key] = hit
    return hit[2]


def mask_to_flags(mask_row_words: np.ndarray, T: int) -> np.ndarray:
    """int32 words [H, W] -> bool flags [H, T] (bit t of word t//32)."""
    w = mask_row_words.astype(np.int64) & 0xFFFFFFFF
    bits = ((w[:, :, None] >> np.arange(32)[None, None, :]) & 1).astype(bool)
    return bits.reshape(w.shape[0], -1)[:, :T]


def compare_decode(state, r, l, q, out, mask, host_kv, seqs, lens=None, sm_scale=1.0):
    """Compare one decoded cell against the oracle on sequences ``seqs``.

    host_kv[b] = (k_bits, v_bits) of the SOURCE cell for sequence b.
    Returns a stats dict; raises AssertionError on a parity failure.
    """
    sr, sl = oa.resolve_source(state.kinds, r, l)
    kind = int(state.kinds[sr, sl])
    tau = float(state.taus[r, l])
    lens = state.lens0 if lens is None else lens
    q_bits = wl.bf16_bits(q)
    out_h = out.cpu().numpy()
    mask_h = mask.cpu().numpy() if mask is not None else None
    og, oo = [], []
    band_total = flagged = 0
    for b in seqs:
        T = int(lens[b])
        if T == 0:
            empty = np.zeros((0, state.w.heads, state.w.head_dim), np.uint16)
            k_bits, v_bits = empty, empty
        else:
            k_bits, v_bits = host_kv[b]
        cache = _cell_cache(k_bits, v_bits, T, kind)
        res = oa.decode(cache, q_bits[b], tau, sm_scale=sm_scale)
        if T > 0 and mask_h is not None:
            gflags = mask_to_flags(mask_h[b], T)
            if kind == oc.KIND_Q4:
                band = oa.ambiguity_band(res["p"], tau)
                diff = (gflags != res["flags"]) & ~band
                if diff.any():
                    h, t = np.argwhere(diff)[0]
                    raise AssertionError(
                        f"mask mismatch cell ({r},{l}) seq {b} head {h} token {t}: gpu {gflags[h, t]} "
                        f"p={res['p'][h, t]:.9g} tau={tau}")
                band_total += int(band.sum())
                flagged += int(res["flags"].sum())
                flags = np.where(band, gflags, res["flags"])
                res = oa.decode(cache, q_bits[b], tau, sm_scale=sm_scale, flags=flags)
            else:
                assert not gflags.any(), "2-bit source must not flag tokens"
        og.append(out_h[b])
        oo.append(res["out"])
    # the band excuses only near-ties: a handful of token-heads, far fewer
    # than the flags (a widened band would excuse a large share of them)
    assert band_total <= 16 + flagged // 50, (
        f"cell ({r},{l}): {band_total} token-heads in the ambiguity band for {flagged} flags")
    og, oo = np.stack(og), np.stack(oo)
    scale = float(np.abs(oo).max()) if oo.size else 0.0
    err = float(np.abs(og - oo).max()) if oo.size else 0.0
    assert np.all(np.isfinite(og)), "non-finite GPU output"
    assert err <= OUT_TOL * max(scale, 1e-30), (
        f"output mismatch cell ({r},{l}): max err {err:.3e} vs L_inf {scale:.3e} (tau={tau}, kind={kind})")
    return {"err": err, "scale": scale, "rel": err / max(scale, 1e-30), "band": band_total,
            "flagged": flagged}


def tau_str(t):
    return "inf" if math.isinf(t) else f"{t:g}"
