"""Decode of one (loop, layer) cell: scores, softmax, tau mask, output.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Float64 throughout.

Sources
-------
* LoopKV abstract ("LoopKV: Loop-Aware KV Cache Compression for Serving
  Looped Transformers", 概要):
  - a cell holds 4-bit or 2-bit codes, or borrows the last loop's cache of
    its layer;
  - at decode the upper two bits of every 4-bit value are used, and the
    lower two are loaded only for tokens whose weight under the loop's own
    query is large enough to need them.

Readings where the pages are silent:
* keys are always read at the source cell's full precision (the weights
  must exist before the mask can be formed): K^ = c*s + z with c = 4*hi + lo
  for a 4-bit source;
* score_t = sm_scale * sum_d q_d K^_{t,d}; p = softmax(score) over all T
  tokens of one (sequence, head); heads are independent;
* "own weights require 4-bit precision" is p_t >= tau with the calling
  cell's tau and the calling cell's query (a reuse cell uses its own q and
  tau on its source's cache); tau = 0 flags every token, tau = +inf none;
* a value whose low plane is not fetched is reconstructed at the centre of
  its high-plane bucket: V^ = (4*hi + 3/2)*s + z; a fetched one is
  V^ = (4*hi + lo)*s + z; 2-bit sources use V^ = c*s + z and have no mask;
* output o = sum_t p_t V^_t, returned in float64 (the library returns fp32);
  an empty sequence (T = 0) gives o = 0.

Pins (tests/test_oracle_attention.py): tau = 0 against full 4-bit attention
and tau = +inf against high-plane-only attention, both through
torch.nn.functional.scaled_dot_product_attention in float64; 2-bit cells the
same way; the midpoint equals the mean of the four full reconstructions of
its bucket; reuse equals the source; mask size at most floor(1/tau); masks
nested in tau; a 50-digit mpmath brute force on tiny inputs;
ambiguity_band by closed-form cases just inside and just outside 1e-3 tau.
"""
from __future__ import annotations

import numpy as np

from .cache import CellCache, KIND_Q4, KIND_Q2, KIND_REUSE
from .codec import GROUP, bf16_bits_to_f32


def resolve_source(kinds, r: int, l: int):
    """(loop, layer) whose cache cell (r, l) reads: (R-1, l) for a reuse cell."""
    kinds = np.asarray(kinds)
    R = kinds.shape[0]
    if kinds[r, l] == KIND_REUSE:
        if r == R - 1:
            raise ValueError("a final-loop cell cannot reuse itself")
        return R - 1, l
    return r, l


def dequant_keys(cache: CellCache) -> np.ndarray:
    """K^ [T, H, D] float64: codes times the scale/zero of their key group."""
    T = cache.T
    g = np.arange(T) // GROUP
    s = cache.k_scale[g].astype(np.float64)
    z = cache.k_zero[g].astype(np.float64)
    return cache.k_codes.astype(np.float64) * s + z


def _value_meta(cache: CellCache):
    T, H, D = cache.v_codes.shape
    j = np.arange(D) // GROUP
    s = cache.v_scale[:, :, j].astype(np.float64)  # [T, H, D]
    z = cache.v_zero[:, :, j].astype(np.float64)
    return s, z


def dequant_values_full(cache: CellCache) -> np.ndarray:
    """V^ [T, H, D] float64 from all stored bits."""
    s, z = _value_meta(cache)
    return cache.v_codes.astype(np.float64) * s + z


def dequant_values_mid(cache: CellCache) -> np.ndarray:
    """V^ [T, H, D] of a 4-bit cell from its high plane only (bucket centre)."""
    if cache.kind != KIND_Q4:
        raise ValueError("only 4-bit cells have a high plane")
    s, z = _value_meta(cache)
    hi = (cache.v_codes >> 2).astype(np.float64)
    return (4.0 * hi + 1.5) * s + z


def scores(cache: CellCache, q_bits: np.ndarray, sm_scale: float = 1.0) -> np.ndarray:
    """score [H, T] = sm_scale * q . K^ (q given as bf16 bits [H, D])."""
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    K = dequant_keys(cache)
    return float(sm_scale) * np.einsum("hd,thd->ht", q, K)


def softmax(sc: np.ndarray):
    """p [H, T] and log-sum-exp [H] of scores [H, T] (stable form)."""
    m = sc.max(axis=-1, keepdims=True)
    e = np.exp(sc - m)
    tot = e.sum(axis=-1, keepdims=True)
    return e / tot, (m + np.log(tot))[:, 0]


def decode(cache: CellCache, q_bits: np.ndarray, tau: float,
           sm_scale: float = 1.0, flags: np.ndarray | None = None) -> dict:
    """Decode one sequence's step over one cell's (source) cache.

    ``tau`` is the calling cell's threshold.  ``flags`` ([H, T] bool) replaces
    the computed mask when given (used to adopt the GPU's decision inside the
    ambiguity band); it is ignored for 2-bit sources.
    Returns dict(out [H, D] float64, flags [H, T], p [H, T], score [H, T],
    lse [H]).
    """
    T, H, D = cache.v_codes.shape
    if T == 0:
        return {"out": np.zeros((H, D)), "flags": np.zeros((H, 0), bool),
                "p": np.zeros((H, 0)), "score": np.zeros((H, 0)),
                "lse": np.full(H, -np.inf)}
    sc = scores(cache, q_bits, sm_scale)
    p, lse = softmax(sc)
    if cache.kind == KIND_Q4:
        if flags is None:
            flags = p >= tau
        flags = np.asarray(flags, bool)
        full = dequant_values_full(cache)
        mid = dequant_values_mid(cache)
        V = np.where(flags.T[:, :, None], full, mid)
    elif cache.kind == KIND_Q2:
        flags = np.zeros((H, T), bool)
        V = dequant_values_full(cache)
    else:
        raise ValueError("decode needs a stored source cell")
    out = np.einsum("ht,thd->hd", p, V)
    return {"out": out, "flags": flags, "p": p, "score": sc, "lse": lse}


def ambiguity_band(p: np.ndarray, tau: float, rel: float = 1e-3) -> np.ndarray:
    """Tokens whose weight lies within rel*tau of tau (either flag is correct)."""
    if not np.isfinite(tau) or tau == 0.0:
        return np.zeros_like(p, dtype=bool)
    return np.abs(p - tau) <= rel * tau
