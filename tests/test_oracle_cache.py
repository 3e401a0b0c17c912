"""Pins of the oracle's cell cache and paged layout (CPU only).

* hand-placed bytes of head-blocks (tests/golden/layout_case.txt: 4-bit,
  16-token pages; layout_q2_p16.txt: 2-bit region order and a later key
  group's metadata on its own first page; layout_q4_p64.txt: the second
  key-metadata slot of 64-token pages);
* pack -> unpack round trip for both cell kinds, page sizes 16/32/64,
  shuffled block tables and ragged tails;
* the cache is a pure function of the sequence: every key group's codes only
  depend on that group's tokens (a prefix's complete groups are unchanged).
"""
import os

import numpy as np
import pytest

from oracle import cache as oc
from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_bf16_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def test_golden_layout_bytes():
    P, D, H, T = 16, 64, 1, 1
    d = np.arange(D)
    c = oc.CellCache(
        kind=oc.KIND_Q4,
        k_codes=(d % 16).astype(np.uint8).reshape(1, 1, D),
        k_scale=np.full((1, 1, D), 2.0, np.float16),
        k_zero=np.full((1, 1, D), -1.0, np.float16),
        v_codes=np.full((1, 1, D), 9, np.uint8),
        v_scale=np.array([[[1.0, 0.5]]], np.float16),
        v_zero=np.array([[[-2.0, 0.25]]], np.float16),
    )
    reg = oc.head_block_regions(oc.KIND_Q4, P, D)
    assert (reg["k_hi"], reg["k_lo"], reg["v_hi"], reg["v_lo"], reg["v_meta"],
            reg["k_meta"], reg["HB"]) == (0, 256, 512, 768, 1024, 1152, 1408)
    pool, defined = oc.pack_pool(c, P, [5, 0, 0, 0, 0, 0, 0, 0], 8)
    blk = pool[0, 5]
    n = 0
    with open(os.path.join(GOLDEN, "layout_case.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            off, val = [int(v) for v in line.split()]
            assert blk[off] == val, (off, blk[off], val)
            assert defined[0, 5, off]
            n += 1
    assert n > 20
    # nothing outside page 5 is defined
    assert not defined[0, :5].any() and not defined[0, 6:].any()


def _check_golden(name, pool, defined):
    """Compare against a fixture of (physical page, offset, byte or '-')."""
    n = 0
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            page, off, val = line.split()
            page, off = int(page), int(off)
            if val == "-":
                assert not defined[0, page, off], (name, page, off)
            else:
                assert defined[0, page, off], (name, page, off)
                assert pool[0, page, off] == int(val), (name, page, off, pool[0, page, off], val)
            n += 1
    return n


def test_golden_layout_2bit_16_token_pages():
    """2-bit head-block order (K | V | V meta | K meta) and a second key group
    whose metadata sits on its own first page, two pages after the first."""
    P, D, T = 16, 32, 40
    t = np.arange(T)[:, None, None]
    d = np.arange(D)[None, None, :]
    c = oc.CellCache(
        kind=oc.KIND_Q2,
        k_codes=((t + d) % 4).astype(np.uint8),
        k_scale=np.array([[[2.0] * D], [[0.5] * D]], np.float16),
        k_zero=np.array([[[-1.0] * D], [[3.0] * D]], np.float16),
        v_codes=np.broadcast_to(t % 4, (T, 1, D)).astype(np.uint8),
        v_scale=(1.0 + np.arange(T) / 8.0).astype(np.float16).reshape(T, 1, 1),
        v_zero=np.full((T, 1, 1), -0.5, np.float16),
    )
    reg = oc.head_block_regions(oc.KIND_Q2, P, D)
    assert (reg["k"], reg["v"], reg["v_meta"], reg["k_meta"], reg["HB"]) == (0, 128, 256, 320, 448)
    pool, defined = oc.pack_pool(c, P, [3, 0, 5], 6)
    assert _check_golden("layout_q2_p16.txt", pool, defined) > 25
    assert not defined[0, [1, 2, 4]].any()


def test_golden_layout_4bit_64_token_pages():
    """Two key-metadata slots per 64-token page: group 1 in slot 1 of the
    first page, group 2 in slot 0 of the next."""
    P, D, T = 64, 32, 70
    t = np.arange(T)[:, None, None]
    d = np.arange(D)[None, None, :]
    g = np.arange(3)[:, None, None]
    c = oc.CellCache(
        kind=oc.KIND_Q4,
        k_codes=((t + d) % 16).astype(np.uint8),
        k_scale=np.broadcast_to(0.25 * (g + 1), (3, 1, D)).astype(np.float16),
        k_zero=np.broadcast_to(-(g + 1.0), (3, 1, D)).astype(np.float16),
        v_codes=np.full((T, 1, D), 9, np.uint8),
        v_scale=np.full((T, 1, 1), 1.0, np.float16),
        v_zero=np.full((T, 1, 1), 0.0, np.float16),
    )
    reg = oc.head_block_regions(oc.KIND_Q4, P, D)
    assert (reg["k_hi"], reg["k_lo"], reg["v_hi"], reg["v_lo"], reg["v_meta"], reg["k_meta"], reg["HB"]) == \
        (0, 512, 1024, 1536, 2048, 2304, 2560)
    pool, defined = oc.pack_pool(c, P, [2, 0], 3)
    assert _check_golden("layout_q4_p64.txt", pool, defined) > 20
    assert not defined[0, 1].any()


@pytest.mark.parametrize("kind", [oc.KIND_Q4, oc.KIND_Q2])
@pytest.mark.parametrize("P", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 31, 33, 100])
def test_pack_unpack_round_trip(kind, P, T):
    rng = np.random.default_rng(T * 7 + P + kind)
    H, D = 2, 64
    kb = _rand_bf16_bits(rng, (T, H, D))
    vb = _rand_bf16_bits(rng, (T, H, D))
    c = oc.build_cell_cache(kb, vb, kind)
    npages_used = -(-T // P)
    num_pages = npages_used + 3
    block_row = rng.permutation(num_pages)[:npages_used]
    pool, defined = oc.pack_pool(c, P, block_row, num_pages)
    back = oc.unpack_pool(pool, kind, P, block_row, T)
    for name in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        a, b = getattr(c, name), getattr(back, name)
        assert np.array_equal(a.view(np.uint8) if a.dtype == np.float16 else a,
                              b.view(np.uint8) if b.dtype == np.float16 else b), name
    reg = oc.head_block_regions(kind, P, D)
    planes = 4 if kind == oc.KIND_Q4 else 2
    ng = -(-T // 32)
    expect = H * (T * planes * reg["row"] + T * (D // 32) * 4 + ng * 4 * D)
    assert defined.sum() == expect


def test_cache_is_pure_function_of_sequence():
    rng = np.random.default_rng(3)
    H, D, T = 2, 64, 77
    kb = _rand_bf16_bits(rng, (T, H, D))
    vb = _rand_bf16_bits(rng, (T, H, D))
    for kind in (oc.KIND_Q4, oc.KIND_Q2):
        full = oc.build_cell_cache(kb, vb, kind)
        for Tp in (32, 40, 64, 65):
            pre = oc.build_cell_cache(kb[:Tp], vb[:Tp], kind)
            done = (Tp // 32) * 32  # complete key groups of the prefix
            assert np.array_equal(pre.k_codes[:done], full.k_codes[:done])
            assert np.array_equal(pre.v_codes, full.v_codes[:Tp])
            assert np.array_equal(pre.v_scale, full.v_scale[:Tp])


def test_group_quantization_matches_per_group_codec():
    """Key codes of group g equal quantizing that group's tokens alone."""
    rng = np.random.default_rng(4)
    H, D, T = 1, 32, 70
    kb = _rand_bf16_bits(rng, (T, H, D), 3.0)
    vb = _rand_bf16_bits(rng, (T, H, D))
    c = oc.build_cell_cache(kb, vb, oc.KIND_Q4)
    K = codec.bf16_bits_to_f32(kb)
    for g, (lo, hi) in enumerate([(0, 32), (32, 64), (64, 70)]):
        for d in (0, 5, 31):
            cc, s, z = codec.quantize(K[lo:hi, 0, d], 4)
            assert np.array_equal(c.k_codes[lo:hi, 0, d], cc)
            assert c.k_scale[g, 0, d] == s and c.k_zero[g, 0, d] == z
