"""Cell cache of one sequence, and its paged bit-plane byte layout.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources
-------
* LoopKV abstract ("LoopKV: Loop-Aware KV Cache Compression for Serving
  Looped Transformers", 概要): every (loop, layer) cell has its own cache,
  holding 4-bit or 2-bit codes, or borrowing the last loop's cache of its
  layer; the upper and lower bit pairs of a 4-bit code are loaded apart, so
  the two planes of a 4-bit cell live in separate rows.
* fugumt LoopVQ page, related-papers list, KIVI entry: keys quantized per
  channel over groups of tokens, values per token over groups of channels.

Readings where the pages are silent:
* group size 32; the key group of token t is t // 32 and a trailing partial
  group is quantized over the tokens present, so the cache is a pure
  function of the sequence (appending re-quantizes the open group);
* a page holds P tokens of every head; the pool is head-major: head h of
  physical page p is the head-block at byte ((h * num_pages) + p) * HB;
* head-block, 4-bit cell:  K_hi rows | K_lo rows | V_hi rows | V_lo rows |
  V meta | K meta;  2-bit cell:  K rows | V rows | V meta | K meta;
  a row is one token's D codes of one plane, D/4 bytes, token-major;
* V meta: per token, per 32-channel group j: fp16 scale then fp16 zero
  (4 bytes), tokens in page order;
* K meta: max(1, P/32) slots of D fp16 scales followed by D fp16 zeros; key
  group g lives in the page holding token 32g, slot (32g mod P) / 32;
* defined bytes are rows and V meta of tokens < T and K meta slots of
  groups holding at least one token; every other byte is unspecified.

Pins (tests/test_oracle_cache.py): round trip pack -> unpack, and the
hand-placed bytes of tests/golden/layout_case.txt (4-bit, 16-token pages),
layout_q2_p16.txt (2-bit region order; a later key group's metadata on its
own first page) and layout_q4_p64.txt (the second key-metadata slot).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .codec import GROUP, bf16_bits_to_f32, quantize, split_planes, join_planes, \
    pack_row, unpack_row

KIND_Q4 = 0
KIND_Q2 = 1
KIND_REUSE = 2


@dataclass
class CellCache:
    """Quantized cache of one stored cell for one sequence of T tokens."""
    kind: int
    k_codes: np.ndarray   # uint8 [T, H, D], 0..15 (Q4) or 0..3 (Q2)
    k_scale: np.ndarray   # float16 [NG, H, D], NG = ceil(T / 32)
    k_zero: np.ndarray    # float16 [NG, H, D]
    v_codes: np.ndarray   # uint8 [T, H, D]
    v_scale: np.ndarray   # float16 [T, H, D / 32]
    v_zero: np.ndarray    # float16 [T, H, D / 32]

    @property
    def T(self) -> int:
        return self.k_codes.shape[0]


def kind_bits(kind: int) -> int:
    if kind == KIND_Q4:
        return 4
    if kind == KIND_Q2:
        return 2
    raise ValueError("only stored cells (4-bit or 2-bit) have a cache")


def build_cell_cache(k_bits: np.ndarray, v_bits: np.ndarray, kind: int) -> CellCache:
    """Quantize one sequence's bf16 keys/values [T, H, D] into a cell cache."""
    bits = kind_bits(kind)
    K = bf16_bits_to_f32(k_bits)
    V = bf16_bits_to_f32(v_bits)
    T, H, D = K.shape
    if D % GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    ng = -(-T // GROUP)
    k_codes = np.zeros((T, H, D), np.uint8)
    k_scale = np.zeros((ng, H, D), np.float16)
    k_zero = np.zeros((ng, H, D), np.float16)
    for g in range(ng):
        lo, hi = g * GROUP, min(T, (g + 1) * GROUP)
        c, s, z = quantize(K[lo:hi], bits, axis=0)
        k_codes[lo:hi] = c
        k_scale[g] = s
        k_zero[g] = z
    Vg = V.reshape(T, H, D // GROUP, GROUP)
    vc, vs, vz = quantize(Vg, bits, axis=-1)
    return CellCache(kind, k_codes, k_scale, k_zero,
                     vc.reshape(T, H, D), vs, vz)


# ----------------------------------------------------------------------------
# paged byte layout
# ----------------------------------------------------------------------------

def head_block_regions(kind: int, P: int, D: int) -> dict:
    """Byte offset of every region inside one head-block, plus its size HB."""
    row = D // 4
    vmeta = P * (D // GROUP) * 4
    kslots = max(1, P // GROUP)
    kmeta = kslots * D * 4
    if kind == KIND_Q4:
        r = {"k_hi": 0, "k_lo": P * row, "v_hi": 2 * P * row, "v_lo": 3 * P * row}
        off = 4 * P * row
    elif kind == KIND_Q2:
        r = {"k": 0, "v": P * row}
        off = 2 * P * row
    else:
        raise ValueError("reuse cells own no pages")
    r["v_meta"] = off
    r["k_meta"] = off + vmeta
    r["HB"] = off + vmeta + kmeta
    r["row"] = row
    r["kslots"] = kslots
    return r


def key_meta_place(g: int, P: int):
    """(logical page, slot) holding key group g's metadata."""
    first = g * GROUP
    return first // P, (first % P) // GROUP


def _f16_bytes(a: np.ndarray) -> np.ndarray:
    """float16 array [..., n] -> little-endian bytes [..., 2n]."""
    a = np.ascontiguousarray(a.astype("<f2"))
    return a.view(np.uint8).reshape(a.shape[:-1] + (a.shape[-1] * 2,))


def pack_pool(cache: CellCache, P: int, block_row, num_pages: int):
    """Write a sequence's cache into a fresh head-major pool.

    Returns (pool uint8 [H, num_pages, HB], defined bool of the same shape).
    ``block_row[lp]`` is the physical page of logical page lp.
    """
    T, H, D = cache.k_codes.shape
    reg = head_block_regions(cache.kind, P, D)
    HB, row = reg["HB"], reg["row"]
    pool = np.zeros((H, num_pages, HB), np.uint8)
    defined = np.zeros((H, num_pages, HB), bool)
    block_row = np.asarray(block_row, dtype=np.int64)

    def put(offset_in_block: np.ndarray, phys: np.ndarray, data: np.ndarray):
        # data [T', H, n] placed at block (h, phys[t]) offset offset_in_block[t] + k
        n = data.shape[-1]
        hh = np.arange(H)[None, :, None]
        pp = phys[:, None, None]
        oo = offset_in_block[:, None, None] + np.arange(n)[None, None, :]
        pool[hh, pp, oo] = data
        defined[hh, pp, oo] = True

    t = np.arange(T)
    phys = block_row[t // P]
    r_in = t % P
    if cache.kind == KIND_Q4:
        khi, klo = split_planes(cache.k_codes)
        vhi, vlo = split_planes(cache.v_codes)
        planes = [("k_hi", khi), ("k_lo", klo), ("v_hi", vhi), ("v_lo", vlo)]
    else:
        planes = [("k", cache.k_codes), ("v", cache.v_codes)]
    for name, codes in planes:
        put(reg[name] + r_in * row, phys, pack_row(codes))
    # value metadata: per token, per channel group j: scale, zero
    nj = D // GROUP
    sz = np.stack([cache.v_scale, cache.v_zero], axis=-1).reshape(T, H, 2 * nj)
    put(reg["v_meta"] + r_in * (nj * 4), phys, _f16_bytes(sz))
    # key metadata: one slot per key group
    ng = cache.k_scale.shape[0]
    g = np.arange(ng)
    lp, slot = key_meta_place(g, P)
    kd = np.concatenate([cache.k_scale, cache.k_zero], axis=-1)  # [NG, H, 2D]
    put(reg["k_meta"] + slot * (4 * D), block_row[lp], _f16_bytes(kd))
    return pool, defined


def _read_f16(block: np.ndarray, off, n: int) -> np.ndarray:
    raw = block[..., off:off + 2 * n]
    return np.ascontiguousarray(raw).view("<f2").astype(np.float16)


def unpack_pool(pool: np.ndarray, kind: int, P: int, block_row, T: int) -> CellCache:
    """Read a sequence's cache back from a head-major pool [H, pages, HB]."""
    H, _, HB = pool.shape
    # recover D from HB: HB is linear in D for fixed kind and P
    probe = head_block_regions(kind, P, 32)["HB"]
    D = 32 * HB // probe
    reg = head_block_regions(kind, P, D)
    if reg["HB"] != HB:
        raise ValueError("pool block size does not match kind / page size")
    row = reg["row"]
    block_row = np.asarray(block_row, dtype=np.int64)
    t = np.arange(T)
    phys = block_row[t // P]
    r_in = t % P

    def rows(name):
        out = np.zeros((T, H, row), np.uint8)
        for tt in range(T):
            o = reg[name] + r_in[tt] * row
            out[tt] = pool[:, phys[tt], o:o + row]
        return unpack_row(out)

    if kind == KIND_Q4:
        kc = join_planes(rows("k_hi"), rows("k_lo"))
        vc = join_planes(rows("v_hi"), rows("v_lo"))
    else:
        kc, vc = rows("k"), rows("v")
    nj = D // GROUP
    vs = np.zeros((T, H, nj), np.float16)
    vz = np.zeros((T, H, nj), np.float16)
    for tt in range(T):
        o = reg["v_meta"] + r_in[tt] * nj * 4
        sz = _read_f16(pool[:, phys[tt]], o, 2 * nj).reshape(H, nj, 2)
        vs[tt], vz[tt] = sz[..., 0], sz[..., 1]
    ng = -(-T // GROUP)
    ks = np.zeros((ng, H, D), np.float16)
    kz = np.zeros((ng, H, D), np.float16)
    for g in range(ng):
        lp, slot = key_meta_place(g, P)
        o = reg["k_meta"] + slot * 4 * D
        kd = _read_f16(pool[:, block_row[lp]], o, 2 * D)
        ks[g], kz[g] = kd[:, :D], kd[:, D:]
    return CellCache(kind, kc, ks, kz, vc, vs, vz)
