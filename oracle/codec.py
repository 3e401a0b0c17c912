"""Group codec: asymmetric uniform quantizer, bit planes, 2-bit row packing.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources
-------
* LoopKV abstract ("LoopKV: Loop-Aware KV Cache Compression for Serving
  Looped Transformers", 概要): a cell keeps 4-bit or 2-bit codes, and the
  upper pair of bits of a 4-bit code must be readable without its lower
  pair.  Hence the plane split of a 4-bit code c into hi = c >> 2 and
  lo = c & 3, with c = 4*hi + lo.
* fugumt LoopVQ page, related-papers list, KIVI entry: asymmetric low-bit
  KV quantization with a per-group floating scale and zero point.

Readings where the pages are silent:
* zero point z is the group minimum rounded DOWN to fp16, scale s is
  (max - z) / (2^b - 1) computed in fp32 and rounded UP to fp16, so the grid
  z + c*s, c = 0 .. 2^b-1, covers [min, max];
* code = clamp(rint((x - z) / s), 0, 2^b - 1), the subtraction and the
  division in IEEE fp32 (round to nearest even), rint ties to even;
  a group with s == 0 (all values equal and exactly representable) has all
  codes 0;
* dequantized value x^ = c*s + z (in float64 here);
* row packing: a row of D codes is D/4 bytes; bits [2i, 2i+1] of byte k hold
  the code of channel 4k + i (little-endian bit fields).

Pins (tests/test_oracle_codec.py): fp16 directed rounding against a
brute-force search over every finite fp16 value; quantization error at most
half a step; code equal to the exact nearest grid point (Fractions, ties to
even); covering grid; constant and single-value groups lossless; hi/lo
recombination over all 16 codes; pack/unpack round trip over all 256 bytes;
hand-derived fixtures in tests/golden/codec_cases.txt.
"""
from __future__ import annotations

import numpy as np

GROUP = 32  # tokens per key group and channels per value group


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16/int16) -> exact float32 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f16_round_down(x: np.ndarray) -> np.ndarray:
    """Largest float16 value that is <= x (x float32).  Returns float16."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)  # round to nearest even
        back = h.astype(np.float32)
    too_big = back > x
    h = np.where(too_big, np.nextafter(h, np.float16(-np.inf)), h)
    return h.astype(np.float16)


def f16_round_up(x: np.ndarray) -> np.ndarray:
    """Smallest float16 value that is >= x (x float32).  Returns float16."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)
        back = h.astype(np.float32)
    too_small = back < x
    h = np.where(too_small, np.nextafter(h, np.float16(np.inf)), h)
    return h.astype(np.float16)


def levels(bits: int) -> int:
    """Largest code of a b-bit quantizer (3 for 2-bit, 15 for 4-bit)."""
    return (1 << bits) - 1


def quantize(x: np.ndarray, bits: int, axis: int = -1):
    """Quantize float32 values (exact bf16 values) in groups along ``axis``.

    Every slice along ``axis`` is one group.  Returns (codes uint8 with x's
    shape, scale float16, zero float16) where scale/zero have ``axis``
    removed.
    """
    x = np.asarray(x, dtype=np.float32)
    top = np.float32(levels(bits))
    mn = x.min(axis=axis, keepdims=True)
    mx = x.max(axis=axis, keepdims=True)
    z16 = f16_round_down(mn)
    z = z16.astype(np.float32)
    r = (mx - z).astype(np.float32)            # fp32 subtraction
    s32 = (r / top).astype(np.float32)         # fp32 IEEE division
    s16 = f16_round_up(s32)
    s = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = ((x - z).astype(np.float32) / s).astype(np.float32)
        c = np.clip(np.rint(t), 0, top)
    c = np.where(s > 0, c, 0).astype(np.uint8)
    return c, np.squeeze(s16, axis=axis), np.squeeze(z16, axis=axis)


def dequantize(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """x^ = c*s + z in float64 (scale/zero already broadcast to codes)."""
    return (codes.astype(np.float64) * scale.astype(np.float64)
            + zero.astype(np.float64))


def split_planes(codes4: np.ndarray):
    """4-bit codes -> (hi, lo) 2-bit planes: hi = c >> 2, lo = c & 3."""
    c = np.asarray(codes4, dtype=np.uint8)
    return (c >> 2).astype(np.uint8), (c & 3).astype(np.uint8)


def join_planes(hi: np.ndarray, lo: np.ndarray) -> np.ndarray:
    """(hi, lo) 2-bit planes -> 4-bit codes 4*hi + lo."""
    return (hi.astype(np.uint8) * 4 + lo.astype(np.uint8)).astype(np.uint8)


def pack_row(codes2: np.ndarray) -> np.ndarray:
    """2-bit codes [..., D] -> bytes [..., D/4]; channel 4k+i at bits 2i of byte k."""
    c = np.asarray(codes2, dtype=np.uint8)
    d = c.shape[-1]
    if d % 4:
        raise ValueError("row length must be a multiple of 4")
    c4 = c.reshape(c.shape[:-1] + (d // 4, 4)).astype(np.uint32)
    out = c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)
    return out.astype(np.uint8)


def unpack_row(row: np.ndarray) -> np.ndarray:
    """Inverse of pack_row: bytes [..., D/4] -> 2-bit codes [..., D]."""
    b = np.asarray(row, dtype=np.uint8)
    parts = [(b >> (2 * i)) & 3 for i in range(4)]
    out = np.stack(parts, axis=-1)
    return out.reshape(b.shape[:-1] + (b.shape[-1] * 4,)).astype(np.uint8)
