"""ctypes binding of include/loopkv.h (argument marshalling only).

Every computation runs in libloopkv.so's HIP kernels.  torch is used only to
hand device pointers and the current HIP stream to the library.  If the
library is not built, loading fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import struct
from ctypes import c_float, c_int, c_int32, c_int64, c_size_t, c_void_p, c_char_p, POINTER

# the in-tree build; LOOPKV_LIB names another build of the same library
# (e.g. one with host sanitizers) to load instead
LIB_PATH = os.environ.get("LOOPKV_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libloopkv.so")

OK = 0
NOOP_REUSE = 1
E_INVAL = -1
E_PLAN = -2
E_CAPACITY = -3
E_HIP = -4

CELL_Q4 = 0
CELL_Q2 = 1
CELL_REUSE = 2

ABI_VERSION = 1

# exported function -> (restype, argtypes)
_SIGNATURES = {
    "loopkv_abi_version": (c_int, []),
    "loopkv_last_error": (c_char_p, []),
    "loopkv_plan_load": (c_int, [c_void_p, c_size_t, POINTER(c_void_p)]),
    "loopkv_plan_free": (None, [c_void_p]),
    "loopkv_plan_dims": (c_int, [c_void_p, POINTER(c_int32)]),
    "loopkv_cell_info": (c_int, [c_void_p, c_int, c_int, POINTER(c_int), POINTER(c_float), POINTER(c_int)]),
    "loopkv_head_block_bytes": (c_size_t, [c_void_p, c_int, c_int]),
    "loopkv_pool_bytes": (c_size_t, [c_void_p, c_int, c_int, c_int64]),
    "loopkv_staging_bytes": (c_size_t, [c_void_p, c_int, c_int, c_int32]),
    "loopkv_decode_workspace_bytes": (c_size_t, [c_void_p, c_int32, c_int32]),
    "loopkv_decode_splits": (c_int, [c_void_p, c_int32, c_int32, c_int32, c_int32, POINTER(c_int32)]),
    "loopkv_append": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "loopkv_decode": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "loopkv_decode_noalloc_bytes": (c_size_t, [c_void_p, c_int, c_int, c_int32, c_int32, c_int32, c_int32]),
    "loopkv_decode_layout": (c_int, [c_void_p, c_int, c_int, c_int32, c_int32, c_int32, c_int32, POINTER(c_int32)]),
    "loopkv_decode_noalloc": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p]),
    "loopkv_profile_enable": (c_int, [c_int]),
    "loopkv_profile_collect": (c_int, [c_int, POINTER(c_int64), POINTER(ctypes.c_double)]),
    "loopkv_read_probe": (c_int, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "loopkv_plan_optimize": (c_int, [c_int32, c_int32, c_void_p, ctypes.c_double, c_int64, c_void_p, c_void_p]),
    "loopkv_vq_codebook_bytes": (c_size_t, [c_void_p]),
    "loopkv_vq_pool_bytes": (c_size_t, [c_void_p, c_int64]),
    "loopkv_vq_workspace_bytes": (c_size_t, [c_void_p, c_int32, c_int32]),
    "loopkv_vq_append": (c_int, [c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                 c_void_p, c_void_p]),
    "loopkv_vq_decode": (c_int, [c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int, c_void_p, c_void_p,
                                 c_void_p, c_float, c_void_p, c_size_t, c_void_p]),
}

KERNEL_SPLIT = 0
KERNEL_MERGE = 1
KERNEL_APPEND = 2


class CellMem(ctypes.Structure):
    """loopkv_cell_mem"""
    _fields_ = [("pool", c_void_p), ("staging", c_void_p), ("num_pages", c_int64),
                ("max_slots", c_int32), ("reserved", c_int32)]


class Batch(ctypes.Structure):
    """loopkv_batch"""
    _fields_ = [("batch", c_int32), ("max_pages", c_int32), ("seq_lens", c_void_p),
                ("slots", c_void_p), ("block_tables", c_void_p), ("max_seq_len", c_int32),
                ("sum_seq_lens", c_int32)]


class DecodeOpts(ctypes.Structure):
    """loopkv_decode_opts"""
    _fields_ = [("sm_scale", c_float), ("num_splits", c_int32), ("workspace", c_void_p),
                ("workspace_bytes", c_size_t), ("mask_bits", c_void_p), ("counters", c_void_p)]


class VqDims(ctypes.Structure):
    """loopkv_vq_dims"""
    _fields_ = [("loops", c_int32), ("heads", c_int32), ("head_dim", c_int32), ("page", c_int32)]


class LoopKVError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"loopkv error {code}: {message}")
        self.code = code
        self.message = message


_lib = None


def lib():
    """Load libloopkv.so once.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m loop_aware_quantized_amd.build`"
                " (the HIP library is required; there is no fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.loopkv_abi_version() != ABI_VERSION:
            raise RuntimeError("libloopkv.so ABI version mismatch")
        _lib = handle
    return _lib


def last_error() -> str:
    return (lib().loopkv_last_error() or b"").decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise LoopKVError(rc, last_error())
    return rc


def _ptr(t) -> int | None:
    """Address of a device tensor, None for None.  Every buffer the library
    takes is device memory, so a host torch tensor is refused here rather
    than handed to a kernel."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", True):
        raise ValueError(f"loopkv: expected a device tensor, got one on {t.device}")
    return t.data_ptr()


def _stream_handle(stream) -> int | None:
    import torch
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ----------------------------------------------------------------------------
# plan blob
# ----------------------------------------------------------------------------

def plan_blob(R: int, L: int, H: int, D: int, P: int, kinds, taus, G: int = 32) -> bytes:
    """Encode a plan: "LKVP", u32 version, i32 R L H D G P, R*L {u8 kind, pad, f32 tau}."""
    out = bytearray(b"LKVP")
    out += struct.pack("<I6i", 1, R, L, H, D, G, P)
    for r in range(R):
        for l in range(L):
            out += struct.pack("<B3xf", int(kinds[r][l]), float(taus[r][l]))
    return bytes(out)


class Plan:
    """Owned handle of a loaded plan (loopkv_plan*)."""

    def __init__(self, blob: bytes):
        h = c_void_p()
        buf = ctypes.create_string_buffer(blob, len(blob))
        _check(lib().loopkv_plan_load(ctypes.cast(buf, c_void_p), len(blob), ctypes.byref(h)))
        self.handle = h
        dims = (c_int32 * 6)()
        _check(lib().loopkv_plan_dims(self.handle, dims))
        self.R, self.L, self.H, self.D, self.G, self.P = list(dims)

    def close(self):
        if self.handle:
            lib().loopkv_plan_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def cell_info(self, loop: int, layer: int):
        k, t, s = c_int(), c_float(), c_int()
        _check(lib().loopkv_cell_info(self.handle, loop, layer, ctypes.byref(k), ctypes.byref(t),
                                      ctypes.byref(s)))
        return k.value, t.value, s.value

    def head_block_bytes(self, loop: int, layer: int) -> int:
        return lib().loopkv_head_block_bytes(self.handle, loop, layer)

    def pool_bytes(self, loop: int, layer: int, num_pages: int) -> int:
        return lib().loopkv_pool_bytes(self.handle, loop, layer, num_pages)

    def staging_bytes(self, loop: int, layer: int, max_slots: int) -> int:
        return lib().loopkv_staging_bytes(self.handle, loop, layer, max_slots)

    def decode_workspace_bytes(self, batch: int, max_seq_len: int) -> int:
        return lib().loopkv_decode_workspace_bytes(self.handle, batch, max_seq_len)

    def decode_splits(self, batch: int, max_seq_len: int, sum_seq_lens: int = 0,
                      num_splits: int = 0) -> tuple[int, int]:
        """(splits per (sequence, head), tokens per split) of loopkv_decode."""
        out = (c_int32 * 2)()
        _check(lib().loopkv_decode_splits(self.handle, batch, max_seq_len, sum_seq_lens, num_splits, out))
        return int(out[0]), int(out[1])


def loopkv_plan_load(blob: bytes) -> Plan:
    return Plan(blob)


def cell_array(plan: Plan, mems: dict):
    """loopkv_cell_mem[R*L] from {(loop, layer): (pool, staging, num_pages, max_slots)}."""
    arr = (CellMem * (plan.R * plan.L))()
    for (r, l), (pool, staging, num_pages, max_slots) in mems.items():
        c = arr[r * plan.L + l]
        c.pool = _ptr(pool)
        c.staging = _ptr(staging)
        c.num_pages = int(num_pages)
        c.max_slots = int(max_slots)
    return arr


def make_batch(seq_lens, block_tables, max_seq_len: int, slots=None, batch: int | None = None,
               max_pages: int | None = None, sum_seq_lens: int = 0) -> Batch:
    """loopkv_batch over int32 device tensors seq_lens [B], block_tables [B][max_pages]."""
    b = Batch()
    b.sum_seq_lens = int(sum_seq_lens) if 0 < sum_seq_lens < 2 ** 31 else 0
    b.batch = int(seq_lens.shape[0] if batch is None else batch)
    b.max_pages = int(block_tables.shape[-1] if max_pages is None else max_pages)
    b.seq_lens = _ptr(seq_lens)
    b.slots = _ptr(slots)
    b.block_tables = _ptr(block_tables)
    b.max_seq_len = int(max_seq_len)
    return b


def make_opts(workspace, sm_scale: float = 1.0, num_splits: int = 0, mask_bits=None,
              counters=None) -> DecodeOpts:
    o = DecodeOpts()
    o.sm_scale = float(sm_scale)
    o.num_splits = int(num_splits)
    o.workspace = _ptr(workspace)
    o.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    o.mask_bits = _ptr(mask_bits)
    o.counters = _ptr(counters)
    return o


def loopkv_append(plan: Plan, cells, loop: int, layer: int, batch: Batch, n_new: int, k, v,
                  stream=None) -> int:
    """Quantize/pack n_new tokens per sequence into cell (loop, layer)."""
    return _check(lib().loopkv_append(plan.handle, ctypes.cast(cells, c_void_p), loop, layer,
                                      ctypes.byref(batch), n_new, _ptr(k), _ptr(v),
                                      _stream_handle(stream)))


def loopkv_decode(plan: Plan, cells, loop: int, layer: int, batch: Batch, q, out,
                  opts: DecodeOpts, stream=None) -> int:
    """One decode step of cell (loop, layer); writes fp32 out [B][H][D]."""
    return _check(lib().loopkv_decode(plan.handle, ctypes.cast(cells, c_void_p), loop, layer,
                                      ctypes.byref(batch), _ptr(q), _ptr(out), ctypes.byref(opts),
                                      _stream_handle(stream)))


def loopkv_decode_layout(plan: Plan, loop: int, layer: int, batch: int, max_seq_len: int, sum_seq_lens: int = 0,
                         num_splits: int = 0):
    """(streamed, records per pair, tokens per split or wave range, waves or 0) of a decode."""
    out = (c_int32 * 4)()
    _check(lib().loopkv_decode_layout(plan.handle, loop, layer, batch, max_seq_len, sum_seq_lens, num_splits, out))
    return tuple(out)


NOALLOC_SCRATCH_BYTES = 32 << 20


def loopkv_decode_noalloc(plan: Plan, cells, loop: int, layer: int, batch: Batch, q, out,
                          opts: DecodeOpts, stream=None) -> int:
    """loopkv_decode on the library's fixed device scratch (opts' workspace ignored)."""
    return _check(lib().loopkv_decode_noalloc(plan.handle, ctypes.cast(cells, c_void_p), loop, layer,
                                              ctypes.byref(batch), _ptr(q), _ptr(out), ctypes.byref(opts),
                                              _stream_handle(stream)))


def loopkv_decode_noalloc_bytes(plan: Plan, loop: int, layer: int, batch: int, max_seq_len: int,
                                sum_seq_lens: int = 0, num_splits: int = 0) -> int:
    """Scratch bytes loopkv_decode_noalloc would use (0 for invalid arguments)."""
    return lib().loopkv_decode_noalloc_bytes(plan.handle, loop, layer, batch, max_seq_len, sum_seq_lens,
                                             num_splits)


def loopkv_profile_enable(on: bool) -> int:
    return _check(lib().loopkv_profile_enable(1 if on else 0))


def loopkv_profile_collect(kernel_class: int):
    """(launches, total_ms) of one kernel class since the last collect."""
    n, ms = c_int64(), ctypes.c_double()
    _check(lib().loopkv_profile_collect(kernel_class, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def loopkv_read_probe(buf, sink=None, stream=None) -> int:
    """Stream-read a device tensor (bandwidth probe)."""
    return _check(lib().loopkv_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                          _stream_handle(stream)))


def loopkv_plan_optimize(damage, damage_budget: float, storage_budget: int):
    """Least-reads plan under damage and storage budgets.

    damage: float64 array [R][L][4] (4-bit, 2-bit, reuse of a 4-bit final
    cell, reuse of a 2-bit final cell).  Returns (kinds int array [R][L],
    (reads, storage, damage) totals); raises LoopKVError (code E_PLAN) when
    no plan meets both budgets.
    """
    import numpy as np
    d = np.ascontiguousarray(damage, dtype=np.float64)
    if d.ndim != 3 or d.shape[2] != 4:
        raise ValueError("damage must be [R][L][4]")
    R, L = d.shape[0], d.shape[1]
    kinds = np.zeros((R, L), np.uint8)
    totals = np.zeros(3, np.float64)
    _check(lib().loopkv_plan_optimize(R, L, d.ctypes.data, float(damage_budget), int(storage_budget),
                                      kinds.ctypes.data, totals.ctypes.data))
    return kinds.astype(np.int64), (int(totals[0]), int(totals[1]), float(totals[2]))


# ----------------------------------------------------------------------------
# joint vector quantization across loop steps
# ----------------------------------------------------------------------------

def vq_dims(loops: int, heads: int, head_dim: int, page: int) -> VqDims:
    return VqDims(loops, heads, head_dim, page)


def vq_codebook_bytes(dims: VqDims) -> int:
    return lib().loopkv_vq_codebook_bytes(ctypes.byref(dims))


def vq_pool_bytes(dims: VqDims, num_pages: int) -> int:
    return lib().loopkv_vq_pool_bytes(ctypes.byref(dims), num_pages)


def vq_workspace_bytes(dims: VqDims, batch: int, max_seq_len: int) -> int:
    return lib().loopkv_vq_workspace_bytes(ctypes.byref(dims), batch, max_seq_len)


def loopkv_vq_append(dims: VqDims, pool, num_pages: int, codebook_k, codebook_v, batch: Batch, n_new: int,
                     k, v, stream=None) -> int:
    """Code n_new tokens of every sequence (k, v: [R][B][n_new][H][D] bf16)."""
    return _check(lib().loopkv_vq_append(ctypes.byref(dims), _ptr(pool), num_pages, _ptr(codebook_k),
                                         _ptr(codebook_v), ctypes.byref(batch), n_new, _ptr(k), _ptr(v),
                                         _stream_handle(stream)))


def loopkv_vq_decode(dims: VqDims, pool, num_pages: int, codebook_k, codebook_v, loop: int, batch: Batch,
                     q, out, workspace, sm_scale: float = 1.0, stream=None) -> int:
    """Decode step of loop `loop` over a layer's joint cache; writes fp32 out [B][H][D]."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _check(lib().loopkv_vq_decode(ctypes.byref(dims), _ptr(pool), num_pages, _ptr(codebook_k),
                                         _ptr(codebook_v), loop, ctypes.byref(batch), _ptr(q), _ptr(out),
                                         float(sm_scale), _ptr(workspace), nbytes, _stream_handle(stream)))
