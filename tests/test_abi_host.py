"""C-ABI library on the host (no GPU): it loads, exports every function that
include/loopkv.h declares, parses and validates plans, answers size queries,
and rejects bad host-visible arguments before launching anything.
"""
import ctypes
import math
import os
import re
import struct

import pytest

from loop_aware_quantized_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loopkv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(abi.LIB_PATH),
                                reason="libloopkv.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(loopkv_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


def test_exports_every_declared_function():
    names = declared_functions()
    assert "loopkv_decode" in names and "loopkv_append" in names and "loopkv_plan_load" in names
    handle = ctypes.CDLL(abi.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert set(names) == set(abi._SIGNATURES), "binding and header disagree"


def test_abi_version():
    assert abi.lib().loopkv_abi_version() == abi.ABI_VERSION == 1


def _blob(R=2, L=2, H=2, D=64, P=16, kinds=None, taus=None, G=32):
    kinds = kinds or [[0, 2], [1, 0]]
    taus = taus or [[0.02] * L for _ in range(R)]
    return abi.plan_blob(R, L, H, D, P, kinds, taus, G=G)


def test_plan_load_and_queries():
    p = abi.Plan(_blob())
    assert (p.R, p.L, p.H, p.D, p.G, p.P) == (2, 2, 2, 64, 32, 16)
    assert p.cell_info(0, 1) == (2, pytest.approx(0.02), 1)   # reuse -> final loop
    assert p.cell_info(1, 0)[0] == 1 and p.cell_info(1, 0)[2] == 1
    # head-block of a 4-bit cell, P=16, D=64: 4 planes * 16 rows * 16 B + 16*2*4 + 64*4
    assert p.head_block_bytes(0, 0) == 4 * 256 + 128 + 256
    assert p.head_block_bytes(1, 0) == 2 * 256 + 128 + 256
    assert p.head_block_bytes(0, 1) == 0
    assert p.pool_bytes(0, 0, 10) == 10 * 2 * 1408
    assert p.staging_bytes(0, 0, 3) == 3 * 2 * 32 * 64 * 2
    assert p.staging_bytes(0, 1, 3) == 0
    assert p.decode_workspace_bytes(4, 1000) > 0
    p.close()


def _load_rc(blob):
    h = ctypes.c_void_p()
    buf = ctypes.create_string_buffer(blob, len(blob))
    rc = abi.lib().loopkv_plan_load(ctypes.cast(buf, ctypes.c_void_p), len(blob), ctypes.byref(h))
    if rc == 0:
        abi.lib().loopkv_plan_free(h)
    return rc, abi.last_error()


@pytest.mark.parametrize("mutate, text", [
    (lambda b: b"XXXX" + b[4:], "magic"),
    (lambda b: b[:4] + struct.pack("<I", 2) + b[8:], "version"),
    (lambda b: b[:20], "shorter"),
    (lambda b: b + b"\0" * 8, "blob size"),
])
def test_plan_rejects_malformed(mutate, text):
    rc, msg = _load_rc(mutate(_blob()))
    assert rc == abi.E_PLAN and text in msg


@pytest.mark.parametrize("kw, text", [
    (dict(kinds=[[0, 0], [2, 0]]), "final loop"),
    (dict(kinds=[[0, 3], [1, 0]]), "unknown kind"),
    (dict(taus=[[math.nan, 0.1], [0.1, 0.1]]), "NaN or negative"),
    (dict(taus=[[-0.1, 0.1], [0.1, 0.1]]), "NaN or negative"),
    (dict(D=96), "head_dim"),
    (dict(P=24), "page size"),
    (dict(G=16), "group size"),
])
def test_plan_rejects_invalid(kw, text):
    rc, msg = _load_rc(_blob(**kw))
    assert rc == abi.E_PLAN and text in msg


def test_plan_accepts_inf_and_zero_tau():
    rc, _ = _load_rc(_blob(taus=[[0.0, math.inf], [math.inf, 0.0]]))
    assert rc == 0


def test_null_arguments():
    assert abi.lib().loopkv_plan_load(None, 0, None) == abi.E_INVAL
    assert abi.lib().loopkv_plan_dims(None, None) == abi.E_INVAL
    assert abi.lib().loopkv_head_block_bytes(None, 0, 0) == 0


class _FakeTensor:
    """Stands in for a device tensor: only its address is used by the binding."""

    def __init__(self, addr, shape=(1,), nbytes=16):
        self.addr, self.shape, self._n = addr, shape, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def test_append_and_decode_reject_bad_host_arguments():
    p = abi.Plan(_blob())
    cells = abi.cell_array(p, {(0, 0): (_FakeTensor(0x1000), _FakeTensor(0x2000), 4, 1),
                                (1, 0): (_FakeTensor(0x3000), _FakeTensor(0x4000), 4, 1),
                                (1, 1): (_FakeTensor(0x5000), _FakeTensor(0x6000), 4, 1)})
    lens = _FakeTensor(0x7000, shape=(1,))
    table = _FakeTensor(0x8000, shape=(1, 4))
    b = abi.make_batch(lens, table, max_seq_len=64)
    k = _FakeTensor(0x9000)
    lib = abi.lib()

    def app(loop, layer, n_new, batch=b, kk=k):
        return lib.loopkv_append(p.handle, ctypes.cast(cells, ctypes.c_void_p), loop, layer,
                                 ctypes.byref(batch), n_new, kk and kk.data_ptr(),
                                 kk and kk.data_ptr(), None)

    assert app(0, 1, 1) == abi.NOOP_REUSE            # reuse cell stores nothing
    assert app(5, 0, 1) == abi.E_INVAL                # no such cell
    assert app(0, 0, 0) == abi.E_INVAL                # n_new < 1
    assert app(0, 0, 1, kk=None) == abi.E_INVAL       # NULL inputs
    big = abi.make_batch(lens, table, max_seq_len=65)  # 4 pages * 16 < 65
    assert app(0, 0, 1, batch=big) == abi.E_INVAL
    assert "max_pages" in abi.last_error()
    two = abi.make_batch(lens, table, max_seq_len=64, batch=2)  # 2 sequences, 1 staging slot
    assert app(0, 0, 1, batch=two) == abi.E_CAPACITY

    out = _FakeTensor(0xA000)
    small_ws = _FakeTensor(0xB000, nbytes=16)

    def dec(loop, layer, opts, batch=b):
        return lib.loopkv_decode(p.handle, ctypes.cast(cells, ctypes.c_void_p), loop, layer,
                                 ctypes.byref(batch), k.data_ptr(), out.data_ptr(),
                                 ctypes.byref(opts), None)

    assert dec(0, 0, abi.make_opts(small_ws)) == abi.E_CAPACITY
    assert "workspace" in abi.last_error()
    assert dec(0, 0, abi.make_opts(small_ws, num_splits=-1)) == abi.E_INVAL
    assert dec(7, 0, abi.make_opts(small_ws)) == abi.E_INVAL
    assert dec(0, 0, abi.make_opts(small_ws), batch=big) == abi.E_INVAL
    # a reuse cell resolves to the final loop's pool of its layer: (1, 1)
    empty = abi.cell_array(p, {(0, 0): (_FakeTensor(0x1000), _FakeTensor(0x2000), 4, 1)})
    rc = lib.loopkv_decode(p.handle, ctypes.cast(empty, ctypes.c_void_p), 0, 1, ctypes.byref(b),
                           k.data_ptr(), out.data_ptr(), ctypes.byref(abi.make_opts(small_ws)), None)
    assert rc == abi.E_INVAL and "source cell pool" in abi.last_error()
    p.close()


def test_batch_limits_alignment_and_scale():
    """Batches above 65535 sequences, misaligned device arrays or outputs and
    a non-finite sm_scale are rejected before anything is launched (the
    addresses below are never dereferenced)."""
    p = abi.Plan(_blob())
    cells = abi.cell_array(p, {(0, 0): (_FakeTensor(0x1000), _FakeTensor(0x2000), 4, 1),
                                (1, 0): (_FakeTensor(0x3000), _FakeTensor(0x4000), 4, 1),
                                (1, 1): (_FakeTensor(0x5000), _FakeTensor(0x6000), 4, 1)})
    lens, table = _FakeTensor(0x7000, shape=(1,)), _FakeTensor(0x8000, shape=(1, 4))
    b = abi.make_batch(lens, table, max_seq_len=64)
    huge = abi.make_batch(lens, table, max_seq_len=64, batch=65536)
    odd_lens = abi.make_batch(_FakeTensor(0x7002, shape=(1,)), table, max_seq_len=64)
    odd_table = abi.make_batch(lens, _FakeTensor(0x8001, shape=(1, 4)), max_seq_len=64)
    lib = abi.lib()
    k = _FakeTensor(0x9000)
    ws = _FakeTensor(0xB000, nbytes=1 << 30)

    def app(batch):
        return lib.loopkv_append(p.handle, ctypes.cast(cells, ctypes.c_void_p), 0, 0, ctypes.byref(batch), 1,
                                 k.data_ptr(), k.data_ptr(), None)

    def dec(batch=b, q=0x9000, out=0xA000, **kw):
        opts = abi.make_opts(ws, **kw)
        return lib.loopkv_decode(p.handle, ctypes.cast(cells, ctypes.c_void_p), 0, 0, ctypes.byref(batch),
                                 q, out, ctypes.byref(opts), None)

    for call in (app, dec):
        assert call(huge) == abi.E_INVAL and "65535" in abi.last_error()
        assert call(odd_lens) == abi.E_INVAL and "4-byte" in abi.last_error()
        assert call(odd_table) == abi.E_INVAL and "4-byte" in abi.last_error()
    assert dec(q=0x9001) == abi.E_INVAL and "aligned" in abi.last_error()
    assert dec(out=0xA002) == abi.E_INVAL and "aligned" in abi.last_error()
    assert dec(mask_bits=_FakeTensor(0xC002)) == abi.E_INVAL
    assert dec(counters=_FakeTensor(0xD004)) == abi.E_INVAL
    assert dec(sm_scale=math.nan) == abi.E_INVAL and "sm_scale" in abi.last_error()
    assert dec(sm_scale=math.inf) == abi.E_INVAL

    d = abi.vq_dims(4, 2, 128, 32)
    vws = abi.vq_workspace_bytes(d, 1, 128)
    vb = abi.make_batch(lens, table, max_seq_len=128)
    vhuge = abi.make_batch(lens, table, max_seq_len=128, batch=65536)

    def vdec(batch=vb, out=0x9000, scale=1.0):
        return lib.loopkv_vq_decode(ctypes.byref(d), 0x1000, 4, 0x2000, 0x3000, 0, ctypes.byref(batch), 0x6000,
                                    out, scale, 0xA000, 1 << 40, None)

    assert vdec(batch=vhuge) == abi.E_INVAL and "65535" in abi.last_error()
    assert vdec(out=0x9002) == abi.E_INVAL
    assert vdec(scale=math.nan) == abi.E_INVAL
    assert lib.loopkv_vq_append(ctypes.byref(d), 0x1000, 4, 0x2000, 0x3000, ctypes.byref(vhuge), 1, 0x4000,
                                0x5000, None) == abi.E_INVAL
    assert vws > 0
    p.close()


def _round_up(x, m):
    return (x + m - 1) // m * m


def test_vq_size_queries():
    """Sizes of the joint-code calls follow their documented layouts."""
    d = abi.vq_dims(4, 16, 128, 32)
    assert abi.vq_codebook_bytes(d) == 4 * 256 * 32 * 4 * 2          # [R][256][D/4][4] fp16
    assert abi.vq_pool_bytes(d, 10) == 16 * 10 * 2 * 32 * 32          # [H][pages]: 2 x P x D/4 bytes
    assert abi.vq_pool_bytes(d, 0) == 0
    # partial records of D + 4 floats, at most one split per 512 tokens
    assert abi.vq_workspace_bytes(d, 3, 1000) == _round_up(3 * 16 * 2 * (128 + 4) * 4, 256)
    assert abi.vq_workspace_bytes(d, 3, 0) == _round_up(3 * 16 * 1 * (128 + 4) * 4, 256)
    d64 = abi.vq_dims(2, 2, 64, 16)
    assert abi.vq_codebook_bytes(d64) == 2 * 256 * 16 * 4 * 2
    for bad in [(1, 16, 128, 32), (5, 16, 128, 32), (4, 0, 128, 32), (4, 1025, 128, 32), (4, 16, 96, 32),
                (4, 16, 128, 8)]:
        bd = abi.vq_dims(*bad)
        assert abi.vq_codebook_bytes(bd) == 0
        assert abi.vq_pool_bytes(bd, 4) == 0
        assert abi.vq_workspace_bytes(bd, 1, 64) == 0
    assert abi.vq_workspace_bytes(d, -1, 64) == 0


def test_vq_calls_reject_bad_host_arguments():
    """Host-visible arguments of loopkv_vq_append / loopkv_vq_decode are
    validated before anything is launched (addresses below are never used)."""
    lib = abi.lib()
    d = abi.vq_dims(4, 2, 128, 32)
    lens = _FakeTensor(0x7000, shape=(1,))
    table = _FakeTensor(0x8000, shape=(1, 4))
    b = abi.make_batch(lens, table, max_seq_len=128)
    big = abi.make_batch(lens, table, max_seq_len=129)        # 4 pages * 32 < 129
    none = abi.make_batch(lens, table, max_seq_len=128, batch=0)

    def app(dims=d, pool=0x1000, cbk=0x2000, cbv=0x3000, batch=b, n_new=1, k=0x4000, v=0x5000):
        return lib.loopkv_vq_append(ctypes.byref(dims), pool, 4, cbk, cbv, ctypes.byref(batch), n_new, k, v, None)

    assert app(dims=abi.vq_dims(5, 2, 128, 32)) == abi.E_INVAL and "loops" in abi.last_error()
    assert app(dims=abi.vq_dims(4, 2, 128, 12)) == abi.E_INVAL and "page" in abi.last_error()
    assert app(n_new=0) == abi.E_INVAL
    assert app(pool=None) == abi.E_INVAL
    assert app(k=0x4004) == abi.E_INVAL and "aligned" in abi.last_error()
    assert app(batch=big) == abi.E_INVAL and "max_pages" in abi.last_error()
    assert app(batch=none) == abi.OK                           # nothing to code

    ws = abi.vq_workspace_bytes(d, 1, 128)

    def dec(loop=0, cbk=0x2000, ws_bytes=ws, batch=b, q=0x6000):
        return lib.loopkv_vq_decode(ctypes.byref(d), 0x1000, 4, cbk, 0x3000, loop, ctypes.byref(batch), q,
                                    0x9000, 1.0, 0xA000, ws_bytes, None)

    assert dec(loop=4) == abi.E_INVAL and "loop" in abi.last_error()
    assert dec(loop=-1) == abi.E_INVAL
    assert dec(cbk=0x2008) == abi.E_INVAL and "16-byte" in abi.last_error()
    assert dec(q=0x6004) == abi.E_INVAL
    assert dec(q=None) == abi.E_INVAL
    assert dec(ws_bytes=ws - 1) == abi.E_CAPACITY and "workspace" in abi.last_error()
    assert dec(batch=big) == abi.E_INVAL
    assert dec(batch=none, ws_bytes=0) == abi.OK               # nothing to decode


def _rup(x, m):
    return (x + m - 1) // m * m


@pytest.mark.parametrize("H,D", [(2, 64), (16, 128)])
def test_decode_splits_fit_the_workspace(H, D):
    """Every split layout (automatic, for uniform and ragged length hints,
    or requested) has whole 64-token tiles, at most 4096 tokens per split
    and, when uniform, no split longer than the longest sequence; it covers
    max_seq_len and fits the workspace loopkv_decode_workspace_bytes
    reserves: per (sequence, head) S partial records of D + 4 floats, S
    candidate counts and S lists of split-length 8-byte entries (streamed
    layouts: one list slot per token of the longest sequence).  Among the cases: 4096 x 16 short ragged
    sequences, where the ragged rule alone would ask for splits 4.5x longer
    than the sequences."""
    p = abi.Plan(_blob(H=H, D=D, kinds=[[0, 2], [1, 0]]))
    checked = 0
    for batch in (1, 7, 64, 512, 4096, 65535):
        for tm in (0, 1, 63, 64, 128, 1000, 4096, 16384, 100000, 600000, 8388608):
            for t_sum in (0, batch * tm // 2, batch * tm):
                for req in (0, 1, 3, 17, 2048):
                    if t_sum >= 2 ** 31:
                        continue
                    try:
                        S, ln = p.decode_splits(batch, tm, t_sum, req)
                    except abi.LoopKVError:
                        # only a requested count can ask for too many splits
                        assert req > 0 and -(-tm // min(4096, _rup(-(-max(tm, 1) // req), 64))) > 2048
                        continue
                    streamed, S2, ln2, waves = abi.loopkv_decode_layout(p, 0, 0, batch, tm, t_sum, req)
                    assert (S2, ln2) == (S, ln)
                    tmax = max(tm, 1)
                    assert ln % 64 == 0 and 64 <= ln <= 4096
                    assert 1 <= S <= 2048 and S * ln >= tmax
                    if streamed:
                        # equal tile ranges over the pairs' tiles end to end: they cover
                        # every tile, and a pair meets at most S of them
                        assert not req and 0 < t_sum < 0.85 * batch * tmax and batch <= 256
                        longest = ln // 64
                        assert longest >= 4 and waves * longest >= H * (-(-t_sum // 64) + batch)
                        assert -(-(-(-tmax // 64)) // longest) + 1 <= S <= -(-tmax // 64)
                        need = batch * H * (S * ((D + 4) * 4 + 4) + _rup(tmax, 64) * 8)
                    else:
                        assert waves == 0 and (S - 1) * ln < tmax and ln <= _rup(tmax, 64)
                        need = batch * H * S * ((D + 4) * 4 + 4 + ln * 8)
                    if req:   # more than requested only where splits would exceed 4096 tokens
                        assert S <= max(req, -(-tmax // 4096))
                    assert p.decode_workspace_bytes(batch, tm) >= need, (batch, tm, t_sum, req, S, ln)
                    checked += 1
    assert checked > 500
    # many short ragged pairs: one split per pair, no longer than the longest sequence
    assert p.decode_splits(4096, 128, 4096 * 80, 0) == (1, 128)
    with pytest.raises(abi.LoopKVError):
        p.decode_splits(-1, 128, 0, 0)
    p.close()


def test_binding_refuses_host_tensors():
    """The binding passes device addresses only: a host torch tensor is
    refused before any call into the library."""
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="device tensor"):
        abi.make_batch(torch.zeros(1, dtype=torch.int32), torch.zeros(1, 4, dtype=torch.int32), max_seq_len=64)


def test_noalloc_decode_sizes_and_host_errors():
    """loopkv_decode_noalloc_bytes is the compact scratch of the chosen split
    layout (partials, counts, and candidate lists only with a tau mask); a
    batch above the fixed scratch, and bad arguments, fail before anything
    touches a device (the addresses below are never dereferenced)."""
    H, D = 16, 128
    p = abi.Plan(abi.plan_blob(2, 2, H, D, 32, [[0, 1], [0, 2 - 2]], [[0.01, 0.01], [math.inf, 0.0]]))
    lib = abi.lib()
    for B, T in ((1, 64), (4, 3000), (8, 4096), (32, 16384)):
        S, ln = p.decode_splits(B, T, 0, 0)
        recs = B * H * S
        base = _round_up(recs * (D + 4) * 4, 256) + _round_up(recs * 4, 256)
        cand = _round_up(recs * ln * 8, 256)
        assert abi.loopkv_decode_noalloc_bytes(p, 0, 0, B, T) == base + cand    # 4-bit, 0 < tau < inf
        assert abi.loopkv_decode_noalloc_bytes(p, 0, 1, B, T) == base           # 2-bit source
        assert abi.loopkv_decode_noalloc_bytes(p, 1, 0, B, T) == base           # tau = +inf
        assert abi.loopkv_decode_noalloc_bytes(p, 1, 1, B, T) == base           # tau = 0
    assert abi.loopkv_decode_noalloc_bytes(p, 0, 7, 1, 64) == 0
    assert abi.loopkv_decode_noalloc_bytes(p, 0, 0, -1, 64) == 0
    assert abi.NOALLOC_SCRATCH_BYTES == 32 << 20
    assert abi.loopkv_decode_noalloc_bytes(p, 0, 0, 32, 16384) > abi.NOALLOC_SCRATCH_BYTES

    pages = 32 * 16384 // 32
    cells = abi.cell_array(p, {c: (_FakeTensor(0x100000 * (i + 1)), _FakeTensor(0x80000000 + 0x100000 * i),
                                   pages, 32) for i, c in enumerate([(0, 0), (0, 1), (1, 0), (1, 1)])})
    lens = _FakeTensor(0x7000, shape=(32,))
    table = _FakeTensor(0x8000, shape=(32, 512))

    def dec(loop, layer, B=32, T=16384, **kw):
        b = abi.make_batch(lens, table, max_seq_len=T, batch=B)
        return lib.loopkv_decode_noalloc(p.handle, ctypes.cast(cells, ctypes.c_void_p), loop, layer,
                                         ctypes.byref(b), 0x9000, 0xA000, ctypes.byref(abi.make_opts(None, **kw)),
                                         None)

    assert dec(0, 0) == abi.E_CAPACITY and "scratch" in abi.last_error()
    assert dec(0, 0, B=0) == abi.OK
    assert dec(0, 9) == abi.E_INVAL
    assert dec(0, 0, num_splits=-1) == abi.E_INVAL
    assert dec(0, 0, sm_scale=math.nan) == abi.E_INVAL
    p.close()
