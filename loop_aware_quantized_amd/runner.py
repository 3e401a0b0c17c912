"""Cache state of one workload on the GPU, driven through the C ABI.

Owns device memory (torch tensors: pools, staging, page tables, lengths,
workspace, queries, outputs) and calls loopkv_append / loopkv_decode.  All
quantization and attention work happens in libloopkv.so.
"""
from __future__ import annotations

import numpy as np

from . import abi
from . import inputs as wl


class CacheState:
    """Pools of every stored cell of a workload, plus batch metadata."""

    def __init__(self, w: wl.Workload, device, kinds=None, taus=None, extra_tokens: int = 0,
                 lengths=None, only_cells=None):
        """only_cells: allocate pools for these stored (loop, layer) cells only
        (decoding a cell whose source has no pool is then an error)."""
        import torch
        self.w = w
        self.device = device
        if kinds is None or taus is None:
            kinds, taus = wl.make_plan(w)
        self.kinds = np.asarray(kinds)
        self.taus = np.asarray(taus, np.float64)
        self.plan = abi.Plan(abi.plan_blob(w.loops, w.layers, w.heads, w.head_dim, w.page,
                                           self.kinds, self.taus))
        self.lens0 = (wl.make_lengths(w) if lengths is None
                      else np.asarray(lengths, np.int32))     # lengths after prefill
        self.capacity = self.lens0.astype(np.int64) + extra_tokens
        table, num_pages = wl.make_block_tables(w, self.capacity)
        self.table_np = table
        self.num_pages = num_pages
        self.block_tables = torch.from_numpy(table).to(device)
        self.max_seq_len = int(self.capacity.max())
        self.stored = [(r, l) for r in range(w.loops) for l in range(w.layers)
                       if self.kinds[r, l] != wl.KIND_REUSE
                       and (only_cells is None or (r, l) in only_cells)]
        self.pools, self.staging = {}, {}
        mems = {}
        for (r, l) in self.stored:
            self.pools[(r, l)] = torch.empty(self.plan.pool_bytes(r, l, num_pages),
                                             dtype=torch.uint8, device=device)
            self.staging[(r, l)] = torch.empty(self.plan.staging_bytes(r, l, w.batch),
                                               dtype=torch.uint8, device=device)
            mems[(r, l)] = (self.pools[(r, l)], self.staging[(r, l)], num_pages, w.batch)
        self.cells = abi.cell_array(self.plan, mems)
        self.workspace = torch.empty(self.plan.decode_workspace_bytes(w.batch, self.max_seq_len),
                                     dtype=torch.uint8, device=device)
        self.lens = torch.from_numpy(self.lens0.astype(np.int32)).to(device)
        self.slots = torch.arange(w.batch, dtype=torch.int32, device=device)
        self._zero = torch.zeros(1, dtype=torch.int32, device=device)

    # --------------------------------------------------------------- prefill
    def cell_index(self, r: int, l: int) -> int:
        return r * self.w.layers + l

    def prefill_cell(self, r: int, l: int, keep_host=None):
        """Draw and append the prefill tokens of stored cell (r, l).

        ``keep_host``: optional set of sequence indices whose bf16 keys and
        values are returned as host bit arrays {b: (k_bits, v_bits)}.
        """
        import torch
        w = self.w
        cell = self.cell_index(r, l)
        kept = {}
        if np.all(self.lens0 == 0):
            return kept                      # nothing to store
        if np.all(self.lens0 == self.lens0[0]):
            T = int(self.lens0[0])
            K, V = wl.cell_kv(w, cell, T, self.device)
            zeros = torch.zeros(w.batch, dtype=torch.int32, device=self.device)
            batch = abi.make_batch(zeros, self.block_tables, self.max_seq_len)
            abi.loopkv_append(self.plan, self.cells, r, l, batch, T, K, V)
            for b in (keep_host or ()):
                kept[b] = (wl.bf16_bits(K[b]), wl.bf16_bits(V[b]))
            del K, V
        else:
            for b in range(w.batch):
                T = int(self.lens0[b])
                if T == 0:
                    continue
                K, V = wl.cell_kv(w, cell, T, self.device, b, b + 1)
                batch = abi.make_batch(self._zero, self.block_tables[b:b + 1], self.max_seq_len,
                                       slots=self.slots[b:b + 1])
                abi.loopkv_append(self.plan, self.cells, r, l, batch, T, K, V)
                if keep_host and b in keep_host:
                    kept[b] = (wl.bf16_bits(K[0]), wl.bf16_bits(V[0]))
                del K, V
        return kept

    def prefill(self, keep=None):
        """Prefill every stored cell.  keep: {(r, l): set(b)} of host copies."""
        kept = {}
        for (r, l) in self.stored:
            want = (keep or {}).get((r, l))
            kept[(r, l)] = self.prefill_cell(r, l, want)
        return kept

    # ---------------------------------------------------------------- decode
    def batch(self, lens=None, max_seq_len=None, sum_seq_lens: int = 0):
        return abi.make_batch(self.lens if lens is None else lens, self.block_tables,
                              self.max_seq_len if max_seq_len is None else max_seq_len,
                              sum_seq_lens=sum_seq_lens)

    def new_mask(self):
        import torch
        words = (self.max_seq_len + 31) // 32
        return torch.zeros(self.w.batch, self.w.heads, words, dtype=torch.int32, device=self.device)

    def decode(self, r: int, l: int, q, out, num_splits: int = 0, mask=None, counters=None,
               lens=None, sm_scale: float = 1.0, sum_seq_lens: int | None = None):
        """Decode cell (r, l).  sum_seq_lens is the host-side length hint; by
        default the prefill lengths' sum when lens is None, else 0 (unknown)."""
        opts = abi.make_opts(self.workspace, sm_scale=sm_scale, num_splits=num_splits,
                             mask_bits=mask, counters=counters)
        if sum_seq_lens is None:
            sum_seq_lens = int(self.lens0.sum()) if lens is None else 0
        return abi.loopkv_decode(self.plan, self.cells, r, l, self.batch(lens, sum_seq_lens=sum_seq_lens),
                                 q, out, opts)

    def append(self, r: int, l: int, k, v, lens_before):
        batch = abi.make_batch(lens_before, self.block_tables, self.max_seq_len)
        return abi.loopkv_append(self.plan, self.cells, r, l, batch, int(k.shape[1]), k, v)


def required_bytes_per_token_head(kind_src: int, head_dim: int) -> int:
    """Plan-required bytes of one token-head read by the split pass.

    4-bit source: K hi+lo planes (D/2) + K metadata (4 B per 32 channels:
    D/8) + V high plane (D/4) + V metadata (D/8) = D bytes;
    2-bit source: K (D/4) + K meta (D/8) + V (D/4) + V meta (D/8) = 3D/4.
    A flagged token adds its V low-plane row (D/4), counted separately.
    """
    return head_dim if kind_src == wl.KIND_Q4 else (3 * head_dim) // 4


class VqState:
    """Joint-code caches (one per layer) of a LoopVQ-style workload."""

    def __init__(self, w: wl.VqWorkload, device, extra_tokens: int = 0, layers=None, lengths=None):
        import torch
        self.w = w
        self.device = device
        self.dims = abi.vq_dims(w.loops, w.heads, w.head_dim, w.page)
        self.lens0 = np.full(w.batch, w.ctx, np.int32) if lengths is None else np.asarray(lengths, np.int32)
        self.capacity = self.lens0.astype(np.int64) + extra_tokens
        table, num_pages = wl.make_block_tables(w, self.capacity)
        self.table_np = table
        self.num_pages = num_pages
        self.block_tables = torch.from_numpy(table).to(device)
        self.max_seq_len = int(self.capacity.max())
        self.layers = list(range(w.layers)) if layers is None else list(layers)
        self.pools, self.codebooks = {}, {}
        for l in self.layers:
            self.pools[l] = torch.zeros(abi.vq_pool_bytes(self.dims, num_pages), dtype=torch.uint8, device=device)
            self.codebooks[l] = wl.vq_codebooks(w, l, device)
        self.workspace = torch.empty(abi.vq_workspace_bytes(self.dims, w.batch, self.max_seq_len),
                                     dtype=torch.uint8, device=device)
        self.lens = torch.from_numpy(self.lens0.astype(np.int32)).to(device)
        self._zero = torch.zeros(1, dtype=torch.int32, device=device)

    def append(self, l: int, k, v, lens_before, table=None, max_seq_len=None):
        table = self.block_tables if table is None else table
        batch = abi.make_batch(lens_before, table, self.max_seq_len if max_seq_len is None else max_seq_len)
        cbk, cbv = self.codebooks[l]
        return abi.loopkv_vq_append(self.dims, self.pools[l], self.num_pages, cbk, cbv, batch,
                                    int(k.shape[2]), k, v)

    def prefill_layer(self, l: int, keep=None):
        """Code every sequence's prefill tokens, one sequence per call.
        keep: set of sequences whose bf16 (K, V) stay on the host."""
        kept = {}
        for b in range(self.w.batch):
            T = int(self.lens0[b])
            if T == 0:
                continue
            k, v = wl.vq_kv(self.w, l, b, 0, T, self.device)
            self.append(l, k, v, self._zero, table=self.block_tables[b:b + 1])
            if keep and b in keep:
                kept[b] = (wl.bf16_bits(k[:, 0]), wl.bf16_bits(v[:, 0]))    # [R][T][H][D]
        return kept

    def decode(self, l: int, loop: int, q, out, lens=None, sm_scale: float = 1.0):
        batch = abi.make_batch(self.lens if lens is None else lens, self.block_tables, self.max_seq_len)
        cbk, cbv = self.codebooks[l]
        return abi.loopkv_vq_decode(self.dims, self.pools[l], self.num_pages, cbk, cbv, loop, batch, q, out,
                                    self.workspace, sm_scale)

    def pool_indices(self, l: int, b: int, T: int):
        """Host copy of sequence b's (key, value) indices [T][H][D/4] from the pool."""
        import torch
        P, H, G = self.w.page, self.w.heads, self.w.head_dim // 4
        n = -(-T // P)
        pages = torch.from_numpy(self.table_np[b, :n].astype(np.int64)).to(self.device)
        blk = self.pools[l].view(H, self.num_pages, 2 * P * G).index_select(1, pages).cpu().numpy()
        k = blk[:, :, :P * G].reshape(H, n * P, G)[:, :T].transpose(1, 0, 2)
        v = blk[:, :, P * G:].reshape(H, n * P, G)[:, :T].transpose(1, 0, 2)
        # group j of token t is stored at byte j ^ (t mod G) of its row
        pos = np.arange(G)[None, :] ^ (np.arange(T) % G)[:, None]          # [T][G]
        return (np.take_along_axis(k, pos[:, None, :], 2), np.take_along_axis(v, pos[:, None, :], 2))
