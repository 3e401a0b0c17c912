"""CPU oracle for the LoopKV plan-driven quantized decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library under ``loop_aware_quantized_amd``;
both sides receive the same seeded inputs and nothing else.

What it follows (pages cited by title and section; no line numbers):

* "LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers",
  abstract (概要 on the mlinfo page, "Full text" on the astralor page):
  every (loop, layer) cell has its own KV cache; a plan fixed ahead of time
  keeps a cell at 4 bits or at 2 bits, or lets it borrow the last loop's
  cache of the same layer; a decoding loop always uses the upper two bits
  of a 4-bit value and loads the lower two only for tokens whose weight,
  under that loop's own query, is large enough to need them.
* The related-papers list (関連論文リスト) on the fugumt LoopVQ page, KIVI
  entry: tuning-free asymmetric low-bit KV quantization.  Its layout (keys
  per channel over token groups, values per token over channel groups, with
  a float scale and zero point) is the codec shape used here.

Precision: the codec's defining steps are fp32/fp16 operations emulated
exactly with numpy float32/float16, because they define stored bytes; every
step after dequantization is float64.

Modules
-------
codec      group quantizer, bit planes, 2-bit row packing
cache      per-sequence cell cache and its paged byte layout
attention  decode of one cell: scores, softmax, tau mask, output
planner    offline plan search by exhaustive enumeration (small grids)
loopvq     joint vector quantization across loop steps and its decode
           ("LoopVQ: Sub 1-bit KV Cache Quantization for Looped
           Transformers", abstract)

Parity status of every function is listed in each module's header, with
the tests under ``tests/`` that pin it to something other than itself:

codec.quantize / f16 rounding  exhaustive fp16 search, exact nearest grid
                               point (Fractions), half-step bound, goldens
codec planes / row packing     all 16 codes, all 256 bytes, goldens
cache.build_cell_cache         per-group codec equality, pure function of
                               the sequence
cache.pack_pool / layout       hand-placed bytes: 4-bit over 16-token pages,
                               2-bit region order with a later key group's
                               metadata on its own page, the second metadata
                               slot of 64-token pages; round trips
attention.decode               SDPA (float64) at tau = 0 and +inf and for
                               2-bit cells, bucket-mean midpoint, mask size
                               and nesting, 50-digit mpmath brute force
attention.ambiguity_band       closed-form inside/outside cases
planner                        hand-computed one-layer cases, closed forms
loopvq                         planted codeword, lossless codebook, SDPA

End-to-end values at the workloads' real shapes are pinned only through
these parts: the pages print no values.
"""
