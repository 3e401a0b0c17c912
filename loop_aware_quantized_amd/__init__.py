"""LoopKV plan-driven quantized decode attention for MI355X (gfx950).

The work runs in the HIP library ``libloopkv.so`` (C ABI in include/loopkv.h);
``abi`` is its thin ctypes binding, ``inputs`` the seeded synthetic workload
generators, ``runner`` the cache and step state used by tests and the benchmark.
"""
__all__ = ["abi", "inputs", "runner"]
