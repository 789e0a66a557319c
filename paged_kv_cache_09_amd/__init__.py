"""PagedAttention decode for AMD MI355X (gfx950): HIP kernels behind a C ABI.

``paged_kv_cache_09_amd.pkv`` is the thin ctypes binding of ``libpkv.so``
(importing it fails loudly if the library is not built).
``paged_kv_cache_09_amd.workloads`` draws the seeded synthetic decode inputs.
"""
