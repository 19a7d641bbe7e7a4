"""GQA/MQA attention over a paged KV cache for MI355X (gfx950).

The compute lives in ``libgqa_paged.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/gqa_paged.h``).  ``ops`` is a thin ctypes binding
over it; ``workloads`` builds seeded synthetic batches.  Importing the package
loads nothing: ``ops`` loads the library on first use and raises if it is
missing.
"""
