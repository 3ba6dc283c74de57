"""CPU oracle for the sparse decode-attention step (test infrastructure only).

Plain, slow NumPy code in float64 (float32 only where the storage format fixes
a float32 step) that states what the decode step computes, one function per
step, each citing the page passage it follows:

* :mod:`oracle.nvfp4`  -- E2M1 / E4M3 codecs of the NVFP4 key copy
* :mod:`oracle.decode` -- pack, block/token scan, top-k selection, sparse
  attention with split partials, log-sum-exp combine

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library
and imports nothing from it; the product path never calls it.
"""
