"""MI355X-native sparse decode attention: 4-bit key scan, top-k, sparse attention.

The compute path is the HIP library ``libbsa.so`` (sources in ``csrc/``), reached
through the ctypes binding in :mod:`block_sparse_attention_pack_amd.binding`.
Importing this package loads nothing; the binding loads the library on first use
and raises if it is missing.
"""

__all__ = ["binding", "workloads"]
