"""MI355X-native raw-token hashed n-gram embedding (hash, gather, scatter-add).

The compute path is the C-ABI library ``libengram.so`` built from ``csrc/``
(HIP kernels for gfx950).  ``gram_hashed_embedding_amd.engram`` is the thin
ctypes binding over it; importing that module loads the library and raises
if it is missing.  ``gram_hashed_embedding_amd.workloads`` draws the seeded
synthetic inputs and needs neither the library nor a GPU.
"""

__all__ = ["engram", "workloads"]
