"""HySparse2 hybrid-block decode and KV-Bridging on MI355X (gfx950).

The compute path is ``libhs2.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/hs2.h``).  ``long_context_kv_hs2_amd.hs2`` is the thin
ctypes binding: it marshals torch tensors' device pointers and the current
stream into the C calls and does no arithmetic of its own.  Importing the
package does not load the library; the first call into ``hs2`` does, and
raises if the library is missing.
"""

__all__ = ["hs2", "inputs"]
