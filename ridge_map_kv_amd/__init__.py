"""RidgeFill upper-layer KV fill, calibration and ridge solve for MI355X (gfx950).

The compute lives in the HIP library libridgefill.so (C ABI, include/ridgefill.h); the
module `ridge_map_kv_amd.binding` marshals torch tensors to it.  Importing this package
does not load the library; `binding.lib()` does, and raises if it is missing.
"""

__all__ = ["configs", "synth", "binding"]
