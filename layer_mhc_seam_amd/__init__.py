"""MI355X-native fused, delayed mHC seam.

The product is ``libmhc_seam.so`` (HIP for gfx950 behind the C ABI declared in
``include/mhc_seam.h``); ``layer_mhc_seam_amd.seam`` is its thin ctypes
binding.  Importing this package loads nothing; the binding loads the library
on first use and raises if it is missing.
"""
