"""QVG (Quant VideoGen) KV-cache compress/decompress for MI355X (gfx950).

The compute path is the HIP library ``libqvg.so`` behind the C ABI declared in
``include/qvg.h``; ``means_residual_compression_amd.qvg`` is its thin ctypes
binding.  ``synth`` holds the seeded input generators.  Importing this package
loads nothing; the binding loads the library on first use and raises if it is
missing.
"""
