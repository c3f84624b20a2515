"""libmxattn: MXFP8 microscaled flash attention for AMD MI355X (gfx950).

The compute path is the HIP shared library ``libmxattn.so`` (C ABI declared in
``include/mxattn.h``); this package only marshals arguments to it. Importing the package
does not load the library; the first call does, and raises if it is missing.
"""
