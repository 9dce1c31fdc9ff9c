"""Batch-1 dense-decoder decode on one AMD MI355X (gfx950).

The compute path is the HIP library `libdecmono.so` (C ABI in include/dec.h);
`binding` marshals arguments to it with ctypes.  Importing this package loads
nothing; `binding.load()` loads the library and raises if it is missing.
"""
__all__ = ["binding", "roofline", "weights_file"]
